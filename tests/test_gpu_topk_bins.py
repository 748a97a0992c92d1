"""GPU parity of idx_topk on rows shaped for the linear first pass of the
long-row instances (1024 threads, 8 key slots). That pass takes bins linear in
the score for rows whose mean lies inside their range, bins linear in the
order key for rows of one sign whose mean crowds one end (heavy tails), and
settles a threshold bin too large to gather from its min and max when all its
keys are equal. Rows of 8000 entries run in one workgroup per row; rows of
20000 are cut into segments whose candidates the last workgroup merges.

Ids are checked bit-exactly against the oracle's selection (ties to the lower
index), in index order or in score order.
"""
import sys

import numpy as np
import pytest

torch = pytest.importorskip("torch")

from tests.helpers import check_ids_exact, to_dev

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)

import block_scoring_top_amd as idx  # noqa: E402


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def heavy_rows(rng, n):
    """One row per case, float32."""
    lognormal = rng.lognormal(0.0, 2.0, n)
    zipf = rng.zipf(1.1, n).astype(np.float64)
    with_inf = rng.lognormal(0.0, 2.0, n)
    with_inf[rng.choice(n, 5, replace=False)] = np.inf
    tied = rng.integers(1, 5, n).astype(np.float64)     # four values, three huge outliers:
    tied[rng.choice(n, 3, replace=False)] = 1e6          # key bins, the threshold bin tied
    outlier = np.ones(n)
    outlier[n // 3] = 1e30                               # every other score equal
    neg_with_dead = -rng.lognormal(0.0, 2.0, n)
    neg_with_dead[rng.choice(n, n // 4, replace=False)] = -np.inf
    rows = [lognormal, -lognormal, zipf, -zipf, with_inf, tied, outlier,
            rng.random(n),                               # uniform [0, 1): value bins
            rng.random(n) * 1e-30,                       # tiny positive scores
            neg_with_dead]
    return np.stack(rows).astype(np.float32)


@pytest.mark.parametrize("N,K,sorted_out", [(8000, 256, False), (8000, 2048, True),
                                            (20000, 300, False), (20000, 2048, True),
                                            (20000, 4096, False)])
def test_topk_heavy_tailed_and_tied_rows(N, K, sorted_out):
    rng = np.random.default_rng(430 + N + K)
    s = heavy_rows(rng, N)
    nv = np.full(s.shape[0], N, dtype=np.int64)
    nv[1::4] = rng.integers(K // 2, N, len(nv[1::4]))
    say(f"[topk bins] N={N} K={K} sorted={sorted_out} rows={s.shape[0]}")
    ids, counts = idx.idx_topk(to_dev(s), K, to_dev(nv.astype(np.int32)), sorted_out)
    torch.cuda.synchronize()
    check_ids_exact(ids.cpu().numpy(), counts.cpu().numpy(), s, nv, K, sorted_out)


def few_valued_rows(rng, B, n):
    """Rows of 2, 3, 5 or 8 distinct small-integer values (exact in bf16): the
    split top-K's segments then hand over candidates of two or three values,
    whose linear-bin counts the merge spreads over several histogram copies.
    Values 0, 1, 2 put the candidates in bins 0, 1024 and 2047 (one LDS bank
    in a single copy)."""
    rows = []
    for r in range(B):
        nvals = (2, 3, 5, 8)[r % 4]
        row = rng.integers(0, nvals, n).astype(np.float32)
        if r % 8 >= 4:
            row -= np.float32(nvals // 2)   # values of both signs
        rows.append(row)
    return np.stack(rows)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("K", [1, 300, 2048])
def test_topk_split_few_valued_rows(dtype, K):
    N, B = 30000, 16
    rng = np.random.default_rng(910 + K)
    s = few_valued_rows(rng, B, N)
    nv = np.full(B, N, dtype=np.int64)
    nv[3::5] = rng.integers(K + 1, N, len(nv[3::5]))
    say(f"[topk few values] {dtype} N={N} K={K} rows={B}")
    t = to_dev(s)
    if dtype == "bf16":
        t = t.to(torch.bfloat16)  # small integers: exact
    ids, counts = idx.idx_topk(t, K, to_dev(nv.astype(np.int32)))
    torch.cuda.synchronize()
    check_ids_exact(ids.cpu().numpy(), counts.cpu().numpy(), s, nv, K, False)


@pytest.mark.parametrize("N,B", [(30000, 16), (8000, 8)])
@pytest.mark.parametrize("K", [300, 2048])
def test_topk_score_order_top_value_copies(N, B, K):
    """Score order where the row's top value has K - 1, K, K + 1 or 3K copies
    (and rows of one value): when the copies fill K, every taken key is that
    value and the pairs stand in index order without a sort; with K - 1 copies
    one lower key joins them and the sort runs."""
    rng = np.random.default_rng(977 + N + K)
    rows = []
    for r in range(B):
        c = (K - 1, K, K + 1, 3 * K, N)[r % 5]
        row = (rng.standard_normal(N) - 10.0).astype(np.float32)
        row[rng.choice(N, c, replace=False)] = 5.0
        rows.append(row)
    s = np.stack(rows)
    nv = np.full(B, N, dtype=np.int64)
    nv[2::3] = rng.integers(K + 1, N, len(nv[2::3]))
    say(f"[topk top-value copies] N={N} K={K} rows={B}")
    ids, counts = idx.idx_topk(to_dev(s), K, to_dev(nv.astype(np.int32)), True)
    torch.cuda.synchronize()
    check_ids_exact(ids.cpu().numpy(), counts.cpu().numpy(), s, nv, K, True)
