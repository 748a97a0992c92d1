"""GPU parity of idx_select on score rows shaped to drive each branch of the
select: the linear-bin first pass with a small threshold bin (gathered and
ranked, with ties), threshold bins too large to gather (tied or clustered rows,
an outlier that squeezes every other score into a few bins), rows of one or two
values, and rows of at most K blocks. Each case runs in the three launch shapes
of the fused select (few requests: 1024-thread workgroups; many requests: short
rows in one key slot, longer rows in four).

Centroid rows are copies drawn from a small pool of distinct rows, so equal
rows give bit-identical scores; the ids are checked bit-exactly against the
oracle's selection on the GPU's own scores (ties to the lower id), in index
order or in score order, and the scores against the oracle's float64 scores.
"""
import sys

import numpy as np
import pytest

torch = pytest.importorskip("torch")

import oracle
import synth
from tests.helpers import RTOL, check_ids_exact, check_scores, to_dev

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)

import block_scoring_top_amd as idx  # noqa: E402

# (requests, N_pad): 1024-thread workgroups; 512 threads, one key slot (rows of
# at most 2048 blocks); 512 threads, four key slots (longer rows)
SHAPES = [(4, 8192), (40, 2048), (40, 5000)]
H, D = 4, 128


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def pooled_inputs(B, N_pad, distinct, seed, K, outlier=None, seq_len=None):
    """c[b] rows are copies of `distinct` random rows (exact score ties); an
    outlier row, when given, is scaled so its score dwarfs the others."""
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((B, H, D)).astype(np.float32)
    if distinct >= N_pad:  # every row its own draw
        c = rng.standard_normal((B, N_pad, D)).astype(np.float32)
    else:
        pool = rng.standard_normal((B, distinct, D)).astype(np.float32)
        pick = rng.integers(0, distinct, (B, N_pad))
        c = np.take_along_axis(pool, pick[:, :, None], axis=1)
    if outlier is not None:
        c[:, 7, :] = np.sign(q.sum(axis=1)) * outlier  # score ~ outlier * sum |q_bar|
    if seq_len is None:
        seq_len = np.full(B, N_pad * synth.PAGE_SIZE, dtype=np.int64)
        seq_len[1::3] = rng.integers(1, N_pad * synth.PAGE_SIZE, len(seq_len[1::3]))
    return synth.IndexerInputs(q=synth.f32_to_bf16_bits(q), c=synth.f32_to_bf16_bits(c),
                               seq_len=np.asarray(seq_len, dtype=np.int32),
                               page_size=synth.PAGE_SIZE, K=K, sorted=False, dtype="bf16",
                               name="pooled")


def check(x, K, sorted_out):
    q, c, sl = to_dev(x.q), to_dev(x.c), to_dev(x.seq_len)
    ids, counts, s = idx.idx_select(q, c, sl, K, sorted=sorted_out, return_scores=True)
    torch.cuda.synchronize()
    ids, counts, s = ids.cpu().numpy(), counts.cpu().numpy(), s.cpu().numpy()
    S, A = oracle.score(x.q, x.c, x.seq_len, x.page_size, x.dtype)
    nv = oracle.n_valid(x.seq_len, x.page_size, x.N_pad)
    check_scores(s, S, A, RTOL[x.dtype])
    check_ids_exact(ids, counts, s, nv, K, sorted_out)
    ids2, counts2, _ = idx.idx_select(q, c, sl, K, sorted=sorted_out)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(ids2.cpu().numpy(), ids)
    np.testing.assert_array_equal(counts2.cpu().numpy(), counts)


@pytest.mark.parametrize("B,N_pad", SHAPES)
@pytest.mark.parametrize("sorted_out", [False, True])
@pytest.mark.parametrize("distinct", [4000, 300, 40])
def test_select_ties(B, N_pad, sorted_out, distinct):
    """Many distinct rows: small threshold bins (gathered). 300 rows: ~7-27
    copies of each score, the threshold bin gathered with ties. 40 rows: more
    copies than the gather takes, the radix passes resolve."""
    x = pooled_inputs(B, N_pad, distinct, 900 + distinct + N_pad, 256)
    say(f"[select paths] ties B={B} N_pad={N_pad} distinct={distinct} sorted={sorted_out}")
    check(x, 256, sorted_out)


@pytest.mark.parametrize("B,N_pad", SHAPES)
@pytest.mark.parametrize("scale", [30.0, 3e4])
@pytest.mark.parametrize("sorted_out", [False, True])
def test_select_outlier(B, N_pad, scale, sorted_out):
    """One block scores far above the rest: the linear bins squeeze the other
    scores into a few bins (at 3e4, every other score shares the lowest bins)."""
    x = pooled_inputs(B, N_pad, 100000, 950 + N_pad, 256, outlier=scale)
    say(f"[select paths] outlier B={B} N_pad={N_pad} scale={scale} sorted={sorted_out}")
    check(x, 256, sorted_out)


@pytest.mark.parametrize("B,N_pad", SHAPES)
@pytest.mark.parametrize("distinct", [1, 2])
@pytest.mark.parametrize("sorted_out", [False, True])
def test_select_one_or_two_values(B, N_pad, distinct, sorted_out):
    """Every block the same row (one score per request: no linear range), or two rows."""
    x = pooled_inputs(B, N_pad, distinct, 970 + distinct + N_pad, 100)
    say(f"[select paths] {distinct} value(s) B={B} N_pad={N_pad} sorted={sorted_out}")
    check(x, 100, sorted_out)


@pytest.mark.parametrize("B,N_pad", SHAPES)
@pytest.mark.parametrize("sorted_out", [False, True])
def test_select_rows_within_k(B, N_pad, sorted_out):
    """Requests of at most K blocks take every block; longer ones select."""
    rng = np.random.default_rng(990 + N_pad)
    seq_len = rng.integers(1, 300 * synth.PAGE_SIZE, B)
    seq_len[0] = N_pad * synth.PAGE_SIZE
    x = pooled_inputs(B, N_pad, 100000, 991 + N_pad, 256, seq_len=seq_len)
    say(f"[select paths] rows within K B={B} N_pad={N_pad} sorted={sorted_out}")
    check(x, 256, sorted_out)
