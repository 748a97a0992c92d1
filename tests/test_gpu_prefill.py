"""GPU parity of idx_select_prefill (per-token scores on the matrix cores and
per-token top-K) against the CPU oracle."""
import sys

import numpy as np
import pytest

torch = pytest.importorskip("torch")

import oracle
import synth
from tests.helpers import RTOL, check_ids_band, check_ids_exact, check_scores, to_dev

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)

import block_scoring_top_amd as idx  # noqa: E402


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def run_prefill(x, K=None, sorted_out=None, with_scores=True):
    K = x.K if K is None else K
    srt = x.sorted if sorted_out is None else sorted_out
    ids, counts, s = idx.idx_select_prefill(to_dev(x.q), to_dev(x.c), to_dev(x.pos0), K,
                                            page_size=x.page_size, sorted=srt,
                                            return_scores=with_scores)
    torch.cuda.synchronize()
    return (ids.cpu().numpy(), counts.cpu().numpy(), None if s is None else s.cpu().numpy())


def full_prefill_check(x, K=None, sorted_out=None, exact_scores=False):
    K = x.K if K is None else K
    srt = x.sorted if sorted_out is None else sorted_out
    say(f"[prefill] {x.name} B={x.B} T={x.T} H={x.H} N_pad={x.N_pad} pos0={list(x.pos0)} K={K} "
        f"sorted={srt}")
    ids, counts, s = run_prefill(x, K, srt)
    S, A, NV = oracle.score_prefill(x.q, x.c, x.pos0, x.page_size, x.dtype)
    R = x.B * x.T
    s2, S2, A2, nv2 = s.reshape(R, -1), S.reshape(R, -1), A.reshape(R, -1), NV.reshape(R)
    if exact_scores:
        np.testing.assert_array_equal(s2.astype(np.float64), S2)
    check_scores(s2, S2, A2, RTOL[x.dtype])
    check_ids_exact(ids.reshape(R, K), counts.reshape(R), s2, nv2, K, srt)
    check_ids_band(ids.reshape(R, K), S2, A2, nv2, K, RTOL[x.dtype])
    ids2, counts2, _ = run_prefill(x, K, srt, with_scores=False)
    np.testing.assert_array_equal(ids2, ids)
    np.testing.assert_array_equal(counts2, counts)


@pytest.mark.parametrize("sorted_out", [False, True])
def test_prefill_small_ragged(sorted_out):
    """37 tokens (a ragged token tile), 300 blocks (a ragged column tile), a
    request that starts inside a page and one that starts at 0."""
    x = synth.make_prefill(2, 37, 3, 128, 300, [3000, 0], 20, 700, name="small")
    full_prefill_check(x, sorted_out=sorted_out)


@pytest.mark.parametrize("H", [1, 4, 16])
def test_prefill_integer_inputs_bit_exact(H):
    """Small integers: the head sums are exact in bf16 and every product sum is
    an exact integer in fp32, so the scores equal the oracle's exactly."""
    x = synth.make_prefill(2, 70, H, 128, 200, [1000, 2500], 32, 701 + H, integer=True,
                           name=f"integer_H{H}")
    full_prefill_check(x, exact_scores=True)


def test_prefill_many_tiles_and_blocks_none_visible():
    """Several token and column tiles; column tiles past every token's blocks,
    and a negative start (counts as 0)."""
    x = synth.make_prefill(3, 100, 4, 128, 1100, [-50, 400, 15000], 64, 702, name="tiles")
    full_prefill_check(x)
    full_prefill_check(x, K=700, sorted_out=True)


def test_prefill_k_larger_than_blocks():
    x = synth.make_prefill(1, 40, 2, 128, 64, [10], 100, 703, name="small_k")
    full_prefill_check(x)


def test_prefill_workload_full_size():
    x = synth.workload(7)
    full_prefill_check(x)
    full_prefill_check(x, sorted_out=True)


# ---- a few tokens over few rows: one fused score + select launch per call ----------------
@pytest.mark.parametrize("T", [1, 2, 4, 8])
@pytest.mark.parametrize("sorted_out", [False, True])
def test_prefill_few_tokens(T, sorted_out):
    """The short-prompt route (T <= 8, B*T <= 256): starts at 0, inside a page,
    negative, and past the table (every block visible), ragged table length."""
    x = synth.make_prefill(5, T, 4, 128, 1537, [0, 333, -9, 24570, 30000], 100, 710 + T,
                           name=f"few_T{T}")
    full_prefill_check(x, sorted_out=sorted_out)


@pytest.mark.parametrize("H", [1, 4, 16])
def test_prefill_few_tokens_integer_inputs_bit_exact(H):
    """Small integers on the short-prompt route: every product and head sum is
    an exact integer in fp32, so the scores equal the oracle's exactly."""
    x = synth.make_prefill(3, 4, H, 128, 300, [1000, 2500, 5], 32, 720 + H, integer=True,
                           name=f"few_integer_H{H}")
    full_prefill_check(x, exact_scores=True)


@pytest.mark.parametrize("B,T", [(32, 8), (33, 8), (1, 9), (128, 2), (129, 2)])
def test_prefill_route_boundaries(B, T):
    """Both sides of the short-prompt limits (B*T = 256 fused, 257 or T = 9 not),
    checked against the oracle the same way."""
    rng = np.random.default_rng(730 + B * T)
    x = synth.make_prefill(B, T, 4, 128, 700, rng.integers(-20, 12000, B), 64, 731 + B,
                           name=f"route_B{B}_T{T}")
    full_prefill_check(x, sorted_out=bool(B & 1))


def test_prefill_workspace_shared_by_both_routes():
    """One zero-filled workspace serves short and long prompts in turn (its
    arrival lines sit at a fixed place whatever the call's shape)."""
    shapes = [(20, 8, 900, 37), (3, 70, 900, 200), (64, 4, 500, 256), (2, 40, 1300, 30),
              (64, 4, 500, 256), (1, 1, 1300, 5)]
    nbytes = max(idx.idx_prefill_workspace_bytes(B, T, N, K) for B, T, N, K in shapes)
    ws = torch.zeros(nbytes, dtype=torch.uint8, device="cuda")
    for i, (B, T, N, K) in enumerate(shapes):
        rng = np.random.default_rng(740 + i)
        x = synth.make_prefill(B, T, 4, 128, N, rng.integers(-5, N * 16, B), K, 740 + i)
        say(f"[prefill shared ws] B={B} T={T} N_pad={N} K={K}")
        ids, counts, s = idx.idx_select_prefill(to_dev(x.q), to_dev(x.c), to_dev(x.pos0), K,
                                                sorted=bool(i & 1), return_scores=True, ws=ws)
        torch.cuda.synchronize()
        S, A, NV = oracle.score_prefill(x.q, x.c, x.pos0, x.page_size, x.dtype)
        R = B * T
        s2 = s.cpu().numpy().reshape(R, -1)
        check_scores(s2, S.reshape(R, -1), A.reshape(R, -1), RTOL["bf16"])
        check_ids_exact(ids.cpu().numpy().reshape(R, K), counts.cpu().numpy().reshape(R), s2,
                        NV.reshape(R), K, bool(i & 1))


@pytest.mark.parametrize("page_size", [1, 5, 64])
def test_prefill_few_tokens_page_sizes(page_size):
    x = synth.make_prefill(3, 3, 4, 128, 900, [0, 61, 2 * 900 * page_size], 50, 750 + page_size,
                           page_size=page_size, name=f"few_page{page_size}")
    full_prefill_check(x)


@pytest.mark.parametrize("T", [1, 3, 8])
def test_prefill_few_tokens_f32(T):
    """fp32 inputs, which the short-prompt route takes (fp32 products and sums)."""
    x = synth.make_prefill(4, T, 4, 128, 1100, [0, 97, -3, 20000], 128, 760 + T, dtype="f32",
                           name=f"few_f32_T{T}")
    full_prefill_check(x, sorted_out=T == 3)


def test_prefill_f32_long_prompt_unsupported():
    x = synth.make_prefill(1, 9, 4, 128, 64, [0], 8, 770, dtype="f32")
    with pytest.raises(idx.IdxError):
        run_prefill(x)


@pytest.mark.parametrize("sorted_out", [False, True])
def test_prefill_few_tokens_long_rows(sorted_out):
    """The short-prompt route past the select's register tile (rows of more than
    8192 blocks) with K = 2048, and tokens on both sides of a block boundary."""
    x = synth.make_prefill(2, 3, 4, 128, 20000, [16 * 15000 - 2, 16 * 20000], 2048, 780,
                           name="few_long")
    full_prefill_check(x, sorted_out=sorted_out)
