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
