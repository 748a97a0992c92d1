"""GPU parity of idx_select_paged (a paged centroid pool) against the CPU oracle.

Covers the page-count regimes and batch sizes of the centroid-scorer sweep,
page lists that share pool rows, invalid list entries, empty and clamped
requests, and the reduction to the dense call when the lists are identities.
"""
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


def run_paged(x, K=None, sorted_out=None, with_scores=True, indptr=None, indices=None,
              max_pages=None):
    K = x.K if K is None else K
    srt = x.sorted if sorted_out is None else sorted_out
    indptr = x.indptr if indptr is None else indptr
    indices = x.indices if indices is None else indices
    mp = x.max_pages if max_pages is None else max_pages
    ids, counts, s = idx.idx_select_paged(
        to_dev(x.q), to_dev(x.c_pool), to_dev(np.asarray(indptr, np.int32)),
        to_dev(np.asarray(indices, np.int32)), K, mp, sorted=srt, return_scores=with_scores)
    torch.cuda.synchronize()
    return (ids.cpu().numpy(), counts.cpu().numpy(),
            None if s is None else s.cpu().numpy())


def full_paged_check(x, K=None, sorted_out=None, indptr=None, indices=None, max_pages=None):
    K = x.K if K is None else K
    srt = x.sorted if sorted_out is None else sorted_out
    indptr = x.indptr if indptr is None else indptr
    indices = x.indices if indices is None else indices
    mp = x.max_pages if max_pages is None else max_pages
    say(f"[paged] {x.name} B={x.B} H={x.H} pool={x.c_pool.shape[0]} max_pages={mp} K={K} "
        f"sorted={srt} dtype={x.dtype}")
    ids, counts, s = run_paged(x, K, srt, True, indptr, indices, mp)
    S, A, n_slots = oracle.score_paged(x.q, x.c_pool, indptr, indices, mp, x.dtype)
    check_scores(s, S, A, RTOL[x.dtype])
    check_ids_exact(ids, counts, s, n_slots, K, srt)
    check_ids_band(ids, S, A, n_slots, K, RTOL[x.dtype])
    ids2, counts2, _ = run_paged(x, K, srt, False, indptr, indices, mp)
    np.testing.assert_array_equal(ids2, ids)
    np.testing.assert_array_equal(counts2, counts)
    return ids, counts, s


@pytest.mark.parametrize("regime", range(len(synth.PAGE_REGIMES)))
@pytest.mark.parametrize("B", synth.PAGED_BATCHES)
def test_paged_sweep(regime, B):
    """The scorer sweep: five page-count regimes x five batch sizes, pool of 16384."""
    x = synth.make_paged(B, 4, 128, synth.POOL_BLOCKS, synth.PAGE_REGIMES[regime], 256, "bf16",
                         600 + 10 * regime + B, name=f"sweep_r{regime}_b{B}")
    full_paged_check(x)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("sorted_out", [False, True])
def test_paged_small_ragged(dtype, sorted_out):
    x = synth.make_paged(5, 3, 128, 700, [1, 333, 0, 700, 65], 50, dtype, 610, name="small")
    full_paged_check(x, sorted_out=sorted_out)


def test_paged_many_requests_and_sorted_large_K():
    rng = np.random.default_rng(611)
    x = synth.make_paged(40, 4, 128, 5000, list(rng.integers(0, 3000, 40)), 1500, "bf16", 611,
                         name="many")
    full_paged_check(x)
    full_paged_check(x, sorted_out=True)


def test_paged_invalid_entries_are_not_candidates():
    x = synth.make_paged(3, 4, 128, 900, [400, 400, 400], 64, "bf16", 612, name="invalid")
    indices = x.indices.copy()
    indices[5] = -1          # below the pool
    indices[400 + 7] = 900   # past the pool
    indices[800 + 9] = 1 << 30
    ids, counts, s = full_paged_check(x, indices=indices)
    assert s[0, 5] == -np.inf and s[1, 7] == -np.inf and s[2, 9] == -np.inf
    assert 5 not in ids[0] and 7 not in ids[1] and 9 not in ids[2]


def test_paged_lists_past_the_index_array_and_clamped_counts():
    x = synth.make_paged(4, 4, 128, 800, [100, 100, 100, 100], 30, "bf16", 613, name="clamp")
    indptr = np.array([0, 100, 100, 350, 420], np.int32)   # request 2 runs past the 400 entries
    # request 1 is empty; request 2 (250 slots) is clamped to max_pages = 200
    full_paged_check(x, indptr=indptr, max_pages=200)


@pytest.mark.parametrize("chunk_log2", [10, 12])
def test_paged_large_chunks_stage_their_lists_in_pieces(chunk_log2):
    """Chunks of 1024 and 4096 slots stage their page lists 256 entries at a
    time: the same ids and scores as the default chunking, and the oracle's,
    with invalid entries among the staged ones."""
    x = synth.make_paged(3, 4, 128, 5000, [4500, 3000, 1300], 200, "bf16", 615, name="chunks")
    indices = x.indices.copy()
    indices[300] = -1
    indices[4500 + 2999] = 5000
    mp = x.max_pages
    say(f"[paged] large chunks 2^{chunk_log2}")
    args = (to_dev(x.q), to_dev(x.c_pool), to_dev(x.indptr.astype(np.int32)),
            to_dev(indices.astype(np.int32)), 200, mp)
    ids, counts, s = idx.idx_select_paged(*args, return_scores=True, chunk_log2=chunk_log2)
    ids_d, counts_d, s_d = idx.idx_select_paged(*args, return_scores=True)
    torch.cuda.synchronize()
    ids, counts, s = ids.cpu().numpy(), counts.cpu().numpy(), s.cpu().numpy()
    S, A, n_slots = oracle.score_paged(x.q, x.c_pool, x.indptr, indices, mp, x.dtype)
    check_scores(s, S, A, RTOL[x.dtype])
    check_ids_exact(ids, counts, s, n_slots, 200, False)
    np.testing.assert_array_equal(ids, ids_d.cpu().numpy())
    np.testing.assert_array_equal(counts, counts_d.cpu().numpy())
    np.testing.assert_array_equal(s.view(np.uint32), s_d.cpu().numpy().view(np.uint32))
    assert s[0, 300] == -np.inf and s[1, 2999] == -np.inf


def test_paged_identity_lists_equal_the_dense_call():
    """Identity page lists over a per-request table: the same ids, counts and
    scores, bit for bit, as idx_select on the dense table."""
    dense = synth.make_indexer(3, 4, 128, 2000, [2000 * 16, 777 * 16, 5 * 16], 100, "bf16", 614,
                               poison=False)
    B, N = dense.B, dense.N_pad
    nv = oracle.n_valid(dense.seq_len, 16, N)
    pool = dense.c.reshape(B * N, 128)
    indptr = np.zeros(B + 1, np.int32)
    indptr[1:] = np.cumsum(nv)
    indices = np.concatenate([b * N + np.arange(nv[b]) for b in range(B)]).astype(np.int32)
    for srt in (False, True):
        ids_d, cnt_d, s_d = idx.idx_select(to_dev(dense.q), to_dev(dense.c), to_dev(dense.seq_len),
                                           100, sorted=srt, return_scores=True)
        ids_p, cnt_p, s_p = idx.idx_select_paged(to_dev(dense.q), to_dev(pool), to_dev(indptr),
                                                 to_dev(indices), 100, N, sorted=srt,
                                                 return_scores=True)
        torch.cuda.synchronize()
        np.testing.assert_array_equal(ids_p.cpu().numpy(), ids_d.cpu().numpy())
        np.testing.assert_array_equal(cnt_p.cpu().numpy(), cnt_d.cpu().numpy())
        np.testing.assert_array_equal(s_p.cpu().numpy().view(np.uint32),
                                      s_d.cpu().numpy().view(np.uint32))


def test_paged_workload_full_size():
    x = synth.workload(6)
    full_paged_check(x)
    full_paged_check(x, sorted_out=True)
