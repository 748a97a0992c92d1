"""GPU parity: the HIP path (through the C ABI) against the CPU oracle.

Small cases span several workgroup chunks and register tiles with ragged tails;
the named workloads run at full size in the launch configuration the bench
times. All inputs are seeded (synth).
"""
import sys

import numpy as np
import pytest

torch = pytest.importorskip("torch")

import oracle
import synth
from tests.helpers import (RTOL, check_assign, check_ids_band, check_ids_exact, check_scores,
                           to_dev)

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)

import block_scoring_top_amd as idx  # noqa: E402


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def run_select(x, K=None, sorted_out=None, chunk_log2=0, with_scores=True):
    K = x.K if K is None else K
    srt = x.sorted if sorted_out is None else sorted_out
    q, c, sl = to_dev(x.q), to_dev(x.c), to_dev(x.seq_len)
    ids, counts, s = idx.idx_select(q, c, sl, K, page_size=x.page_size, sorted=srt,
                                    return_scores=with_scores, chunk_log2=chunk_log2)
    torch.cuda.synchronize()
    return (ids.cpu().numpy(), counts.cpu().numpy(),
            None if s is None else s.cpu().numpy())


def full_select_check(x, K=None, sorted_out=None, chunk_log2=0):
    K = x.K if K is None else K
    srt = x.sorted if sorted_out is None else sorted_out
    say(f"[select] {x.name} B={x.B} H={x.H} N_pad={x.N_pad} K={K} sorted={srt} "
        f"dtype={x.dtype} chunk_log2={chunk_log2}")
    ids, counts, s = run_select(x, K, srt, chunk_log2)
    S, A = oracle.score(x.q, x.c, x.seq_len, x.page_size, x.dtype)
    nv = oracle.n_valid(x.seq_len, x.page_size, x.N_pad)
    rel = check_scores(s, S, A, RTOL[x.dtype])
    check_ids_exact(ids, counts, s, nv, K, srt)
    check_ids_band(ids, S, A, nv, K, RTOL[x.dtype])
    ids2, counts2, _ = run_select(x, K, srt, chunk_log2, with_scores=False)
    np.testing.assert_array_equal(ids2, ids)
    np.testing.assert_array_equal(counts2, counts)
    return rel


# ---------------------------------------------------------------------------------------
# idx_score
# ---------------------------------------------------------------------------------------
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_score_small_ragged(dtype):
    x = synth.make_indexer(3, 4, 128, 1001, [16000, 5 * 16 + 3, 0], 8, dtype, 101)
    say(f"[score] small ragged {dtype}")
    s = idx.idx_score(to_dev(x.q), to_dev(x.c), to_dev(x.seq_len), 16)
    torch.cuda.synchronize()
    S, A = oracle.score(x.q, x.c, x.seq_len, 16, dtype)
    check_scores(s.cpu().numpy(), S, A, RTOL[dtype])


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("H", [1, 3, 16, 64])
def test_score_integer_inputs_bit_exact(dtype, H):
    """Small integers: every partial sum is exact in fp32, so scores are exact."""
    x = synth.make_integer_indexer(2, H, 128, 300, [300 * 16, 77 * 16 - 5], 8, dtype, 102 + H)
    say(f"[score] integer H={H} {dtype}")
    s = idx.idx_score(to_dev(x.q), to_dev(x.c), to_dev(x.seq_len), 16)
    torch.cuda.synchronize()
    S, _ = oracle.score(x.q, x.c, x.seq_len, 16, dtype)
    np.testing.assert_array_equal(s.cpu().numpy().astype(np.float64), S)


# ---------------------------------------------------------------------------------------
# idx_select: small cases, grids and edge cases
# ---------------------------------------------------------------------------------------
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("K", [1, 7, 256, 300])
@pytest.mark.parametrize("sorted_out", [False, True])
def test_select_small(dtype, K, sorted_out):
    x = synth.make_indexer(4, 4, 128, 1001, [16016, 5 * 16 + 3, 0, 300 * 16 + 1], K, dtype,
                           200 + K)
    full_select_check(x, K, sorted_out)


@pytest.mark.parametrize("chunk_log2", [4, 5, 6, 8, 11])
def test_select_grid_does_not_change_ids(chunk_log2):
    x = synth.make_indexer(3, 4, 128, 4000, [4000 * 16, 1234 * 16, 17], 128, "bf16", 300)
    full_select_check(x, 128, False, chunk_log2)


@pytest.mark.parametrize("chunk_log2", [0, 4, 7])
def test_select_many_requests(chunk_log2):
    """More than 32 requests: 256-thread workgroups, 8 key slots per thread."""
    rng = np.random.default_rng(306)
    seq = rng.integers(0, 1200 * 16, 40)
    seq[:3] = [0, 1, 1200 * 16]
    x = synth.make_indexer(40, 8, 128, 1200, seq, 100, "bf16", 306)
    full_select_check(x, 100, False, chunk_log2)
    full_select_check(x, 100, True, chunk_log2)


def test_select_many_requests_medium_rows():
    """More than 32 requests, tables between 2048 and 8192 blocks (8 key slots)."""
    rng = np.random.default_rng(311)
    seq = rng.integers(0, 5000 * 16, 36)
    seq[:2] = [5000 * 16, 2049 * 16]
    x = synth.make_indexer(36, 4, 128, 5000, seq, 700, "bf16", 311)
    full_select_check(x, 700, False)
    full_select_check(x, 700, True)


@pytest.mark.parametrize("K", [2, 64, 65, 1024, 1025, 2049, 4096])
def test_select_sorted_sizes(K):
    """Score order around the sort's size steps: in-thread, in-wave and across
    waves, with 1024-thread workgroups (few requests) and 256-thread workgroups
    (many requests; above 1024 ids the sort runs in LDS)."""
    x = synth.make_indexer(3, 4, 128, 6000, [6000 * 16, 4100 * 16, 700 * 16], K, "bf16", 320 + K)
    full_select_check(x, K, True)
    rng = np.random.default_rng(340 + K)
    seq = rng.integers(0, 5000 * 16, 40)
    seq[:2] = [5000 * 16, 3000 * 16]
    x = synth.make_indexer(40, 2, 128, 5000, seq, K, "bf16", 340 + K)
    full_select_check(x, K, True)


def test_select_many_requests_multi_tile():
    """More than 32 requests with rows longer than one 8192-key register tile."""
    x = synth.make_indexer(33, 2, 128, 9000, [9000 * 16] * 30 + [8193 * 16, 5, 8192 * 16],
                           300, "bf16", 307)
    full_select_check(x, 300, False)


def test_select_multi_tile_rows():
    """Rows longer than one register tile (8192 keys) take the streaming path."""
    x = synth.make_indexer(2, 2, 128, 20000, [20000 * 16, 9000 * 16 - 3], 500, "bf16", 301)
    full_select_check(x, 500, False)
    full_select_check(x, 500, True)


def test_select_maximum_requests_and_heads():
    """The largest request count one call takes (16384, one arrival line each)
    with short tables, and the largest head count (64)."""
    rng = np.random.default_rng(320)
    seq = rng.integers(0, 40 * 16, 16384)
    seq[:3] = [0, 1, 40 * 16]
    x = synth.make_indexer(16384, 2, 128, 40, seq, 9, "bf16", 320)
    full_select_check(x, 9, False)
    x = synth.make_indexer(3, 64, 128, 3000, [3000 * 16, 1500 * 16 + 5, 16], 100, "bf16", 321)
    full_select_check(x, 100, True)


def test_select_constant_centroids_tie_to_lowest_ids():
    x = synth.make_indexer(2, 4, 128, 600, [600 * 16, 333 * 16], 50, "f32", 302)
    x.c[:] = x.c[:, :1, :]  # every block has the same centroid: all scores tie
    say("[select] constant centroids")
    ids, counts, s = run_select(x, 50, True)
    for b in range(2):
        assert np.all(s[b, : [600, 333][b]] == s[b, 0])
        np.testing.assert_array_equal(ids[b], np.arange(50))


def test_select_integer_ties_and_signed_zeros():
    """Integer data with many exact ties and zero scores; ids bit-exact."""
    x = synth.make_integer_indexer(3, 2, 128, 700, [700 * 16, 400 * 16, 9 * 16], 64, "bf16",
                                   303, lo=-1, hi=1)
    for srt in (False, True):
        full_select_check(x, 64, srt)


def test_select_fewer_valid_than_k_and_empty():
    x = synth.make_indexer(3, 4, 128, 512, [5 * 16, 0, 1], 256, "bf16", 304)
    ids, counts, _ = run_select(x, 256, False)
    np.testing.assert_array_equal(counts, [5, 0, 1])
    np.testing.assert_array_equal(ids[0, :5], np.arange(5))
    assert (ids[0, 5:] == -1).all() and (ids[1] == -1).all()
    assert ids[2, 0] == 0 and (ids[2, 1:] == -1).all()


def test_select_workspace_reused_across_shapes():
    """One workspace serves a small batch with long rows, then a larger batch."""
    small = synth.make_indexer(3, 4, 128, 9000, [9000 * 16, 4000 * 16, 77], 64, "bf16", 308)
    big = synth.make_indexer(100, 4, 128, 300, [300 * 16] * 100, 64, "bf16", 309)
    nbytes = max(idx.idx_workspace_bytes(3, 9000, 4, 64), idx.idx_workspace_bytes(100, 300, 4, 64))
    ws = torch.zeros(nbytes, dtype=torch.uint8, device="cuda")
    for x in (small, big, small):
        say(f"[select] shared workspace B={x.B}")
        ids, counts, s = idx.idx_select(to_dev(x.q), to_dev(x.c), to_dev(x.seq_len), 64, ws=ws,
                                        return_scores=True)
        torch.cuda.synchronize()
        nv = oracle.n_valid(x.seq_len, 16, x.N_pad)
        check_ids_exact(ids.cpu().numpy(), counts.cpu().numpy(), s.cpu().numpy(), nv, 64, False)
        # the arrival counters (the first 2 MiB) are back at zero; staging is scratch
        assert int(torch.count_nonzero(ws[:2 << 20])) == 0, "arrival counters left nonzero"
        ids2, _, _ = idx.idx_select(to_dev(x.q), to_dev(x.c), to_dev(x.seq_len), 64, ws=ws)
        torch.cuda.synchronize()
        assert torch.equal(ids2, ids) and int(torch.count_nonzero(ws[:2 << 20])) == 0


def test_select_is_deterministic():
    x = synth.make_indexer(4, 4, 128, 8192, [4096, 16384, 65536, 131072], 256, "bf16", 305)
    a = run_select(x, 256, False, with_scores=True)
    b = run_select(x, 256, False, with_scores=True)
    for u, v in zip(a, b):
        np.testing.assert_array_equal(u, v)


# ---------------------------------------------------------------------------------------
# idx_topk
# ---------------------------------------------------------------------------------------
def run_topk(scores, K, n_valid=None, sorted_out=False):
    nvd = None if n_valid is None else to_dev(np.asarray(n_valid, np.int32))
    ids, counts = idx.idx_topk(to_dev(scores), K, nvd, sorted_out)
    torch.cuda.synchronize()
    return ids.cpu().numpy(), counts.cpu().numpy()


@pytest.mark.parametrize("sorted_out", [False, True])
def test_topk_adversarial_rows(sorted_out):
    rng = np.random.default_rng(400)
    N = 5000
    rows = [np.where(rng.random(N) < 0.5, 0.0, -0.0).astype(np.float32),
            np.full(N, -np.inf, np.float32),
            np.concatenate([np.full(10, np.inf), rng.standard_normal(N - 10)]).astype(np.float32),
            rng.integers(-2, 3, N).astype(np.float32),
            np.full(N, 3.5, np.float32),
            rng.standard_normal(N).astype(np.float32)]
    s = np.stack(rows)
    nv = [N, N, N, N, 37, 0]
    for K in (1, 100, 2048, 4096, 5000):
        if sorted_out and K > 4096:
            continue  # sorted output is limited to K <= 4096
        say(f"[topk] adversarial K={K} sorted={sorted_out}")
        ids, counts = run_topk(s, K, nv, sorted_out)
        check_ids_exact(ids, counts, s, np.array(nv), K, sorted_out)


@pytest.mark.parametrize("K,sorted_out", [(1, False), (300, False), (300, True), (1024, True),
                                          (1100, True), (2000, False)])
def test_topk_many_short_rows(K, sorted_out):
    """600 rows of at most 2048 entries: 256-thread workgroups (1024-thread ones
    when more than 1024 ids are to be ordered), every stress distribution."""
    N = 1999 if sorted_out else 2048   # unaligned and aligned rows
    x = synth.make_topk(600, N, K, 410 + K)
    nv = np.random.default_rng(411).integers(0, N, 600)
    nv[:3] = [0, 1, N]
    say(f"[topk] many short rows K={K} sorted={sorted_out}")
    ids, counts = run_topk(x.scores, K, nv, sorted_out)
    check_ids_exact(ids, counts, x.scores, nv, K, sorted_out)


@pytest.mark.parametrize("K,sorted_out", [(1, False), (777, True), (4096, True), (6000, False)])
def test_topk_long_rows_split_into_segments(K, sorted_out):
    """Few long rows: several workgroups per row select segments, the last one
    merges; lengths end inside, at and just past segment boundaries, ties across
    segments (all-equal and quantised rows) go to the lower index."""
    B, N = 20, 50000
    x = synth.make_topk(B, N, K, 420 + K)
    nv = np.random.default_rng(421).integers(0, N, B)
    nv[:7] = [0, 1, N, 12500, 12501, 12499, 25000]
    say(f"[topk] split rows K={K} sorted={sorted_out}")
    ids, counts = run_topk(x.scores, K, nv, sorted_out)
    check_ids_exact(ids, counts, x.scores, nv, K, sorted_out)
    ids2, counts2 = run_topk(x.scores, K, nv, sorted_out)   # the workspace is reusable
    np.testing.assert_array_equal(ids2, ids)
    np.testing.assert_array_equal(counts2, counts)


def test_topk_workspace_serves_later_calls_with_other_row_counts():
    """One workspace for split calls whose row counts grow and shrink: an earlier
    call's segment candidates must not lie where a later call's arrival counters
    are (a counter left nonzero leaves its row unmerged and its outputs
    unwritten). Outputs poisoned with 0xa5 bytes before every call."""
    shapes = [(9, 20675, 37), (20, 22957, 2), (5, 30000, 2048), (64, 30000, 2048),
              (3, 40000, 100), (40, 20000, 700), (9, 20675, 37)]
    nbytes = max(idx.idx_topk_workspace_bytes(B, N, K) for B, N, K in shapes)
    ws = torch.zeros(nbytes, dtype=torch.uint8, device="cuda")
    for i, (B, N, K) in enumerate(shapes):
        assert idx.idx_topk_workspace_bytes(B, N, K) > 0  # the split path
        x = synth.make_topk(B, N, K, 430 + i)
        say(f"[topk] shared workspace, call {i}: B={B} N={N} K={K}")
        ids = torch.full((B, K), -1515870811, dtype=torch.int32, device="cuda")
        counts = torch.full((B,), -1515870811, dtype=torch.int32, device="cuda")
        idx.idx_topk(to_dev(x.scores), K, None, i % 2 == 1, ids=ids, counts=counts, ws=ws)
        torch.cuda.synchronize()
        check_ids_exact(ids.cpu().numpy(), counts.cpu().numpy(), x.scores, None, K, i % 2 == 1)


@pytest.mark.parametrize("N", [1, 3, 1000, 8191, 8192, 32768, 32769, 70001])
def test_topk_lengths(N):
    """Row lengths around the layouts: one 2-slot tile (up to 8191 entries a
    row stays whole), two segments of 4096 staged in LDS (8192), 8-slot
    segments (32769 and longer rows), and the 2- and 8-slot merges."""
    x = synth.make_topk(9, N, 300, 401 + N)
    say(f"[topk] N={N}")
    for srt in (False, True):
        ids, counts = run_topk(x.scores, 300, None, srt)
        check_ids_exact(ids, counts, x.scores, None, 300, srt)


# ---------------------------------------------------------------------------------------
# idx_assign
# ---------------------------------------------------------------------------------------
def run_assign(xb, cb):
    a, best = idx.idx_assign(to_dev(xb), to_dev(cb), return_best=True)
    torch.cuda.synchronize()
    return a.cpu().numpy(), best.cpu().numpy()


# C covers 1 to 8, 16 and 17 tiles of 64 centroids (the tile loop is unrolled
# by six and software-pipelined over two accumulator sets), whole and partial
@pytest.mark.parametrize("N,C", [(1, 1), (700, 64), (700, 65), (1000, 100), (2000, 130),
                                 (1800, 256), (1700, 300), (1500, 384), (900, 390),
                                 (1500, 449), (4097, 1024), (3000, 1031)])
def test_assign_small(N, C):
    x = synth.make_assign(N, C, 128, 500 + N)
    say(f"[assign] N={N} C={C}")
    a, best = run_assign(x.x, x.c)
    check_assign(a, best, x.x, x.c)
    np.testing.assert_array_equal(a, x.comp)


def test_assign_integer_inputs_exact_with_ties():
    rng = np.random.default_rng(502)
    cb = synth.f32_to_bf16_bits(rng.integers(-2, 3, (200, 128)).astype(np.float32))
    cb[150] = cb[20]
    cb[199] = cb[20]
    xb = synth.f32_to_bf16_bits(rng.integers(-2, 3, (3000, 128)).astype(np.float32))
    xb[:64] = cb[20]
    say("[assign] integer ties")
    a, best = run_assign(xb, cb)
    a_ref, S, _ = oracle.assign(xb, cb)
    np.testing.assert_array_equal(a, a_ref)
    np.testing.assert_array_equal(2.0 * best.astype(np.float64), S[np.arange(3000), a_ref])
    assert (a[:64] == 20).all()


# ---------------------------------------------------------------------------------------
# the named workloads at full size
# ---------------------------------------------------------------------------------------
@pytest.mark.parametrize("w", [1, 2, 4])
def test_workload_select(w):
    x = synth.workload(w)
    rel = full_select_check(x)
    say(f"  max |err|/A = {rel:.3e}")
    if x.sorted is False:
        full_select_check(x, sorted_out=True)


def test_workload_topk():
    x = synth.workload(3)
    for srt in (False, True):
        say(f"[topk] workload 3 sorted={srt}")
        ids, counts = run_topk(x.scores, x.K, None, srt)
        check_ids_exact(ids, counts, x.scores, None, x.K, srt)


def test_workload_assign():
    x = synth.workload(5)
    say("[assign] workload 5 (2^20 points, C=1024)")
    a, best = run_assign(x.x, x.c)
    # every point's generating component is its nearest centroid (holds at any size)
    np.testing.assert_array_equal(a, x.comp)
    rng = np.random.default_rng(5)
    rows = np.concatenate([np.arange(64), rng.choice(x.x.shape[0], 8192, replace=False),
                           np.arange(x.x.shape[0] - 64, x.x.shape[0])])
    assert check_assign(a, best, x.x, x.c, rows) == 0


@pytest.mark.gpu
def test_floor_mfma_sums_in_closed_form():
    """Each thread's 64 accumulator words after `iters` rounds of 32x32x16
    products of all-ones operands hold 16 * iters each: 1024 * iters in all."""
    import torch
    frags = torch.full((8192,), 0x3F80, dtype=torch.int16, device="cuda")  # bf16 1.0
    for blocks, iters in ((1, 8), (3, 40), (300, 128)):
        sink = torch.full((256 * blocks,), -1.0, dtype=torch.float32, device="cuda")
        idx.idx_floor_mfma(frags, blocks, iters, sink)
        torch.cuda.synchronize()
        assert (sink.cpu().numpy() == 1024.0 * iters).all(), (blocks, iters)


@pytest.mark.gpu
def test_floor_launches_run_and_leave_the_ticket_at_zero():
    import torch
    src = torch.arange(1 << 20, dtype=torch.int32, device="cuda")
    sink = torch.full((512,), 7.0, dtype=torch.float32, device="cuda")
    ticket = torch.zeros(1, dtype=torch.int32, device="cuda")
    idx.idx_floor_empty(128)
    for blocks, threads in ((1, 256), (37, 256), (512, 1024)):
        sink.fill_(7.0)
        idx.idx_floor_read(src, 4 << 20, sink, ticket, blocks, threads)
        torch.cuda.synchronize()
        assert int(ticket.item()) == 0
        # every workgroup wrote its word (xor of its share of the arange)
        w = sink[:blocks].view(torch.int32).cpu().numpy()
        n16 = (4 << 20) // 16
        per = -(-n16 // blocks)
        a = np.arange(1 << 20, dtype=np.int64).reshape(-1, 4)
        for g in range(blocks):
            part = a[g * per:min((g + 1) * per, n16)]
            assert int(w[g]) == int(np.bitwise_xor.reduce(part.ravel()))
