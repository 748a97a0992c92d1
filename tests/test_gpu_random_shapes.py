"""Seeded random call shapes against the oracle. Each case draws its shape from a
fixed seed (so a failure names a reproducible case): idx_select over both input
types, score order or index order, the 8-bit radix variant, head counts up to
64, row lengths from one block to 20000, K from 1 to 4096, request lengths at
and around the block and row boundaries, also through a resolved plan and
through idx_select_noalloc; idx_topk and idx_topk_bf16 over the nine stress
distributions with and without per-row valid counts; idx_select_paged with
empty, clamped and invalid page lists; idx_select_prefill with ragged token
and block tiles; idx_assign; idx_pool_keys. Outputs are poisoned with 0xa5
bytes first; ids, their order, the -1 padding and the counts are compared word
for word with the oracle's selection from the GPU's own scores, and the scores
against fp64 within the tolerance of their type ("Round 18 Track C", section
2: bitwise parity over many shapes, poisoned unused slots). All calls of one
entry point share the binding's workspace, as a caller's calls would."""
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

POISON = -1515870811  # 0xa5a5a5a5


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def draw_select(seed):
    rng = np.random.default_rng(7000 + seed)
    dtype = ["bf16", "f32"][int(rng.integers(2))]
    B = int(rng.integers(1, 10))
    H = int(rng.choice([1, 2, 3, 4, 7, 16, 64]))
    N_pad = int([rng.integers(1, 300), rng.integers(300, 3000),
                 rng.integers(3000, 20001)][int(rng.integers(3))])
    while B * N_pad * H > 3_000_000 and N_pad > 1:  # keep the fp64 oracle quick
        N_pad //= 2
    K = int([1, 2, rng.integers(1, 65), rng.integers(65, 600),
             rng.integers(600, 4097)][int(rng.integers(5))])
    srt = bool(rng.integers(2))
    radix8 = bool(rng.random() < 0.3)
    page = int([16, 16, 1, 7, 64][int(rng.integers(5))])
    top = N_pad * page
    picks = [0, 1, page - 1, page, page + 1, top - 1, top, top + 5, page * min(K, N_pad),
             page * min(K, N_pad) + 1]
    seq = [int(picks[int(rng.integers(len(picks)))]) if rng.random() < 0.5
           else int(rng.integers(0, top + 1)) for _ in range(B)]
    seq = [max(0, s) for s in seq]
    chunk_log2 = int([0, 0, rng.integers(4, 15)][int(rng.integers(3))])
    return dict(dtype=dtype, B=B, H=H, N_pad=N_pad, K=K, srt=srt, radix8=radix8, seq=seq,
                page=page, chunk_log2=chunk_log2)


@pytest.mark.parametrize("seed", range(96))
def test_random_select_shapes(seed):
    p = draw_select(seed)
    say(f"[random select {seed}] {p}")
    x = synth.make_indexer(p["B"], p["H"], 128, p["N_pad"], p["seq"], p["K"], p["dtype"],
                           7100 + seed, sorted_out=p["srt"], page_size=p["page"])
    q, c, sl = to_dev(x.q), to_dev(x.c), to_dev(x.seq_len)
    B, K, pg = p["B"], p["K"], p["page"]
    ids = torch.full((B, K), POISON, dtype=torch.int32, device="cuda")
    counts = torch.full((B,), POISON, dtype=torch.int32, device="cuda")
    _, _, s = idx.idx_select(q, c, sl, K, page_size=pg, sorted=p["srt"], ids=ids, counts=counts,
                             return_scores=True, radix8=p["radix8"])
    torch.cuda.synchronize()
    s = s.cpu().numpy()
    S, A = oracle.score(x.q, x.c, x.seq_len, x.page_size, x.dtype)
    nv = oracle.n_valid(x.seq_len, x.page_size, x.N_pad)
    check_scores(s, S, A, RTOL[x.dtype])
    ids_np, counts_np = ids.cpu().numpy(), counts.cpu().numpy()
    check_ids_exact(ids_np, counts_np, s, nv, K, p["srt"])
    check_ids_band(ids_np, S, A, nv, K, RTOL[x.dtype])
    # the standalone scoring kernel on the same inputs
    check_scores(idx.idx_score(q, c, sl, page_size=pg).cpu().numpy(), S, A, RTOL[x.dtype])
    # the form without a score output (staged scores, any chunking) returns the same words
    ids2 = torch.full((B, K), POISON, dtype=torch.int32, device="cuda")
    counts2 = torch.full((B,), POISON, dtype=torch.int32, device="cuda")
    idx.idx_select(q, c, sl, K, page_size=pg, sorted=p["srt"], ids=ids2, counts=counts2,
                   radix8=p["radix8"], chunk_log2=p["chunk_log2"])
    torch.cuda.synchronize()
    np.testing.assert_array_equal(ids2.cpu().numpy(), ids_np)
    np.testing.assert_array_equal(counts2.cpu().numpy(), counts_np)
    if seed % 2 == 0 and not p["radix8"]:  # a resolved plan returns the same words
        dt = torch.bfloat16 if p["dtype"] == "bf16" else torch.float32
        plan = idx.plan_for(B, p["H"], p["N_pad"], K, dt, page_size=pg, sorted=p["srt"])
        ids3, counts3, _ = plan(q, c, sl)
        torch.cuda.synchronize()
        np.testing.assert_array_equal(ids3.cpu().numpy(), ids_np)
        np.testing.assert_array_equal(counts3.cpu().numpy(), counts_np)
    if seed % 2 == 1 and B * ((p["N_pad"] + 3) // 4 * 4) * 4 <= (16 << 20) - 4096 * 128:
        ids4 = torch.full((B, K), POISON, dtype=torch.int32, device="cuda")
        counts4 = torch.full((B,), POISON, dtype=torch.int32, device="cuda")
        idx.idx_select_noalloc(q, c, sl, K, page_size=pg, sorted=p["srt"], ids=ids4,
                               counts=counts4, radix8=p["radix8"])
        torch.cuda.synchronize()
        np.testing.assert_array_equal(ids4.cpu().numpy(), ids_np)
        np.testing.assert_array_equal(counts4.cpu().numpy(), counts_np)


def draw_topk(seed):
    rng = np.random.default_rng(8000 + seed)
    B = int(rng.integers(1, 71))
    N = int([rng.integers(1, 2049), rng.integers(2049, 8193),
             rng.integers(8193, 40001)][int(rng.integers(3))])
    while B * N > 600_000 and B > 1:
        B //= 2
    K = int([1, 2, rng.integers(1, 65), rng.integers(65, 1025),
             rng.integers(1025, 4097)][int(rng.integers(5))])
    srt = bool(rng.integers(2))
    with_nv = bool(rng.integers(2))
    nv = None
    if with_nv:
        # counts outside [0, N] are clamped by the library
        picks = [0, 1, K - 1, K, K + 1, N - 1, N, -5, N + 7]
        nv = np.array([picks[int(rng.integers(len(picks)))] if rng.random() < 0.5
                       else int(rng.integers(0, N + 1)) for _ in range(B)], np.int32)
    return dict(B=B, N=N, K=K, srt=srt, nv=nv, radix8=bool(rng.random() < 0.3))


def run_topk(scores_h, scores_d, p, bf16):
    B, K = p["B"], p["K"]
    ids = torch.full((B, K), POISON, dtype=torch.int32, device="cuda")
    counts = torch.full((B,), POISON, dtype=torch.int32, device="cuda")
    nvd = None if p["nv"] is None else torch.from_numpy(p["nv"]).to("cuda")
    if bf16:
        idx.idx_topk_bf16(scores_d, K, nvd, p["srt"], ids=ids, counts=counts)
    else:
        idx.idx_topk(scores_d, K, nvd, p["srt"], ids=ids, counts=counts, radix8=p["radix8"])
    torch.cuda.synchronize()
    nv = None if p["nv"] is None else np.clip(p["nv"], 0, p["N"])
    check_ids_exact(ids.cpu().numpy(), counts.cpu().numpy(), scores_h, nv, K, p["srt"])


@pytest.mark.parametrize("seed", range(96))
def test_random_topk_shapes(seed):
    p = draw_topk(seed)
    say(f"[random topk {seed}] B={p['B']} N={p['N']} K={p['K']} sorted={p['srt']} "
        f"valid counts={p['nv'] is not None} radix8={p['radix8']}")
    x = synth.make_topk(p["B"], p["N"], p["K"], 8100 + seed)
    run_topk(x.scores, to_dev(x.scores), p, False)


@pytest.mark.parametrize("seed", range(48))
def test_random_topk_bf16_shapes(seed):
    p = draw_topk(1000 + seed)
    say(f"[random topk bf16 {seed}] B={p['B']} N={p['N']} K={p['K']} sorted={p['srt']} "
        f"valid counts={p['nv'] is not None}")
    x = synth.make_topk(p["B"], p["N"], p["K"], 8200 + seed)
    bits = synth.f32_to_bf16_bits(x.scores)
    # the oracle selects from the same bf16 values, widened exactly
    run_topk(synth.bf16_bits_to_f32(bits), to_dev(bits), p, True)


@pytest.mark.parametrize("seed", range(48))
def test_random_paged_shapes(seed):
    rng = np.random.default_rng(9000 + seed)
    dtype = ["bf16", "f32"][int(rng.integers(2))]
    B = int(rng.integers(1, 41))
    H = int(rng.choice([1, 4, 16]))
    n_rows = int([rng.integers(1, 64), rng.integers(64, 20001)][int(rng.integers(2))])
    hi = min(n_rows, 6000)
    counts = [int([0, 1, hi, rng.integers(0, hi + 1)][int(rng.integers(4))]) for _ in range(B)]
    while sum(counts) * H > 1_500_000:
        counts = [n // 2 for n in counts]
    K = int([1, 2, rng.integers(1, 300), rng.integers(300, 4097)][int(rng.integers(4))])
    srt = bool(rng.integers(2))
    mx = max(max(counts), 1)
    max_pages = int([mx, max(1, mx // 2), mx + 37][int(rng.integers(3))])
    x = synth.make_paged(B, H, 128, n_rows, counts, K, dtype, 9100 + seed, sorted_out=srt,
                         max_pages=max_pages)
    indices = x.indices.copy()
    if indices.size and rng.random() < 0.5:  # entries that name no page
        bad = rng.choice(indices.size, min(indices.size, 5), replace=False)
        indices[bad] = np.where(rng.random(bad.size) < 0.5, -1, n_rows + 3)
    say(f"[random paged {seed}] {dtype} B={B} H={H} pool={n_rows} pages={counts[:6]} "
        f"max_pages={max_pages} K={K} sorted={srt}")
    qd, cd = to_dev(x.q), to_dev(x.c_pool)
    ipd, ixd = to_dev(x.indptr), to_dev(indices)
    ids = torch.full((B, K), POISON, dtype=torch.int32, device="cuda")
    cnt = torch.full((B,), POISON, dtype=torch.int32, device="cuda")
    _, _, s = idx.idx_select_paged(qd, cd, ipd, ixd, K, max_pages, sorted=srt, ids=ids,
                                   counts=cnt, return_scores=True)
    torch.cuda.synchronize()
    s = s.cpu().numpy()
    S, A, n_slots = oracle.score_paged(x.q, x.c_pool, x.indptr, indices, max_pages, dtype)
    check_scores(s, S, A, RTOL[dtype])
    ids_np, cnt_np = ids.cpu().numpy(), cnt.cpu().numpy()
    check_ids_exact(ids_np, cnt_np, s, n_slots, K, srt)
    check_ids_band(ids_np, S, A, n_slots, K, RTOL[dtype])
    ids2 = torch.full((B, K), POISON, dtype=torch.int32, device="cuda")
    idx.idx_select_paged(qd, cd, ipd, ixd, K, max_pages, sorted=srt, ids=ids2)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(ids2.cpu().numpy(), ids_np)


@pytest.mark.parametrize("seed", range(32))
def test_random_prefill_shapes(seed):
    rng = np.random.default_rng(9500 + seed)
    B = int(rng.integers(1, 4))
    T = int([1, rng.integers(1, 33), rng.integers(33, 160)][int(rng.integers(3))])
    H = int(rng.choice([1, 3, 4, 16]))
    N_pad = int([rng.integers(1, 64), rng.integers(64, 2600)][int(rng.integers(2))])
    while B * T * N_pad * H > 6_000_000 and N_pad > 1:
        N_pad //= 2
    pos0 = [int([-7, 0, rng.integers(0, 16 * N_pad + 1), 16 * N_pad][int(rng.integers(4))])
            for _ in range(B)]
    K = int([1, rng.integers(1, 300), rng.integers(300, 1500)][int(rng.integers(3))])
    srt = bool(rng.integers(2))
    dt = "f32" if T <= 8 and rng.integers(2) else "bf16"   # fp32: short prompts only
    say(f"[random prefill {seed}] B={B} T={T} H={H} N_pad={N_pad} pos0={pos0} K={K} "
        f"sorted={srt} {dt}")
    x = synth.make_prefill(B, T, H, 128, N_pad, pos0, K, 9600 + seed, dtype=dt, sorted_out=srt)
    qd, cd, pd = to_dev(x.q), to_dev(x.c), to_dev(x.pos0)
    ids = torch.full((B, T, K), POISON, dtype=torch.int32, device="cuda")
    cnt = torch.full((B, T), POISON, dtype=torch.int32, device="cuda")
    _, _, s = idx.idx_select_prefill(qd, cd, pd, K, sorted=srt, ids=ids, counts=cnt,
                                     return_scores=True)
    torch.cuda.synchronize()
    R = B * T
    s = s.cpu().numpy().reshape(R, -1)
    S, A, NV = oracle.score_prefill(x.q, x.c, x.pos0, x.page_size, x.dtype)
    S, A, NV = S.reshape(R, -1), A.reshape(R, -1), NV.reshape(R)
    check_scores(s, S, A, RTOL[x.dtype])
    ids_np, cnt_np = ids.cpu().numpy().reshape(R, K), cnt.cpu().numpy().reshape(R)
    check_ids_exact(ids_np, cnt_np, s, NV, K, srt)
    check_ids_band(ids_np, S, A, NV, K, RTOL[x.dtype])
    ids2 = torch.full((B, T, K), POISON, dtype=torch.int32, device="cuda")
    idx.idx_select_prefill(qd, cd, pd, K, sorted=srt, ids=ids2)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(ids2.cpu().numpy().reshape(R, K), ids_np)


@pytest.mark.parametrize("seed", range(24))
def test_random_assign_shapes(seed):
    from tests.helpers import check_assign
    rng = np.random.default_rng(9800 + seed)
    N = int([1, rng.integers(1, 300), rng.integers(300, 6000)][int(rng.integers(3))])
    C = int([1, rng.integers(1, 64), rng.integers(64, 1600)][int(rng.integers(3))])
    say(f"[random assign {seed}] N={N} C={C}")
    x = synth.make_assign(N, C, 128, 9900 + seed)
    a = torch.full((N,), POISON, dtype=torch.int32, device="cuda")
    best = torch.full((N,), float("nan"), dtype=torch.float32, device="cuda")
    idx.idx_assign(to_dev(x.x), to_dev(x.c), assign=a, best=best, return_best=True)
    torch.cuda.synchronize()
    a_np, b_np = a.cpu().numpy(), best.cpu().numpy()
    check_assign(a_np, b_np, x.x, x.c)
    np.testing.assert_array_equal(a_np, x.comp)


@pytest.mark.parametrize("seed", range(24))
def test_random_pool_shapes(seed):
    from tests.test_gpu_pool import pool_check
    rng = np.random.default_rng(9950 + seed)
    B = int(rng.integers(1, 6))
    page = int(rng.choice([1, 3, 16, 64]))
    N_pad = int(rng.integers(1, 400))
    S_pad = int(rng.integers(1, N_pad * page + 40))
    seq = [int([0, 1, S_pad, rng.integers(0, S_pad + 1), S_pad + 9][int(rng.integers(5))])
           for _ in range(B)]
    dtype = ["bf16", "f32"][int(rng.integers(2))]
    say(f"[random pool {seed}] B={B} S_pad={S_pad} N_pad={N_pad} page={page} seq={seq} {dtype}")
    pool_check(synth.make_keys(B, S_pad, 128, N_pad, seq, dtype, 9960 + seed, page_size=page,
                               name=f"random_{seed}"))


@pytest.mark.parametrize("seed", range(12))
def test_random_graph_replays(seed):
    """Random select and top-K shapes captured into one HIP graph (two calls of
    each, workspaces passed in), replayed three times with the outputs poisoned
    before each replay and eager calls of other shapes on the same workspaces
    between replays: every replay's ids and counts equal the oracle's."""
    p = draw_select(500 + seed)
    t = draw_topk(500 + seed)
    say(f"[random graph {seed}] select {p} topk B={t['B']} N={t['N']} K={t['K']}")
    x = synth.make_indexer(p["B"], p["H"], 128, p["N_pad"], p["seq"], p["K"], p["dtype"],
                           7300 + seed, sorted_out=p["srt"], page_size=p["page"])
    q, c, sl = to_dev(x.q), to_dev(x.c), to_dev(x.seq_len)
    B, K, pg = p["B"], p["K"], p["page"]
    y = synth.make_topk(t["B"], t["N"], t["K"], 8300 + seed)
    sc = to_dev(y.scores)
    nvd = None if t["nv"] is None else torch.from_numpy(t["nv"]).to("cuda")
    ws_s = torch.zeros(idx.idx_workspace_bytes(B, p["N_pad"], p["H"], K), dtype=torch.uint8,
                       device="cuda")
    ws_t = torch.zeros(max(256, idx.idx_topk_workspace_bytes(t["B"], t["N"], t["K"])),
                       dtype=torch.uint8, device="cuda")
    # the GPU's scores of this select, checked against fp64, fix the expected ids
    _, _, s = idx.idx_select(q, c, sl, K, page_size=pg, sorted=p["srt"], return_scores=True,
                             ws=ws_s)
    torch.cuda.synchronize()
    s = s.cpu().numpy()
    S, A = oracle.score(x.q, x.c, x.seq_len, x.page_size, x.dtype)
    check_scores(s, S, A, RTOL[x.dtype])
    nv = oracle.n_valid(x.seq_len, x.page_size, x.N_pad)
    ids = torch.empty(B, K, dtype=torch.int32, device="cuda")
    counts = torch.empty(B, dtype=torch.int32, device="cuda")
    tids = torch.empty(t["B"], t["K"], dtype=torch.int32, device="cuda")
    tcounts = torch.empty(t["B"], dtype=torch.int32, device="cuda")

    def calls():
        idx.idx_select(q, c, sl, K, page_size=pg, sorted=p["srt"], ids=ids, counts=counts,
                       ws=ws_s)
        idx.idx_topk(sc, t["K"], nvd, t["srt"], ids=tids, counts=tcounts, ws=ws_t)

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        calls()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        calls()
        calls()
    other = draw_select(600 + seed)
    xo = synth.make_indexer(min(other["B"], B), p["H"], 128, p["N_pad"],
                            other["seq"][:min(other["B"], B)], K, p["dtype"], 7400 + seed,
                            page_size=pg)
    for rep in range(3):
        for o in (ids, counts, tids, tcounts):
            o.fill_(POISON)
        g.replay()
        torch.cuda.synchronize()
        check_ids_exact(ids.cpu().numpy(), counts.cpu().numpy(), s, nv, K, p["srt"])
        check_ids_exact(tids.cpu().numpy(), tcounts.cpu().numpy(), y.scores,
                        None if t["nv"] is None else np.clip(t["nv"], 0, t["N"]), t["K"],
                        t["srt"])
        # eager work of another shape on the same workspaces between the replays
        idx.idx_select(to_dev(xo.q), to_dev(xo.c), to_dev(xo.seq_len), K, page_size=pg,
                       ws=ws_s)
        idx.idx_topk(sc[: max(1, t["B"] // 2)], t["K"], None, not t["srt"], ws=ws_t)
        torch.cuda.synchronize()


@pytest.mark.parametrize("seed", range(8))
def test_random_long_select_rows(seed):
    """Requests longer than a 1024-thread workgroup's register tile (32768
    entries): the selecting workgroup streams the staged row through its tile."""
    rng = np.random.default_rng(7700 + seed)
    dtype = ["bf16", "f32"][int(rng.integers(2))]
    B = int(rng.integers(1, 4))
    H = int(rng.choice([1, 4]))
    N_pad = int(rng.integers(32769, 80001))
    K = int([1, rng.integers(2, 300), rng.integers(300, 4097)][int(rng.integers(3))])
    srt = bool(rng.integers(2))
    top = N_pad * 16
    seq = [int([top, top - 1, rng.integers(0, top + 1), 16 * 32768 + 16][int(rng.integers(4))])
           for _ in range(B)]
    say(f"[random long rows {seed}] {dtype} B={B} H={H} N_pad={N_pad} K={K} sorted={srt} "
        f"seq={seq}")
    x = synth.make_indexer(B, H, 128, N_pad, seq, K, dtype, 7800 + seed, sorted_out=srt)
    q, c, sl = to_dev(x.q), to_dev(x.c), to_dev(x.seq_len)
    ids = torch.full((B, K), POISON, dtype=torch.int32, device="cuda")
    counts = torch.full((B,), POISON, dtype=torch.int32, device="cuda")
    _, _, s = idx.idx_select(q, c, sl, K, sorted=srt, ids=ids, counts=counts, return_scores=True)
    torch.cuda.synchronize()
    s = s.cpu().numpy()
    S, A = oracle.score(x.q, x.c, x.seq_len, x.page_size, x.dtype)
    nv = oracle.n_valid(x.seq_len, x.page_size, x.N_pad)
    check_scores(s, S, A, RTOL[x.dtype])
    ids_np, counts_np = ids.cpu().numpy(), counts.cpu().numpy()
    check_ids_exact(ids_np, counts_np, s, nv, K, srt)
    check_ids_band(ids_np, S, A, nv, K, RTOL[x.dtype])
    ids2 = torch.full((B, K), POISON, dtype=torch.int32, device="cuda")
    idx.idx_select(q, c, sl, K, sorted=srt, ids=ids2)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(ids2.cpu().numpy(), ids_np)


@pytest.mark.parametrize("seed", range(16))
def test_random_select_many_requests(seed):
    """More than 32 requests: the 512-thread instances (one or four key slots,
    blocked or striped rows), and score-ordered K above 1024 back on the
    1024-thread ones."""
    rng = np.random.default_rng(7900 + seed)
    dtype = ["bf16", "f32"][int(rng.integers(2))]
    B = int(rng.integers(33, 301))
    H = int(rng.choice([1, 4, 16]))
    N_pad = int([rng.integers(1, 600), rng.integers(600, 2049), rng.integers(2049, 9000)][
        int(rng.integers(3))])
    while B * N_pad * H > 3_000_000 and N_pad > 1:
        N_pad //= 2
    K = int([1, rng.integers(2, 257), rng.integers(257, 1025), rng.integers(1025, 2049)][
        int(rng.integers(4))])
    srt = bool(rng.integers(2))
    top = N_pad * 16
    seq = [int([0, top, rng.integers(0, top + 1), 16 * min(K, N_pad)][int(rng.integers(4))])
           for _ in range(B)]
    say(f"[random many requests {seed}] {dtype} B={B} H={H} N_pad={N_pad} K={K} sorted={srt}")
    x = synth.make_indexer(B, H, 128, N_pad, seq, K, dtype, 7950 + seed, sorted_out=srt)
    q, c, sl = to_dev(x.q), to_dev(x.c), to_dev(x.seq_len)
    ids = torch.full((B, K), POISON, dtype=torch.int32, device="cuda")
    counts = torch.full((B,), POISON, dtype=torch.int32, device="cuda")
    _, _, s = idx.idx_select(q, c, sl, K, sorted=srt, ids=ids, counts=counts, return_scores=True)
    torch.cuda.synchronize()
    s = s.cpu().numpy()
    S, A = oracle.score(x.q, x.c, x.seq_len, x.page_size, x.dtype)
    nv = oracle.n_valid(x.seq_len, x.page_size, x.N_pad)
    check_scores(s, S, A, RTOL[x.dtype])
    ids_np, counts_np = ids.cpu().numpy(), counts.cpu().numpy()
    check_ids_exact(ids_np, counts_np, s, nv, K, srt)
    check_ids_band(ids_np, S, A, nv, K, RTOL[x.dtype])
    ids2 = torch.full((B, K), POISON, dtype=torch.int32, device="cuda")
    idx.idx_select(q, c, sl, K, sorted=srt, ids=ids2)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(ids2.cpu().numpy(), ids_np)


@pytest.mark.parametrize("seed", range(12))
def test_random_topk_many_short_rows(seed):
    """At least 512 rows of at most 2048 entries: the 256-thread instances (K up
    to 1024), fp32 and bf16 rows, with and without valid counts."""
    rng = np.random.default_rng(8600 + seed)
    B = int(rng.integers(512, 3001))
    N = int([rng.integers(1, 200), rng.integers(200, 2049)][int(rng.integers(2))])
    K = int([1, rng.integers(2, 65), rng.integers(65, 1025)][int(rng.integers(3))])
    srt = bool(rng.integers(2))
    nv = None
    if rng.integers(2):
        nv = np.clip(rng.integers(-3, N + 5, B), -3, N + 5).astype(np.int32)
    bf16 = bool(rng.integers(2))
    p = dict(B=B, N=N, K=K, srt=srt, nv=nv, radix8=not bf16 and bool(rng.random() < 0.3))
    say(f"[random many short rows {seed}] B={B} N={N} K={K} sorted={srt} "
        f"valid counts={nv is not None} bf16={bf16} radix8={p['radix8']}")
    x = synth.make_topk(B, N, K, 8700 + seed)
    if bf16:
        bits = synth.f32_to_bf16_bits(x.scores)
        run_topk(synth.bf16_bits_to_f32(bits), to_dev(bits), p, True)
    else:
        run_topk(x.scores, to_dev(x.scores), p, False)


@pytest.mark.parametrize("seed", range(8))
def test_random_prefill_many_tokens(seed):
    """At least 512 (request, token) rows of at most 2048 blocks: the prompt
    selects run in the narrow instances (512 threads, one key slot, or 256
    threads in score order)."""
    rng = np.random.default_rng(9700 + seed)
    B = int(rng.integers(1, 4))
    T = int(max(rng.integers(200, 701), -(-512 // B)))
    H = int(rng.choice([1, 4]))
    N_pad = int(rng.integers(1, 2049))
    while B * T * N_pad * H > 8_000_000 and N_pad > 1:
        N_pad //= 2
    pos0 = [int([0, rng.integers(0, 16 * N_pad + 1), 16 * N_pad][int(rng.integers(3))])
            for _ in range(B)]
    K = int([1, rng.integers(2, 300), rng.integers(300, 1025)][int(rng.integers(3))])
    srt = bool(rng.integers(2))
    say(f"[random prefill many tokens {seed}] B={B} T={T} H={H} N_pad={N_pad} pos0={pos0} "
        f"K={K} sorted={srt}")
    x = synth.make_prefill(B, T, H, 128, N_pad, pos0, K, 9750 + seed, sorted_out=srt)
    qd, cd, pd = to_dev(x.q), to_dev(x.c), to_dev(x.pos0)
    ids = torch.full((B, T, K), POISON, dtype=torch.int32, device="cuda")
    cnt = torch.full((B, T), POISON, dtype=torch.int32, device="cuda")
    _, _, s = idx.idx_select_prefill(qd, cd, pd, K, sorted=srt, ids=ids, counts=cnt,
                                     return_scores=True)
    torch.cuda.synchronize()
    R = B * T
    s = s.cpu().numpy().reshape(R, -1)
    S, A, NV = oracle.score_prefill(x.q, x.c, x.pos0, x.page_size, x.dtype)
    S, A, NV = S.reshape(R, -1), A.reshape(R, -1), NV.reshape(R)
    check_scores(s, S, A, RTOL[x.dtype])
    check_ids_exact(ids.cpu().numpy().reshape(R, K), cnt.cpu().numpy().reshape(R), s, NV, K, srt)


def test_random_shapes_on_concurrent_streams():
    """Calls of different shapes in flight together on four streams, each with
    the binding's workspace of its own stream: every output equals the oracle's
    (no state is shared between calls other than their workspaces)."""
    streams = [torch.cuda.Stream() for _ in range(4)]
    jobs = []
    for i, st in enumerate(streams):
        p = draw_select(800 + i)
        x = synth.make_indexer(p["B"], p["H"], 128, p["N_pad"], p["seq"], p["K"], p["dtype"],
                               8800 + i, sorted_out=p["srt"], page_size=p["page"])
        t = draw_topk(800 + i)
        y = synth.make_topk(t["B"], t["N"], t["K"], 8900 + i)
        q, c, sl, sc = to_dev(x.q), to_dev(x.c), to_dev(x.seq_len), to_dev(y.scores)
        nvd = None if t["nv"] is None else torch.from_numpy(t["nv"]).to("cuda")
        torch.cuda.synchronize()
        jobs.append((p, x, q, c, sl, t, y, sc, nvd, st))
    outs = []
    for p, x, q, c, sl, t, y, sc, nvd, st in jobs:
        st.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(st):
            a = idx.idx_select(q, c, sl, p["K"], page_size=p["page"], sorted=p["srt"],
                               return_scores=True)
            b = idx.idx_topk(sc, t["K"], nvd, t["srt"])
        outs.append((a, b))
    torch.cuda.synchronize()
    for (p, x, q, c, sl, t, y, sc, nvd, st), (a, b) in zip(jobs, outs):
        say(f"[concurrent] select B={p['B']} N_pad={p['N_pad']} K={p['K']}; "
            f"topk B={t['B']} N={t['N']} K={t['K']}")
        ids, counts, s = (v.cpu().numpy() for v in a)
        S, A = oracle.score(x.q, x.c, x.seq_len, x.page_size, x.dtype)
        check_scores(s, S, A, RTOL[x.dtype])
        check_ids_exact(ids, counts, s, oracle.n_valid(x.seq_len, x.page_size, x.N_pad), p["K"],
                        p["srt"])
        nv = None if t["nv"] is None else np.clip(t["nv"], 0, t["N"])
        check_ids_exact(b[0].cpu().numpy(), b[1].cpu().numpy(), y.scores, nv, t["K"], t["srt"])
