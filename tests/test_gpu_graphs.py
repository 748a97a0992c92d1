"""Every entry point captured into a HIP graph (launch amortisation: one graph
launch per batch of calls). Each replay's own outputs are checked against the
CPU oracle (ids bit-exact against the oracle's selection from the replay's own
scores, scores within tolerance, the fp64 band), with eager work between the
replays. Every workspace is allocated before the capture."""
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

POISON = -1515870811  # 0xa5a5a5a5


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def replays_checked(name, call, outs, check, poison=POISON, replays=4):
    """Capture three calls of call() (which writes into the preallocated `outs`),
    then replay the graph `replays` times: before each replay the outputs are
    poisoned, after it check(host copies of outs) runs the oracle comparison; an
    eager call runs between the replays and is checked the same way."""
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        call()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for _ in range(3):
            call()
    host = lambda: [o.cpu().numpy() for o in outs]
    for rep in range(replays):
        say(f"[graph] {name} replay {rep}")
        for o in outs:
            o.fill_(poison)
        g.replay()
        torch.cuda.synchronize()
        check(*host())
        for o in outs:
            o.fill_(poison)
        call()                      # eager work between replays
        torch.cuda.synchronize()
        check(*host())


@pytest.mark.parametrize("sorted_out", [False, True])
def test_graph_select_against_oracle(sorted_out):
    x = synth.make_indexer(4, 4, 128, 8192, [4096, 16384, 65536, 131072], 256, "bf16", 310)
    q, c, sl = to_dev(x.q), to_dev(x.c), to_dev(x.seq_len)
    ws = torch.zeros(idx.idx_workspace_bytes(4, 8192, 4, 256), dtype=torch.uint8, device="cuda")
    ids = torch.empty(4, 256, dtype=torch.int32, device="cuda")
    counts = torch.empty(4, dtype=torch.int32, device="cuda")
    s = torch.empty(4, 8192, dtype=torch.float32, device="cuda")
    S, A = oracle.score(x.q, x.c, x.seq_len, 16, "bf16")
    nv = oracle.n_valid(x.seq_len, 16, 8192)

    def check(ids_h, counts_h, s_h):
        check_scores(s_h, S, A, RTOL["bf16"])
        check_ids_exact(ids_h, counts_h, s_h, nv, 256, sorted_out)
        check_ids_band(ids_h, S, A, nv, 256, RTOL["bf16"])

    replays_checked(f"select sorted={sorted_out}",
                    lambda: idx.idx_select(q, c, sl, 256, sorted=sorted_out, ids=ids,
                                           counts=counts, scores_out=s, ws=ws),
                    [ids, counts, s], check)


def test_graph_select_without_scores_against_oracle():
    """The timed form (no score output): the ids of each replay against the
    oracle's selection from the GPU's scores of an eager call."""
    x = synth.make_indexer(128, 16, 128, 2048,
                           np.random.default_rng(311).integers(8192, 32769, 128), 256, "bf16",
                           311)
    q, c, sl = to_dev(x.q), to_dev(x.c), to_dev(x.seq_len)
    ws = torch.zeros(idx.idx_workspace_bytes(128, 2048, 16, 256), dtype=torch.uint8,
                     device="cuda")
    _, _, s = idx.idx_select(q, c, sl, 256, return_scores=True, ws=ws)
    torch.cuda.synchronize()
    s = s.cpu().numpy()
    S, A = oracle.score(x.q, x.c, x.seq_len, 16, "bf16")
    nv = oracle.n_valid(x.seq_len, 16, 2048)
    check_scores(s, S, A, RTOL["bf16"])
    ids = torch.empty(128, 256, dtype=torch.int32, device="cuda")
    counts = torch.empty(128, dtype=torch.int32, device="cuda")

    def check(ids_h, counts_h):
        check_ids_exact(ids_h, counts_h, s, nv, 256, False)

    replays_checked("select gqa", lambda: idx.idx_select(q, c, sl, 256, ids=ids, counts=counts,
                                                         ws=ws),
                    [ids, counts], check)


def test_graph_noalloc_against_oracle():
    x = synth.make_indexer(3, 4, 128, 1001, [16000, 83, 0], 64, "bf16", 312)
    q, c, sl = to_dev(x.q), to_dev(x.c), to_dev(x.seq_len)
    ids = torch.empty(3, 64, dtype=torch.int32, device="cuda")
    counts = torch.empty(3, dtype=torch.int32, device="cuda")
    s = torch.empty(3, 1001, dtype=torch.float32, device="cuda")
    S, A = oracle.score(x.q, x.c, x.seq_len, 16, "bf16")
    nv = oracle.n_valid(x.seq_len, 16, 1001)

    def check(ids_h, counts_h, s_h):
        check_scores(s_h, S, A, RTOL["bf16"])
        check_ids_exact(ids_h, counts_h, s_h, nv, 64, True)

    replays_checked("noalloc", lambda: idx.idx_select_noalloc(q, c, sl, 64, sorted=True, ids=ids,
                                                              counts=counts, scores_out=s),
                    [ids, counts, s], check)


@pytest.mark.parametrize("B,N,K", [(70, 5000, 300), (64, 30000, 2048)])
def test_graph_topk_against_oracle(B, N, K):
    x = synth.make_topk(B, N, K, 900 + B)
    sc = to_dev(x.scores)
    ids = torch.empty(B, K, dtype=torch.int32, device="cuda")
    counts = torch.empty(B, dtype=torch.int32, device="cuda")
    ws = torch.zeros(max(256, idx.idx_topk_workspace_bytes(B, N, K)), dtype=torch.uint8,
                     device="cuda")

    for srt in (False, True):
        def check(ids_h, counts_h):
            check_ids_exact(ids_h, counts_h, x.scores, None, K, srt)

        replays_checked(f"topk {B}x{N} sorted={srt}",
                        lambda: idx.idx_topk(sc, K, None, srt, ids=ids, counts=counts, ws=ws),
                        [ids, counts], check, replays=2)


def test_graph_paged_against_oracle():
    x = synth.make_paged(16, 4, 128, 16384, (1024, 256), 256, "bf16", 901)
    q, c, ip, ix = to_dev(x.q), to_dev(x.c_pool), to_dev(x.indptr), to_dev(x.indices)
    ids = torch.empty(16, 256, dtype=torch.int32, device="cuda")
    counts = torch.empty(16, dtype=torch.int32, device="cuda")
    s = torch.empty(16, x.max_pages, dtype=torch.float32, device="cuda")
    ws = torch.zeros(idx.idx_workspace_bytes(16, x.max_pages, 4, 256), dtype=torch.uint8,
                     device="cuda")
    S, A, n = oracle.score_paged(x.q, x.c_pool, x.indptr, x.indices, x.max_pages, "bf16")

    def check(ids_h, counts_h, s_h):
        check_scores(s_h, S, A, RTOL["bf16"])
        check_ids_exact(ids_h, counts_h, s_h, n, 256, False)
        check_ids_band(ids_h, S, A, n, 256, RTOL["bf16"])

    replays_checked("paged", lambda: idx.idx_select_paged(q, c, ip, ix, 256, x.max_pages, ids=ids,
                                                          counts=counts, scores_out=s, ws=ws),
                    [ids, counts, s], check)


@pytest.mark.parametrize("T", [100, 4])   # matrix-core scores + top-K; one fused launch
def test_graph_prefill_against_oracle(T):
    x = synth.make_prefill(2, T, 4, 128, 600, [2000, 7000], 64, 902)
    q, c, p0 = to_dev(x.q), to_dev(x.c), to_dev(x.pos0)
    ids = torch.empty(2, T, 64, dtype=torch.int32, device="cuda")
    counts = torch.empty(2, T, dtype=torch.int32, device="cuda")
    s = torch.empty(2, T, 600, dtype=torch.float32, device="cuda")
    ws = torch.zeros(idx.idx_prefill_workspace_bytes(2, T, 600, 64, 1), dtype=torch.uint8,
                     device="cuda")
    S, A, NV = oracle.score_prefill(x.q, x.c, x.pos0, 16, "bf16")
    R = 2 * T

    def check(ids_h, counts_h, s_h):
        sh = s_h.reshape(R, -1)
        check_scores(sh, S.reshape(R, -1), A.reshape(R, -1), RTOL["bf16"])
        check_ids_exact(ids_h.reshape(R, -1), counts_h.reshape(R), sh, NV.reshape(R), 64, True)

    replays_checked(f"prefill T={T}", lambda: idx.idx_select_prefill(q, c, p0, 64, sorted=True, ids=ids,
                                                              counts=counts, scores_out=s, ws=ws),
                    [ids, counts, s], check)


def test_graph_pool_keys_against_oracle():
    x = synth.make_keys(3, 3000, 128, 200, [3000, 1234, 7], "bf16", 903)
    k, sl = to_dev(x.k), to_dev(x.seq_len)
    c = torch.zeros(3, 200, 128, dtype=torch.bfloat16, device="cuda")
    cv = c.view(torch.int16)
    C, M, nv = oracle.pool_keys(x.k, x.seq_len, 200, 16, "bf16")

    def check(bits):
        got = synth.bf16_bits_to_f32(bits.view(np.uint16)).astype(np.float64)
        for b in range(3):
            m = int(nv[b])
            err = np.abs(got[b, :m] - C[b, :m])
            tol = 2.0 ** -8 * np.abs(C[b, :m]) + 2.0 ** -17 * M[b, :m]
            assert not (err > tol).any(), b

    replays_checked("pool", lambda: idx.idx_pool_keys(k, sl, 200, 16, c=c), [cv], check,
                    poison=-1)


def test_graph_assign_against_oracle():
    x = synth.make_assign(50000, 300, 128, 904)
    xd, cd = to_dev(x.x), to_dev(x.c)
    a = torch.empty(50000, dtype=torch.int32, device="cuda")
    best = torch.empty(50000, dtype=torch.float32, device="cuda")
    ws = torch.zeros(idx.idx_assign_workspace_bytes(300, 128), dtype=torch.uint8, device="cuda")
    rows = np.random.default_rng(904).choice(50000, 4096, replace=False)

    def check(a_h, best_h):
        np.testing.assert_array_equal(a_h, x.comp)
        assert check_assign(a_h, best_h, x.x, x.c, rows) == 0

    replays_checked("assign", lambda: idx.idx_assign(xd, cd, assign=a, best=best, ws=ws),
                    [a, best], check, poison=0)


# the refused call leaves the capture empty, which torch reports as a warning
@pytest.mark.filterwarnings("ignore:The CUDA Graph is empty")
def test_workspace_is_not_allocated_inside_a_capture():
    """A captured call whose workspace was never created for the capturing stream
    is refused (an allocation and its zero fill would be recorded in the graph)."""
    x = synth.make_assign(1000, 64, 128, 905)
    xd, cd = to_dev(x.x), to_dev(x.c)
    idx._ws_cache.clear()
    g = torch.cuda.CUDAGraph()
    with pytest.raises(RuntimeError, match="graph is being captured"):
        with torch.cuda.graph(g):
            idx.idx_assign(xd, cd)
