"""Every entry point captured into a HIP graph (launch amortisation: one graph
launch per batch of calls): every replay equals the eager call, with eager work
between the replays."""
import sys

import numpy as np
import pytest

torch = pytest.importorskip("torch")

import synth
from tests.helpers import to_dev

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)

import block_scoring_top_amd as idx  # noqa: E402


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def graph_matches_eager(name, call, outs):
    """call() writes into the preallocated tensors `outs`; all workspaces are
    created by the eager calls before the capture."""
    call()
    torch.cuda.synchronize()
    ref = [o.clone() for o in outs]
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        call()
    torch.cuda.current_stream().wait_stream(side)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for _ in range(3):
            call()
    for rep in range(4):
        say(f"[graph] {name} replay {rep}")
        for o in outs:
            o.fill_(-7)
        g.replay()
        torch.cuda.synchronize()
        for o, r in zip(outs, ref):
            assert torch.equal(o, r), (name, rep)
        call()                      # eager work between replays
        torch.cuda.synchronize()
        for o, r in zip(outs, ref):
            assert torch.equal(o, r), (name, rep, "eager")


def test_graph_topk():
    x = synth.make_topk(70, 5000, 300, 900)
    s = to_dev(x.scores)
    ids = torch.empty(70, 300, dtype=torch.int32, device="cuda")
    counts = torch.empty(70, dtype=torch.int32, device="cuda")
    graph_matches_eager("topk", lambda: idx.idx_topk(s, 300, None, True, ids=ids, counts=counts),
                        [ids, counts])


def test_graph_paged():
    x = synth.make_paged(16, 4, 128, 16384, (1024, 256), 256, "bf16", 901)
    q, c, ip, ix = to_dev(x.q), to_dev(x.c_pool), to_dev(x.indptr), to_dev(x.indices)
    ids = torch.empty(16, 256, dtype=torch.int32, device="cuda")
    counts = torch.empty(16, dtype=torch.int32, device="cuda")
    ws = torch.zeros(idx.idx_workspace_bytes(16, x.max_pages, 4, 256), dtype=torch.uint8,
                     device="cuda")
    graph_matches_eager("paged", lambda: idx.idx_select_paged(q, c, ip, ix, 256, x.max_pages,
                                                              ids=ids, counts=counts, ws=ws),
                        [ids, counts])


def test_graph_prefill():
    x = synth.make_prefill(2, 100, 4, 128, 600, [2000, 7000], 64, 902)
    q, c, p0 = to_dev(x.q), to_dev(x.c), to_dev(x.pos0)
    ids = torch.empty(2, 100, 64, dtype=torch.int32, device="cuda")
    counts = torch.empty(2, 100, dtype=torch.int32, device="cuda")
    graph_matches_eager("prefill", lambda: idx.idx_select_prefill(q, c, p0, 64, sorted=True,
                                                                  ids=ids, counts=counts),
                        [ids, counts])


def test_graph_pool_keys():
    x = synth.make_keys(3, 3000, 128, 200, [3000, 1234, 7], "bf16", 903)
    k, sl = to_dev(x.k), to_dev(x.seq_len)
    c = torch.zeros(3, 200, 128, dtype=torch.bfloat16, device="cuda")
    cv = c.view(torch.int16)
    # the rows each request's blocks fill (rows past them are never written)
    rows = [cv[0, :188], cv[1, :78], cv[2, :1]]
    graph_matches_eager("pool", lambda: idx.idx_pool_keys(k, sl, 200, 16, c=c), rows)


def test_graph_assign():
    x = synth.make_assign(50000, 300, 128, 904)
    xd, cd = to_dev(x.x), to_dev(x.c)
    a = torch.empty(50000, dtype=torch.int32, device="cuda")
    graph_matches_eager("assign", lambda: idx.idx_assign(xd, cd, assign=a), [a])
