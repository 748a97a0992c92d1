"""Plans ("Export Cake KMeans plan-runtime suite", Summary: a launch plan
resolved once per call signature, a cache of them, and graph capture of the
planned calls): plan calls and every replay of a captured graph of them are
checked against the CPU oracle (ids bit-exact against the oracle's selection
from the GPU's own scores, scores within tolerance, the fp64 band)."""
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


def inputs(w):
    if w == "decode":
        return synth.workload(2)
    if w == "gqa":
        return synth.make_indexer(128, 16, 128, 2048,
                                  np.random.default_rng(60).integers(8192, 32769, 128), 256,
                                  "bf16", 60, name="plan_gqa")
    return synth.make_indexer(3, 4, 128, 1001, [16000, 83, 0], 64, "f32", 61, name="plan_f32")


def oracle_check(x, ids, counts, s, srt):
    S, A = oracle.score(x.q, x.c, x.seq_len, x.page_size, x.dtype)
    nv = oracle.n_valid(x.seq_len, x.page_size, x.N_pad)
    check_scores(s, S, A, RTOL[x.dtype])
    check_ids_exact(ids, counts, s, nv, x.K, srt)
    check_ids_band(ids, S, A, nv, x.K, RTOL[x.dtype])


@pytest.mark.parametrize("w", ["decode", "gqa", "f32"])
@pytest.mark.parametrize("srt", [False, True])
def test_plan_calls_against_oracle(w, srt):
    x = inputs(w)
    dt = torch.bfloat16 if x.dtype == "bf16" else torch.float32
    plan = idx.plan_for(x.B, x.H, x.N_pad, x.K, dt, x.page_size, srt)
    assert idx.plan_for(x.B, x.H, x.N_pad, x.K, dt, x.page_size, srt) is plan
    q, c, sl = to_dev(x.q), to_dev(x.c), to_dev(x.seq_len)
    say(f"[plan] {w} sorted={srt}")
    ids = torch.full((x.B, x.K), POISON, dtype=torch.int32, device="cuda")
    counts = torch.full((x.B,), POISON, dtype=torch.int32, device="cuda")
    s = torch.empty(x.B, x.N_pad, dtype=torch.float32, device="cuda")
    plan(q, c, sl, ids, counts, s)
    torch.cuda.synchronize()
    oracle_check(x, ids.cpu().numpy(), counts.cpu().numpy(), s.cpu().numpy(), srt)
    # without the score output: the same ids as idx_select
    ids2, counts2, _ = plan(q, c, sl)
    ref, rc, _ = idx.idx_select(q, c, sl, x.K, page_size=x.page_size, sorted=srt)
    torch.cuda.synchronize()
    assert torch.equal(ids2, ref) and torch.equal(counts2, rc)
    assert torch.equal(ids2, ids)


def test_plan_graph_replays_against_oracle():
    x = inputs("decode")
    plan = idx.SelectPlan(x.B, x.H, x.N_pad, x.K)
    q, c, sl = to_dev(x.q), to_dev(x.c), to_dev(x.seq_len)
    ids = torch.empty(x.B, x.K, dtype=torch.int32, device="cuda")
    counts = torch.empty(x.B, dtype=torch.int32, device="cuda")
    s = torch.empty(x.B, x.N_pad, dtype=torch.float32, device="cuda")
    g = plan.capture(q, c, sl, ids, counts, s, calls=3)
    for rep in range(4):
        say(f"[plan] graph replay {rep}")
        ids.fill_(POISON)
        counts.fill_(POISON)
        s.fill_(float("nan"))
        g.replay()
        torch.cuda.synchronize()
        oracle_check(x, ids.cpu().numpy(), counts.cpu().numpy(), s.cpu().numpy(), False)
        plan(q, c, sl, ids, counts)  # eager work between replays
        torch.cuda.synchronize()


def test_plan_rejects_other_signatures():
    x = inputs("decode")
    plan = idx.SelectPlan(x.B, x.H, x.N_pad, x.K)
    q, c, sl = to_dev(x.q), to_dev(x.c), to_dev(x.seq_len)
    with pytest.raises(ValueError):
        plan(q[:2].contiguous(), c[:2].contiguous(), sl[:2].contiguous())
    with pytest.raises(ValueError):
        plan(q.float(), c.float(), sl)
