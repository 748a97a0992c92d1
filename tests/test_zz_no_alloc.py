"""idx_select_noalloc, the entry point that allocates nothing (its arrival
counters and staging live in the library's static per-GPU scratch), against
idx_select on the same inputs: ids and counts bit-exact, and its own scores
against the oracle. Two calls in a row, the second smaller, then the first
shape again, so that scratch left by a larger call cannot leak into a smaller
one and the counters are back at zero."""
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

POISON = np.int32(np.uint32(0xA5A5A5A5).view(np.int32))


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def both(x, sorted_out):
    """Outputs of idx_select (own workspace) and idx_select_noalloc, ids and counts
    pre-filled with 0xa5 bytes."""
    q, c, sl = to_dev(x.q), to_dev(x.c), to_dev(x.seq_len)
    out = []
    for fn in (idx.idx_select, idx.idx_select_noalloc):
        ids = torch.full((x.B, x.K), int(POISON), dtype=torch.int32, device="cuda")
        counts = torch.full((x.B,), int(POISON), dtype=torch.int32, device="cuda")
        fn(q, c, sl, x.K, page_size=x.page_size, sorted=sorted_out, ids=ids, counts=counts)
        torch.cuda.synchronize()
        out.append((ids.cpu().numpy(), counts.cpu().numpy()))
    return out


def scores_check(x, sorted_out):
    """The no-allocation call's own scores against the oracle (C2), its ids
    against the oracle's selection from them (C1) and from fp64 (C3)."""
    q, c, sl = to_dev(x.q), to_dev(x.c), to_dev(x.seq_len)
    ids, counts, s = idx.idx_select_noalloc(q, c, sl, x.K, page_size=x.page_size,
                                            sorted=sorted_out, return_scores=True)
    torch.cuda.synchronize()
    ids, counts, s = ids.cpu().numpy(), counts.cpu().numpy(), s.cpu().numpy()
    S, A = oracle.score(x.q, x.c, x.seq_len, x.page_size, x.dtype)
    nv = oracle.n_valid(x.seq_len, x.page_size, x.N_pad)
    check_scores(s, S, A, RTOL[x.dtype])
    check_ids_exact(ids, counts, s, nv, x.K, sorted_out)
    check_ids_band(ids, S, A, nv, x.K, RTOL[x.dtype])


CASES = [
    # the large GQA batch shape (B=128, H=16, 2048-block tables, K=256), bf16
    lambda: synth.make_indexer(128, 16, 128, 2048,
                               np.random.default_rng(41).integers(8192, 32769, 128), 256,
                               "bf16", 41, name="noalloc_gqa"),
    # smaller: four ragged fp32 requests, one of them empty
    lambda: synth.make_indexer(4, 4, 128, 1000, [16000, 83, 0, 9999], 64, "f32", 42,
                               name="noalloc_small"),
]


@pytest.mark.parametrize("sorted_out", [False, True])
def test_noalloc_matches_idx_select_on_two_calls_in_a_row(sorted_out):
    xs = [mk() for mk in CASES]
    for x in xs + xs[:1]:
        say(f"[noalloc] {x.name} B={x.B} H={x.H} N_pad={x.N_pad} K={x.K} sorted={sorted_out}")
        (ids_ref, cnt_ref), (ids, cnt) = both(x, sorted_out)
        np.testing.assert_array_equal(cnt, cnt_ref)
        np.testing.assert_array_equal(ids, ids_ref)
    for x in xs:
        scores_check(x, sorted_out)


def test_noalloc_rejects_shapes_beyond_its_scratch():
    x = synth.make_indexer(1, 4, 128, 64, [1024], 8, "bf16", 43, name="noalloc_reject")
    q, c, sl = to_dev(x.q), to_dev(x.c), to_dev(x.seq_len)
    # 4097 requests: more arrival lines than the scratch holds
    qb = q.expand(4097, -1, -1).contiguous()
    cb = c.expand(4097, -1, -1).contiguous()
    slb = sl.expand(4097).contiguous()
    with pytest.raises(idx.IdxError) as e:
        idx.idx_select_noalloc(qb, cb, slb, 8)
    assert e.value.status == -5
    # staging beyond the scratch (64 requests x 65536 blocks x 4 B = 16 MiB), but
    # accepted when the scores go to the caller's buffer instead
    cbig = torch.zeros(64, 65536, 128, dtype=torch.bfloat16, device="cuda")
    qs = q.expand(64, -1, -1).contiguous()
    sls = torch.full((64,), 160, dtype=torch.int32, device="cuda")
    with pytest.raises(idx.IdxError) as e:
        idx.idx_select_noalloc(qs, cbig, sls, 8)
    assert e.value.status == -5
    ids, counts, s = idx.idx_select_noalloc(qs, cbig, sls, 8, return_scores=True)
    torch.cuda.synchronize()
    assert (counts.cpu().numpy() == 8).all()
