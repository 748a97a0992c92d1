"""Boundary sweep of the selection ("Round 18 Track C", section 2: ids compared
bitwise over a list of context lengths, with unused output slots poisoned with
0xa5 bytes). One batch per K holds one request per valid-block count in
{0, 1, 2, K-1, K, K+1, 255, 256, 257, 1023, 1024, 1025, 2047, 2048, 2049, 4095,
4096, 4097, N_pad}; the token counts are not multiples of the page size. Every
output word (ids, padding and counts) is compared with the oracle's selection
from the GPU's own scores, in the fused select and in idx_topk, in both output
orders and in every workgroup shape the host chooses between. Also: fp32 inputs
with N(0,1) values at 16 and 64 query heads against the 1e-5 tolerance."""
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
KS = [1, 2, 64, 255, 256, 257, 2048]


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def counts_list(K, N_pad):
    v = {0, 1, 2, K - 1, K, K + 1, 255, 256, 257, 1023, 1024, 1025, 2047, 2048, 2049, 4095, 4096,
         4097, N_pad}
    return sorted(n for n in v if 0 <= n <= N_pad)


def seq_lens(nv, rng, page=16):
    """Token counts whose block count is nv: a partly filled last page (1..page
    tokens in it) where nv > 0."""
    nv = np.asarray(nv, dtype=np.int64)
    r = rng.integers(1, page + 1, nv.size)
    return np.where(nv > 0, (nv - 1) * page + r, 0).astype(np.int32)


def exact_words(ids_gpu, counts_gpu, s_gpu, nv, K, srt):
    """Every id slot and count equal to the oracle's, padding -1 included (the
    poison value would show wherever a slot was not written)."""
    ids_ref, counts_ref = oracle.select(s_gpu, nv, K, srt)
    np.testing.assert_array_equal(counts_gpu, counts_ref)
    np.testing.assert_array_equal(ids_gpu, ids_ref)


# (N_pad, copies of the count list): 1024-thread workgroups for up to 32
# requests; 512-thread ones with four key slots (blocked) or one (rows of at
# most 2048 blocks) for more
SHAPES = [(4500, 1), (4500, 3), (2048, 3)]


@pytest.mark.parametrize("K", KS)
@pytest.mark.parametrize("N_pad,copies", SHAPES)
def test_boundary_sweep_select(K, N_pad, copies):
    rng = np.random.default_rng(1000 + K + N_pad + copies)
    nv = np.concatenate([counts_list(K, N_pad)] * copies)
    sl = seq_lens(nv, rng)
    x = synth.make_indexer(nv.size, 4, 128, N_pad, sl, K, "bf16", int(rng.integers(1 << 30)),
                           name="sweep")
    q, c, sld = to_dev(x.q), to_dev(x.c), to_dev(x.seq_len)
    S, A = oracle.score(x.q, x.c, x.seq_len, 16, "bf16")
    nvo = oracle.n_valid(x.seq_len, 16, N_pad)
    np.testing.assert_array_equal(nvo, nv)
    for srt in (False, True):
        say(f"[sweep] select B={x.B} N_pad={N_pad} K={K} sorted={srt}")
        ids = torch.full((x.B, K), POISON, dtype=torch.int32, device="cuda")
        counts = torch.full((x.B,), POISON, dtype=torch.int32, device="cuda")
        s = torch.full((x.B, N_pad), float("nan"), dtype=torch.float32, device="cuda")
        idx.idx_select(q, c, sld, K, sorted=srt, ids=ids, counts=counts, scores_out=s)
        torch.cuda.synchronize()
        s_h = s.cpu().numpy()
        check_scores(s_h, S, A, RTOL["bf16"])
        exact_words(ids.cpu().numpy(), counts.cpu().numpy(), s_h, nv, K, srt)
        check_ids_band(ids.cpu().numpy(), S, A, nv, K, RTOL["bf16"])
        # the same call without the score output (the staged path)
        ids2 = torch.full((x.B, K), POISON, dtype=torch.int32, device="cuda")
        counts2 = torch.full((x.B,), POISON, dtype=torch.int32, device="cuda")
        idx.idx_select(q, c, sld, K, sorted=srt, ids=ids2, counts=counts2)
        torch.cuda.synchronize()
        exact_words(ids2.cpu().numpy(), counts2.cpu().numpy(), s_h, nv, K, srt)


@pytest.mark.parametrize("K", KS)
def test_boundary_sweep_topk(K):
    """idx_topk over rows with the same valid counts, tied and untied values."""
    rng = np.random.default_rng(2000 + K)
    N = 4500
    nv = np.concatenate([counts_list(K, N)] * 2).astype(np.int32)
    B = nv.size
    sc = rng.standard_normal((B, N)).astype(np.float32)
    sc[1::2] = np.floor(sc[1::2] * 4.0)  # every second row: a few tied values
    sd, nvd = to_dev(sc), to_dev(nv)
    ws = torch.zeros(max(256, idx.idx_topk_workspace_bytes(B, N, K)), dtype=torch.uint8,
                     device="cuda")
    for srt in (False, True):
        say(f"[sweep] topk B={B} N={N} K={K} sorted={srt}")
        ids = torch.full((B, K), POISON, dtype=torch.int32, device="cuda")
        counts = torch.full((B,), POISON, dtype=torch.int32, device="cuda")
        idx.idx_topk(sd, K, nvd, srt, ids=ids, counts=counts, ws=ws)
        torch.cuda.synchronize()
        exact_words(ids.cpu().numpy(), counts.cpu().numpy(), sc, nv, K, srt)


@pytest.mark.parametrize("H", [16, 64])
@pytest.mark.parametrize("srt", [False, True])
def test_fp32_random_inputs_many_heads(H, srt):
    """N(0,1) fp32 queries and centroids: scores within 1e-5 * A, ids exact
    against the GPU's scores and inside the band of the fp64 ones."""
    seq = [16 * 3000 - 5, 16 * 1024, 77, 16 * 4000]
    x = synth.make_indexer(4, H, 128, 4000, seq, 256, "f32", 3000 + H, sorted_out=srt,
                           name=f"f32_h{H}")
    q, c, sl = to_dev(x.q), to_dev(x.c), to_dev(x.seq_len)
    say(f"[f32] H={H} sorted={srt}")
    ids, counts, s = idx.idx_select(q, c, sl, 256, sorted=srt, return_scores=True)
    torch.cuda.synchronize()
    ids, counts, s = ids.cpu().numpy(), counts.cpu().numpy(), s.cpu().numpy()
    S, A = oracle.score(x.q, x.c, x.seq_len, 16, "f32")
    nv = oracle.n_valid(x.seq_len, 16, 4000)
    rel = check_scores(s, S, A, RTOL["f32"])
    say(f"  max |err|/A = {rel:.3e}")
    check_ids_exact(ids, counts, s, nv, 256, srt)
    check_ids_band(ids, S, A, nv, 256, RTOL["f32"])
    # idx_score's own kernel on the same inputs
    s2 = idx.idx_score(q, c, sl)
    torch.cuda.synchronize()
    check_scores(s2.cpu().numpy(), S, A, RTOL["f32"])
