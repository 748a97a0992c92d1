"""Rows whose linear threshold bin holds many distinct keys: a tight cluster of
scores plus a few wide outliers that stretch the row's range, so the bin of the
K-th score holds hundreds of different keys (more than the rank gather takes,
fewer than the bitonic refinement's cap, or more for the longest rows, which
fall back to the radix passes). Ids, order, padding and counts are compared
word for word with the oracle's selection (from the GPU's own scores for the
fused select)."""
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


clustered = synth.clustered_rows


def topk_check(scores, K, srt, bf16=False):
    B, N = scores.shape
    ids = torch.full((B, K), POISON, dtype=torch.int32, device="cuda")
    counts = torch.full((B,), POISON, dtype=torch.int32, device="cuda")
    ws = torch.zeros(max(256, idx.idx_topk_workspace_bytes(B, N, K)), dtype=torch.uint8,
                     device="cuda")
    if bf16:
        bits = synth.f32_to_bf16_bits(scores)
        sd = torch.from_numpy(bits.view(np.int16)).to("cuda").view(torch.bfloat16)
        vals = oracle.bf16_decode(bits)
    else:
        sd = to_dev(scores)
        vals = scores
    idx.idx_topk(sd, K, None, srt, ids=ids, counts=counts, ws=ws)
    torch.cuda.synchronize()
    check_ids_exact(ids.cpu().numpy(), counts.cpu().numpy(), vals, None, K, srt)


@pytest.mark.parametrize("B,N,K", [(64, 8000, 1024), (64, 8000, 256), (64, 30000, 2048),
                                   (9, 7999, 700), (1024, 2048, 256), (3, 100000, 500)])
@pytest.mark.parametrize("srt", [False, True])
def test_clustered_topk_rows(B, N, K, srt):
    rng = np.random.default_rng(4000 + B + N + K)
    say(f"[refine] topk {B}x{N} K={K} sorted={srt}")
    topk_check(clustered(rng, B, N), K, srt)


@pytest.mark.parametrize("srt", [False, True])
def test_clustered_topk_rows_bf16(srt):
    rng = np.random.default_rng(4100)
    say(f"[refine] topk bf16 64x8000 K=1024 sorted={srt}")
    topk_check(clustered(rng, 64, 8000, sigma=2.0, wide=200.0), 1024, srt, bf16=True)


@pytest.mark.parametrize("B,N_pad", [(4, 8192), (128, 2048), (40, 5000)])
@pytest.mark.parametrize("srt", [False, True])
def test_clustered_fused_select(B, N_pad, srt):
    """Centroids near one common vector (plus small noise), a few of them scaled
    up: the scores cluster tightly with wide outliers."""
    rng = np.random.default_rng(4200 + B)
    base = rng.standard_normal(128).astype(np.float32)
    c = base + 0.02 * rng.standard_normal((B, N_pad, 128)).astype(np.float32)
    big = rng.random((B, N_pad)) < 0.03
    c[big] *= 4.0
    q = rng.standard_normal((B, 4, 128)).astype(np.float32)
    seq = np.minimum(rng.integers(N_pad * 8, N_pad * 16 + 1, B), N_pad * 16)
    K = 256
    cb, qb = synth.f32_to_bf16_bits(c), synth.f32_to_bf16_bits(q)
    x = synth.IndexerInputs(q=qb, c=cb, seq_len=seq.astype(np.int32), page_size=16, K=K,
                            sorted=srt, dtype="bf16", name="clustered")
    say(f"[refine] select B={B} N_pad={N_pad} sorted={srt}")
    ids = torch.full((B, K), POISON, dtype=torch.int32, device="cuda")
    counts = torch.full((B,), POISON, dtype=torch.int32, device="cuda")
    _, _, s = idx.idx_select(to_dev(qb), to_dev(cb), to_dev(x.seq_len), K, sorted=srt, ids=ids,
                             counts=counts, return_scores=True)
    torch.cuda.synchronize()
    s = s.cpu().numpy()
    S, A = oracle.score(x.q, x.c, x.seq_len, 16, "bf16")
    nv = oracle.n_valid(x.seq_len, 16, N_pad)
    check_scores(s, S, A, RTOL["bf16"])
    check_ids_exact(ids.cpu().numpy(), counts.cpu().numpy(), s, nv, K, srt)
    check_ids_band(ids.cpu().numpy(), S, A, nv, K, RTOL["bf16"])
