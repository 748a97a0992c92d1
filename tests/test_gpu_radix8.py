"""IDX_RADIX8: the select with four 8-bit radix passes and no linear-bin pass
(the radix of the proposal seed in "Iterate Topk", section 6, and of the
four-pass loop in "Round 18 Track C", section 1 Target 1). It is defined to
return exactly what the library's own select returns, so ids, their order, the
-1 padding and the counts are compared word for word with the oracle's
selection: for idx_topk from the input scores, for idx_select from the GPU's
own scores (themselves checked against fp64). Outputs are poisoned with 0xa5
bytes first. Every launch shape: idx_topk's many short rows, 2- and 8-slot
rows and rows split into merged segments; idx_select's 1024-thread blocked and
striped workgroups and 512-thread ones with one or four key slots."""
import sys

import numpy as np
import pytest

torch = pytest.importorskip("torch")

import oracle
import synth
from tests.helpers import RTOL, check_ids_exact, check_scores, to_dev

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)

import block_scoring_top_amd as idx  # noqa: E402

POISON = -1515870811  # 0xa5a5a5a5


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def topk_radix8(scores, K, srt, nv=None):
    B, N = scores.shape
    ids = torch.full((B, K), POISON, dtype=torch.int32, device="cuda")
    counts = torch.full((B,), POISON, dtype=torch.int32, device="cuda")
    ws = torch.zeros(max(256, idx.idx_topk_workspace_bytes(B, N, K)), dtype=torch.uint8,
                     device="cuda")
    nvd = None if nv is None else torch.from_numpy(np.asarray(nv, np.int32)).to("cuda")
    idx.idx_topk(to_dev(scores), K, nvd, srt, ids=ids, counts=counts, ws=ws, radix8=True)
    torch.cuda.synchronize()
    check_ids_exact(ids.cpu().numpy(), counts.cpu().numpy(), scores, nv, K, srt)


# (rows, N, K): 256-thread workgroups (many rows of <= 2048); one 1024-thread
# workgroup per row in 2 slots (<= 8192 entries) or 8 (longer, many rows); few
# long rows cut into segments and merged (4 and 8 segments)
@pytest.mark.parametrize("B,N,K", [(1024, 2048, 256), (64, 8000, 1024), (9, 7999, 300),
                                   (600, 20000, 500), (9, 30000, 2048), (3, 100000, 100)])
@pytest.mark.parametrize("srt", [False, True])
def test_radix8_topk_stress_rows(B, N, K, srt):
    x = synth.make_topk(B, N, K, 8100 + B + N)
    say(f"[radix8] topk {B}x{N} K={K} sorted={srt}")
    topk_radix8(x.scores, K, srt)


@pytest.mark.parametrize("srt", [False, True])
def test_radix8_topk_clustered_and_valid_counts(srt):
    rng = np.random.default_rng(8200)
    say(f"[radix8] topk clustered 64x8000 K=1024 sorted={srt}")
    topk_radix8(synth.clustered_rows(rng, 64, 8000), 1024, srt)
    K, N = 256, 4500
    nv = np.array([0, 1, K - 1, K, K + 1, 1023, 1024, 1025, 4095, 4096, 4097, N] * 2, np.int32)
    say(f"[radix8] topk valid counts sorted={srt}")
    topk_radix8(synth.make_topk(nv.size, N, K, 8201).scores, K, srt, nv)


def test_radix8_topk_zeros_ties_and_neg_inf():
    rng = np.random.default_rng(8300)
    v = rng.choice(np.array([-0.0, 0.0, 1.0, -1.0, 2.0, -np.inf], np.float32), (8, 5000))
    v[2] = 0.0
    v[5] = -np.inf
    for srt in (False, True):
        say(f"[radix8] topk zeros, ties, -inf sorted={srt}")
        topk_radix8(v, 700, srt)


def select_radix8(x, K, srt):
    q, c, sl = to_dev(x.q), to_dev(x.c), to_dev(x.seq_len)
    B = x.q.shape[0]
    ids = torch.full((B, K), POISON, dtype=torch.int32, device="cuda")
    counts = torch.full((B,), POISON, dtype=torch.int32, device="cuda")
    _, _, s = idx.idx_select(q, c, sl, K, page_size=x.page_size, sorted=srt, ids=ids,
                             counts=counts, return_scores=True, radix8=True)
    torch.cuda.synchronize()
    s = s.cpu().numpy()
    S, A = oracle.score(x.q, x.c, x.seq_len, x.page_size, x.dtype)
    nv = oracle.n_valid(x.seq_len, x.page_size, x.N_pad)
    check_scores(s, S, A, RTOL[x.dtype])
    ids_np, counts_np = ids.cpu().numpy(), counts.cpu().numpy()
    check_ids_exact(ids_np, counts_np, s, nv, K, srt)
    # the library's own select on the same inputs returns the same words
    ids2, counts2, _ = idx.idx_select(q, c, sl, K, page_size=x.page_size, sorted=srt)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(ids2.cpu().numpy(), ids_np)
    np.testing.assert_array_equal(counts2.cpu().numpy(), counts_np)


# (B, H, N_pad): 1024-thread workgroups, blocked (N_pad <= 8192) and striped;
# 512-thread ones with one slot (N_pad <= 2048), four blocked, four striped
SELECT_SHAPES = [(4, 4, 8192), (2, 4, 20000), (128, 16, 2048), (64, 4, 4096), (40, 4, 10000)]


@pytest.mark.parametrize("B,H,N_pad", SELECT_SHAPES)
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("srt", [False, True])
def test_radix8_select_shapes(B, H, N_pad, dtype, srt):
    rng = np.random.default_rng(8400 + B + N_pad)
    seq = rng.integers(1, N_pad * 16 + 1, B)
    seq[0] = N_pad * 16
    x = synth.make_indexer(B, H, 128, N_pad, seq, 256, dtype, 8401 + B + N_pad, sorted_out=srt)
    say(f"[radix8] select B={B} H={H} N_pad={N_pad} {dtype} sorted={srt}")
    select_radix8(x, 256, srt)


def test_radix8_select_tiny_fp32_score_order():
    """The tiny fp32 call: one request of 1024 blocks, K = 256 in score order."""
    x = synth.make_indexer(1, 4, 128, 1024, [1024 * 16], 256, "f32", 8500, sorted_out=True)
    say("[radix8] select tiny fp32 sorted")
    select_radix8(x, 256, True)


def test_radix8_rejected_where_not_built():
    s = torch.zeros(4, 100, dtype=torch.bfloat16, device="cuda")
    with pytest.raises(idx.IdxError):
        idx.idx_topk_bf16(s, 10, radix8=True)
