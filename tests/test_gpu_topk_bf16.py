"""idx_topk_bf16 (bf16 scores, 16-bit keys: "Iterate Topk", section 6) against the
oracle's selection from the exact values of the same bf16 patterns: ids, their
order, the -1 padding and the counts compared word for word, outputs poisoned
with 0xa5 bytes first. Every launch shape the host chooses between: few long
rows cut into segments and merged, one 2-slot or 8-slot workgroup per row, and
many short rows in 256-thread workgroups."""
import sys

import numpy as np
import pytest

torch = pytest.importorskip("torch")

import oracle
import synth

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)

import block_scoring_top_amd as idx  # noqa: E402

POISON = -1515870811  # 0xa5a5a5a5


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def bf16_rows(B, N, seed, dists=None):
    """The top-K stress rows (nine rotating distributions) rounded to bf16."""
    x = synth.make_topk(B, N, 1, seed, dists=dists)
    return synth.f32_to_bf16_bits(x.scores)


def dev_bf16(bits):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to("cuda").view(
        torch.bfloat16)


def run_and_check(bits, K, srt, nv=None):
    B, N = bits.shape
    ids = torch.full((B, K), POISON, dtype=torch.int32, device="cuda")
    counts = torch.full((B,), POISON, dtype=torch.int32, device="cuda")
    ws = torch.zeros(max(256, idx.idx_topk_workspace_bytes(B, N, K)), dtype=torch.uint8,
                     device="cuda")
    nvd = None if nv is None else torch.from_numpy(np.asarray(nv, np.int32)).to("cuda")
    idx.idx_topk_bf16(dev_bf16(bits), K, nvd, srt, ids=ids, counts=counts, ws=ws)
    torch.cuda.synchronize()
    vals = oracle.bf16_decode(bits)
    ids_ref, counts_ref = oracle.select(vals, nv, K, srt)
    np.testing.assert_array_equal(counts.cpu().numpy(), counts_ref)
    got = ids.cpu().numpy()
    for b in range(B):
        if not np.array_equal(got[b], ids_ref[b]):
            d = np.nonzero(got[b] != ids_ref[b])[0]
            raise AssertionError(f"row {b}: {d.size} slots differ, first at {d[0]}: "
                                 f"gpu {got[b, d[0]]} oracle {ids_ref[b, d[0]]}")


@pytest.mark.parametrize("srt", [False, True])
def test_bf16_stress_rows_split_and_merged(srt):
    """64 rows x 30000, K = 2048: segments selected apart, merged by the last."""
    bits = bf16_rows(64, 30000, 70)
    say(f"[bf16] 64x30000 K=2048 sorted={srt}")
    run_and_check(bits, 2048, srt)


@pytest.mark.parametrize("B,N,K", [(64, 8000, 1024), (9, 7999, 300), (4, 100000, 100),
                                   (3, 40001, 4096), (1024, 2048, 256), (600, 1500, 1000)])
@pytest.mark.parametrize("srt", [False, True])
def test_bf16_row_shapes(B, N, K, srt):
    bits = bf16_rows(B, N, 71 + B + N)
    say(f"[bf16] {B}x{N} K={K} sorted={srt}")
    run_and_check(bits, K, srt)


@pytest.mark.parametrize("srt", [False, True])
def test_bf16_valid_counts_at_the_boundaries(srt):
    K, N = 256, 4500
    nv = np.array([0, 1, 2, K - 1, K, K + 1, 255, 256, 257, 1023, 1024, 1025, 2047, 2048, 2049,
                   4095, 4096, 4097, N] * 2, dtype=np.int32)
    bits = bf16_rows(nv.size, N, 72)
    say(f"[bf16] valid counts sorted={srt}")
    run_and_check(bits, K, srt, nv)


def test_bf16_signed_zeros_ties_and_neg_inf():
    rng = np.random.default_rng(73)
    B, N, K = 8, 5000, 700
    v = rng.choice(np.array([-0.0, 0.0, 1.0, -1.0, 2.0, -np.inf], np.float32), (B, N))
    v[2] = 0.0
    v[3] = -0.0
    v[4, ::2] = -np.inf
    v[5] = -np.inf               # no candidates at all
    bits = synth.f32_to_bf16_bits(v)
    for srt in (False, True):
        say(f"[bf16] zeros, ties, -inf sorted={srt}")
        run_and_check(bits, K, srt)


def test_bf16_dtype_dispatch_through_idx_topk():
    bits = bf16_rows(16, 3000, 74)
    ids_a, _ = idx.idx_topk(dev_bf16(bits), 100)
    ids_b, _ = idx.idx_topk_bf16(dev_bf16(bits), 100)
    torch.cuda.synchronize()
    assert torch.equal(ids_a, ids_b)
