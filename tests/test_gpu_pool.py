"""GPU parity of idx_pool_keys (block means of the keys) against the CPU oracle,
and the pooled centroids feeding idx_select."""
import sys

import numpy as np
import pytest

torch = pytest.importorskip("torch")

import oracle
import synth
from tests.helpers import check_ids_exact, to_dev

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)

import block_scoring_top_amd as idx  # noqa: E402

SENTINEL_BF16 = np.uint16(0x7F7F)   # a finite bf16 pattern a mean of N(0,1) keys cannot hit


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def out_values(c_gpu, dtype):
    a = c_gpu.cpu()
    if dtype == "bf16":
        bits = a.view(torch.int16).numpy().view(np.uint16)
        return bits, synth.bf16_bits_to_f32(bits).astype(np.float64)
    v = a.numpy()
    return v.view(np.uint32), v.astype(np.float64)


def pool_check(x):
    """Within the fp32-sum bound plus the output rounding; rows past each
    request's blocks are left as they were."""
    say(f"[pool] {x.name} B={x.B} S_pad={x.k.shape[1]} N_pad={x.N_pad} page={x.page_size} "
        f"{x.dtype}")
    kd = to_dev(x.k)
    if x.dtype == "bf16":
        c0 = np.full((x.B, x.N_pad, 128), SENTINEL_BF16, np.uint16)
    else:
        c0 = np.full((x.B, x.N_pad, 128), 7.5e37, np.float32)
    c = to_dev(c0)
    idx.idx_pool_keys(kd, to_dev(x.seq_len), x.N_pad, x.page_size, c=c)
    torch.cuda.synchronize()
    bits, got = out_values(c, x.dtype)
    C, M, nv = oracle.pool_keys(x.k, x.seq_len, x.N_pad, x.page_size, x.dtype)
    for b in range(x.B):
        m = int(nv[b])
        err = np.abs(got[b, :m] - C[b, :m])
        if x.dtype == "bf16":
            tol = 2.0 ** -8 * np.abs(C[b, :m]) + 2.0 ** -17 * M[b, :m]
        else:
            tol = 2.0 ** -23 * np.abs(C[b, :m]) + 2.0 ** -19 * M[b, :m]
        bad = np.argwhere(err > tol)
        assert bad.size == 0, f"request {b}: {len(bad)} values out of tolerance, first {bad[0]}"
        untouched = bits[b, m:]
        want = SENTINEL_BF16 if x.dtype == "bf16" else np.float32(7.5e37).view(np.uint32)
        assert (untouched == want).all(), f"request {b}: rows past its blocks were written"
    return c, C, nv


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("page", [16, 7])
def test_pool_small_ragged(dtype, page):
    x = synth.make_keys(4, 700, 128, 100, [700, 0, 333, 5000], dtype, 800 + page, page_size=page,
                        name="ragged")
    pool_check(x)


def test_pool_blocks_of_equal_keys_are_exact():
    """Every token of a block holds the same key: the mean is that key, bit for bit."""
    rng = np.random.default_rng(801)
    base = synth.f32_to_bf16_bits(rng.standard_normal((2, 40, 128)).astype(np.float32))
    k = np.repeat(base, 16, axis=1)                        # [2, 640, 128]
    x = synth.KeysInputs(k=k, seq_len=np.array([640, 630], np.int32), N_pad=40, page_size=16,
                         dtype="bf16", name="equal")
    c, _, nv = pool_check(x)
    bits, _ = out_values(c, "bf16")
    np.testing.assert_array_equal(bits[0], base[0])
    np.testing.assert_array_equal(bits[1, :nv[1]], base[1, :nv[1]])


def test_pooled_centroids_feed_the_select():
    """Pool, then select on the pooled table: the ids equal the oracle's
    selection on the scores of exactly those centroids."""
    x = synth.make_keys(3, 4096, 128, 256, [4096, 1000, 17], "bf16", 802, name="feed")
    q = synth.f32_to_bf16_bits(np.random.default_rng(803).standard_normal((3, 4, 128))
                               .astype(np.float32))
    c = idx.idx_pool_keys(to_dev(x.k), to_dev(x.seq_len), x.N_pad, 16)
    ids, counts, s = idx.idx_select(to_dev(q), c, to_dev(x.seq_len), 64, return_scores=True)
    torch.cuda.synchronize()
    c_bits = c.cpu().view(torch.int16).numpy().view(np.uint16)
    S, A = oracle.score(q, c_bits, x.seq_len, 16, "bf16")
    s_np = s.cpu().numpy()
    valid = S != -np.inf
    assert (np.abs(s_np[valid] - S[valid]) <= 2e-3 * A[valid]).all()
    nv = oracle.n_valid(x.seq_len, 16, x.N_pad)
    check_ids_exact(ids.cpu().numpy(), counts.cpu().numpy(), s_np, nv, 64, False)


def test_pool_workload_full_size():
    pool_check(synth.workload(8))
