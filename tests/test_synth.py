"""Pins of the seeded input generators (no GPU)."""
import hashlib

import numpy as np
import torch

import synth


def test_bf16_rounding_matches_torch():
    rng = np.random.default_rng(0)
    x = np.concatenate([rng.standard_normal(100000).astype(np.float32),
                        rng.lognormal(0, 8, 10000).astype(np.float32),
                        np.array([1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, -0.0, 0.0, 65504.0,
                                  3.0e38, 1e-40], np.float32)])
    ours = synth.f32_to_bf16_bits(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(ours, ref)
    back = synth.bf16_bits_to_f32(ours)
    np.testing.assert_array_equal(back, torch.from_numpy(x).to(torch.bfloat16).float().numpy())


def _digest(*arrays):
    h = hashlib.sha256()
    for a in arrays:
        h.update(np.ascontiguousarray(a).tobytes())
    return h.hexdigest()[:16]


def test_generators_are_deterministic():
    a = synth.workload(2)
    b = synth.workload(2)
    assert _digest(a.q, a.c, a.seq_len) == _digest(b.q, b.c, b.seq_len)
    c = synth.workload(2, seed=99)
    assert _digest(a.q) != _digest(c.q)


def test_workload_shapes_and_structure():
    w1 = synth.workload(1)
    assert w1.q.shape == (1, 4, 128) and w1.c.shape == (1, 1024, 128) and w1.q.dtype == np.float32
    assert w1.K == 256 and w1.sorted
    w2 = synth.workload(2)
    assert w2.c.shape == (4, 8192, 128) and w2.c.dtype == np.uint16
    assert list(w2.seq_len) == [4096, 16384, 65536, 131072]
    assert (w2.c[0, 256:] == 0xFFFF).all() and (w2.c[0, :256] != 0xFFFF).all()
    w3 = synth.workload(3)
    assert w3.scores.shape == (64, 30000) and w3.K == 2048
    assert w3.dists[:9] == synth.TOPK_DISTS and w3.dists[9] == "normal"
    r8 = w3.scores[8]
    assert (r8 == -np.inf).sum() == 15000
    assert (w3.scores[4] == 1.0).all()
    assert set(np.unique(w3.scores[5])) <= set(range(8))
    assert np.all(np.diff(w3.scores[6]) >= 0) and np.all(np.diff(w3.scores[7]) <= 0)
    w4 = synth.workload(4)
    assert w4.q.shape == (128, 16, 128) and w4.c.shape == (128, 2048, 128)
    assert w4.seq_len.min() >= 8192 and w4.seq_len.max() <= 32768


def test_bf16_and_clustered_topk_workloads():
    w3, w9 = synth.workload(3), synth.workload(9)
    assert w9.scores.dtype == np.uint16 and w9.scores.shape == w3.scores.shape
    # workload 9 is workload 3's rows rounded to bf16
    np.testing.assert_array_equal(w9.scores, synth.f32_to_bf16_bits(w3.scores))
    w10 = synth.workload(10)
    assert w10.scores.shape == (64, 8000) and w10.K == 1024
    v = w10.scores
    inside = np.abs(v) < 1.0
    assert 0.9 < inside.mean() < 0.99            # the tight cluster
    assert np.abs(v).max() > 20.0                # the wide outliers stretch the range


def test_assign_generator_structure():
    x = synth.make_assign(1000, 64, 128, 5)
    assert x.x.shape == (1000, 128) and x.c.shape == (64, 128)
    xf = synth.bf16_bits_to_f32(x.x)
    cf = synth.bf16_bits_to_f32(x.c)
    dev = xf - cf[x.comp]
    assert 0.08 < dev.std() < 0.12
