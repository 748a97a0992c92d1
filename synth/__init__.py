"""Seeded synthetic inputs for the block-scoring + top-K indexer.

This module only draws random numbers and lays them out; it holds none of the
method's arithmetic (no scoring, no masking, no selection). Both the oracle
tests and the GPU path consume exactly the arrays produced here.

Shapes follow the workloads the pages tune on:
  * "Iterate Centroids Score" (memory-file template, benchmark protocol):
    query rows against a table of block centroids, head_dim 128, a few query
    heads, n_blocks in the thousands.
  * "Round 18 Track C ... qsa_score Query Hoisting" (section 1, Target 2):
    4 fp32 query heads of 128 dims scored against per-block keys.
  * "Iterate Topk" (memory-file template): top-K over per-segment scores drawn
    from a rotation of distributions.
  * "Export Cake KMeans plan-runtime suite" (Summary): nearest-centroid
    assignment of bf16 points.
No public dataset is involved; every input is synthetic.

bf16 values are carried as raw uint16 bit patterns. A float32 draw is rounded
to bf16 by round-to-nearest-even on its bit pattern (inputs never hold NaN).
"""
from __future__ import annotations

import dataclasses

import numpy as np

PAGE_SIZE = 16
BF16_POISON = np.uint16(0xFFFF)  # a bf16 NaN pattern used to fill padded tail rows


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bf16 (nearest, ties to even); return uint16 bits."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    r = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return r.astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Widen bf16 bit patterns to float32 (exact)."""
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


@dataclasses.dataclass
class IndexerInputs:
    """One indexer batch: q[B,H,D], c[B,N_pad,D], seq_len[B] (tokens)."""
    q: np.ndarray            # float32 or uint16 (bf16 bits)
    c: np.ndarray            # float32 or uint16 (bf16 bits)
    seq_len: np.ndarray      # int32 [B]
    page_size: int
    K: int
    sorted: bool
    dtype: str               # "f32" or "bf16"
    name: str

    @property
    def B(self):
        return self.q.shape[0]

    @property
    def H(self):
        return self.q.shape[1]

    @property
    def D(self):
        return self.q.shape[2]

    @property
    def N_pad(self):
        return self.c.shape[1]


@dataclasses.dataclass
class PagedInputs:
    """One paged indexer batch: q[B,H,D], a pool c_pool[n_rows,D] and per-request
    page lists indices[indptr[b]:indptr[b+1]] (CSR)."""
    q: np.ndarray            # float32 or uint16 (bf16 bits)
    c_pool: np.ndarray       # float32 or uint16 (bf16 bits)
    indptr: np.ndarray       # int32 [B+1]
    indices: np.ndarray      # int32 [indptr[B]]
    max_pages: int
    K: int
    sorted: bool
    dtype: str
    name: str

    @property
    def B(self):
        return self.q.shape[0]

    @property
    def H(self):
        return self.q.shape[1]


@dataclasses.dataclass
class TopkInputs:
    scores: np.ndarray       # float32 [B, N]
    K: int
    dists: list
    name: str


@dataclasses.dataclass
class AssignInputs:
    x: np.ndarray            # uint16 bf16 bits [N, D]
    c: np.ndarray            # uint16 bf16 bits [C, D]
    comp: np.ndarray         # int64 [N]: the mixture component each point was drawn from
    name: str


def _normal_f32(rng, shape):
    return rng.standard_normal(shape, dtype=np.float32)


def _poison_tail(c_bits: np.ndarray, seq_len: np.ndarray, page_size: int):
    """Fill centroid rows past each request's last page with NaN (a bf16 NaN
    pattern for bf16 bits, a float NaN for fp32), so that any read of a masked
    row shows up in a result."""
    n_pad = c_bits.shape[1]
    fill = np.float32(np.nan) if c_bits.dtype == np.float32 else BF16_POISON
    for b, s in enumerate(seq_len):
        nv = min(n_pad, -(-int(s) // page_size))
        c_bits[b, nv:, :] = fill


def make_indexer(B, H, D, N_pad, seq_len, K, dtype, seed, sorted_out=False,
                 page_size=PAGE_SIZE, name="custom", poison=True):
    """q and c i.i.d. N(0,1) (fp32, or rounded to bf16); padded tail poisoned."""
    rng = np.random.default_rng(seed)
    seq_len = np.asarray(seq_len, dtype=np.int64)
    if seq_len.ndim == 0:
        seq_len = np.full(B, int(seq_len))
    q = _normal_f32(rng, (B, H, D))
    c = _normal_f32(rng, (B, N_pad, D))
    if dtype == "bf16":
        q = f32_to_bf16_bits(q)
        c = f32_to_bf16_bits(c)
    if poison:
        _poison_tail(c, seq_len, page_size)
    return IndexerInputs(q=q, c=c, seq_len=seq_len.astype(np.int32), page_size=page_size,
                         K=K, sorted=sorted_out, dtype=dtype, name=name)


def make_integer_indexer(B, H, D, N_pad, seq_len, K, dtype, seed, lo=-3, hi=3,
                         page_size=PAGE_SIZE, name="integer"):
    """q, c with small integer entries: every partial sum is an exact integer in fp32."""
    rng = np.random.default_rng(seed)
    q = rng.integers(lo, hi, (B, H, D), endpoint=True).astype(np.float32)
    c = rng.integers(lo, hi, (B, N_pad, D), endpoint=True).astype(np.float32)
    seq_len = np.asarray(seq_len, dtype=np.int32)
    if dtype == "bf16":
        q = f32_to_bf16_bits(q)
        c = f32_to_bf16_bits(c)
    return IndexerInputs(q=q, c=c, seq_len=seq_len, page_size=page_size, K=K,
                         sorted=False, dtype=dtype, name=name)


# ---- paged centroid pools ("Iterate Centroids Score", benchmark protocol) -------------
# page-count regimes N(mean, std) per request; the pages name the smallest and the
# largest, and the three between are taken as the doublings in between
PAGE_REGIMES = [(256, 64), (512, 128), (1024, 256), (2048, 512), (4096, 1024)]
PAGED_BATCHES = [1, 4, 16, 32, 64]
POOL_BLOCKS = 16384


def make_paged(B, H, D, n_rows, pages, K, dtype, seed, sorted_out=False, max_pages=None,
               name="custom"):
    """q i.i.d. N(0,1); a pool of n_rows N(0,1) centroids; request b's page list is
    pages[b] distinct pool rows drawn uniformly (lists of different requests may
    share rows). pages: per-request counts, or (mean, std) of a normal regime
    (rounded, clipped to [1, n_rows])."""
    rng = np.random.default_rng(seed)
    if isinstance(pages, tuple):
        mu, sd = pages
        counts = np.clip(np.rint(rng.normal(mu, sd, B)), 1, n_rows).astype(np.int64)
    else:
        counts = np.asarray(pages, dtype=np.int64)
    q = _normal_f32(rng, (B, H, D))
    pool = _normal_f32(rng, (n_rows, D))
    lists = [rng.choice(n_rows, int(n), replace=False) for n in counts]
    indptr = np.zeros(B + 1, dtype=np.int64)
    indptr[1:] = np.cumsum(counts)
    indices = (np.concatenate(lists) if len(lists) else np.zeros(0)).astype(np.int32)
    if dtype == "bf16":
        q = f32_to_bf16_bits(q)
        pool = f32_to_bf16_bits(pool)
    mp = int(counts.max()) if max_pages is None else int(max_pages)
    return PagedInputs(q=q, c_pool=pool, indptr=indptr.astype(np.int32), indices=indices,
                       max_pages=mp, K=K, sorted=sorted_out, dtype=dtype, name=name)


# ---- keys of the cache, pooled into block centroids -----------------------------------
@dataclasses.dataclass
class KeysInputs:
    """Keys k[B,S_pad,D] of B requests holding seq_len[b] tokens each."""
    k: np.ndarray            # float32 or uint16 (bf16 bits)
    seq_len: np.ndarray      # int32 [B]
    N_pad: int
    page_size: int
    dtype: str
    name: str

    @property
    def B(self):
        return self.k.shape[0]


def make_keys(B, S_pad, D, N_pad, seq_len, dtype, seed, page_size=PAGE_SIZE, name="custom"):
    """Keys i.i.d. N(0,1) (rounded to bf16); token rows past a request's length
    poisoned with a bf16 NaN."""
    rng = np.random.default_rng(seed)
    k = _normal_f32(rng, (B, S_pad, D))
    seq_len = np.asarray(seq_len, dtype=np.int64)
    if dtype == "bf16":
        k = f32_to_bf16_bits(k)
        for b, sl in enumerate(seq_len):
            k[b, max(int(sl), 0):] = BF16_POISON
    return KeysInputs(k=k, seq_len=seq_len.astype(np.int32), N_pad=N_pad, page_size=page_size,
                      dtype=dtype, name=name)


# ---- prompt (prefill) tokens ("Round 15 Track C Audit", section 1 Target 1) -----------
@dataclasses.dataclass
class PrefillInputs:
    """T prompt tokens per request: q[B,T,H,D], c[B,N_pad,D], pos0[B]."""
    q: np.ndarray            # uint16 bf16 bits (or float32)
    c: np.ndarray
    pos0: np.ndarray         # int32 [B]
    page_size: int
    K: int
    sorted: bool
    dtype: str
    name: str

    @property
    def B(self):
        return self.q.shape[0]

    @property
    def T(self):
        return self.q.shape[1]

    @property
    def H(self):
        return self.q.shape[2]

    @property
    def N_pad(self):
        return self.c.shape[1]


def make_prefill(B, T, H, D, N_pad, pos0, K, seed, dtype="bf16", sorted_out=False,
                 page_size=PAGE_SIZE, integer=False, name="custom"):
    """q and c i.i.d. N(0,1), fp32 or rounded to bf16 (or small integers);
    centroid rows past the last token's block poisoned with NaN."""
    rng = np.random.default_rng(seed)
    pos0 = np.asarray(pos0, dtype=np.int64)
    if integer:
        q = rng.integers(-3, 3, (B, T, H, D), endpoint=True).astype(np.float32)
        c = rng.integers(-3, 3, (B, N_pad, D), endpoint=True).astype(np.float32)
    else:
        q = _normal_f32(rng, (B, T, H, D))
        c = _normal_f32(rng, (B, N_pad, D))
    if dtype == "bf16":
        q = f32_to_bf16_bits(q)
        c = f32_to_bf16_bits(c)
    _poison_tail(c, np.maximum(pos0, 0) + T, page_size)
    return PrefillInputs(q=q, c=c, pos0=pos0.astype(np.int32), page_size=page_size, K=K,
                         sorted=sorted_out, dtype=dtype, name=name)


# ---- the distribution rotation of the top-K stress rows -------------------------------
TOPK_DISTS = ["normal", "uniform", "lognormal", "zipf", "all_equal", "quant8",
              "sorted_asc", "sorted_desc", "normal_half_neginf"]


def topk_row(rng, dist: str, n: int) -> np.ndarray:
    if dist == "normal":
        return rng.standard_normal(n).astype(np.float32)
    if dist == "uniform":
        return rng.random(n).astype(np.float32)
    if dist == "lognormal":
        return rng.lognormal(0.0, 2.0, n).astype(np.float32)
    if dist == "zipf":
        return rng.zipf(1.1, n).astype(np.float32)
    if dist == "all_equal":
        return np.ones(n, dtype=np.float32)
    if dist == "quant8":
        return rng.integers(0, 8, n).astype(np.float32)
    if dist == "sorted_asc":
        return np.sort(rng.standard_normal(n)).astype(np.float32)
    if dist == "sorted_desc":
        return np.sort(rng.standard_normal(n))[::-1].astype(np.float32)
    if dist == "normal_half_neginf":
        r = rng.standard_normal(n).astype(np.float32)
        r[rng.permutation(n)[: n // 2]] = -np.inf
        return r
    raise ValueError(dist)


def clustered_rows(rng, B, N, sigma=0.2, wide=10.0, frac=0.05):
    """Rows whose scores form a tight cluster (N(0, sigma)) plus a fraction of
    wide outliers (N(0, wide)) that stretch the row's range: the linear bin of
    the K-th score then holds hundreds of distinct keys."""
    v = rng.normal(0.0, sigma, (B, N))
    out = rng.random((B, N)) < frac
    v[out] = rng.normal(0.0, wide, int(out.sum()))
    return v.astype(np.float32)


def make_topk(B, N, K, seed, dists=None, name="custom"):
    rng = np.random.default_rng(seed)
    dists = TOPK_DISTS if dists is None else dists
    rows, used = [], []
    for r in range(B):
        d = dists[r % len(dists)]
        rows.append(topk_row(rng, d, N))
        used.append(d)
    return TopkInputs(scores=np.stack(rows).astype(np.float32), K=K, dists=used, name=name)


def make_assign(N, C, D, seed, sigma=0.1, name="custom"):
    """Points drawn from a mixture of C Gaussians (std sigma) around bf16 centres
    drawn from N(0,1); the centroids are those centres."""
    rng = np.random.default_rng(seed)
    centres = f32_to_bf16_bits(_normal_f32(rng, (C, D)))
    comp = rng.integers(0, C, N)
    noise = _normal_f32(rng, (N, D))
    x = bf16_bits_to_f32(centres)[comp] + np.float32(sigma) * noise
    return AssignInputs(x=f32_to_bf16_bits(x), c=centres, comp=comp, name=name)


# ---- the five named workloads ----------------------------------------------------------
WORKLOADS = {
    1: "tiny fp32 indexer: B=1 H=4 D=128 N=1024 K=256 sorted",
    2: "variable-length decode batch: B=4 H=4 D=128 bf16 N_pad=8192 K=256",
    3: "top-K stress: 64 rows x 30000 fp32, K=2048, 9-distribution rotation",
    4: "large GQA decode batch: B=128 H=16 D=128 bf16 N_pad=2048 K=256",
    5: "nearest-centroid assignment: 2^20 x 128 bf16 points, C=1024",
    6: "paged pool: B=64 H=4 D=128 bf16, pages per request N(4096,1024) of 16384, K=256",
    7: "prompt tokens: B=2 T=512 H=4 D=128 bf16, pos0 {4096, 30000}, N_pad=1920, K=256",
    8: "pooled keys: B=4 bf16 keys, seq_len {4096, 16384, 65536, 131072}, 16-token blocks",
    9: "top-K stress in bf16: the 64 x 30000 stress rows rounded to bf16, K=2048",
    10: "clustered top-K rows: 64 x 8000 fp32, 95% N(0, 0.2) and 5% N(0, 10), K=1024",
}


def workload(n: int, seed: int | None = None):
    """Inputs of workload n (1..8), seeded with n unless a seed is given."""
    s = n if seed is None else seed
    if n == 1:
        return make_indexer(1, 4, 128, 1024, [16384], 256, "f32", s, sorted_out=True,
                            name="w1_tiny_f32")
    if n == 2:
        return make_indexer(4, 4, 128, 8192, [4096, 16384, 65536, 131072], 256, "bf16", s,
                            name="w2_varlen_bf16")
    if n == 3:
        return make_topk(64, 30000, 2048, s, name="w3_topk_stress")
    if n == 4:
        rng = np.random.default_rng(s)
        seq_len = rng.integers(8192, 32768, 128, endpoint=True)
        # q and c continue from the same generator state, after seq_len
        q = f32_to_bf16_bits(_normal_f32(rng, (128, 16, 128)))
        c = f32_to_bf16_bits(_normal_f32(rng, (128, 2048, 128)))
        _poison_tail(c, seq_len, PAGE_SIZE)
        return IndexerInputs(q=q, c=c, seq_len=seq_len.astype(np.int32), page_size=PAGE_SIZE,
                             K=256, sorted=False, dtype="bf16", name="w4_gqa_bf16")
    if n == 5:
        return make_assign(1 << 20, 1024, 128, s, name="w5_kmeans_assign")
    if n == 6:
        return make_paged(64, 4, 128, POOL_BLOCKS, PAGE_REGIMES[-1], 256, "bf16", s,
                          name="w6_paged_bf16")
    if n == 7:
        return make_prefill(2, 512, 4, 128, 1920, [4096, 30000], 256, s, name="w7_prefill_bf16")
    if n == 8:
        return make_keys(4, 131072, 128, 8192, [4096, 16384, 65536, 131072], "bf16", s,
                         name="w8_pool_keys_bf16")
    if n == 9:
        # the rows of the top-K stress workload (its seed, 3, unless one is given)
        x = make_topk(64, 30000, 2048, 3 if seed is None else seed, name="w9_topk_stress_bf16")
        x.scores = f32_to_bf16_bits(x.scores)
        return x
    if n == 10:
        rng = np.random.default_rng(s)
        return TopkInputs(scores=clustered_rows(rng, 64, 8000), K=1024, dists=["clustered"] * 64,
                          name="w10_topk_clustered")
    raise ValueError(n)
