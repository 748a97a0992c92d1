"""CPU oracle for the block-scoring + top-K indexer.  TEST INFRASTRUCTURE ONLY.

Only the test suite, the smoke check and the benchmark's CPU-baseline leg may
import this package. The GPU library never calls it and shares no code with it.

It is a plain, slow, obviously correct restatement of what the indexer
computes, in float64 numpy with library primitives (a matrix product, a stable
sort, an argmax) as its only building blocks:

  pool_keys  c[b,n,:] = mean of the keys of the tokens of block n ("Round 15
          Track C Audit", section 2: the pooled keys are a stage of the indexer;
          reading: a block's pooled key is the mean of its tokens' keys).
  score   s[b,n] = sum_h sum_d q[b,h,d] * c[b,n,d] for every block n that holds
          tokens of request b; blocks past the request's last token are -inf.
          ("Iterate Centroids Score": the indexer's scorer rates each request's
          candidate pages from its query rows and the table of block
          centroids, feeding the downstream top-K; "Round 18 Track C", section
          1 Target 2: the per-block score sums the query heads' dot products
          with the block key over 128 dims.)
  score_paged  the same score for pages addressed through per-request page
          lists into a shared pool of centroids ("Iterate Centroids Score",
          submission contract and benchmark protocol: the scorer reads a
          request's pages through its context, from a pool of 16384 blocks).
  score_prefill  per-token scores of T prompt tokens, each token seeing the
          blocks up to the one that holds it ("Round 15 Track C Audit",
          section 1 Target 1: the prompt path scores tiles of query tokens
          against the block keys before each token's top-K).
  select  the K highest-scoring valid blocks of each row, ties to the lower
          block id ("Iterate Topk": top-K indices from per-segment scores;
          "Round 18 Track C", section 2: ids compared exactly, with
          adversarial ties and signed zeros).
  assign  a[i] = argmax_j (2 x_i.c_j - |c_j|^2), ties to the lower j
          ("Export Cake KMeans plan-runtime suite", Summary: KMeans assignment
          of bf16 points to centroids, with the centroid norms computed inside
          the call).

Readings of points the pages leave open (each stated where used):
  * a request's last, partly filled page is a candidate: n_valid =
    ceil(seq_len / page_size), capped at the padded table length;
  * -inf scores are never selected; NaN is outside the contract;
  * -0.0 and +0.0 are equal scores (a tie, broken by lower id);
  * fewer than K candidates: all of them are returned, the rest of the row is
    padded with -1;
  * the default output order is ascending block id (a set in canonical form);
    the sorted order is (score descending, id ascending).

Parity against the pages' own printed figures is unpinned: the pages print no
worked example with values. The oracle is pinned instead by closed forms,
brute force on tiny inputs and invariants (see tests/test_oracle_pins.py).
"""
from __future__ import annotations

import numpy as np

__all__ = ["bf16_decode", "to_f64", "n_valid", "pool_keys", "score", "score_paged",
           "score_prefill", "select", "select_row", "assign", "assign_scores"]


def bf16_decode(bits: np.ndarray) -> np.ndarray:
    """bf16 bit patterns -> float64. A bf16 value is the top half of a float32."""
    b = np.ascontiguousarray(bits, dtype=np.uint16)
    return (b.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def to_f64(a: np.ndarray, dtype: str) -> np.ndarray:
    if dtype == "bf16":
        return bf16_decode(a)
    if dtype == "f32":
        return np.asarray(a, dtype=np.float32).astype(np.float64)
    raise ValueError(dtype)


def n_valid(seq_len, page_size: int, n_pad: int) -> np.ndarray:
    """Blocks holding at least one token of the request, capped at the table length.

    Reading: the partly filled last page is a candidate ("Round 15 Track C Audit",
    section 1 Target 1 gives the tail block its own 'dead' state but never says
    it is dropped), so the count is the ceiling of seq_len / page_size.
    """
    s = np.asarray(seq_len, dtype=np.int64)
    return np.minimum(n_pad, (s + page_size - 1) // page_size)


def pool_keys(k, seq_len, n_pad: int, page_size: int, dtype: str):
    """Block means of the keys in float64, and the absolute means (error scale).

    k [B, S_pad, D]; request b holds tokens 0 .. seq_len[b]-1 (clamped to
    [0, S_pad]). For n < n_valid: C[b,n] = mean of k[b,s] over the tokens s of
    block n, s in [n*page_size, min((n+1)*page_size, seq_len[b])); M[b,n] = the
    mean of |k[b,s]|. Rows past n_valid are NaN (not produced).
    Returns (C, M, nv).
    """
    kf = to_f64(k, dtype)
    B, S_pad, D = kf.shape
    sl = np.clip(np.asarray(seq_len, dtype=np.int64), 0, S_pad)
    nv = n_valid(sl, page_size, n_pad)
    C = np.full((B, n_pad, D), np.nan)
    M = np.full((B, n_pad, D), np.nan)
    for b in range(B):
        for n in range(int(nv[b])):
            toks = kf[b, n * page_size:min((n + 1) * page_size, int(sl[b]))]
            C[b, n] = toks.mean(axis=0)
            M[b, n] = np.abs(toks).mean(axis=0)
    return C, M, nv


def score(q, c, seq_len, page_size: int, dtype: str):
    """Block scores in float64 and their rounding-error scale.

    Returns (S, A), both float64 [B, N_pad]:
      S[b,n] = sum_h sum_d q[b,h,d] c[b,n,d]   for n < n_valid[b], else -inf;
      A[b,n] = sum_h sum_d |q[b,h,d] c[b,n,d]| for n < n_valid[b], else 0.
    A is the classical scale of a dot product's rounding error
    (|fl(x.y) - x.y| <= gamma_n sum |x_i y_i|).
    Blocks past n_valid are not read (their contents are unspecified).
    ("Iterate Centroids Score", intro and memory template; "Round 18 Track C",
    section 1 Target 2.)
    """
    qf = to_f64(q, dtype)
    B, H, D = qf.shape
    N_pad = c.shape[1]
    nv = n_valid(seq_len, page_size, N_pad)
    S = np.full((B, N_pad), -np.inf)
    A = np.zeros((B, N_pad))
    for b in range(B):
        m = int(nv[b])
        if m == 0:
            continue
        cb = to_f64(c[b, :m], dtype)               # [m, D]
        per_head = cb @ qf[b].T                    # [m, H]: sum over d for each head
        S[b, :m] = per_head.sum(axis=1)            # then sum over heads
        A[b, :m] = (np.abs(cb) @ np.abs(qf[b]).T).sum(axis=1)
    return S, A


def score_paged(q, c_pool, indptr, indices, max_pages: int, dtype: str):
    """Scores of paged requests in float64, their error scale and slot counts.

    Request b owns slots i = 0 .. n_b - 1, n_b = min(max(indptr[b+1] - indptr[b],
    0), max_pages); slot i is pool row indices[indptr[b] + i]. A slot whose list
    position lies outside the list, or whose row lies outside the pool, is not
    a candidate (reading: such an entry names no page; it scores -inf).
    Returns (S, A, n_slots): S, A float64 [B, max_pages] as in score(), -inf / 0
    past a request's slots; n_slots int64 [B].
    ("Iterate Centroids Score", submission contract and benchmark protocol.)
    """
    qf = to_f64(q, dtype)
    B = qf.shape[0]
    pool = to_f64(c_pool, dtype)
    indptr = np.asarray(indptr, dtype=np.int64)
    indices = np.asarray(indices, dtype=np.int64)
    S = np.full((B, max_pages), -np.inf)
    A = np.zeros((B, max_pages))
    n_slots = np.zeros(B, dtype=np.int64)
    for b in range(B):
        lo = int(indptr[b])
        n = min(max(int(indptr[b + 1]) - lo, 0), max_pages)
        n_slots[b] = n
        pos = lo + np.arange(n)
        ok = (pos >= 0) & (pos < len(indices))
        rows = np.full(n, -1, dtype=np.int64)
        rows[ok] = indices[pos[ok]]
        ok &= (rows >= 0) & (rows < pool.shape[0])
        if not ok.any():
            continue
        cb = pool[rows[ok]]                         # [m, D], gathered through the list
        S[b, :n][ok] = (cb @ qf[b].T).sum(axis=1)   # sum over d per head, then over heads
        A[b, :n][ok] = (np.abs(cb) @ np.abs(qf[b]).T).sum(axis=1)
    return S, A, n_slots


def score_prefill(q, c, pos0, page_size: int, dtype: str):
    """Per-token scores of prompt tokens in float64, their error scale and counts.

    q [B,T,H,D], c [B,N_pad,D]. Token t of request b sits at position
    pos0[b] + t (negative pos0 counts as 0) and sees the blocks n < n_valid(
    pos0[b] + t + 1 tokens) -- the blocks up to the one that holds it (reading:
    causal attention over the prompt, with the same block count rule as the
    decode call).
    Returns (S, A, NV): S, A float64 [B,T,N_pad] as in score(); NV int64 [B,T].
    """
    qf = to_f64(q, dtype)
    B, T, H, D = qf.shape
    N_pad = c.shape[1]
    S = np.full((B, T, N_pad), -np.inf)
    A = np.zeros((B, T, N_pad))
    NV = np.zeros((B, T), dtype=np.int64)
    for b in range(B):
        p0 = max(int(pos0[b]), 0)
        nv = n_valid(p0 + np.arange(T) + 1, page_size, N_pad)
        NV[b] = nv
        m = int(nv.max())
        if m == 0:
            continue
        cb = to_f64(c[b, :m], dtype)                                   # [m, D]
        per = (cb @ qf[b].reshape(T * H, D).T).reshape(m, T, H).sum(axis=2)      # [m, T]
        per_abs = (np.abs(cb) @ np.abs(qf[b]).reshape(T * H, D).T).reshape(m, T, H).sum(axis=2)
        for t in range(T):
            S[b, t, :nv[t]] = per[:nv[t], t]
            A[b, t, :nv[t]] = per_abs[:nv[t], t]
    return S, A, NV


def select_row(s: np.ndarray, nv: int, K: int, sorted_out: bool) -> np.ndarray:
    """Top-K of one row: ids of the K largest scores among blocks < nv, ties to the
    lower id; -inf never selected. Returns int32[K], padded with -1.

    A stable sort by descending score keeps equal scores (signed zeros included,
    since -0.0 == +0.0) in ascending id order, which is the lower-id tie-break.
    """
    s = np.asarray(s)
    head = s[:nv]
    if np.isnan(head).any():
        raise ValueError("NaN score: outside the indexer's contract")
    cand = np.nonzero(head != -np.inf)[0]
    order = cand[np.argsort(-head[cand], kind="stable")]
    chosen = order[:K]
    if not sorted_out:
        chosen = np.sort(chosen)
    out = np.full(K, -1, dtype=np.int32)
    out[: len(chosen)] = chosen
    return out


def select(scores: np.ndarray, nv, K: int, sorted_out: bool = False):
    """Row-wise top-K ("Iterate Topk", intro). Returns (ids int32 [B,K], counts int32 [B])."""
    B, N = scores.shape
    nv = np.full(B, N) if nv is None else np.asarray(nv)
    ids = np.empty((B, K), dtype=np.int32)
    for b in range(B):
        ids[b] = select_row(scores[b], int(min(nv[b], N)), K, sorted_out)
    counts = (ids >= 0).sum(axis=1).astype(np.int32)
    return ids, counts


def assign_scores(x_bits: np.ndarray, c_bits: np.ndarray):
    """k-means assignment scores for the given points, float64 [n, C]:
    S[i,j] = 2 x_i.c_j - |c_j|^2, and the error scale A[i,j] = 2 sum|x c| + |c_j|^2.
    ("Export Cake KMeans plan-runtime suite", Summary and hot-path metric: the
    centroid norms are part of the assignment call.)"""
    x = bf16_decode(x_bits)
    c = bf16_decode(c_bits)
    cn = (c * c).sum(axis=1)
    S = 2.0 * (x @ c.T) - cn[None, :]
    A = 2.0 * (np.abs(x) @ np.abs(c).T) + cn[None, :]
    return S, A


def assign(x_bits: np.ndarray, c_bits: np.ndarray):
    """Nearest-centroid assignment: a[i] = argmax_j S[i,j], ties to the lower j
    (argmax returns the first maximum). Returns (a int32 [n], S, A)."""
    S, A = assign_scores(x_bits, c_bits)
    a = np.argmax(S, axis=1).astype(np.int32)
    return a, S, A
