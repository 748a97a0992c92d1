"""Pins of the CPU oracle against facts that do not come from the oracle itself:
values the pages print, closed forms, brute force on tiny inputs, exact rational
arithmetic, library routines of a different kind, and invariants.

Each test is chosen so that a plausible slip in the oracle (a dropped head, a
wrong sign, a transposed operand, an off-by-one in the mask, a broken
tie-break) fails at least one of them.
"""
import heapq
import itertools
import os
from fractions import Fraction

import numpy as np
import pytest

import oracle
import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# ----------------------------------------------------------------------------------------
# block counts (the masking rule)
# ----------------------------------------------------------------------------------------
def _golden_rows(name):
    rows = []
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            rows.append(line.split())
    return rows


def test_block_counts_match_the_pages():
    rows = _golden_rows("block_counts.txt")
    assert len(rows) >= 3
    for bs, ntok, nb, _cite in rows:
        got = oracle.n_valid([int(ntok)], int(bs), 1 << 30)[0]
        assert got == int(nb), (bs, ntok, nb)


def test_block_count_cap_and_zero():
    assert list(oracle.n_valid([0, 1, 16, 17, 10 ** 9], 16, 100)) == [0, 1, 1, 2, 100]


# ----------------------------------------------------------------------------------------
# bf16 decoding (from the format's definition: sign, 8 exponent bits, 7 fraction bits)
# ----------------------------------------------------------------------------------------
def test_bf16_decode_known_patterns():
    bits = np.array([0x3F80, 0xC000, 0x0000, 0x8000, 0x7F80, 0xFF80, 0x3F81, 0x0001, 0x4049],
                    dtype=np.uint16)
    want = [1.0, -2.0, 0.0, -0.0, np.inf, -np.inf, 1.0 + 2.0 ** -7, 2.0 ** -133, 3.140625]
    got = oracle.bf16_decode(bits)
    for g, w in zip(got, want):
        assert g == w and np.signbit(g) == np.signbit(w)


# ----------------------------------------------------------------------------------------
# scores: closed forms
# ----------------------------------------------------------------------------------------
def _f32(x):
    return np.asarray(x, dtype=np.float32)


def test_score_all_ones_centroids_is_sum_of_queries():
    """c_n = (1,...,1) for every block: each score is the plain sum of all query entries."""
    rng = np.random.default_rng(11)
    q = _f32(rng.integers(-4, 5, (2, 3, 16)))
    c = np.ones((2, 10, 16), dtype=np.float32)
    S, _ = oracle.score(q, c, [160, 70], 16, "f32")
    for b in range(2):
        total = sum(int(v) for v in q[b].ravel())
        nv = [10, 5][b]
        assert np.all(S[b, :nv] == total)
        assert np.all(S[b, nv:] == -np.inf)


def test_score_one_hot_counts_matching_heads():
    """q_h = e_{i_h}, c_n = alpha_n e_{j_n}: s_n = alpha_n * #{h : i_h == j_n}."""
    rng = np.random.default_rng(12)
    B, H, D, N = 3, 8, 32, 40
    i_h = rng.integers(0, 4, (B, H))
    j_n = rng.integers(0, 6, (B, N))
    alpha = rng.integers(-9, 10, (B, N))
    q = np.zeros((B, H, D), np.float32)
    c = np.zeros((B, N, D), np.float32)
    for b in range(B):
        for h in range(H):
            q[b, h, i_h[b, h]] = 1.0
        for n in range(N):
            c[b, n, j_n[b, n]] = alpha[b, n]
    S, A = oracle.score(q, c, [N * 16] * B, 16, "f32")
    for b in range(B):
        for n in range(N):
            k = sum(1 for h in range(H) if i_h[b, h] == j_n[b, n])
            assert S[b, n] == alpha[b, n] * k
            assert A[b, n] == abs(alpha[b, n]) * k


def test_score_one_hot_column_pick():
    """c_n = e_j picks column j of every head: s = sum_h q[h, j] (no products involved)."""
    rng = np.random.default_rng(13)
    q = rng.standard_normal((1, 5, 8)).astype(np.float32)
    c = np.zeros((1, 8, 8), np.float32)
    for n in range(8):
        c[0, n, n] = 1.0
    S, _ = oracle.score(q, c, [8 * 16], 16, "f32")
    for n in range(8):
        want = sum(Fraction(float(v)) for v in q[0, :, n])
        assert Fraction(S[0, n]) == want


def test_score_exact_against_rationals():
    """Brute force in exact rational arithmetic: float64 result within 1e-15 * A."""
    rng = np.random.default_rng(14)
    B, H, D, N = 2, 3, 12, 7
    q = rng.standard_normal((B, H, D)).astype(np.float32)
    c = rng.standard_normal((B, N, D)).astype(np.float32)
    S, A = oracle.score(q, c, [N * 16, 3 * 16 + 1], 16, "f32")
    for b in range(B):
        nv = [N, 4][b]
        for n in range(N):
            if n >= nv:
                assert S[b, n] == -np.inf and A[b, n] == 0
                continue
            exact = sum(Fraction(float(q[b, h, d])) * Fraction(float(c[b, n, d]))
                        for h in range(H) for d in range(D))
            assert abs(Fraction(S[b, n]) - exact) <= Fraction(1e-15) * Fraction(A[b, n])


def test_score_bf16_integer_inputs_are_exact():
    x = synth.make_integer_indexer(2, 4, 128, 64, [64 * 16, 20 * 16 + 3], 8, "bf16", 15)
    S, _ = oracle.score(x.q, x.c, x.seq_len, 16, "bf16")
    qf = synth.bf16_bits_to_f32(x.q).astype(np.int64)
    cf = synth.bf16_bits_to_f32(x.c).astype(np.int64)
    for b in range(2):
        nv = [64, 21][b]
        for n in range(0, nv, 7):
            want = int(sum(int(qf[b, h] @ cf[b, n]) for h in range(4)))
            assert S[b, n] == want
        assert np.all(S[b, nv:] == -np.inf)


def test_score_heads_are_additive_and_blocks_are_not_mixed():
    rng = np.random.default_rng(16)
    q = rng.standard_normal((1, 4, 16)).astype(np.float32)
    c = rng.standard_normal((1, 9, 16)).astype(np.float32)
    S, _ = oracle.score(q, c, [9 * 16], 16, "f32")
    parts = sum(oracle.score(q[:, h:h + 1], c, [9 * 16], 16, "f32")[0] for h in range(4))
    np.testing.assert_allclose(S, parts, rtol=0, atol=1e-12)
    perm = rng.permutation(9)
    Sp, _ = oracle.score(q, c[:, perm], [9 * 16], 16, "f32")
    np.testing.assert_array_equal(Sp[0], S[0, perm])
    S2, _ = oracle.score(2 * q, c, [9 * 16], 16, "f32")
    np.testing.assert_array_equal(S2, 2 * S)


def test_score_never_reads_masked_rows():
    x = synth.make_indexer(2, 4, 128, 64, [100, 0], 8, "bf16", 17)
    assert (x.c[0, 7:] == 0xFFFF).all() and (x.c[1] == 0xFFFF).all()
    S, A = oracle.score(x.q, x.c, x.seq_len, 16, "bf16")
    assert np.isfinite(S[0, :7]).all()
    assert (S[0, 7:] == -np.inf).all() and (S[1] == -np.inf).all()
    assert not np.isnan(A).any()


# ----------------------------------------------------------------------------------------
# paged scores: page lists into a shared pool
# ----------------------------------------------------------------------------------------
def test_score_paged_exact_against_rationals_through_the_lists():
    """Brute force: each slot's exact rational score through its list entry."""
    rng = np.random.default_rng(30)
    B, H, D, R = 3, 2, 10, 9
    q = rng.standard_normal((B, H, D)).astype(np.float32)
    pool = rng.standard_normal((R, D)).astype(np.float32)
    indptr = np.array([0, 4, 4, 11])
    indices = np.array([8, 0, 8, 3, 5, 1, 2, 7, 6, 4, 0])   # row 8 listed twice by request 0
    S, A, n = oracle.score_paged(q, pool, indptr, indices, 6, "f32")
    np.testing.assert_array_equal(n, [4, 0, 6])              # request 2 clamped to 6 slots
    for b in range(B):
        for i in range(6):
            if i >= n[b]:
                assert S[b, i] == -np.inf and A[b, i] == 0
                continue
            r = indices[indptr[b] + i]
            exact = sum(Fraction(float(q[b, h, d])) * Fraction(float(pool[r, d]))
                        for h in range(H) for d in range(D))
            assert abs(Fraction(S[b, i]) - exact) <= Fraction(1e-15) * Fraction(A[b, i])
    assert S[0, 0] == S[0, 2]                                # the same row scores the same


def test_score_paged_one_hot_pool():
    """Pool row j = alpha_j e_(j mod D), heads e_(i_h): s = alpha_row * #{h: i_h = row mod D}."""
    D, R = 16, 40
    alpha = np.arange(1, R + 1, dtype=np.float32)
    pool = np.zeros((R, D), np.float32)
    pool[np.arange(R), np.arange(R) % D] = alpha
    heads = [[3, 3, 5], [0, 7, 7]]
    q = np.zeros((2, 3, D), np.float32)
    for b in range(2):
        for h, i in enumerate(heads[b]):
            q[b, h, i] = 1
    indptr = np.array([0, 5, 9])
    indices = np.array([3, 19, 35, 5, 0, 7, 23, 16, 39])
    S, _, _ = oracle.score_paged(q, pool, indptr, indices, 5, "f32")
    for b in range(2):
        for i in range(indptr[b + 1] - indptr[b]):
            r = indices[indptr[b] + i]
            assert S[b, i] == alpha[r] * sum(1 for x in heads[b] if x == r % D)


def test_score_paged_invalid_entries_and_missing_list_positions():
    rng = np.random.default_rng(31)
    q = rng.standard_normal((2, 2, 8)).astype(np.float32)
    pool = rng.standard_normal((5, 8)).astype(np.float32)
    indptr = np.array([0, 4, 9])        # request 1 runs past the 7 list entries
    indices = np.array([1, -1, 5, 4, 0, 2, 3])
    S, A, n = oracle.score_paged(q, pool, indptr, indices, 5, "f32")
    np.testing.assert_array_equal(n, [4, 5])
    assert np.isfinite(S[0, [0, 3]]).all() and (S[0, [1, 2]] == -np.inf).all()
    assert np.isfinite(S[1, :3]).all() and (S[1, 3:] == -np.inf).all()
    assert (A[S == -np.inf] == 0).all()
    ids, counts = oracle.select(S, n, 5, False)
    np.testing.assert_array_equal(counts, [2, 3])
    np.testing.assert_array_equal(ids[0], [0, 3, -1, -1, -1])


def test_score_paged_identity_lists_reduce_to_dense_tables():
    """Special case: lists that walk a per-request table in order are the dense
    score of that table (the dense form is pinned by the closed forms above)."""
    x = synth.make_indexer(3, 4, 32, 50, [50 * 16, 21 * 16 + 2, 0], 8, "bf16", 32, poison=False)
    nv = oracle.n_valid(x.seq_len, 16, 50)
    pool = x.c.reshape(3 * 50, 32)
    indptr = np.concatenate([[0], np.cumsum(nv)])
    indices = np.concatenate([b * 50 + np.arange(nv[b]) for b in range(3)])
    S, A, n = oracle.score_paged(x.q, pool, indptr, indices, 50, "bf16")
    Sd, Ad = oracle.score(x.q, x.c, x.seq_len, 16, "bf16")
    np.testing.assert_array_equal(n, nv)
    np.testing.assert_allclose(S, Sd, rtol=1e-13, atol=0)
    np.testing.assert_allclose(A, Ad, rtol=1e-13, atol=0)


# ----------------------------------------------------------------------------------------
# prompt (prefill) tokens: each token sees the blocks up to its own
# ----------------------------------------------------------------------------------------
def test_score_prefill_block_counts_by_hand():
    """Page 4, first token at position 5: tokens at positions 5..12 see 6..13
    tokens, i.e. 2, 2, 2, 3, 3, 3, 3, 4 blocks; capped at N_pad = 3 for the rest."""
    q = np.ones((1, 8, 1, 4), np.float32)
    c = np.ones((1, 3, 4), np.float32)
    S, _, NV = oracle.score_prefill(q, c, [5], 4, "f32")
    np.testing.assert_array_equal(NV[0], [2, 2, 2, 3, 3, 3, 3, 3])
    for t in range(8):
        assert np.isfinite(S[0, t, :NV[0, t]]).all() and (S[0, t, NV[0, t]:] == -np.inf).all()
    _, _, NV0 = oracle.score_prefill(q, c, [-7], 4, "f32")    # negative start counts as 0
    np.testing.assert_array_equal(NV0[0], [1, 1, 1, 1, 2, 2, 2, 2])


def test_score_prefill_exact_against_rationals():
    rng = np.random.default_rng(40)
    B, T, H, D, N = 2, 5, 3, 6, 4
    q = rng.standard_normal((B, T, H, D)).astype(np.float32)
    c = rng.standard_normal((B, N, D)).astype(np.float32)
    S, A, NV = oracle.score_prefill(q, c, [0, 9], 4, "f32")
    for b in range(B):
        for t in range(T):
            for n in range(N):
                if n >= NV[b, t]:
                    assert S[b, t, n] == -np.inf and A[b, t, n] == 0
                    continue
                exact = sum(Fraction(float(q[b, t, h, d])) * Fraction(float(c[b, n, d]))
                            for h in range(H) for d in range(D))
                assert abs(Fraction(S[b, t, n]) - exact) <= Fraction(1e-15) * Fraction(A[b, t, n])


def test_score_prefill_each_token_is_a_decode_call():
    """Special case: token t alone is the decode score of a request holding
    pos0 + t + 1 tokens (the decode form is pinned by the closed forms above)."""
    x = synth.make_prefill(2, 9, 4, 32, 40, [17, 300], 8, 41)
    S, A, NV = oracle.score_prefill(x.q, x.c, x.pos0, 16, "bf16")
    for t in range(9):
        Sd, Ad = oracle.score(x.q[:, t], x.c, x.pos0.astype(np.int64) + t + 1, 16, "bf16")
        np.testing.assert_allclose(S[:, t], Sd, rtol=1e-13, atol=0)
        np.testing.assert_allclose(A[:, t], Ad, rtol=1e-13, atol=0)


# ----------------------------------------------------------------------------------------
# pooled keys: block means
# ----------------------------------------------------------------------------------------
def test_pool_keys_closed_forms():
    """An arithmetic progression of keys has its midpoint as block mean; a
    partial last block averages only the tokens held; constant keys pool to
    themselves."""
    S_pad, D = 40, 4
    tok = np.arange(S_pad, dtype=np.float32)
    k = np.stack([np.stack([tok, 2 * tok, np.full(S_pad, 3.0), -tok], axis=1)] * 2).astype(np.float32)
    C, M, nv = oracle.pool_keys(k, [37, 16], 10, 8, "f32")
    np.testing.assert_array_equal(nv, [5, 2])
    # request 0: blocks of tokens 0..7, 8..15, 16..23, 24..31 and 32..36
    for n, (lo, hi) in enumerate([(0, 8), (8, 16), (16, 24), (24, 32), (32, 37)]):
        mid = (lo + hi - 1) / 2
        np.testing.assert_array_equal(C[0, n], [mid, 2 * mid, 3.0, -mid])
        np.testing.assert_array_equal(M[0, n], [mid, 2 * mid, 3.0, mid])
    assert np.isnan(C[0, 5:]).all() and np.isnan(C[1, 2:]).all()


def test_pool_keys_exact_against_rationals_and_clamps():
    rng = np.random.default_rng(50)
    k = rng.standard_normal((2, 13, 5)).astype(np.float32)
    C, _, nv = oracle.pool_keys(k, [13, 99], 4, 3, "f32")   # 99 tokens clamp to the 13 held
    np.testing.assert_array_equal(nv, [4, 4])               # ceil(13/3) = 5 blocks, capped at 4
    for b in range(2):
        for n in range(4):
            toks = range(3 * n, min(3 * n + 3, 13))
            for d in range(5):
                exact = sum(Fraction(float(k[b, s, d])) for s in toks) / len(toks)
                assert abs(Fraction(C[b, n, d]) - exact) <= Fraction(1e-15) * (abs(exact) + 1)


# ----------------------------------------------------------------------------------------
# selection: brute force by rank, exhaustively on tiny rows
# ----------------------------------------------------------------------------------------
def _rank_select(s, nv, K, sorted_out):
    """Selection by the rank definition (no sorting): rank(i) counts the valid,
    non -inf entries that beat i (larger score, or equal score and lower id)."""
    cand = [i for i in range(nv) if s[i] != -np.inf]
    rank = {}
    for i in cand:
        rank[i] = sum(1 for j in cand if s[j] > s[i] or (s[j] == s[i] and j < i))
    chosen = [i for i in cand if rank[i] < K]
    if sorted_out:
        chosen.sort(key=lambda i: rank[i])
    else:
        chosen.sort()
    return chosen + [-1] * (K - len(chosen))


VALUES = [-np.inf, -1.0, -0.0, 0.0, 1.0, 2.0]


@pytest.mark.parametrize("L", [0, 1, 2, 3, 4, 5])
def test_select_matches_rank_definition_exhaustively(L):
    for row in itertools.product(VALUES, repeat=L):
        s = np.array(row, dtype=np.float32)
        for nv in ([L] if L < 4 else [L, L - 2]):
            for K in range(1, L + 2):
                for srt in (False, True):
                    got = oracle.select_row(s, nv, K, srt)
                    assert list(got) == _rank_select(s, nv, K, srt), (row, nv, K, srt)


def test_select_matches_rank_definition_on_random_rows():
    """Longer rows than the exhaustive case, drawn from a fixed seed: tied
    values, signed zeros and -inf, valid counts inside the row, K around the
    number of candidates, both output orders."""
    rng = np.random.default_rng(3131)
    pool = np.array([-np.inf, -2.5, -1.0, -0.0, 0.0, 0.5, 1.0, 1.5, 3.0], dtype=np.float32)
    for _ in range(300):
        L = int(rng.integers(0, 61))
        s = pool[rng.integers(0, pool.size, L)] if rng.random() < 0.7 else \
            rng.standard_normal(L).astype(np.float32)
        nv = int(rng.integers(0, L + 1))
        K = int(rng.integers(1, L + 3))
        srt = bool(rng.integers(2))
        assert list(oracle.select_row(s, nv, K, srt)) == _rank_select(s, nv, K, srt), (
            list(s), nv, K, srt)


def test_select_rank_definition_on_each_stress_distribution():
    """O(N^2) rank counting (vectorised) on one row of each distribution."""
    x = synth.make_topk(9, 2500, 300, 31)
    for r in range(9):
        s = x.scores[r].astype(np.float64)
        cand = s != -np.inf
        beats = (s[None, :] > s[:, None]) | ((s[None, :] == s[:, None]) &
                                            (np.arange(2500)[None, :] < np.arange(2500)[:, None]))
        beats &= cand[None, :]
        rank = beats.sum(axis=1)
        for srt in (False, True):
            got = oracle.select_row(x.scores[r], 2500, 300, srt)
            sel = np.nonzero(cand & (rank < 300))[0]
            want = sel[np.argsort(rank[sel])] if srt else sel
            want = list(want) + [-1] * (300 - len(want))
            assert list(got) == want, x.dists[r]


def test_select_against_heapq_on_full_stress_rows():
    """A different library routine (a heap, keyed on (score, -id)) on full-size rows."""
    x = synth.workload(3)
    ids, counts = oracle.select(x.scores, None, x.K, sorted_out=True)
    for r in range(9):
        s = x.scores[r]
        cand = [i for i in range(s.size) if s[i] != -np.inf]
        top = heapq.nlargest(x.K, cand, key=lambda i: (float(s[i]), -i))
        assert list(ids[r, : len(top)]) == top, x.dists[r]
        assert counts[r] == len(top)


def test_select_special_cases():
    K = 7
    eq = np.ones(30, np.float32)
    assert list(oracle.select_row(eq, 30, K, False)) == list(range(K))
    desc = np.arange(30, 0, -1).astype(np.float32)
    assert list(oracle.select_row(desc, 30, K, True)) == list(range(K))
    asc = np.arange(30).astype(np.float32)
    assert list(oracle.select_row(asc, 30, K, False)) == list(range(23, 30))
    assert list(oracle.select_row(asc, 30, K, True)) == list(range(29, 22, -1))
    assert list(oracle.select_row(asc, 5, K, False)) == [0, 1, 2, 3, 4, -1, -1]
    assert list(oracle.select_row(asc, 0, K, False)) == [-1] * K
    neg = np.full(10, -np.inf, np.float32)
    neg[[3, 8]] = [-5.0, 4.0]
    assert list(oracle.select_row(neg, 10, 4, True)) == [8, 3, -1, -1]
    z = np.array([0.0, -0.0, 0.0, -0.0], np.float32)
    assert list(oracle.select_row(z, 4, 2, True)) == [0, 1]
    with pytest.raises(ValueError):
        oracle.select_row(np.array([1.0, np.nan], np.float32), 2, 1, False)


def test_select_invariants_on_the_stress_workload():
    x = synth.workload(3)
    ids, counts = oracle.select(x.scores, None, x.K)
    for r in range(x.scores.shape[0]):
        s = x.scores[r]
        cand = np.nonzero(s != -np.inf)[0]
        m = min(x.K, cand.size)
        sel = ids[r, :m]
        assert counts[r] == m and (ids[r, m:] == -1).all()
        assert np.all(np.diff(sel) > 0)                       # distinct, ascending
        assert np.all(s[sel] != -np.inf)
        mask = np.zeros(s.size, bool)
        mask[sel] = True
        unsel = s[~mask & (s != -np.inf)]
        if unsel.size:
            kth = s[sel].min()
            assert kth >= unsel.max()
            ties = np.nonzero(s == kth)[0]                    # lowest ids win the tie
            taken = ties[mask[ties]]
            assert np.array_equal(taken, ties[: taken.size])


# ----------------------------------------------------------------------------------------
# k-means assignment
# ----------------------------------------------------------------------------------------
def test_assign_score_equals_distance_form():
    """2 x.c - |c|^2 = |x|^2 - |x - c|^2: the nearest centroid maximises the score."""
    rng = np.random.default_rng(21)
    x = synth.f32_to_bf16_bits(rng.standard_normal((50, 16)).astype(np.float32))
    c = synth.f32_to_bf16_bits(rng.standard_normal((30, 16)).astype(np.float32))
    a, S, _ = oracle.assign(x, c)
    xf = synth.bf16_bits_to_f32(x).astype(np.float64)
    cf = synth.bf16_bits_to_f32(c).astype(np.float64)
    d2 = ((xf[:, None, :] - cf[None, :, :]) ** 2).sum(-1)
    np.testing.assert_allclose(S, (xf ** 2).sum(1)[:, None] - d2, rtol=0, atol=1e-9)
    np.testing.assert_array_equal(a, np.argmin(d2, axis=1))


def test_assign_exact_rationals_and_lower_index_ties():
    rng = np.random.default_rng(22)
    c = synth.f32_to_bf16_bits(rng.integers(-3, 4, (6, 4)).astype(np.float32))
    c[4] = c[1]                                    # duplicate centroid: ties go to 1
    x = synth.f32_to_bf16_bits(rng.integers(-3, 4, (40, 4)).astype(np.float32))
    x[:5] = c[1]
    a, _, _ = oracle.assign(x, c)
    xf = [[Fraction(float(v)) for v in r] for r in synth.bf16_bits_to_f32(x)]
    cf = [[Fraction(float(v)) for v in r] for r in synth.bf16_bits_to_f32(c)]
    for i in range(40):
        sc = [2 * sum(p * q for p, q in zip(xf[i], cj)) - sum(v * v for v in cj) for cj in cf]
        best = max(sc)
        assert a[i] == sc.index(best)
    assert (a[:5] == 1).all()


def test_assign_recovers_the_generating_component():
    x = synth.make_assign(4096, 1024, 128, 5)
    a, _, _ = oracle.assign(x.x, x.c)
    np.testing.assert_array_equal(a, x.comp)
