"""Pins for the CPU oracle: closed forms, library special cases, brute force and
invariants, each independent of the oracle's own code path.

A plausible slip anywhere in the oracle (a dropped term, a wrong sign or index,
the wrong end of a tie, a transposed operand) fails at least one of these.
"""
import itertools
import math
from fractions import Fraction

import numpy as np
import pytest
import scipy.special
import torch
from hypothesis import given, settings, strategies as st, HealthCheck

from oracle import (ParityMismatch, Pattern, Rope, UnitCache, global_scores, prefill_keep, prefill_output,
                    prefill_scores, run_unit, run_unit_global)

torch.set_default_dtype(torch.float64)


def _rand(n, d, seed, dtype=np.float64):
    g = np.random.default_rng(seed)
    return g.standard_normal((n, d)), g.standard_normal((n, d)), g.standard_normal((n, d))


def _sdpa_rows(Q, K, V, mask):
    """Library attention (torch, float64, CPU) with a boolean keep-mask [N, N]."""
    q = torch.from_numpy(Q)[None, None]
    k = torch.from_numpy(K)[None, None]
    v = torch.from_numpy(V)[None, None]
    m = torch.from_numpy(mask)[None, None]
    return torch.nn.functional.scaled_dot_product_attention(q, k, v, attn_mask=m)[0, 0].numpy()


def _library_causal_weights(Q, K):
    """Causal softmax weights from scipy (masked entries at -inf)."""
    d = Q.shape[1]
    x = (Q @ K.T) / math.sqrt(d)
    x = np.where(np.tril(np.ones_like(x, dtype=bool)), x, -np.inf)
    return scipy.special.softmax(x, axis=1)


# ----------------------------------------------------------------------------- prefill scores
@pytest.mark.parametrize("L,d,seed", [(1, 4, 0), (7, 3, 1), (64, 16, 2), (130, 64, 3)])
def test_prefill_column_sums_match_library_softmax(L, d, seed):
    Q, K, _ = _rand(L, d, seed)
    ps = prefill_scores(Q, K, 1 / math.sqrt(d))
    W = _library_causal_weights(Q, K)
    np.testing.assert_allclose(ps.col_sum, W.sum(axis=0), rtol=1e-12, atol=1e-14)
    # row statistics: m_r + log(l_r) is the row's log-sum-exp
    x = (Q @ K.T) / math.sqrt(d)
    lse = np.array([scipy.special.logsumexp(x[r, : r + 1]) for r in range(L)])
    np.testing.assert_allclose(ps.row_max + np.log(ps.row_sum), lse, rtol=1e-12, atol=1e-12)
    # every row is stochastic, so the column sums total L; row 0 sees only itself
    assert abs(ps.col_sum.sum() - L) < 1e-9 * L
    assert ps.col_sum[0] >= 1.0 - 1e-12
    assert ps.col_sum[-1] == pytest.approx(W[-1, -1], rel=1e-12)


@pytest.mark.parametrize("L,d,seed", [(1, 4, 10), (9, 3, 11), (70, 16, 12), (129, 64, 13)])
def test_prefill_output_matches_library_attention(L, d, seed):
    # the prompt's own output is full causal attention: torch SDPA (float64)
    Q, K, V = _rand(L, d, seed)
    O = prefill_output(Q, K, V, 1 / math.sqrt(d))
    ref = _sdpa_rows(Q, K, V, np.tril(np.ones((L, L), dtype=bool)))
    np.testing.assert_allclose(O, ref, rtol=1e-12, atol=1e-12)


def test_prefill_output_identical_keys_is_running_mean():
    # equal keys: row r weights positions 0..r equally, so o_r is the mean of v_0..v_r
    L, d = 23, 5
    g = np.random.default_rng(14)
    Q = g.standard_normal((L, d))
    K = np.tile(g.standard_normal(d), (L, 1))
    V = g.standard_normal((L, d))
    O = prefill_output(Q, K, V, 0.37)
    ref = np.cumsum(V, axis=0) / np.arange(1, L + 1)[:, None]
    np.testing.assert_allclose(O, ref, rtol=1e-12, atol=1e-12)


def test_prefill_single_token():
    ps = prefill_scores(np.ones((1, 2)), np.ones((1, 2)), 0.5)
    assert ps.col_sum.tolist() == [1.0]


def test_prefill_identical_keys_harmonic_closed_form():
    # all keys equal -> every row is uniform over its prefix: c_j = H_L - H_j
    L, d = 256, 8
    g = np.random.default_rng(5)
    Q = g.standard_normal((L, d))
    K = np.tile(g.standard_normal(d), (L, 1))
    ps = prefill_scores(Q, K, 1 / math.sqrt(d))
    H = [Fraction(0)]
    for n in range(1, L + 1):
        H.append(H[-1] + Fraction(1, n))
    expect = np.array([float(H[L] - H[j]) for j in range(L)])
    np.testing.assert_allclose(ps.col_sum, expect, rtol=1e-12)
    assert ps.col_sum[0] == pytest.approx(6.124344962817279, rel=1e-12)  # H_256
    assert ps.col_sum[-1] == pytest.approx(1 / 256, rel=1e-12)


def test_prefill_scale_is_one_over_sqrt_d():
    # a transposed operand or a wrong scale changes these weights
    Q = np.array([[1.0, 0.0], [0.0, 2.0]])
    K = np.array([[2.0, 0.0], [0.0, 1.0]])
    ps = prefill_scores(Q, K, 1 / math.sqrt(2))
    # row 1: logits q1.k0 = 0, q1.k1 = 2 -> weights 1/(1+e^{sqrt 2}), e^{sqrt 2}/(1+e^{sqrt 2})
    w1 = math.exp(math.sqrt(2)) / (1 + math.exp(math.sqrt(2)))
    assert ps.col_sum[1] == pytest.approx(w1, rel=1e-14)
    assert ps.col_sum[0] == pytest.approx(1 + (1 - w1), rel=1e-14)


# ----------------------------------------------------------------------------- prefill selection
def _brute_keep(c, heavy, recent):
    L = len(c)
    if L <= heavy + recent:
        return list(range(L))
    pool = range(L - recent)
    # j is kept iff fewer than `heavy` pool members beat it (higher score, or equal score
    # and higher position)
    kept = [j for j in pool if sum(1 for t in pool if (c[t] > c[j]) or (c[t] == c[j] and t > j)) < heavy]
    return sorted(kept + list(range(L - recent, L)))


@settings(max_examples=300, deadline=None)
@given(st.lists(st.sampled_from([0.0, 0.25, 0.5, 1.0, 1.5, 3.0]), min_size=0, max_size=14),
       st.integers(0, 5), st.integers(0, 5))
def test_prefill_keep_matches_brute_force(vals, heavy, recent):
    if heavy + recent == 0:
        return
    c = np.array(vals, dtype=np.float64)
    kept, _ = prefill_keep(c, heavy, recent)
    assert kept == _brute_keep(c, heavy, recent)
    assert len(kept) == min(len(c), heavy + recent)


def test_prefill_keep_tie_keeps_higher_position():
    c = np.array([1.0, 1.0, 1.0, 0.5, 0.2, 0.1])
    kept, _ = prefill_keep(c, heavy=2, recent=2)
    assert kept == [1, 2, 4, 5]


def test_prefill_keep_threshold_is_L_greater_than_k():
    c = np.arange(6, dtype=float)
    assert prefill_keep(c, 3, 3)[0] == list(range(6))       # L == k keeps all
    c7 = np.array([5.0, 4.0, 3.0, 2.0, 1.0, 0.0, 0.0])
    # L = 7 > k = 6: recent = {4, 5, 6}; heavy = best 3 of {0..3}
    assert prefill_keep(c7, 3, 3)[0] == [0, 1, 2, 4, 5, 6]


def test_prefill_keep_replay_band():
    c = np.array([1.0, 1.0 + 1e-7, 0.5, 3.0, 0.1, 0.1])
    kept, _ = prefill_keep(c, heavy=2, recent=2)
    assert kept == [1, 3, 4, 5]
    kept2, info = prefill_keep(c, heavy=2, recent=2, prefer=[0, 3, 4, 5])
    assert kept2 == [0, 3, 4, 5] and info["tie_adopted"]
    with pytest.raises(ParityMismatch):
        prefill_keep(c, heavy=2, recent=2, prefer=[2, 3, 4, 5])


# ----------------------------------------------------------------------------- full attention
@pytest.mark.parametrize("L,T,d,heavy,recent", [(10, 14, 8, 24, 0), (10, 14, 8, 0, 24), (0, 9, 4, 5, 5),
                                                (5, 30, 16, 20, 20), (1, 5, 2, 3, 3)])
def test_budget_covering_sequence_equals_full_attention(L, T, d, heavy, recent):
    N = L + T
    if heavy + recent < N:
        pytest.skip("budget smaller than the sequence")
    Q, K, V = _rand(N, d, 11 + L)
    res = run_unit(Q, K, V, L, heavy, recent)
    assert (res["evicted"] == -1).all()
    full = _sdpa_rows(Q, K, V, np.tril(np.ones((N, N), dtype=bool)))
    np.testing.assert_allclose(res["out"], full[L:], rtol=1e-12, atol=1e-12)
    W = _library_causal_weights(Q, K)
    pos, score, _, _ = res["cache"].snapshot()
    assert pos.tolist() == list(range(N))
    np.testing.assert_allclose(score, W.sum(axis=0), rtol=1e-11, atol=1e-13)


# ----------------------------------------------------------------------------- sliding window
@pytest.mark.parametrize("L,T,recent", [(3, 25, 4), (12, 20, 5), (0, 15, 1), (9, 9, 9)])
def test_no_heavy_budget_is_sliding_window(L, T, recent):
    d = 6
    N = L + T
    Q, K, V = _rand(N, d, 100 + L)
    res = run_unit(Q, K, V, L, 0, recent)
    band = np.zeros((N, N), dtype=bool)
    for i in range(N):
        band[i, max(0, i - recent): i + 1] = True  # window of recent+1 entries (the new one included)
    win = _sdpa_rows(Q, K, V, band)
    for t in range(T):
        i = L + t
        n_cached_before = min(recent, i) if L <= recent else recent
        # once the cache holds `recent` entries, the step sees exactly [i-recent, i]
        if n_cached_before == recent:
            np.testing.assert_allclose(res["out"][t], win[i], rtol=1e-12, atol=1e-12)
            assert res["evicted"][t] == i - recent
        else:
            assert res["evicted"][t] == -1


# ----------------------------------------------------------------------------- identical keys
@pytest.mark.parametrize("L,T,heavy,recent", [(40, 30, 6, 5), (8, 40, 6, 5), (30, 20, 4, 0), (30, 20, 0, 4)])
def test_identical_keys_closed_form(L, T, heavy, recent):
    d = 5
    N = L + T
    g = np.random.default_rng(7)
    Q = g.standard_normal((N, d))
    K = np.tile(g.standard_normal(d), (N, 1))
    V = g.standard_normal((N, d))
    k = heavy + recent
    res = run_unit(Q, K, V, L, heavy, recent)
    # prefill keeps {0..heavy-1} plus the last `recent` positions (uniform rows favour early tokens)
    if L > k:
        assert res["kept"] == list(range(heavy)) + list(range(L - recent, L))
    for t in range(T):
        i = L + t
        cached = min(k, i) if L <= k else k
        if cached < k:
            assert res["evicted"][t] == -1
            G = list(range(i + 1)) if L <= k else None
        else:
            assert res["evicted"][t] == i - recent, (t, res["evicted"][t])
            G = list(range(heavy)) + list(range(i - recent, i + 1)) if recent > 0 else list(range(heavy)) + [i]
        if G is not None:
            # uniform weights over the attended set
            np.testing.assert_allclose(res["out"][t], V[G].mean(axis=0), rtol=1e-12, atol=1e-12)
    pos = sorted(res["cache"].pos.tolist())
    if recent > 0:
        assert pos == list(range(heavy)) + list(range(N - recent, N))


# ----------------------------------------------------------------------------- brute-force eviction
def _brute_force_run(Q, K, V, L, heavy, recent):
    """Independent simulation: dict state, scipy softmax, exact Fraction sums, and
    the eviction rule as the pages state it -- remove the entry whose removal
    leaves the largest total score (argmax of F over G minus one entry)."""
    d = Q.shape[1]
    k = heavy + recent
    s = 1 / math.sqrt(d)
    score = {}
    # prompt: column sums of the causal softmax, accumulated row by row
    for r in range(L):
        w = scipy.special.softmax(s * (K[: r + 1] @ Q[r]))
        for j in range(r + 1):
            score[j] = score.get(j, Fraction(0)) + Fraction(float(w[j]))
    S = list(range(L))
    if L > k:
        pool = list(range(L - recent))
        # keep the heavy best: rank by (score, position) descending
        best = sorted(pool, key=lambda j: (score[j], j), reverse=True)[:heavy]
        S = sorted(best + list(range(L - recent, L)))
    log = []
    for i in range(L, Q.shape[0]):
        G = S + [i]
        w = scipy.special.softmax(s * (K[G] @ Q[i]))
        score[i] = Fraction(0)
        for j, wj in zip(G, w):
            score[j] += Fraction(float(wj))
        if len(S) < k:
            S = G
            log.append(-1)
            continue
        total = sum(score[j] for j in G)
        cands = [v for v in G if v <= i - recent]
        bestF = max(total - score[v] for v in cands)
        u = min(v for v in cands if total - score[v] == bestF)  # ties: lowest position
        S = [j for j in G if j != u]
        log.append(u)
    return log, sorted(S)


KEYS2 = {"strong": (3.0, 0.0), "mid": (0.5, 0.7), "weak": (-1.0, 0.3), "dead": (-3000.0, 0.0)}


@settings(max_examples=200, deadline=None, suppress_health_check=[HealthCheck.too_slow])
@given(st.lists(st.sampled_from(sorted(KEYS2)), min_size=1, max_size=12),
       st.integers(0, 5), st.integers(0, 3), st.integers(0, 3))
def test_eviction_matches_brute_force(kinds, L, heavy, recent):
    if heavy + recent == 0:
        return
    N = len(kinds)
    L = min(L, N)
    K = np.array([KEYS2[x] for x in kinds])
    Q = np.tile([1.0, 0.0], (N, 1))
    V = np.arange(N * 2, dtype=float).reshape(N, 2)
    res = run_unit(Q, K, V, L, heavy, recent)
    log, S = _brute_force_run(Q, K, V, L, heavy, recent)
    assert res["evicted"].tolist() == log
    assert sorted(res["cache"].pos.tolist()) == S


def test_dead_tokens_tie_evicts_lowest_position():
    # tokens 1 and 2 get exactly zero weight from every row -> equal scores (0);
    # the lowest of the tied positions goes first
    K = np.array([KEYS2["strong"], KEYS2["dead"], KEYS2["dead"], KEYS2["strong"], KEYS2["strong"]])
    Q = np.tile([1.0, 0.0], (5, 1))
    V = np.zeros((5, 2))
    res = run_unit(Q, K, V, 3, 3, 0)
    assert res["evicted"].tolist() == [1, 2]


# ----------------------------------------------------------------------------- invariants
@pytest.mark.parametrize("L,T,heavy,recent,seed", [(50, 80, 7, 6, 0), (5, 60, 3, 9, 1), (40, 40, 10, 0, 2),
                                                   (0, 70, 4, 4, 3), (33, 50, 0, 8, 4)])
def test_invariants_every_step(L, T, heavy, recent, seed):
    d = 8
    Q, K, V = _rand(L + T, d, seed)
    Q = Q * 2.0
    cache, _, _ = UnitCache.from_prompt(Q[:L], K[:L], V[:L], heavy, recent)
    k = heavy + recent
    gone = set(range(L)) - set(cache.pos.tolist())
    for t in range(T):
        i = L + t
        before = set(cache.pos.tolist())
        o, u, info = cache.step(Q[i], K[i], V[i])
        after = set(cache.pos.tolist())
        assert abs(info["weights"].sum() - 1) < 1e-12
        assert len(after) == min(k, cache.rows)
        assert after - before <= {i}
        assert len(before - after) <= 1
        if u >= 0:
            assert u <= i - recent and u not in after
            gone.add(u)
        assert not (after & gone)                     # an evicted position never returns
        window = set(range(max(0, i - recent + 1), i + 1))
        assert window <= after                        # the recent window stays resident
        # mass: the scores total the rows processed minus the mass evicted
        assert abs(cache.score.sum() - (cache.rows - cache.evicted_mass)) < 1e-9 * cache.rows


def test_slot_order_does_not_matter():
    d, L, T = 8, 30, 40
    Q, K, V = _rand(L + T, d, 9)
    a, _, _ = UnitCache.from_prompt(Q[:L], K[:L], V[:L], 6, 5)
    b, _, _ = UnitCache.from_prompt(Q[:L], K[:L], V[:L], 6, 5)
    g = np.random.default_rng(0)
    for t in range(T):
        i = L + t
        if t % 7 == 3:
            perm = g.permutation(len(b.pos))
            b.pos, b.K, b.V, b.score = b.pos[perm], b.K[perm], b.V[perm], b.score[perm]
        oa, ua, _ = a.step(Q[i], K[i], V[i])
        ob, ub, _ = b.step(Q[i], K[i], V[i])
        assert ua == ub
        np.testing.assert_allclose(oa, ob, rtol=1e-12, atol=1e-13)


@pytest.mark.parametrize("L,T,M,heavy,recent,seed", [(40, 90, 37, 8, 6, 0), (20, 60, 1, 5, 0, 1), (0, 50, 25, 4, 4, 2)])
def test_snapshot_mode_continues_the_run(L, T, M, heavy, recent, seed):
    # snapshot mode: a cache rebuilt from the state after M steps (positions,
    # scores, K/V rows in any slot order, next position) runs the remaining steps
    # exactly as the uninterrupted run does
    d = 8
    Q, K, V = _rand(L + T, d, seed)
    Q = Q * 2.0
    full = run_unit(Q, K, V, L, heavy, recent)
    part = run_unit(Q[:L + M], K[:L + M], V[:L + M], L, heavy, recent)
    c = part["cache"]
    perm = np.random.default_rng(seed).permutation(len(c.pos))
    snap = UnitCache(heavy=heavy, recent=recent, scale=c.scale, d=d, pos=c.pos[perm].copy(), K=c.K[perm].copy(),
                     V=c.V[perm].copy(), score=c.score[perm].copy(), next_pos=L + M)
    for t in range(M, T):
        o, u, _ = snap.step(Q[L + t], K[L + t], V[L + t])
        assert u == full["evicted"][t]
        np.testing.assert_allclose(o, full["out"][t], rtol=1e-12, atol=1e-13)
    fp, fs, fk, fv = full["cache"].snapshot()
    sp, ss, sk, sv = snap.snapshot()
    assert np.array_equal(fp, sp) and np.array_equal(fk, sk) and np.array_equal(fv, sv)
    np.testing.assert_allclose(ss, fs, rtol=1e-12)


def test_decode_replay_band_and_mismatch():
    K = np.array([[1.0, 0], [1.0, 0], [0.0, 0.0]])
    Q = np.tile([1.0, 0.0], (3, 1))
    V = np.zeros((3, 2))
    # tokens 0 and 1 have identical keys; with L=2 (k=2, recent=0), step 2 evicts
    res = run_unit(Q, K, V, 2, 2, 0)
    u = int(res["evicted"][0])
    with pytest.raises(ParityMismatch):
        run_unit(Q, K, V, 2, 2, 0, replay_evicted=[-1])
    res2 = run_unit(Q, K, V, 2, 2, 0, replay_evicted=[u])
    assert res2["evicted"].tolist() == [u]


def test_decode_replay_adopts_only_within_band():
    K = np.array([KEYS2["strong"], KEYS2["dead"], KEYS2["dead"], KEYS2["strong"]])
    Q = np.tile([1.0, 0.0], (4, 1))
    V = np.zeros((4, 2))
    assert run_unit(Q, K, V, 3, 3, 0)["evicted"].tolist() == [1]
    assert run_unit(Q, K, V, 3, 3, 0, replay_evicted=[2])["evicted"].tolist() == [2]
    with pytest.raises(ParityMismatch):
        run_unit(Q, K, V, 3, 3, 0, replay_evicted=[0])


# ----------------------------------------------------------------------------- global comparator
def _brute_topk_sets(scores, L, T, heavy, recent):
    """Cached position sets after each decode step under fixed scores, by direct
    enumeration: the recent window plus the K_h best (score, then position) of
    every earlier position; all positions while the budget is not yet full."""
    k = heavy + recent
    sets = []
    for t in range(T):
        i = L + t
        if i + 1 <= k:
            sets.append(set(range(i + 1)))
            continue
        pool = list(range(0, i - recent + 1))
        best = sorted(pool, key=lambda j: (scores[j], j), reverse=True)[:heavy]
        sets.append(set(best) | set(range(i - recent + 1, i + 1)))
    return sets


def _replay_sets(res, L, T, k):
    kept = set(res["kept"])
    out = []
    for t in range(T):
        kept = kept | {L + t}
        u = int(res["evicted"][t])
        if u >= 0:
            kept = kept - {u}
        assert len(kept) == min(L + t + 1, k)
        out.append(set(kept))
    return out


@pytest.mark.parametrize("N,d,seed", [(1, 4, 20), (33, 8, 21), (140, 16, 22)])
def test_global_scores_match_library_softmax(N, d, seed):
    Q, K, _ = _rand(N, d, seed)
    np.testing.assert_allclose(global_scores(Q, K, 1 / math.sqrt(d)), _library_causal_weights(Q, K).sum(axis=0),
                               rtol=1e-12)


@pytest.mark.parametrize("L,T,heavy,recent,seed", [(30, 40, 6, 5, 0), (4, 50, 5, 3, 1), (25, 30, 7, 0, 2),
                                                   (25, 30, 0, 6, 3), (10, 10, 20, 20, 4)])
def test_fixed_scores_keep_top_heavy_by_brute_force(L, T, heavy, recent, seed):
    # fixed scores (with deliberate ties): the cache is always the window plus the
    # K_h best earlier positions
    g = np.random.default_rng(seed)
    N, d = L + T, 6
    Q, K, V = (g.standard_normal((N, d)) for _ in range(3))
    scores = g.integers(0, 6, size=N).astype(float) / 4
    res = run_unit(Q, K, V, L, heavy, recent, fixed=scores)
    assert _replay_sets(res, L, T, heavy + recent) == _brute_topk_sets(scores, L, T, heavy, recent)


def test_fixed_decreasing_scores_is_sink_plus_window_attention():
    # scores that fall with position keep the first K_h tokens forever: every
    # output is attention over the sinks plus the window (torch SDPA, float64)
    L, T, heavy, recent, d = 12, 30, 4, 5, 8
    N = L + T
    Q, K, V = _rand(N, d, 23)
    res = run_unit(Q, K, V, L, heavy, recent, fixed=np.arange(N, 0, -1).astype(float))
    mask = np.zeros((N, N), dtype=bool)
    for i in range(N):
        mask[i, : min(heavy, i + 1)] = True
        mask[i, max(0, i - recent): i + 1] = True
    np.testing.assert_allclose(res["out"], _sdpa_rows(Q, K, V, mask)[L:], rtol=1e-10, atol=1e-10)


@pytest.mark.parametrize("L,T,heavy,recent,seed", [(20, 30, 5, 4, 30), (0, 40, 6, 6, 31), (35, 25, 8, 0, 32)])
def test_global_run_follows_library_scores(L, T, heavy, recent, seed):
    # the comparator ranks by the column sums of the whole sequence's causal
    # softmax (scipy), and its cache is the brute-force top set of those scores
    Q, K, V = _rand(L + T, 8, seed)
    res = run_unit_global(Q, K, V, L, heavy, recent)
    lib = _library_causal_weights(Q, K).sum(axis=0)
    np.testing.assert_allclose(res["scores"], lib, rtol=1e-12)
    assert _replay_sets(res, L, T, heavy + recent) == _brute_topk_sets(lib, L, T, heavy, recent)


# ----------------------------------------------------------------------------- sparse pattern + heavy hitters
def _pattern_protects(kind, per, wid, j, i):
    # strided: every per-th token counted back from the query; fixed: the last
    # wid tokens of every block of per
    if kind == "strided":
        return (i - j) % per == 0
    if kind == "fixed":
        return j % per >= per - wid
    return False


def _brute_pattern_sets(scores, L, T, heavy, recent, kind, per, wid):
    """Direct simulation with fixed scores, on plain sets: the prompt keeps its
    window plus the heavy best by (protected, score, position); every step adds
    the new token and, over budget, removes the lowest-scored unprotected
    candidate (position <= i - recent), or the lowest-scored candidate when all
    are protected."""
    k = heavy + recent
    if L <= k:
        S = set(range(L))
    else:
        pool = range(L - recent)
        best = sorted(pool, key=lambda j: (_pattern_protects(kind, per, wid, j, L), scores[j], j), reverse=True)
        S = set(best[:heavy]) | set(range(L - recent, L))
    out = []
    for t in range(T):
        i = L + t
        S.add(i)
        if len(S) > k:
            cands = [j for j in S if j <= i - recent]
            free = [j for j in cands if not _pattern_protects(kind, per, wid, j, i)]
            S.remove(min(free or cands, key=lambda j: (scores[j], j)))
        out.append(set(S))
    return out


@pytest.mark.parametrize("kind,per,wid", [("strided", 4, 1), ("strided", 7, 1), ("fixed", 8, 2), ("fixed", 5, 4)])
@pytest.mark.parametrize("L,T,heavy,recent,seed", [(30, 40, 6, 5, 0), (4, 50, 5, 3, 1), (25, 30, 7, 0, 2),
                                                   (25, 30, 0, 6, 3), (40, 60, 3, 2, 4)])
def test_pattern_matches_set_simulation(kind, per, wid, L, T, heavy, recent, seed):
    g = np.random.default_rng(seed)
    N = L + T
    Q, K, V = (g.standard_normal((N, 6)) for _ in range(3))
    scores = g.integers(0, 6, size=N).astype(float) / 4
    res = run_unit(Q, K, V, L, heavy, recent, fixed=scores, pattern=Pattern(kind, per, wid))
    assert _replay_sets(res, L, T, heavy + recent) == _brute_pattern_sets(scores, L, T, heavy, recent, kind, per, wid)


@pytest.mark.parametrize("pattern", [Pattern("fixed", 6, 6), Pattern("strided", 1, 1)])
def test_pattern_protecting_everything_is_plain_h2o(pattern):
    # a pattern that protects every position orders nothing: H2O's own choices
    L, T, heavy, recent = 40, 60, 6, 5
    Q, K, V = _rand(L + T, 8, 40)
    a = run_unit(Q, K, V, L, heavy, recent, pattern=pattern)
    b = run_unit(Q, K, V, L, heavy, recent)
    assert a["kept"] == b["kept"] and a["evicted"].tolist() == b["evicted"].tolist()
    np.testing.assert_array_equal(a["out"], b["out"])


def test_fixed_pattern_fixed_scores_closed_form():
    # a fixed pattern is the same for every query, so with fixed scores the cache
    # is the window plus the K_h best earlier positions by (protected, score, pos)
    L, T, heavy, recent, per, wid = 30, 50, 8, 4, 7, 2
    g = np.random.default_rng(41)
    N = L + T
    Q, K, V = (g.standard_normal((N, 6)) for _ in range(3))
    scores = g.integers(0, 5, size=N).astype(float)
    res = run_unit(Q, K, V, L, heavy, recent, fixed=scores, pattern=Pattern("fixed", per, wid))
    for t, S in enumerate(_replay_sets(res, L, T, heavy + recent)):
        i = L + t
        pool = range(i - recent + 1)
        best = sorted(pool, key=lambda j: (j % per >= per - wid, scores[j], j), reverse=True)[:heavy]
        assert S == set(best) | set(range(i - recent + 1, i + 1)), t


def test_pattern_with_no_heavy_budget_is_sliding_window():
    # K_h = 0: the only candidate is the token leaving the window, protected or not
    L, T, recent = 20, 40, 6
    Q, K, V = _rand(L + T, 8, 42)
    for pat in (Pattern("strided", 3, 1), Pattern("fixed", 5, 2)):
        res = run_unit(Q, K, V, L, 0, recent, pattern=pat)
        assert res["evicted"].tolist() == [i - recent for i in range(L, L + T)]


# ----------------------------------------------------------------------------- position rolling (rotary embedding)
def _complex_rope(X, pos, base=10000.0):
    """Rotary embedding written as complex multiplication: the pair (x_m, x_{m+d/2})
    is the complex number x_m + i x_{m+d/2}, turned by pos * base^(-2m/d) radians."""
    X = np.asarray(X, np.float64)
    h = X.shape[1] // 2
    z = X[:, :h] + 1j * X[:, h:]
    w = np.exp(1j * np.outer(np.asarray(pos, np.float64), base ** (-np.arange(0, X.shape[1], 2) / X.shape[1])))
    r = z * w
    return np.concatenate([r.real, r.imag], axis=1)


def test_rope_rotation_matches_complex_multiplication():
    g = np.random.default_rng(50)
    X = g.standard_normal((9, 16))
    pos = np.array([0, 1, 2, 7, 100, 1000, 4095, 12, 3])
    np.testing.assert_allclose(Rope(500.0).rotate(X, pos), _complex_rope(X, pos, 500.0), rtol=1e-12, atol=1e-12)


def test_rope_scores_depend_on_position_gaps_only():
    g = np.random.default_rng(51)
    q, k = g.standard_normal((1, 32)), g.standard_normal((1, 32))
    r = Rope()
    base = (r.rotate(q, [40]) @ r.rotate(k, [17]).T).item()
    for t in (-17, 5, 900):
        assert abs((r.rotate(q, [40 + t]) @ r.rotate(k, [17 + t]).T).item() - base) < 1e-10


def test_rope_prompt_operands():
    # the prompt's rotated operands are the exact rotation to positions 0..L-1
    g = np.random.default_rng(53)
    X = g.standard_normal((300, 64)).astype(np.float32)
    got = Rope(10000.0).prompt(X)
    np.testing.assert_allclose(got, _complex_rope(X, np.arange(300)), rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("L,T,heavy,recent", [(12, 20, 40, 40), (0, 25, 30, 30)])
def test_rope_full_budget_is_rope_attention(L, T, heavy, recent):
    # nothing is evicted, so ranks are text positions: torch SDPA on q, k rotated
    # to their own positions (complex formulation)
    N, d = L + T, 8
    Q, K, V = _rand(N, d, 54)
    res = run_unit(Q, K, V, L, heavy, recent, rope=Rope(100.0))
    ref = _sdpa_rows(_complex_rope(Q, np.arange(N), 100.0), _complex_rope(K, np.arange(N), 100.0), V,
                     np.tril(np.ones((N, N), dtype=bool)))
    np.testing.assert_allclose(res["out"], ref[L:], rtol=1e-10, atol=1e-10)


def test_rope_sliding_window_is_rope_band_attention():
    # K_h = 0 keeps a contiguous window, so rank gaps equal position gaps
    L, T, recent, d = 10, 30, 5, 8
    N = L + T
    Q, K, V = _rand(N, d, 55)
    res = run_unit(Q, K, V, L, 0, recent, rope=Rope(50.0))
    band = np.zeros((N, N), dtype=bool)
    for i in range(N):
        band[i, max(0, i - recent): i + 1] = True
    ref = _sdpa_rows(_complex_rope(Q, np.arange(N), 50.0), _complex_rope(K, np.arange(N), 50.0), V, band)
    np.testing.assert_allclose(res["out"], ref[L:], rtol=1e-10, atol=1e-10)


@pytest.mark.parametrize("L,T,heavy,recent", [(30, 40, 6, 5), (20, 30, 5, 0)])
def test_rope_rolling_with_heavy_hitters_by_enumeration(L, T, heavy, recent):
    # fixed scores fix every step's attended set (window + best earlier positions);
    # the entries sit at their index in the sorted position list, the new token
    # last; logits from the complex formulation, softmax from scipy
    N, d, base = L + T, 8, 30.0
    g = np.random.default_rng(56 + recent)
    Q, K, V = (g.standard_normal((N, d)) for _ in range(3))
    scores = g.permutation(N).astype(float)
    res = run_unit(Q, K, V, L, heavy, recent, fixed=scores, rope=Rope(base))
    sets = _brute_topk_sets(scores, L, T, heavy, recent)
    prev = set(res["kept"])
    for t in range(T):
        i = L + t
        G = sorted(prev | {i})
        x = np.array([(_complex_rope(K[j][None], [r], base) @ _complex_rope(Q[i][None], [len(G) - 1], base).T).item()
                      for r, j in enumerate(G)]) / math.sqrt(d)
        o = scipy.special.softmax(x) @ V[G]
        np.testing.assert_allclose(res["out"][t], o, rtol=1e-10, atol=1e-10)
        prev = sets[t]


def test_rope_prompt_column_sums_match_library():
    L, d = 64, 16
    Q, K, _ = _rand(L, d, 57)
    res = run_unit(Q, K, K, L, 8, 8, rope=Rope(10000.0))
    lib = _library_causal_weights(_complex_rope(Q, np.arange(L)), _complex_rope(K, np.arange(L))).sum(axis=0)
    np.testing.assert_allclose(res["prefill"].col_sum, lib, rtol=1e-10)
