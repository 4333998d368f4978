"""Plant plausible mistakes in a copy of the oracle (CPU only) and check that the
independent pins catch every one of them.

Each mutation is a source edit of ``oracle/h2o_oracle.py`` loaded as a fresh
module; the real oracle is untouched.  A mutation counts as caught when any pin
fails (an assertion or an exception).
"""
import math
import os
import sys
import types
from fractions import Fraction

import numpy as np
import pytest
import scipy.special

from test_oracle_pins import (KEYS2, _brute_force_run, _brute_keep, _brute_pattern_sets, _brute_topk_sets,
                              _library_causal_weights, _replay_sets, _sdpa_rows)

SRC = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "oracle", "h2o_oracle.py")

MUTATIONS = {
    "ties evict the highest position": (
        "u = min(cand, key=lambda t: (prot[t], G_score[t], G_pos[t]))",
        "u = min(cand, key=lambda t: (prot[t], G_score[t], -G_pos[t]))"),
    "argmax instead of argmin": (
        "u = min(cand, key=lambda t: (prot[t], G_score[t], G_pos[t]))",
        "u = max(cand, key=lambda t: (prot[t], G_score[t], G_pos[t]))"),
    "candidate bound off by one": (
        "cand = np.nonzero(G_pos <= i - self.recent)[0]",
        "cand = np.nonzero(G_pos < i - self.recent)[0]"),
    "recent window not protected": (
        "cand = np.nonzero(G_pos <= i - self.recent)[0]",
        "cand = np.nonzero(G_pos <= i)[0]"),
    "new token's own weight dropped": (
        "G_score = np.concatenate([self.score, [0.0]]) + a",
        "G_score = np.concatenate([self.score + a[:-1], [0.0]])"),
    "decode weights not accumulated": (
        "G_score = np.concatenate([self.score, [0.0]]) + a",
        "G_score = np.concatenate([self.score, [a[-1]]])"),
    "prefill ties keep the lower position": (
        "best_first = sorted(pool, key=lambda j: (prot[j], c[j], j), reverse=True)",
        "best_first = sorted(pool, key=lambda j: (prot[j], c[j], -j), reverse=True)"),
    "prefill keeps the worst": (
        "best_first = sorted(pool, key=lambda j: (prot[j], c[j], j), reverse=True)",
        "best_first = sorted(pool, key=lambda j: (prot[j], c[j], j))"),
    "scale 1/d": ("return 1.0 / np.sqrt(float(d))", "return 1.0 / float(d)"),
    "row sums instead of column sums": ("col_sum=A.sum(axis=0)", "col_sum=A.sum(axis=1)"),
    "transposed operands": ("x = scale * (K[: r + 1] @ Q[r])", "x = scale * (Q[: r + 1] @ K[r])"),
    "diagonal excluded": ("x = scale * (K[: r + 1] @ Q[r])",
                          "x = scale * (K[: r + 1] @ Q[r]) - np.where(np.arange(r + 1) == r, 1e300, 0.0) * (r > 0)"),
    # (the selection threshold L > k vs L >= k is not a mutation: with the pool
    # [0, L - recent), a prompt of exactly k tokens keeps everything either way)
    "prefill recent window shifted": ("recent_pos = list(range(L - recent, L))",
                                      "recent_pos = list(range(L - recent - 1, L - 1))"),
    "cache allowed to overfill": ("if len(self.pos) < self.k:", "if len(self.pos) <= self.k:"),
    "prefill scores not seeded": ("cache.score = c[kept].copy()",
                                  "cache.score = np.zeros(len(kept))"),
    "recent pool overlaps": ("pool = list(range(L - recent))", "pool = list(range(L))"),
    "prefill output from transposed weights": ("return A @ np.asarray(V, np.float64)",
                                               "return A.T @ np.asarray(V, np.float64)"),
    "prefill output mixes keys": ("return A @ np.asarray(V, np.float64)", "return A @ np.asarray(K, np.float64)"),
    "prefill output one row late": ("return A @ np.asarray(V, np.float64)",
                                    "return np.vstack([np.zeros((1, V.shape[1])), (A @ V)[:-1]])"),
    "fixed scores still accumulate": ("G_score = np.concatenate([self.score, [self.fixed[i]]])",
                                      "G_score = np.concatenate([self.score, [self.fixed[i]]]) + a"),
    "new token's fixed score dropped": ("G_score = np.concatenate([self.score, [self.fixed[i]]])",
                                        "G_score = np.concatenate([self.score, [0.0]])"),
    "fixed prompt ranked by its own column sums": (
        "c = ps.col_sum if fixed is None else cache.fixed[:L]",
        "c = prefill_scores(Qp, Kp, scale).col_sum"),
    "global scores from the prompt rows only": (
        "g = global_scores(Q, K, scale)",
        "g = np.concatenate([global_scores(Q[:max(prompt_len, 1)], K[:max(prompt_len, 1)], scale), "
        "np.zeros(len(Q) - max(prompt_len, 1))])"),
    "protected entries evicted first": (
        "u = min(cand, key=lambda t: (prot[t], G_score[t], G_pos[t]))",
        "u = min(cand, key=lambda t: (not prot[t], G_score[t], G_pos[t]))"),
    "pattern ignored at eviction": (
        "u = min(cand, key=lambda t: (prot[t], G_score[t], G_pos[t]))",
        "u = min(cand, key=lambda t: (G_score[t], G_pos[t]))"),
    "prefill ignores the pattern": (
        "best_first = sorted(pool, key=lambda j: (prot[j], c[j], j), reverse=True)",
        "best_first = sorted(pool, key=lambda j: (c[j], j), reverse=True)"),
    "strided offset off by one": ("return (i - j) % self.period == 0", "return (i - 1 - j) % self.period == 0"),
    "fixed pattern takes the block heads": ("return j % self.period >= self.period - self.width",
                                            "return j % self.period < self.width"),
    "rolling uses text positions": (
        'rank[np.argsort(G_pos, kind="stable")] = np.arange(len(G_pos))',
        "rank[:] = G_pos - G_pos.max() + len(G_pos) - 1"),
    "rotation sign flipped": ("return np.concatenate([x * c - y * s, x * s + y * c], axis=1)\n",
                              "return np.concatenate([x * c + y * s, -x * s + y * c], axis=1)\n"),
    "rotation pairs adjacent elements": ("x, y = X[:, :h], X[:, h:]", "x, y = X[:, 0::2], X[:, 1::2]"),
    "prompt rotated to reversed positions": ("return self.rotate(X, np.arange(X.shape[0]))",
                                             "return self.rotate(X, np.arange(X.shape[0])[::-1])"),
    "prompt rotation order swapped": ("return self.rotate(X, np.arange(X.shape[0]))",
                                      "return np.roll(self.rotate(np.roll(X, X.shape[1] // 2, axis=1), "
                                      "np.arange(X.shape[0])), X.shape[1] // 2, axis=1)"),
    "new token one position late": ("qr = self.rope.rotate(q[None], [len(G_pos) - 1])[0]",
                                    "qr = self.rope.rotate(q[None], [len(G_pos)])[0]"),
    "prompt scored unrotated": ("prefill_scores(rope.prompt(Qp), rope.prompt(Kp), scale)",
                                "prefill_scores(Qp, Kp, scale)"),
    "rope frequencies halved": ("** (-2.0 * np.arange(d // 2) / d)", "** (-1.0 * np.arange(d // 2) / d)"),
    "evicted entries stay in the normaliser": (
        "a = softmax(x)\n        o = a @ G_V",
        "a = softmax(x)\n        a = a * (len(x) / (len(x) + self.evicted_mass))\n        o = a @ G_V"),
}


_COUNTER = [0]


def _load(src_text):
    _COUNTER[0] += 1
    name = f"mutant_oracle_{_COUNTER[0]}"
    mod = types.ModuleType(name)
    sys.modules[name] = mod  # dataclasses look their module up here
    exec(compile(src_text, name, "exec"), mod.__dict__)
    return mod


def _checks(m):
    """Yields pins; each raises on disagreement."""
    g = np.random.default_rng(1)

    def full_attention():
        N, L, d = 20, 6, 8
        Q, K, V = (g.standard_normal((N, d)) for _ in range(3))
        res = m.run_unit(Q, K, V, L, N, N)
        full = _sdpa_rows(Q, K, V, np.tril(np.ones((N, N), dtype=bool)))
        np.testing.assert_allclose(res["out"], full[L:], rtol=1e-10, atol=1e-10)
        W = _library_causal_weights(Q, K)
        pos, score, _, _ = res["cache"].snapshot()
        assert pos.tolist() == list(range(N))
        np.testing.assert_allclose(score, W.sum(axis=0), rtol=1e-10)

    def prefill_library():
        L, d = 40, 16
        Q, K = g.standard_normal((L, d)), g.standard_normal((L, d))
        ps = m.prefill_scores(Q, K, m.default_scale(d))
        np.testing.assert_allclose(ps.col_sum, _library_causal_weights(Q, K).sum(axis=0), rtol=1e-10)

    def prefill_out():
        L, d = 33, 7
        Q, K, V = (g.standard_normal((L, d)) for _ in range(3))
        O = m.prefill_output(Q, K, V, 1 / math.sqrt(d))
        ref = _sdpa_rows(Q, K, V, np.tril(np.ones((L, L), dtype=bool)))
        np.testing.assert_allclose(O, ref, rtol=1e-10, atol=1e-10)
        Ks = np.tile(K[0], (L, 1))
        O = m.prefill_output(Q, Ks, V, 0.37)
        np.testing.assert_allclose(O, np.cumsum(V, axis=0) / np.arange(1, L + 1)[:, None], rtol=1e-10)

    def global_comparator():
        for (L, T, h, r) in [(20, 30, 5, 4), (25, 20, 6, 0), (3, 30, 4, 4)]:
            Q, K, V = (g.standard_normal((L + T, 6)) for _ in range(3))
            res = m.run_unit_global(Q, K, V, L, h, r)
            lib = _library_causal_weights(Q, K).sum(axis=0)
            np.testing.assert_allclose(res["scores"], lib, rtol=1e-10)
            assert _replay_sets(res, L, T, h + r) == _brute_topk_sets(lib, L, T, h, r)
        for (L, T, h, r) in [(30, 40, 6, 5), (4, 50, 5, 3), (25, 30, 7, 0)]:
            Q, K, V = (g.standard_normal((L + T, 6)) for _ in range(3))
            sc = g.integers(0, 6, size=L + T).astype(float) / 4  # ties on purpose
            res = m.run_unit(Q, K, V, L, h, r, fixed=sc)
            assert _replay_sets(res, L, T, h + r) == _brute_topk_sets(sc, L, T, h, r)

    def sparse_pattern():
        for (kind, per, wid) in [("strided", 5, 1), ("fixed", 8, 2), ("fixed", 6, 3)]:
            for (L, T, h, r) in [(30, 40, 6, 5), (4, 50, 5, 3), (25, 30, 7, 0)]:
                Q, K, V = (g.standard_normal((L + T, 6)) for _ in range(3))
                sc = g.integers(0, 6, size=L + T).astype(float) / 4
                res = m.run_unit(Q, K, V, L, h, r, fixed=sc, pattern=m.Pattern(kind, per, wid))
                assert _replay_sets(res, L, T, h + r) == _brute_pattern_sets(sc, L, T, h, r, kind, per, wid)

    def rolling():
        from test_oracle_pins import _complex_rope
        N, d, base = 40, 8, 30.0
        Q, K, V = (g.standard_normal((N, d)) for _ in range(3))
        res = m.run_unit(Q, K, V, 10, 40, 40, rope=m.Rope(base))  # nothing evicted
        ref = _sdpa_rows(_complex_rope(Q, np.arange(N), base), _complex_rope(K, np.arange(N), base), V,
                         np.tril(np.ones((N, N), dtype=bool)))
        np.testing.assert_allclose(res["out"], ref[10:], rtol=1e-10, atol=1e-10)
        lib = _library_causal_weights(_complex_rope(Q[:10], np.arange(10), base),
                                      _complex_rope(K[:10], np.arange(10), base)).sum(axis=0)
        np.testing.assert_allclose(res["prefill"].col_sum, lib, rtol=1e-10)
        np.testing.assert_allclose(m.Rope(base).prompt(Q), _complex_rope(Q, np.arange(N), base), rtol=1e-12,
                                   atol=1e-12)
        L, T, h, r = 30, 40, 6, 5
        Q, K, V = (g.standard_normal((L + T, d)) for _ in range(3))
        sc = g.permutation(L + T).astype(float)
        res = m.run_unit(Q, K, V, L, h, r, fixed=sc, rope=m.Rope(base))
        sets = _brute_topk_sets(sc, L, T, h, r)
        prev = set(res["kept"])
        for t in range(T):
            i = L + t
            G = sorted(prev | {i})
            x = np.array([(_complex_rope(K[j][None], [rk], base) @
                           _complex_rope(Q[i][None], [len(G) - 1], base).T).item() for rk, j in enumerate(G)])
            o = scipy.special.softmax(x / math.sqrt(d)) @ V[G]
            np.testing.assert_allclose(res["out"][t], o, rtol=1e-10, atol=1e-10)
            prev = sets[t]

    def sliding_window():
        N, L, R, d = 30, 9, 4, 6
        Q, K, V = (g.standard_normal((N, d)) for _ in range(3))
        res = m.run_unit(Q, K, V, L, 0, R)
        band = np.zeros((N, N), dtype=bool)
        for i in range(N):
            band[i, max(0, i - R): i + 1] = True
        win = _sdpa_rows(Q, K, V, band)
        np.testing.assert_allclose(res["out"], win[L:], rtol=1e-10, atol=1e-10)
        assert res["evicted"].tolist() == [i - R for i in range(L, N)]

    def identical_keys():
        L, T, h, r, d = 40, 30, 6, 5, 5
        Q = g.standard_normal((L + T, d))
        K = np.tile(g.standard_normal(d), (L + T, 1))
        V = g.standard_normal((L + T, d))
        res = m.run_unit(Q, K, V, L, h, r)
        assert res["kept"] == list(range(h)) + list(range(L - r, L))
        assert res["evicted"].tolist() == [L + t - r for t in range(T)]
        H = [Fraction(0)]
        for n in range(1, L + 1):
            H.append(H[-1] + Fraction(1, n))
        np.testing.assert_allclose(res["prefill"].col_sum, [float(H[L] - H[j]) for j in range(L)], rtol=1e-12)

    def brute_force():
        kinds_list = [
            ["strong", "dead", "dead", "strong", "mid", "weak", "strong", "dead", "mid", "mid", "weak", "strong"],
            ["mid", "mid", "weak", "weak", "strong", "dead", "mid", "strong", "weak", "mid", "dead", "weak"],
        ]
        for kinds in kinds_list:
            for (L, h, r) in [(3, 3, 0), (5, 2, 2), (0, 2, 1), (7, 1, 3), (8, 2, 2)]:
                N = len(kinds)
                K = np.array([KEYS2[x] for x in kinds])
                Q = np.tile([1.0, 0.0], (N, 1))
                V = np.arange(N * 2, dtype=float).reshape(N, 2)
                res = m.run_unit(Q, K, V, L, h, r)
                log, S = _brute_force_run(Q, K, V, L, h, r)
                assert res["evicted"].tolist() == log
                assert sorted(res["cache"].pos.tolist()) == S

    def keep_brute():
        for _ in range(200):
            n = int(g.integers(0, 12))
            c = g.choice([0.0, 0.5, 1.0, 2.0], size=n)
            h, r = int(g.integers(0, 4)), int(g.integers(0, 4))
            if h + r == 0:
                continue
            assert m.prefill_keep(c, h, r)[0] == _brute_keep(c, h, r)

    def mass():
        N, L, d = 60, 20, 8
        Q, K, V = (g.standard_normal((N, d)) for _ in range(3))
        res = m.run_unit(Q, K, V, L, 5, 4)
        c = res["cache"]
        assert len(c.pos) == 9
        assert abs(c.score.sum() - (c.rows - c.evicted_mass)) < 1e-9 * c.rows

    return [full_attention, prefill_library, prefill_out, global_comparator, sparse_pattern, rolling, sliding_window, identical_keys, brute_force, keep_brute, mass]


def test_unmutated_oracle_passes_every_check():
    m = _load(open(SRC).read())
    for chk in _checks(m):
        chk()


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_mutation_is_caught(name):
    old, new = MUTATIONS[name]
    src = open(SRC).read()
    assert src.count(old) >= 1, f"mutation anchor not found: {old!r}"
    m = _load(src.replace(old, new, 1))
    caught = []
    for chk in _checks(m):
        try:
            chk()
        except Exception as e:  # noqa: BLE001 - any failure is a catch
            caught.append((chk.__name__, type(e).__name__))
    assert caught, f"mutation '{name}' passed every pin"
