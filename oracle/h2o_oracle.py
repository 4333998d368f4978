"""CPU oracle for H2O budgeted attention.  TEST INFRASTRUCTURE ONLY.

Only the tests, the package's ``smoke()`` check and the benchmark's CPU-baseline
leg may import this module.  The product path (the HIP library and its Python
binding) never imports, links or runs it, and the two share no code: the only
thing both sides read is the seeded input generator in ``workload/``.

Everything is plain float64 NumPy, one *unit* (one layer / batch element / head)
at a time, on the same storage-rounded inputs the GPU receives (bfloat16 and
float32 values are exact in float64).  H2O is a greedy heuristic, not a faster
route to an exactly defined result, so the oracle runs its steps in the order
the pages give them.

Sources (page title, then section):

* [Report] "H2O: Heavy-Hitter Oracle for Efficient Generative Inference of Large
  Language Models — 深度解读报告" (zako-mio llm-papers-knowledge-base):
  §2.3 (heavy hitters are found greedily from the attention each token has
  received so far), §3.1 (budgeted generation: |S_i| = k, at most one eviction
  per step, evicted entries leave the softmax normaliser D_i), §3.3 (the
  paper's Definition 4.3 / Algorithm 1 eviction rule), §3.4 (system layout:
  preallocated cache overwritten in place, heavy-hitter region plus recent
  ring, the prefill rule and the decode rule).
* [Card] "H2O: Heavy-Hitter Oracle for Efficient Generative Inference of Large
  Language Models" (phantomic12 inference-research paper card): a running
  accumulated-attention score per token, lowest-scoring entries evicted when the
  cache is full, recent tokens kept for locality.

Readings taken where the pages are silent or garbled (each is marked ``READING``
below): the score is the attention a token has *received* (a column sum), the
new token's self-attention counts, attention comes before eviction, one victim
per step drawn from the heavy hitters plus the token leaving the recent window,
ties evict the lowest position, the prefill pool for heavy hitters excludes the
recent window, selection happens only when the prompt exceeds the budget,
scale = 1/sqrt(d), and scores never decay.
"""
from __future__ import annotations

from collections import defaultdict
from dataclasses import dataclass, field

import numpy as np

TIE_RTOL = 1e-5


class ParityMismatch(AssertionError):
    """A replayed decision that is not among the oracle's acceptable choices."""


def default_scale(d: int) -> float:
    """READING: logits are q.k / sqrt(d) (standard scaled dot-product attention)."""
    return 1.0 / np.sqrt(float(d))


def softmax(x: np.ndarray) -> np.ndarray:
    """Softmax of a 1-D float64 vector (max subtracted; exact in real arithmetic)."""
    m = np.max(x)
    e = np.exp(x - m)
    return e / e.sum()


# =============================================================================== prefill
@dataclass
class PrefillScores:
    col_sum: np.ndarray   # c_j: attention received by prompt token j from all prompt rows
    row_max: np.ndarray   # max_j x_rj  (x = scale * q_r . k_j, j <= r)
    row_sum: np.ndarray   # sum_j exp(x_rj - row_max_r)
    weights: np.ndarray   # the causal attention matrix A[r, j] (zero above the diagonal)


def prefill_scores(Q: np.ndarray, K: np.ndarray, scale: float) -> PrefillScores:
    """Column sums of the prompt's causal softmax attention.

    Row r of the prompt attends to positions 0..r (diagonal included) with
    weights a_rj = softmax_j(scale * q_r . k_j).  Token j's score is the total
    attention it receives, c_j = sum over r >= j of a_rj.  [Report §2.3, §3.3;
    Card]  READING: the pages call the statistic a "row sum" of attention, which
    is degenerate for a softmax row (it is always 1); the accumulated attention
    *received* is the reading the rest of the pages support (a token stays
    because later tokens keep attending to it).
    """
    Q = np.asarray(Q, np.float64)
    K = np.asarray(K, np.float64)
    L = Q.shape[0]
    A = np.zeros((L, L))
    row_max = np.zeros(L)
    row_sum = np.zeros(L)
    for r in range(L):
        x = scale * (K[: r + 1] @ Q[r])
        row_max[r] = x.max()
        e = np.exp(x - row_max[r])
        row_sum[r] = e.sum()
        A[r, : r + 1] = e / row_sum[r]
    return PrefillScores(col_sum=A.sum(axis=0), row_max=row_max, row_sum=row_sum, weights=A)


def prefill_output(Q: np.ndarray, K: np.ndarray, V: np.ndarray, scale: float) -> np.ndarray:
    """The prompt's own attention output o_r = sum over j <= r of a_rj v_j, with the
    causal weights of ``prefill_scores``.  The prompt is attended in full: H2O
    bounds the cache only from the first generated token on.  [Report §3.4,
    prefill rule]
    """
    A = prefill_scores(Q, K, scale).weights
    return A @ np.asarray(V, np.float64)


# =============================================================================== position rolling
@dataclass(frozen=True)
class Rope:
    """Rotary position embedding applied at positions inside the cache ("position
    rolling"): the positions are the ranks of the attended entries, not their
    positions in the text.  [Report §4.4, Q1: H2O with position rolling streams
    4 million tokens]

    READINGS (the pages name the technique only): rotary embedding over the pairs
    (m, m + d/2) with frequencies theta_m = base^(-2m/d); at a decode step the
    attended entries (the cached ones plus the new token) take positions
    0, 1, ... in position order, so the new token sits at the last one and a
    cached entry's rotation depends on how many entries lie between; the cache
    keeps keys unrotated.  The prompt is attended before anything is evicted, so
    its positions are its ranks.  Every rotation here is exact (float64), for the
    prompt's score operands as for the decode steps."""

    base: float = 10000.0

    def theta(self, d: int) -> np.ndarray:
        return float(self.base) ** (-2.0 * np.arange(d // 2) / d)

    def rotate(self, X: np.ndarray, pos) -> np.ndarray:
        """Exact rotation of the rows of X [n, d] to positions ``pos`` [n]: each
        pair (x_m, x_{m+d/2}) turns by the angle pos * theta_m."""
        X = np.asarray(X, np.float64)
        h = X.shape[1] // 2
        ang = np.asarray(pos, np.float64)[:, None] * self.theta(X.shape[1])[None, :]
        c, s = np.cos(ang), np.sin(ang)
        x, y = X[:, :h], X[:, h:]
        return np.concatenate([x * c - y * s, x * s + y * c], axis=1)

    def prompt(self, X: np.ndarray) -> np.ndarray:
        """Rows of X [L, d] rotated to their own positions 0..L-1 (the prompt's
        score operands), exactly."""
        X = np.asarray(X, np.float64)
        return self.rotate(X, np.arange(X.shape[0]))


@dataclass(frozen=True)
class Pattern:
    """A Sparse-Transformer attention pattern whose positions H2O keeps in
    preference to its heavy hitters, the heavy hitters filling the rest of the
    budget.  [Report §4.5 (Table 2): heavy hitters added to strided and fixed
    sparse patterns]

    * ``strided`` with period l: at step i the positions j with (i - j) mod l = 0
      (every l-th token counted back from the query).
    * ``fixed`` with period l and width c: the last c positions of every block of
      l tokens (j mod l >= l - c), the same for every query.

    READINGS: the pattern only orders the cache's own entries (an evicted token
    never returns, so the pattern is honoured as far as the cache still holds it);
    keep/evict rank by (protected, score, position), so a protected entry is
    evicted only when every candidate is protected; the prefill ranks the prompt
    as seen by the first generated token (i = L)."""

    kind: str = "none"  # "none", "strided" or "fixed"
    period: int = 1
    width: int = 1

    def protected(self, j: int, i: int) -> bool:
        if self.kind == "strided":
            return (i - j) % self.period == 0
        if self.kind == "fixed":
            return j % self.period >= self.period - self.width
        return False


NO_PATTERN = Pattern()


def prefill_keep(c: np.ndarray, heavy: int, recent: int, prefer=None, tie_rtol: float = TIE_RTOL,
                 pattern: Pattern = NO_PATTERN):
    """Positions kept after the prompt.  [Report §3.4, prefill rule]

    If the prompt fits the budget (L <= k = heavy + recent) every position is
    kept.  Otherwise the last ``recent`` positions are kept, plus the ``heavy``
    best-scored positions among the rest.  READINGS: the heavy-hitter pool is
    [0, L - recent) so the two sets are disjoint and total k; the selection
    threshold is L > k (the pages' "prompt at least 2K" keeps everything at
    L = 2K under both readings); "best" is the reverse of the eviction order, so
    on equal scores the higher position is kept.  With a ``pattern`` the
    positions it protects (for the first generated token, i = L) rank above all
    others.

    ``prefer`` (optional): another kept set.  If it differs from the oracle's only
    by positions whose scores lie within ``tie_rtol`` (relative) of the boundary
    score, it is adopted; otherwise ``ParityMismatch`` is raised.

    Returns ``(kept, info)`` with ``kept`` a sorted list of positions.
    """
    L = len(c)
    k = heavy + recent
    info = {"selected": L > k, "tie_adopted": False, "band": []}
    if L <= k:
        kept = list(range(L))
        if prefer is not None and sorted(prefer) != kept:
            raise ParityMismatch(f"prefill keeps all {L} positions, other side kept {len(prefer)}")
        return kept, info
    pool = list(range(L - recent))
    recent_pos = list(range(L - recent, L))
    prot = {j: pattern.protected(j, L) for j in pool}
    best_first = sorted(pool, key=lambda j: (prot[j], c[j], j), reverse=True)
    heavy_set = best_first[:heavy]
    kept = sorted(heavy_set + recent_pos)
    if prefer is not None:
        prefer = sorted(int(p) for p in prefer)
        if prefer != kept:
            if heavy == 0:
                raise ParityMismatch("no heavy hitters to choose, yet the kept sets differ")
            t = c[best_first[heavy - 1]]
            pt = prot[best_first[heavy - 1]]
            band = {j for j in pool if prot[j] == pt and abs(c[j] - t) <= tie_rtol * abs(t)}
            info["band"] = sorted(band)
            pset, kset = set(prefer), set(kept)
            ok = (len(prefer) == k and set(recent_pos) <= pset
                  and len(pset & set(pool)) == heavy and (pset ^ kset) <= band)
            if not ok:
                raise ParityMismatch(
                    f"kept sets differ outside the near-tie band: only other={sorted(pset - kset)[:8]} "
                    f"only oracle={sorted(kset - pset)[:8]} boundary score={t!r}")
            kept = prefer
            info["tie_adopted"] = True
    return kept, info


# =============================================================================== decode
@dataclass
class UnitCache:
    """The budgeted cache of one unit: the kept set S, each entry's K/V rows and
    accumulated score.  Entry order carries no meaning.  [Report §3.1, §3.4]"""

    heavy: int
    recent: int
    scale: float
    d: int
    pos: np.ndarray = field(default_factory=lambda: np.zeros(0, np.int64))
    K: np.ndarray = None
    V: np.ndarray = None
    score: np.ndarray = field(default_factory=lambda: np.zeros(0))
    next_pos: int = 0
    evicted_mass: float = 0.0
    rows: int = 0  # attention rows processed (prompt rows + decode steps)
    fixed: np.ndarray = None  # per-position scores fixed in advance (global comparator), or None
    pattern: Pattern = NO_PATTERN  # sparse pattern kept in preference to heavy hitters
    rope: Rope = None  # rotary embedding at positions inside the cache, or None

    def __post_init__(self):
        if self.K is None:
            self.K = np.zeros((0, self.d))
        if self.V is None:
            self.V = np.zeros((0, self.d))

    @property
    def k(self) -> int:
        return self.heavy + self.recent

    # ------------------------------------------------------------------ prefill
    @classmethod
    def from_prompt(cls, Qp, Kp, Vp, heavy: int, recent: int, scale: float | None = None,
                    prefer_kept=None, tie_rtol: float = TIE_RTOL, fixed=None,
                    pattern: Pattern = NO_PATTERN, rope: Rope = None):
        """Prefill: score the prompt, keep per ``prefill_keep``, seed the scores
        of the kept entries with their column sums.  READING: prefill column sums
        seed the running scores (the decode steps keep adding to them).

        ``fixed``: scores for every position of the sequence, fixed in advance
        (the global comparator).  The prompt is then ranked by ``fixed[:L]``
        instead of its own column sums, and decode steps add nothing.  ``rope``:
        the prompt is scored on its rotated queries and keys; the cache keeps
        the keys unrotated."""
        Qp, Kp, Vp = (np.asarray(x, np.float64) for x in (Qp, Kp, Vp))
        L, d = Kp.shape if Kp.ndim == 2 else (0, Qp.shape[-1])
        scale = default_scale(d) if scale is None else scale
        cache = cls(heavy=heavy, recent=recent, scale=scale, d=d, pattern=pattern, rope=rope)
        if fixed is not None:
            cache.fixed = np.asarray(fixed, np.float64)
        if L == 0:
            return cache, None, {"selected": False, "tie_adopted": False, "band": []}
        if fixed is None:
            ps = prefill_scores(Qp, Kp, scale) if rope is None else prefill_scores(rope.prompt(Qp), rope.prompt(Kp), scale)
        else:
            ps = None
        c = ps.col_sum if fixed is None else cache.fixed[:L]
        kept, info = prefill_keep(c, heavy, recent, prefer=prefer_kept, tie_rtol=tie_rtol, pattern=pattern)
        kept = np.asarray(kept, np.int64)
        cache.pos = kept
        cache.K = Kp[kept].copy()
        cache.V = Vp[kept].copy()
        cache.score = c[kept].copy()
        dropped = np.setdiff1d(np.arange(L), kept)
        cache.evicted_mass = float(c[dropped].sum())
        cache.next_pos = L
        cache.rows = L
        return cache, ps, info

    # ------------------------------------------------------------------ one decode step
    def step(self, q, k_new, v_new, prefer_victim=None, tie_rtol: float = TIE_RTOL):
        """One generated token at position i = next_pos.

        1. G = S ∪ {i}.  Attend over G only: x_j = scale * q . k_j and
           a = softmax(x) over G, so evicted entries carry no weight and are absent
           from the normaliser.  o = sum_j a_j v_j.  [Report §3.1 (D_i)]
           READING: attention happens before eviction; step i's scores decide it.
        2. Every entry of G adds the attention it just received to its score; the
           new token's score starts at its own weight a_i.  [Report §3.3; Card]
           READING: scores only accumulate (no decay, no reset).  With fixed
           scores (the global comparator) nothing is added and the new token's
           score is its fixed score.
        3. While |S| < k, S = G and nothing is evicted.  Otherwise one entry u
           leaves: the candidates are the entries at positions j <= i - recent
           (the heavy hitters plus the token that just left the recent window;
           with recent = 0 the new token itself is a candidate), and u is the
           candidate whose removal leaves the largest total score, i.e. the one
           with the lowest score, ties going to the lowest position.
           [Report §3.3 (Algorithm 1), §3.4 (decode rule); Card]
           READINGS: the pages' "oldest recent token leaves and each head evicts
           one heavy hitter" is one removal, not two (|S_i| = k and at most one
           eviction per step); the token leaving the window joins the candidates.
           With a sparse ``pattern`` the candidates it protects at step i are
           evicted only when every candidate is protected (see ``Pattern``).

        ``prefer_victim``: another side's decision for this step (a position, or
        -1 for no eviction).  It is adopted when it lies within ``tie_rtol``
        (relative) of the lowest candidate score; any other difference raises
        ``ParityMismatch``.

        Returns ``(o, evicted_position_or_minus1, info)``.
        """
        i = self.next_pos
        q = np.asarray(q, np.float64)
        G_pos = np.concatenate([self.pos, [i]])
        G_K = np.vstack([self.K, np.asarray(k_new, np.float64)[None]])
        G_V = np.vstack([self.V, np.asarray(v_new, np.float64)[None]])
        if self.rope is None:
            x = self.scale * (G_K @ q)
        else:
            # position rolling: the attended entries sit at their ranks 0..|G|-1
            # in position order; the new token (the latest) at |G| - 1
            rank = np.empty(len(G_pos), np.int64)
            rank[np.argsort(G_pos, kind="stable")] = np.arange(len(G_pos))
            qr = self.rope.rotate(q[None], [len(G_pos) - 1])[0]
            x = self.scale * (self.rope.rotate(G_K, rank) @ qr)
        a = softmax(x)
        o = a @ G_V
        if self.fixed is None:
            G_score = np.concatenate([self.score, [0.0]]) + a
        else:
            G_score = np.concatenate([self.score, [self.fixed[i]]])
        info = {"tie_adopted": False, "band": [], "weights": a, "positions": G_pos}
        self.rows += 1
        self.next_pos = i + 1
        if len(self.pos) < self.k:
            if prefer_victim is not None and int(prefer_victim) != -1:
                raise ParityMismatch(f"position {i}: cache not full, other side evicted {prefer_victim}")
            self.pos, self.K, self.V, self.score = G_pos, G_K, G_V, G_score
            return o, -1, info
        cand = np.nonzero(G_pos <= i - self.recent)[0]
        if self.pattern.kind == "none":
            prot = defaultdict(bool)  # nothing is protected
        else:
            prot = {t: self.pattern.protected(int(G_pos[t]), i) for t in cand}
        u = min(cand, key=lambda t: (prot[t], G_score[t], G_pos[t]))
        if prefer_victim is not None and int(prefer_victim) != int(G_pos[u]):
            smin = G_score[u]
            band = [t for t in cand if prot[t] == prot[u] and G_score[t] <= smin + tie_rtol * abs(smin)]
            info["band"] = [int(G_pos[t]) for t in band]
            hit = [t for t in band if int(G_pos[t]) == int(prefer_victim)]
            if not hit:
                raise ParityMismatch(
                    f"position {i}: oracle evicts {int(G_pos[u])} (score {smin!r}), other side "
                    f"{prefer_victim}, not within {tie_rtol} of the lowest candidate score")
            u = hit[0]
            info["tie_adopted"] = True
        keep = np.ones(len(G_pos), bool)
        keep[u] = False
        self.evicted_mass += float(G_score[u])
        evicted = int(G_pos[u])
        self.pos, self.K, self.V, self.score = G_pos[keep], G_K[keep], G_V[keep], G_score[keep]
        return o, evicted, info

    def snapshot(self):
        """(positions, scores, K, V) sorted by position."""
        order = np.argsort(self.pos)
        return self.pos[order].copy(), self.score[order].copy(), self.K[order].copy(), self.V[order].copy()


# =============================================================================== driver
def run_unit(Q, K, V, prompt_len: int, heavy: int, recent: int, scale: float | None = None,
             replay_kept=None, replay_evicted=None, tie_rtol: float = TIE_RTOL,
             keep_weights: bool = False, fixed=None, pattern: Pattern = NO_PATTERN, rope: Rope = None):
    """Prefill then decode one unit over positions 0..N-1 of ``Q, K, V`` ([N, d]).

    ``replay_kept`` / ``replay_evicted``: the other side's prefill kept set and
    per-step eviction log; they are adopted only at near-ties (see
    ``prefill_keep`` and ``UnitCache.step``).  ``fixed``: per-position scores
    [N] fixed in advance (see ``run_unit_global``); None for H2O itself.
    ``pattern``: a sparse pattern kept in preference to heavy hitters.
    ``rope``: rotary embedding at positions inside the cache (position rolling).

    Returns a dict: prefill stats (or None), ``kept`` (sorted prefill kept set),
    ``out`` [T, d], ``evicted`` [T], the final ``cache`` and tie counters.
    """
    Q, K, V = (np.asarray(x, np.float64) for x in (Q, K, V))
    N, d = Q.shape
    L = prompt_len
    cache, ps, pinfo = UnitCache.from_prompt(Q[:L], K[:L], V[:L], heavy, recent, scale,
                                             prefer_kept=replay_kept, tie_rtol=tie_rtol, fixed=fixed,
                                             pattern=pattern, rope=rope)
    kept = [int(p) for p in cache.pos]
    T = N - L
    out = np.zeros((T, d))
    evicted = np.zeros(T, np.int64)
    ties = 0
    weights = []
    for t in range(T):
        pv = None if replay_evicted is None else int(replay_evicted[t])
        o, u, info = cache.step(Q[L + t], K[L + t], V[L + t], prefer_victim=pv, tie_rtol=tie_rtol)
        out[t] = o
        evicted[t] = u
        ties += int(info["tie_adopted"])
        if keep_weights:
            weights.append((info["positions"], info["weights"]))
    return {"prefill": ps, "kept": kept, "prefill_tie_adopted": pinfo["tie_adopted"],
            "out": out, "evicted": evicted, "cache": cache, "decode_ties_adopted": ties,
            "weights": weights}


# =============================================================================== global comparator
def global_scores(Q, K, scale: float) -> np.ndarray:
    """The attention each token receives from every row of the whole sequence:
    c_j = sum over r >= j of a_rj, with a the causal softmax over all N rows
    (prompt and generated alike).  This is the score a heavy-hitter rule could
    use if it saw the future; the pages contrast it with the greedy local score.
    [Report §2.3, the local-versus-global comparison of Figure 2(d)]
    READING: "global" means the column sums of the full causal attention of the
    sequence the unit will see, computed once."""
    return prefill_scores(Q, K, scale).col_sum


def run_unit_global(Q, K, V, prompt_len: int, heavy: int, recent: int, scale: float | None = None,
                    replay_kept=None, replay_evicted=None, tie_rtol: float = TIE_RTOL, rope: Rope = None):
    """The global comparator: the same prefill keep and decode eviction rule as
    ``run_unit``, but every token's score is its global score (``global_scores``
    over all N rows), fixed in advance; decode steps accumulate nothing.  The
    attention itself is unchanged (normalised over the cached entries only).
    [Report §2.3, Figure 2(d)]
    READING: the recent window, the candidate set (positions <= i - K_r), the tie
    rule and the one-victim-per-step budget are those of H2O; only the score
    differs.  Returns ``run_unit``'s dict plus ``scores`` (the global scores)."""
    Q, K, V = (np.asarray(x, np.float64) for x in (Q, K, V))
    scale = default_scale(Q.shape[1]) if scale is None else scale
    g = global_scores(Q, K, scale) if rope is None else global_scores(rope.prompt(Q), rope.prompt(K), scale)
    res = run_unit(Q, K, V, prompt_len, heavy, recent, scale, replay_kept=replay_kept,
                   replay_evicted=replay_evicted, tie_rtol=tie_rtol, fixed=g, rope=rope)
    res["scores"] = g
    return res
