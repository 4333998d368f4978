"""Per-unit comparison of the GPU results with the CPU oracle.

Runs in worker processes (imports numpy and the oracle only; never torch or the
GPU library).  Tolerances:
  * attention output: 2e-3 absolute per element;
  * scores (prefill column sums, final accumulated scores): 1e-4 relative;
  * prefill row statistics: row max 2e-4 absolute (logit units), row sum 1e-4
    relative (fp32 sums of exactly-multiplied bf16 products, derived bound);
  * kept sets and evicted positions: exact, except near-ties (1e-5 relative),
    where the oracle adopts the GPU's choice and continues.
"""
from __future__ import annotations

import numpy as np

from oracle import NO_PATTERN, ParityMismatch, Pattern, Rope, run_unit, run_unit_global

OUT_ATOL = 2e-3
SCORE_RTOL = 1e-4
# log of each prompt row's softmax normaliser: the row maximum (2e-4 absolute)
# plus the log of the shifted sum (1e-4 relative, i.e. 1e-4 absolute in the log)
LSE_ATOL = 3e-4


def _rel(a, b):
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    return np.abs(a - b) / np.maximum(np.abs(b), 1e-30)


def check_unit(p: dict) -> dict:
    """``p``: Q, K, V [N, d] (float32, storage-rounded), L, heavy, recent, and the
    GPU's results for the unit: kept, evicted [T], out [T, d] (or sampled
    steps), stats (row_lse, col_sum) or None, final (pos, score, k, v).

    ``p["mode"]``: "local" (H2O, the default), "global" (the global-score
    comparator; ``p["gscores"]`` holds the GPU's column scores of the whole
    sequence) or "fixed" (scores ``p["fixed"]`` given to both sides, so every
    decision must agree exactly, with no near-tie adoption).  ``p["pattern"]``:
    (kind, period, width) of a sparse pattern kept before heavy hitters;
    ``p["rope"]``: (base,) of the rotary embedding at positions inside
    the cache; ``p["scale"]``: the logit scale when not 1/sqrt(d)."""
    tag = p["tag"]
    mode = p.get("mode", "local")
    pattern = Pattern(*p["pattern"]) if p.get("pattern") else NO_PATTERN
    rope = Rope(*p["rope"]) if p.get("rope") else None
    res = {"tag": tag, "ok": True, "msg": ""}
    try:
        if mode == "global":
            o = run_unit_global(p["Q"], p["K"], p["V"], p["L"], p["heavy"], p["recent"], p.get("scale"),
                                replay_kept=p["kept"], replay_evicted=p["evicted"], rope=rope)
        else:
            o = run_unit(p["Q"], p["K"], p["V"], p["L"], p["heavy"], p["recent"], p.get("scale"),
                         replay_kept=p["kept"], replay_evicted=p["evicted"],
                         fixed=p["fixed"] if mode == "fixed" else None, pattern=pattern, rope=rope)
    except ParityMismatch as e:
        return {"tag": tag, "ok": False, "msg": f"decision mismatch: {e}"}
    res["ties"] = int(o["decode_ties_adopted"]) + int(o["prefill_tie_adopted"])
    msgs = []
    if mode == "fixed" and res["ties"]:
        msgs.append(f"{res['ties']} decisions differ under identical fixed scores")
    if mode == "global":
        e_g = float(np.max(_rel(p["gscores"], o["scores"])))
        res["colsum_rel"] = e_g
        if e_g > SCORE_RTOL:
            msgs.append(f"global column score rel {e_g:.3g}")
    # prefill statistics
    st = p.get("stats")
    if st is not None and o["prefill"] is not None:
        ps = o["prefill"]
        e_lse = np.max(np.abs(st[0] - (ps.row_max + np.log(ps.row_sum))))
        e_c = np.max(_rel(st[1], ps.col_sum))
        res.update(lse_err=float(e_lse), colsum_rel=float(e_c))
        if e_lse > LSE_ATOL:
            msgs.append(f"row lse err {e_lse:.3g}")
        if e_c > SCORE_RTOL:
            j = int(np.argmax(_rel(st[1], ps.col_sum)))
            msgs.append(f"col_sum rel {e_c:.3g} at {j}: gpu {st[1][j]!r} oracle {ps.col_sum[j]!r}")
    # per-step outputs and evictions
    if not np.array_equal(np.asarray(p["evicted"]), o["evicted"]):
        msgs.append("evicted log differs after replay")
    steps = p.get("out_steps")
    out_ref = o["out"] if steps is None else o["out"][steps]
    if len(out_ref):
        e_o = float(np.max(np.abs(p["out"] - out_ref)))
        res["out_err"] = e_o
        if e_o > OUT_ATOL:
            msgs.append(f"out err {e_o:.3g}")
    # final cache: same positions, scores within tolerance, K/V rows exact
    pos, score, kr, vr = o["cache"].snapshot()
    gpos, gscore, gk, gv = p["final"]
    valid = gpos >= 0
    order = np.argsort(gpos[valid])
    gp = gpos[valid][order]
    if not np.array_equal(gp, pos):
        msgs.append(f"final positions differ: gpu {gp[:10]} oracle {pos[:10]}")
    else:
        e_s = float(np.max(_rel(gscore[valid][order], score))) if len(pos) else 0.0
        res["score_rel"] = e_s
        if e_s > SCORE_RTOL:
            msgs.append(f"score rel {e_s:.3g}")
        if not (np.array_equal(gk[valid][order], kr) and np.array_equal(gv[valid][order], vr)):
            msgs.append("cached K/V rows differ from the inputs at those positions")
    if msgs:
        res["ok"] = False
        res["msg"] = "; ".join(msgs)
    return res


def continue_unit(p: dict) -> dict:
    """Snapshot mode: the oracle starts from the GPU's cache of one unit (``p["snap"]``:
    positions, scores with the compensation folded in, K and V rows) at position
    ``p["next_pos"]`` and runs the decode steps of ``p["q"], p["k"], p["v"]``
    ([T, d]), adopting the GPU's eviction ``p["evicted"]`` only at near-ties.
    Compared: every step's output with ``p["out"]`` (2e-3 absolute), every
    eviction (exact), and the cache after the steps with ``p["after"]``
    (positions exact, scores 1e-4 relative, K/V rows exact)."""
    from oracle import TIE_RTOL, UnitCache, default_scale

    tag = p["tag"]
    pos, score, K, V = p["snap"]
    d = K.shape[1]
    uc = UnitCache(heavy=p["heavy"], recent=p["recent"], scale=default_scale(d), d=d,
                   pos=np.asarray(pos, np.int64), K=np.asarray(K, np.float64), V=np.asarray(V, np.float64),
                   score=np.asarray(score, np.float64), next_pos=int(p["next_pos"]))
    res = {"tag": tag, "ok": True, "msg": "", "ties": 0, "out_err": 0.0, "score_rel": 0.0}
    try:
        for t in range(len(p["q"])):
            o, u, info = uc.step(p["q"][t], p["k"][t], p["v"][t], prefer_victim=int(p["evicted"][t]),
                                 tie_rtol=TIE_RTOL)
            res["ties"] += int(info["tie_adopted"])
            res["out_err"] = max(res["out_err"], float(np.max(np.abs(p["out"][t] - o))))
    except ParityMismatch as e:
        return {"tag": tag, "ok": False, "msg": f"decision mismatch: {e}"}
    msgs = []
    if res["out_err"] > OUT_ATOL:
        msgs.append(f"out err {res['out_err']:.3g}")
    op, osc, ok_, ov = uc.snapshot()
    gpos, gscore, gk, gv = p["after"]
    order = np.argsort(gpos)
    if not np.array_equal(gpos[order], op):
        msgs.append("positions differ after the steps")
    else:
        res["score_rel"] = float(np.max(_rel(gscore[order], osc)))
        if res["score_rel"] > SCORE_RTOL:
            msgs.append(f"score rel {res['score_rel']:.3g}")
        if not (np.array_equal(gk[order], ok_) and np.array_equal(gv[order], ov)):
            msgs.append("cached K/V rows differ from the inputs at those positions")
    if msgs:
        res["ok"] = False
        res["msg"] = "; ".join(msgs)
    return res


# The prompt's own attention output: per-element bound rel * m_re + abs with
# m_re = sum_j a_rj |v_je| (the derivation is in test_gpu_prefill_out.py);
# with position rolling the relative part gains 4 max_j e_rj, e_rj = scale ROT
# sum_e |q_re k_je|.
PROMPT_OUT_REL = {"f32": 2e-5, "bf16": 2.0 ** -16 + 2e-5}
PROMPT_OUT_ABS = {"f32": 1e-6, "bf16": 1e-6}
PROMPT_OUT_ROT = {"f32": 2.0 ** -22, "bf16": 3 * 2.0 ** -18}


def check_prompt_output(p):
    """Compare one unit's [L, d] prompt output ``p["o"]`` with the oracle: every
    element within OUT_ATOL and within the derived bound.  ``p``: dtype, Q, K, V
    (float arrays [L, d]), o, tag, rope_base (0: none).  Returns the worst
    err/bound; raises AssertionError on a miss."""
    import math

    from oracle import prefill_output, prefill_scores

    Q, K, V = (np.asarray(p[x], np.float64) for x in ("Q", "K", "V"))
    o, tag, dt = p["o"], p["tag"], p["dtype"]
    rope = Rope(base=p["rope_base"]) if p.get("rope_base") else None
    if rope is not None:
        Q, K = rope.prompt(Q), rope.prompt(K)
    scale = 1.0 / math.sqrt(Q.shape[1])
    ref = prefill_output(Q, K, V, scale)
    mag = prefill_scores(Q, K, scale).weights @ np.abs(V)
    rel = PROMPT_OUT_REL[dt]
    if rope is not None:
        e = scale * PROMPT_OUT_ROT[dt] * (np.abs(Q) @ np.abs(K).T)
        rel = rel + 4 * np.max(np.tril(e), axis=1, keepdims=True)
    bound = rel * mag + PROMPT_OUT_ABS[dt]
    assert np.isfinite(o).all(), f"{tag}: output not fully written"
    err = np.abs(np.asarray(o, np.float64) - ref)
    assert float(err.max()) <= OUT_ATOL, f"{tag}: max abs error {float(err.max()):.3g} above {OUT_ATOL}"
    worst = float((err / bound).max())
    bad = np.argwhere(err > bound)
    assert bad.size == 0, (f"{tag}: {len(bad)} elements outside the bound, first (row, col) "
                           f"{bad[0].tolist()}: got {o[tuple(bad[0])]}, oracle {ref[tuple(bad[0])]}")
    return worst
