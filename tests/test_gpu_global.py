"""The global-score comparator through the C ABI against the oracle (needs an
MI355X): column scores of a whole sequence, the keep/evict rule under fixed
scores (identical scores on both sides, so every decision must match exactly),
and the comparator end to end (column scores over all N tokens, then the scored
prefill and decode, near-ties replayed as for H2O)."""
import numpy as np
import pytest
import torch

from workload import get, scaled, synth

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)

from gpu_harness import check_payloads, log, run_gpu, run_gpu_scored, unit_payload  # noqa: E402
from kv_cache_eviction_prefill_amd import H2OCache  # noqa: E402

DEV = torch.device("cuda", 0)


def _inputs(w):
    Q, K, V = synth.batch_qkv(w, 0)
    return Q, K, V, tuple(synth.to_torch(w, x, DEV) for x in (Q, K, V))


@pytest.mark.parametrize("wl,d,N,B,H", [
    ("tiny-fp32", 64, 320, 1, 1), ("tiny-fp32", 128, 33, 1, 2),
    ("opt6.7b-layer-b16", 128, 1, 1, 2), ("opt6.7b-layer-b16", 128, 77, 2, 3),
    ("opt6.7b-layer-b16", 64, 600, 1, 2), ("opt6.7b-layer-b16", 128, 1024, 2, 2),
])
def test_column_scores_match_oracle(wl, d, N, B, H):
    from oracle import global_scores

    w = scaled(get(wl), batch=B, heads=H, head_dim=d, prompt_len=N, decode_steps=0, n_anchors=max(1, N // 50))
    Q, K, _, (q, k, _) = _inputs(w)
    cache = H2OCache(B, H, d, 4, 4, dtype=w.dtype, max_prompt=N)
    c = cache.column_scores(q, k).cpu().numpy()
    cache.close()
    worst = 0.0
    for b in range(B):
        for h in range(H):
            ref = global_scores(Q[b, h].astype(np.float64), K[b, h].astype(np.float64), 1 / np.sqrt(d))
            rel = np.abs(c[b, h] - ref) / ref
            worst = max(worst, float(rel.max()))
    log(f"column scores {w.dtype} d={d} N={N}: worst rel {worst:.3g}")
    assert worst <= 1e-4
    assert np.allclose(c.sum(axis=-1), N, rtol=1e-4)  # every row is stochastic


@pytest.mark.parametrize("d,L,T,heavy,recent,B,H", [
    (128, 77, 40, 6, 5, 2, 3),     # ragged prompt
    (128, 200, 33, 20, 0, 1, 4),   # K_r = 0: the new token competes
    (64, 150, 60, 0, 9, 2, 2),     # K_h = 0: sliding window
    (128, 20, 60, 30, 10, 2, 2),   # prompt shorter than the budget
    (128, 0, 80, 12, 12, 1, 2),    # empty prompt
    (128, 700, 80, 150, 150, 1, 4),  # split path (few units, large budget)
])
def test_fixed_scores_decisions_exact(d, L, T, heavy, recent, B, H):
    w = scaled(get("opt6.7b-layer-b16"), batch=B, heads=H, head_dim=d, prompt_len=L, decode_steps=T,
               heavy_budget=heavy, recent_budget=recent, n_anchors=max(1, (L + T) // 50))
    Q, K, V, (q, k, v) = _inputs(w)
    g = np.random.default_rng(L * 7 + T)
    fixed = (g.integers(0, 64, size=(B, H, L + T)) / 16).astype(np.float32)  # many exact ties
    g_res = run_gpu_scored(q, k, v, L, heavy, recent, "bf16", torch.from_numpy(fixed).to(DEV))
    payloads = []
    for b in range(B):
        for h in range(H):
            pl = unit_payload(g_res, b, h, Q[b, h], K[b, h], V[b, h], L, heavy, recent)
            pl.update(mode="fixed", fixed=fixed[b, h].astype(np.float64))
            payloads.append(pl)
    results, bad = check_payloads(payloads)
    assert not bad, bad[:3]
    for r in results:
        assert r["ties"] == 0 and r.get("score_rel", 0.0) == 0.0, r


@pytest.mark.parametrize("d,L,T,heavy,recent,B,H", [
    (128, 256, 128, 26, 26, 2, 4),
    (64, 100, 150, 10, 10, 2, 2),
    (128, 300, 100, 40, 0, 1, 3),
])
def test_global_comparator_end_to_end(d, L, T, heavy, recent, B, H):
    w = scaled(get("opt6.7b-layer-b16"), batch=B, heads=H, head_dim=d, prompt_len=L, decode_steps=T,
               heavy_budget=heavy, recent_budget=recent, n_anchors=max(1, (L + T) // 50))
    Q, K, V, (q, k, v) = _inputs(w)
    g_res = run_gpu_scored(q, k, v, L, heavy, recent, "bf16")
    payloads = []
    for b in range(B):
        for h in range(H):
            pl = unit_payload(g_res, b, h, Q[b, h], K[b, h], V[b, h], L, heavy, recent)
            pl.update(mode="global", gscores=g_res["gscores"][b, h].astype(np.float64))
            payloads.append(pl)
    results, bad = check_payloads(payloads)
    assert not bad, bad[:3]
    for r in results:
        assert "colsum_rel" in r and "out_err" in r, r


@pytest.mark.parametrize("anchor,alpha", [("fixed", 3.0), ("fixed", 32.0), ("zipf", 40.0)])
def test_comparator_quality_report(anchor, alpha):
    # What the greedy local score loses against the global one, on the OPT-6.7B
    # layer shape (512 units, 512 + 512, 20 % budget): each variant's decode
    # outputs against full attention (a budget covering the whole sequence).  The
    # workload's own anchors (alpha = 3) shift an anchor's logit by only
    # alpha / sqrt(d) ~ 0.27, so its attention has no real heavy hitters; the
    # stronger settings (fixed anchors at +2.8, Zipf-ranked strengths) do.  The
    # numbers are a measurement of the method on synthetic inputs, logged, not a
    # pass criterion; the test checks only that the full-budget run evicts nothing.
    w = scaled(get("opt6.7b-layer-b16"), anchor=anchor, alpha=alpha)
    L, T, kh, kr = w.prompt_len, w.decode_steps, w.heavy_budget, w.recent_budget
    _, _, _, (q, k, v) = _inputs(w)
    N = L + T
    full = run_gpu(q, k, v, L, N // 2, N - N // 2, "bf16")
    assert (full["evicted"] == -1).all()
    ref = full["out"].astype(np.float64)
    runs = {"h2o (local)": run_gpu(q, k, v, L, kh, kr, "bf16"),
            "global": run_gpu_scored(q, k, v, L, kh, kr, "bf16"),
            "recent window only": run_gpu(q, k, v, L, 0, kh + kr, "bf16"),
            "heavy hitters only": run_gpu(q, k, v, L, kh + kr, 0, "bf16")}
    for name, r in runs.items():
        o = r["out"].astype(np.float64)
        err = np.abs(o - ref)
        rel = np.linalg.norm((o - ref).reshape(-1)) / np.linalg.norm(ref.reshape(-1))
        log(f"comparator [{anchor} anchors, alpha {alpha:g}] {name}: k = {kh + kr} of {N}: "
            f"mean |o - o_full| {err.mean():.4g}, max {err.max():.4g}, relative L2 {rel:.4g}")
        assert np.isfinite(o).all()
