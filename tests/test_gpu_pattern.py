"""Heavy hitters added to a sparse attention pattern, through the C ABI against
the oracle (needs an MI355X): the keep/evict rule under fixed scores that both
sides receive (every decision must match exactly), and H2O's own scores with the
pattern (near-ties replayed as usual), for the strided and the fixed pattern."""
import numpy as np
import pytest
import torch

from workload import get, scaled, synth

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)

from gpu_harness import check_payloads, log, run_gpu, run_gpu_scored, unit_payload  # noqa: E402
from kv_cache_eviction_prefill_amd import H2OCache, h2o  # noqa: E402

DEV = torch.device("cuda", 0)
PATTERNS = [("strided", 8, 1), ("fixed", 16, 4)]


def _workload(d, L, T, heavy, recent, B, H):
    w = scaled(get("opt6.7b-layer-b16"), batch=B, heads=H, head_dim=d, prompt_len=L, decode_steps=T,
               heavy_budget=heavy, recent_budget=recent, n_anchors=max(1, (L + T) // 50))
    Q, K, V = synth.batch_qkv(w, 0)
    return w, Q, K, V, tuple(synth.to_torch(w, x, DEV) for x in (Q, K, V))


def _check(g, w, Q, K, V, pattern, **extra):
    payloads = []
    for b in range(w.batch):
        for h in range(w.heads):
            pl = unit_payload(g, b, h, Q[b, h], K[b, h], V[b, h], w.prompt_len, w.heavy_budget, w.recent_budget)
            pl.update(pattern=pattern, **{k: (v[b, h] if isinstance(v, np.ndarray) else v) for k, v in extra.items()})
            payloads.append(pl)
    results, bad = check_payloads(payloads)
    assert not bad, bad[:3]
    return results


@pytest.mark.parametrize("pattern", PATTERNS)
@pytest.mark.parametrize("d,L,T,heavy,recent,B,H", [
    (128, 200, 60, 20, 6, 2, 3),    # prompt selection with protected positions
    (128, 150, 50, 24, 0, 1, 4),    # K_r = 0: the new token competes (strided protects it)
    (64, 40, 120, 12, 8, 2, 2),     # prompt shorter than the budget
    (128, 700, 60, 150, 150, 1, 4),  # split path
])
def test_pattern_fixed_scores_decisions_exact(pattern, d, L, T, heavy, recent, B, H):
    w, Q, K, V, (q, k, v) = _workload(d, L, T, heavy, recent, B, H)
    rng = np.random.default_rng(L + 3 * T)
    fixed = (rng.integers(0, 64, size=(B, H, L + T)) / 16).astype(np.float32)
    g = run_gpu_scored(q, k, v, L, heavy, recent, "bf16", torch.from_numpy(fixed).to(DEV), pattern=pattern)
    log(f"case pattern {pattern} fixed scores d={d} L={L} T={T} K_h={heavy} K_r={recent}")
    res = _check(g, w, Q, K, V, pattern, mode="fixed", fixed=fixed.astype(np.float64))
    for r in res:
        assert r["ties"] == 0 and r.get("score_rel", 0.0) == 0.0, r
    # the pattern is not idle here: without it the decisions differ
    plain = run_gpu_scored(q, k, v, L, heavy, recent, "bf16", torch.from_numpy(fixed).to(DEV))
    assert not np.array_equal(plain["evicted"], g["evicted"])


@pytest.mark.parametrize("pattern", PATTERNS)
@pytest.mark.parametrize("d,L,T,heavy,recent,B,H", [
    (128, 300, 80, 30, 10, 2, 3),
    (64, 120, 100, 16, 0, 2, 2),
])
def test_pattern_h2o_scores_match_oracle(pattern, d, L, T, heavy, recent, B, H):
    w, Q, K, V, (q, k, v) = _workload(d, L, T, heavy, recent, B, H)
    g = run_gpu(q, k, v, L, heavy, recent, "bf16", pattern=pattern)
    log(f"case pattern {pattern} d={d} L={L} T={T} K_h={heavy} K_r={recent}")
    res = _check(g, w, Q, K, V, pattern)
    for r in res:
        assert "score_rel" in r and "out_err" in r, r


def test_set_pattern_validation_and_reset():
    c = H2OCache(1, 2, 64, 4, 4, dtype="bf16", max_prompt=16)
    for args in [(7, 4, 1), (h2o.H2O_PATTERN_STRIDED, 0, 1), (h2o.H2O_PATTERN_FIXED, 4, 0),
                 (h2o.H2O_PATTERN_FIXED, 4, 5)]:
        assert h2o.h2o_cache_set_pattern(c.handle, *args) == h2o.H2O_ERR_INVALID_ARG
    assert h2o.h2o_cache_set_pattern(c.handle, h2o.H2O_PATTERN_FIXED, 4, 4) == h2o.H2O_OK
    assert h2o.h2o_cache_set_pattern(c.handle, h2o.H2O_PATTERN_NONE, 0, 0) == h2o.H2O_OK
    c.close()


def test_explicit_no_pattern_is_plain_h2o():
    # pattern "none" set explicitly: bit-identical to a cache that never had one
    w, Q, K, V, (q, k, v) = _workload(128, 200, 40, 20, 6, 1, 2)
    a = run_gpu(q, k, v, 200, 20, 6, "bf16", pattern=("none", 1, 1))
    b = run_gpu(q, k, v, 200, 20, 6, "bf16")
    assert np.array_equal(a["evicted"], b["evicted"])
    assert np.array_equal(a["out"].view(np.uint32), b["out"].view(np.uint32))
