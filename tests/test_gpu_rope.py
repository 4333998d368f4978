"""Position rolling (rotary embedding at positions inside the cache) through the
C ABI against the oracle (needs an MI355X): prompt statistics on the rotated,
storage-rounded prompt, decode outputs with the rank-gap rotation, evictions,
the split path and the global comparator."""
import numpy as np
import pytest
import torch

from workload import get, scaled, synth

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)

from gpu_harness import check_payloads, log, run_gpu, run_gpu_scored, unit_payload  # noqa: E402

DEV = torch.device("cuda", 0)


def _inputs(w):
    Q, K, V = synth.batch_qkv(w, 0)
    return Q, K, V, tuple(synth.to_torch(w, x, DEV) for x in (Q, K, V))


def _check(g, w, Q, K, V, base, **extra):
    payloads = []
    for b in range(w.batch):
        for h in range(w.heads):
            pl = unit_payload(g, b, h, Q[b, h], K[b, h], V[b, h], w.prompt_len, w.heavy_budget, w.recent_budget)
            pl.update(rope=(base,), **{k: (v[b, h] if isinstance(v, np.ndarray) else v)
                                                for k, v in extra.items()})
            payloads.append(pl)
    results, bad = check_payloads(payloads)
    assert not bad, bad[:3]
    return results


@pytest.mark.parametrize("wl,d,L,T,heavy,recent,B,H,base", [
    ("tiny-fp32", 64, 256, 64, 26, 26, 1, 1, 10000.0),
    ("tiny-fp32", 128, 70, 60, 10, 6, 1, 2, 500.0),
    ("opt6.7b-layer-b16", 128, 300, 120, 30, 10, 2, 3, 10000.0),   # heavy hitters: ranks differ from positions
    ("opt6.7b-layer-b16", 64, 150, 80, 12, 0, 2, 2, 10000.0),      # K_r = 0
    ("opt6.7b-layer-b16", 128, 40, 60, 80, 80, 1, 3, 10000.0),     # nothing evicted: ranks are positions
    ("opt6.7b-layer-b16", 128, 700, 80, 150, 150, 1, 4, 10000.0),  # split path
    ("opt6.7b-layer-b16", 128, 1, 200, 20, 20, 2, 2, 100.0),       # one-token prompt, fast rotation
])
def test_rolling_matches_oracle(wl, d, L, T, heavy, recent, B, H, base):
    w = scaled(get(wl), batch=B, heads=H, head_dim=d, prompt_len=L, decode_steps=T, heavy_budget=heavy,
               recent_budget=recent, n_anchors=max(1, (L + T) // 50))
    Q, K, V, (q, k, v) = _inputs(w)
    log(f"case rolling {w.dtype} d={d} L={L} T={T} K_h={heavy} K_r={recent} base={base}")
    g = run_gpu(q, k, v, L, heavy, recent, w.dtype, rope_base=base)
    res = _check(g, w, Q, K, V, base)
    for r in res:
        assert "out_err" in r and "score_rel" in r and (L == 0 or "colsum_rel" in r), r


def test_rolling_global_comparator():
    w = scaled(get("opt6.7b-layer-b16"), batch=2, heads=2, prompt_len=200, decode_steps=100, heavy_budget=20,
               recent_budget=20, n_anchors=6)
    Q, K, V, (q, k, v) = _inputs(w)
    g = run_gpu_scored(q, k, v, 200, 20, 20, "bf16", rope_base=10000.0)
    res = _check(g, w, Q, K, V, 10000.0, mode="global", gscores=g["gscores"].astype(np.float64))
    for r in res:
        assert "colsum_rel" in r and "out_err" in r, r


def test_rolling_changes_the_outputs():
    # the rotation is not idle: with and without it the outputs differ
    w = scaled(get("opt6.7b-layer-b16"), batch=1, heads=2, prompt_len=100, decode_steps=40, heavy_budget=10,
               recent_budget=10, n_anchors=3)
    _, _, _, (q, k, v) = _inputs(w)
    a = run_gpu(q, k, v, 100, 10, 10, "bf16", rope_base=10000.0)
    b = run_gpu(q, k, v, 100, 10, 10, "bf16")
    assert np.abs(a["out"] - b["out"]).max() > 1e-2
