"""The prompt's own attention output (optional ``out`` of the prefill) against the
oracle, through the C ABI (needs an MI355X).

Every element must lie within 2e-3 absolute of the oracle (the attention-output
tolerance).  A tighter bound derived from the arithmetic is checked as well, per
element (r, e), with m_re = sum_j a_rj |v_je|:
  - f32 caches: logits, normaliser and weights in fp32, so every weight carries a
    relative error of a few fp32 ulps times the logit magnitude; 2e-5 m_re
    covers it.
  - bf16 caches: each weight enters the product with V as two bf16 parts, hi (its
    top 8 significant bits) and lo = bf16(weight - hi), whose sum is the weight
    to 2^-16 relative, so |o - o_exact| <= (2^-16 + 2e-5) m_re.
With position rolling the logits come from rotated operands that are not bf16
values: the kernels carry each as hi + lo (to 2^-18 relative, the lo.lo product
left out), fp32 ones in fp32 (2^-22), so the logit x_rj = scale q_r.k_j is off
by at most e_rj = scale ROT sum_e |q_re k_je|, each weight by at most twice the
row's largest e_rj relative, and the bound gains 4 max_j e_rj m_re.
A wrong weight, key or value row gives errors of the order of m_re itself.
"""
import numpy as np
import pytest
import torch

from workload import get, scaled, synth

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)

from gpu_harness import log, parallel_map  # noqa: E402
from kv_cache_eviction_prefill_amd import H2OCache  # noqa: E402
from oracle import Rope  # noqa: E402

from _oracle_worker import OUT_ATOL, check_prompt_output  # noqa: E402
from _oracle_worker import PROMPT_OUT_ABS as ABS  # noqa: E402
from _oracle_worker import PROMPT_OUT_REL as REL  # noqa: E402

DEV = torch.device("cuda", 0)


def _gpu_prefill_out(w, q, k, v, rope_base=0.0):
    B, H, L, d = q.shape
    cache = H2OCache(B, H, d, w.heavy_budget, w.recent_budget, dtype=w.dtype, max_prompt=L, rope_base=rope_base)
    out = torch.full((B, H, L, d), float("nan"), dtype=torch.float32, device=DEV)
    cache.prefill(q, k, v, out=out)
    res = {"out": out, "kept": cache.read(), "stats": cache.prefill_stats()}
    cache.close()
    return res


def _check_unit(w, Q, K, V, o, tag, rope=None):
    """Compare one unit's [L, d] output with the oracle (2e-3 absolute and the
    derived bound); returns the worst err/bound.  ``rope``: the prompt is
    attended on its queries and keys rotated to their positions."""
    return check_prompt_output({"dtype": w.dtype, "Q": Q, "K": K, "V": V, "o": o, "tag": tag,
                                "rope_base": rope.base if rope is not None else 0.0})


def _run(w, units=None, rope_base=0.0):
    Q, K, V = synth.batch_qkv(w, 0, 0, w.prompt_len)
    q, k, v = (synth.to_torch(w, x, DEV) for x in (Q, K, V))
    g = _gpu_prefill_out(w, q, k, v, rope_base)
    g["out"] = g["out"].cpu().numpy()
    units = units or [(b, h) for b in range(w.batch) for h in range(w.heads)]
    rope = Rope(rope_base) if rope_base > 0 else None
    worst = max(_check_unit(w, Q[b, h], K[b, h], V[b, h], g["out"][b, h], f"b{b}h{h}", rope) for b, h in units)
    log(f"prefill output {w.dtype} d={w.head_dim} L={w.prompt_len} rope={rope_base} units={len(units)}: "
        f"worst err/bound {worst:.3f}")
    return g, (q, k, v)


def test_tiny_fp32_prefill_output():
    _run(get("tiny-fp32"))


@pytest.mark.parametrize("d,L", [(128, 70), (64, 1), (64, 129)])
def test_fp32_shapes(d, L):
    _run(scaled(get("tiny-fp32"), batch=2, heads=2, head_dim=d, prompt_len=L, decode_steps=0,
                n_anchors=max(1, L // 50)))


@pytest.mark.parametrize("d,L,B,H", [
    (128, 1, 2, 2),       # one row: o_0 = v_0
    (128, 31, 2, 2),      # shorter than one key tile
    (128, 77, 2, 3),      # ragged, inside one 128-row block
    (64, 128, 2, 2),      # exactly one row block
    (64, 513, 1, 2),      # five row blocks and a one-row tail
    (128, 300, 1, 4),     # three row blocks, ragged
    (128, 1000, 1, 2),    # many key tiles, two rows of blocks per pair
])
def test_bf16_shapes(d, L, B, H):
    w = scaled(get("opt6.7b-layer-b16"), batch=B, heads=H, head_dim=d, prompt_len=L, decode_steps=0,
               n_anchors=max(1, L // 50))
    _run(w)


@pytest.mark.parametrize("dtype,d,L,B,H", [
    ("bf16", 128, 300, 1, 3),   # split operands (hi, lo) in the output pass, ragged
    ("bf16", 64, 129, 2, 2),
    ("bf16", 128, 1, 1, 2),
    ("f32", 64, 70, 1, 2),
])
def test_rolling_prefill_output(dtype, d, L, B, H):
    # position rolling: the prompt is attended on q and k rotated to their positions
    base = get("tiny-fp32") if dtype == "f32" else get("opt6.7b-layer-b16")
    w = scaled(base, batch=B, heads=H, head_dim=d, prompt_len=L, decode_steps=0, n_anchors=max(1, L // 50))
    _run(w, rope_base=10000.0)


def test_output_leaves_cache_and_statistics_unchanged():
    w = scaled(get("opt6.7b-layer-b16"), batch=2, heads=3, prompt_len=300, decode_steps=0,
               heavy_budget=30, recent_budget=30)
    g, (q, k, v) = _run(w)
    cache = H2OCache(w.batch, w.heads, w.head_dim, 30, 30, dtype="bf16", max_prompt=300)
    cache.prefill(q, k, v)
    plain = {"kept": cache.read(), "stats": cache.prefill_stats()}
    cache.close()
    for key in ("pos", "score", "k", "v"):
        assert np.array_equal(np.asarray(g["kept"][key]), np.asarray(plain["kept"][key])), key
    for s in range(len(plain["stats"])):
        assert np.array_equal(g["stats"][s].view(np.uint32), plain["stats"][s].view(np.uint32))


def test_identical_keys_running_mean():
    # equal keys: row r weights positions 0..r equally
    w = scaled(get("opt6.7b-layer-b16"), batch=1, heads=2, prompt_len=260, decode_steps=0, n_anchors=5)
    Q, K, V = synth.batch_qkv(w, 0, 0, w.prompt_len)
    K[:] = K[:, :, :1].copy()
    q, k, v = (synth.to_torch(w, x, DEV) for x in (Q, K, V))
    g = _gpu_prefill_out(w, q, k, v)
    g["out"] = g["out"].cpu().numpy()
    n = np.arange(1, w.prompt_len + 1)[:, None]
    mean = np.cumsum(V.astype(np.float64), axis=2) / n
    mag = np.cumsum(np.abs(V.astype(np.float64)), axis=2) / n
    assert (np.abs(g["out"] - mean) <= OUT_ATOL).all()
    assert (np.abs(g["out"] - mean) <= REL["bf16"] * mag + ABS["bf16"]).all()


def test_bench_shape_every_unit():
    # the benchmark's launch configuration (2048 units, prompt 2048, d = 128),
    # every unit checked by the oracle (worker processes)
    w = get("opt6.7b-32L-b64")
    L = w.prompt_len
    q, k, v = synth.torch_qkv(w, 0, 0, L, DEV)
    log(f"prefill output at full shape: B={w.batch} H={w.heads} L={L}")
    g = _gpu_prefill_out(w, q, k, v)
    out = g["out"].cpu().numpy()
    payloads = [{"dtype": w.dtype, "Q": q[b, h].to(torch.float32).cpu().numpy(),
                 "K": k[b, h].to(torch.float32).cpu().numpy(), "V": v[b, h].to(torch.float32).cpu().numpy(),
                 "o": out[b, h], "tag": f"b{b}h{h}", "rope_base": 0.0}
                for b in range(w.batch) for h in range(w.heads)]
    del q, k, v, g
    torch.cuda.empty_cache()
    worst = parallel_map(check_prompt_output, payloads)
    assert len(worst) == w.batch * w.heads
    log(f"full shape: {len(worst)} units, worst err/bound {max(worst):.3f}")
