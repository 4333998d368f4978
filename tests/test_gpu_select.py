"""The prefill selection on the GPU against the oracle on score patterns that
reach every branch of the radix select (needs an MI355X).  The prompt is ranked
by scores both sides receive (the scored prefill), so the kept set and every
later decision must match exactly: scores all equal (no score bit differs, the
positions decide), a tie straddling the boundary, values spread over the whole
exponent range, zeros and subnormals, a long prompt whose tied positions need
two position digits, a protected pattern (the key's top bit), and the extreme
budgets K_h = 1 and K_h = pool - 1."""
import numpy as np
import pytest
import torch

from workload import get, scaled, synth

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)

from gpu_harness import check_payloads, log, run_gpu_scored, unit_payload  # noqa: E402

DEV = torch.device("cuda", 0)


def _scores(kind, rng, B, H, N):
    shape = (B, H, N)
    if kind == "all-equal":
        s = np.ones(shape)
    elif kind == "boundary-tie":
        # a few clear winners, then one value shared by most of the pool, so the
        # K_h-th best lies inside a large group of equal scores
        s = np.full(shape, 0.75)
        s[..., rng.permutation(N)[: N // 20]] = 2.0 + rng.random((B, H, N // 20))
        s[..., rng.permutation(N)[: N // 4]] = 0.25
    elif kind == "wide-range":
        # distinct powers 2^(a/4), a spread over [-400, 400): every exponent bit varies
        a = np.stack([np.stack([rng.permutation(800)[:N] for _ in range(H)]) for _ in range(B)])
        s = 2.0 ** ((a - 400) / 4.0)
    elif kind == "zeros-subnormal":
        s = rng.choice(np.array([0.0, 1e-45, 3e-44, 1e-40, 2.5e-39, 1e-30, 0.5]), size=shape)
    elif kind == "discrete":
        s = rng.integers(0, 64, size=shape) / 16
    else:
        raise ValueError(kind)
    return s.astype(np.float32)


def _run(kind, d, L, T, heavy, recent, B=1, H=2, dtype="bf16", pattern=None, seed=0):
    base = get("opt6.7b-layer-b16") if dtype == "bf16" else get("tiny-fp32")
    w = scaled(base, batch=B, heads=H, head_dim=d, prompt_len=L, decode_steps=T, heavy_budget=heavy,
               recent_budget=recent, n_anchors=max(1, (L + T) // 50))
    Q, K, V = synth.batch_qkv(w, 0)
    q, k, v = (synth.to_torch(w, x, DEV) for x in (Q, K, V))
    fixed = _scores(kind, np.random.default_rng(seed + L), B, H, L + T)
    log(f"case select {kind}: {dtype} d={d} L={L} T={T} K_h={heavy} K_r={recent} pattern={pattern}")
    g = run_gpu_scored(q, k, v, L, heavy, recent, dtype, torch.from_numpy(fixed).to(DEV), pattern=pattern)
    payloads = []
    for b in range(B):
        for h in range(H):
            pl = unit_payload(g, b, h, Q[b, h], K[b, h], V[b, h], L, heavy, recent)
            pl.update(mode="fixed", fixed=fixed[b, h].astype(np.float64), pattern=pattern)
            payloads.append(pl)
    results, bad = check_payloads(payloads)
    assert not bad, bad[:3]
    for r in results:
        assert r["ties"] == 0 and r.get("score_rel", 0.0) == 0.0, r
    return g, fixed


@pytest.mark.parametrize("kind", ["all-equal", "boundary-tie", "wide-range", "zeros-subnormal", "discrete"])
def test_select_branches_bf16(kind):
    g, fixed = _run(kind, 128, 700, 8, 100, 50)
    if kind == "all-equal":
        # equal scores keep the highest positions of the pool
        pool = 700 - 50
        for h in range(2):
            assert g["kept"]["pos"][0, h][g["kept"]["pos"][0, h] >= 0].min() == pool - 100


@pytest.mark.parametrize("kind", ["all-equal", "discrete"])
def test_select_long_prompt_two_position_digits(kind):
    # pool positions need 14 bits: the tie pass takes two 8-bit digits
    _run(kind, 128, 9000, 4, 1000, 200)


@pytest.mark.parametrize("kind", ["all-equal", "discrete", "wide-range"])
def test_select_with_pattern_top_bit(kind):
    _run(kind, 128, 600, 8, 80, 40, pattern=("strided", 8, 1))


@pytest.mark.parametrize("heavy,recent,L", [(1, 30, 400), (60, 20, 81), (1, 0, 300), (299, 0, 300)])
def test_select_extreme_budgets(heavy, recent, L):
    # K_h = 1; K_h = pool - 1 (L = k + 1); K_r = 0 with K_h = 1 and K_h = pool - 1
    _run("discrete", 128, L, 6, heavy, recent)


@pytest.mark.parametrize("kind", ["all-equal", "boundary-tie", "wide-range"])
def test_select_fp32_cache(kind):
    _run(kind, 64, 500, 6, 60, 30, dtype="f32")
