"""The library's limits on the GPU against the oracle (needs an MI355X): the
largest budget (k = 12288 slots) on the split path and on the single-block
path, head_dim 64 at the benchmark's full launch shape, small budgets over
many units (the 128-thread decode blocks) for both storage types and head sizes,
larger bf16 budgets over many units (the one-wave decode blocks) and short split
slices (the one-wave partial blocks).  Inputs come from
the device-side generator; the oracle reads the sampled units' inputs back from
those tensors and runs each unit in full."""
import numpy as np
import pytest
import torch

from workload import get, scaled, synth

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)

from gpu_harness import check_payloads, log, run_gpu, unit_payload  # noqa: E402

DEV = torch.device("cuda", 0)
K_MAX = 12288


def _run(w, units, T):
    L = w.prompt_len
    q, k, v = synth.torch_qkv(w, 0, 0, L + T, DEV)
    log(f"case {w.name}: B={w.batch} H={w.heads} d={w.head_dim} L={L} T={T} k={w.k}; {len(units)} sampled units")
    g = run_gpu(q, k, v, L, w.heavy_budget, w.recent_budget, w.dtype, out_units=units)
    payloads = []
    for n, (b, h) in enumerate(units):
        Q, K, V = (x[b, h].to(torch.float32).cpu().numpy() for x in (q, k, v))
        payloads.append(unit_payload(g, b, h, Q, K, V, L, w.heavy_budget, w.recent_budget, out_index=n,
                                     tag=f"{w.name}/b{b}h{h}"))
    del q, k, v
    torch.cuda.empty_cache()
    results, bad = check_payloads(payloads)
    assert not bad, bad[:3]
    for r in results:
        assert "score_rel" in r and "out_err" in r and "colsum_rel" in r, r
    # the budget holds exactly
    assert ((g["final"]["pos"] >= 0).sum(-1) == min(L + T, w.k)).all()
    return g


def test_largest_budget_split_path():
    # 2 units: each unit's 12288 slots are spread over 64 blocks, the finish launch
    # loads most of its metadata inside the loop
    w = scaled(get("llama7b-stream-4m"), batch=1, heads=2, prompt_len=12400, decode_steps=24,
               heavy_budget=K_MAX // 2, recent_budget=K_MAX // 2, n_anchors=64)
    _run(w, [(0, 0), (0, 1)], 24)


def test_largest_budget_single_block_path():
    # 512 units (one block per unit): 48 KB of logits in LDS per block
    w = scaled(get("opt6.7b-32L-b64"), layers=1, batch=4, heads=128, head_dim=64, prompt_len=12300,
               decode_steps=8, heavy_budget=K_MAX // 2, recent_budget=K_MAX // 2, n_anchors=64)
    _run(w, [(0, 3), (3, 100)], 8)


def test_head_dim_64_at_full_shape():
    # the benchmark's 2048 units and 2048-token prompt, head_dim 64
    w = scaled(get("opt6.7b-32L-b64"), layers=1, head_dim=64, decode_steps=96)
    rng = np.random.default_rng(64)
    idx = rng.choice(w.batch * w.heads, size=6, replace=False)
    _run(w, [(int(i) // w.heads, int(i) % w.heads) for i in sorted(idx)], 96)


@pytest.mark.parametrize("base,d", [("opt6.7b-layer-b16", 128), ("opt6.7b-layer-b16", 64), ("tiny-fp32", 64),
                                    ("tiny-fp32", 128)])
def test_small_budget_many_units(base, d):
    # 1,024 units with k = 32 and 1,024 units with k = 128 (the largest budget on
    # the 128-thread blocks), prompt longer than the budget
    for heavy, recent in ((20, 12), (64, 64)):
        w = scaled(get(base), layers=1, batch=32, heads=32, head_dim=d, prompt_len=300, decode_steps=40,
                   heavy_budget=heavy, recent_budget=recent, n_anchors=6)
        rng = np.random.default_rng(d + heavy)
        idx = rng.choice(w.batch * w.heads, size=4, replace=False)
        _run(w, [(int(i) // w.heads, int(i) % w.heads) for i in sorted(idx)], 40)


@pytest.mark.parametrize("variant", ["rope", "pattern", "fixed"])
def test_small_budget_blocks_with_variants(variant):
    # the 128-thread decode blocks (k <= 128 over >= 1024 units) with position
    # rolling, with a sparse pattern and with fixed scores
    from gpu_harness import run_gpu_scored

    L, T, heavy, recent = 200, 30, 24, 16
    w = scaled(get("opt6.7b-layer-b16"), layers=1, batch=32, heads=32, prompt_len=L, decode_steps=T,
               heavy_budget=heavy, recent_budget=recent, n_anchors=5)
    q, k, v = synth.torch_qkv(w, 0, 0, L + T, DEV)
    units = [(1, 3), (17, 30)]
    extra, fixed = {}, None
    if variant == "rope":
        g = run_gpu(q, k, v, L, heavy, recent, "bf16", out_units=units, rope_base=10000.0)
        extra = {"rope": (10000.0,)}
    elif variant == "pattern":
        g = run_gpu(q, k, v, L, heavy, recent, "bf16", out_units=units, pattern=("strided", 8, 1))
        extra = {"pattern": ("strided", 8, 1)}
    else:
        fixed = (np.random.default_rng(5).integers(0, 64, size=(w.batch, w.heads, L + T)) / 16).astype(np.float32)
        g = run_gpu_scored(q, k, v, L, heavy, recent, "bf16", torch.from_numpy(fixed).to(DEV))
    log(f"case small-budget blocks with {variant}: 1024 units, k={heavy + recent}")
    payloads = []
    for n, (b, h) in enumerate(units):
        Q, K, V = (x[b, h].to(torch.float32).cpu().numpy() for x in (q, k, v))
        pl = unit_payload(g, b, h, Q, K, V, L, heavy, recent, out_index=None if fixed is not None else n)
        pl.update(extra)
        if fixed is not None:
            pl.update(mode="fixed", fixed=fixed[b, h].astype(np.float64))
        payloads.append(pl)
    results, bad = check_payloads(payloads)
    assert not bad, bad[:3]
    for r in results:
        assert "score_rel" in r and "out_err" in r, r


def test_small_budget_blocks_cache_filling():
    # 1,024 units on the 128-thread blocks with a prompt shorter than the budget:
    # the cache fills during decode (new tokens take free slots), then evicts
    w = scaled(get("opt6.7b-layer-b16"), layers=1, batch=32, heads=32, prompt_len=50, decode_steps=120,
               heavy_budget=64, recent_budget=64, n_anchors=4)
    g = _run(w, [(0, 0), (13, 7), (31, 31)], 120)
    ev = g["evicted"]
    assert (ev[: 128 - 50] == -1).all() and (ev[128 - 50:] >= 0).all()


@pytest.mark.parametrize("heavy,recent", [(65, 64), (150, 150)])
def test_one_wave_blocks(heavy, recent):
    # bf16 d=128, 1,024 units with k = 129 (the smallest budget on the one-wave
    # blocks) and k = 300 (slots not a multiple of the 32 in flight per wave)
    w = scaled(get("opt6.7b-layer-b16"), layers=1, batch=32, heads=32, prompt_len=420, decode_steps=40,
               heavy_budget=heavy, recent_budget=recent, n_anchors=6)
    rng = np.random.default_rng(heavy + recent)
    idx = rng.choice(w.batch * w.heads, size=4, replace=False)
    _run(w, [(int(i) // w.heads, int(i) % w.heads) for i in sorted(idx)], 40)


@pytest.mark.parametrize("variant,heavy,recent", [("rope", 90, 70), ("rope", 170, 130), ("pattern", 90, 70),
                                                  ("fixed", 90, 70)])
def test_one_wave_blocks_with_variants(variant, heavy, recent):
    # 1,024 bf16 units at k = 160 (and 300 with rolling: slots not a multiple of
    # the 32 in flight per block): the pattern and fixed-score variants run on
    # the one-wave blocks, position rolling on the two-wave blocks
    from gpu_harness import run_gpu_scored

    L, T = 330, 30
    w = scaled(get("opt6.7b-layer-b16"), layers=1, batch=32, heads=32, prompt_len=L, decode_steps=T,
               heavy_budget=heavy, recent_budget=recent, n_anchors=5)
    q, k, v = synth.torch_qkv(w, 0, 0, L + T, DEV)
    units = [(2, 5), (30, 17)]
    extra, fixed = {}, None
    if variant == "rope":
        g = run_gpu(q, k, v, L, heavy, recent, "bf16", out_units=units, rope_base=10000.0)
        extra = {"rope": (10000.0,)}
    elif variant == "pattern":
        g = run_gpu(q, k, v, L, heavy, recent, "bf16", out_units=units, pattern=("fixed", 16, 2))
        extra = {"pattern": ("fixed", 16, 2)}
    else:
        fixed = (np.random.default_rng(6).integers(0, 64, size=(w.batch, w.heads, L + T)) / 16).astype(np.float32)
        g = run_gpu_scored(q, k, v, L, heavy, recent, "bf16", torch.from_numpy(fixed).to(DEV))
    log(f"case one-wave blocks with {variant}: 1024 units, k={heavy + recent}")
    payloads = []
    for n, (b, h) in enumerate(units):
        Q, K, V = (x[b, h].to(torch.float32).cpu().numpy() for x in (q, k, v))
        pl = unit_payload(g, b, h, Q, K, V, L, heavy, recent, out_index=None if fixed is not None else n)
        pl.update(extra)
        if fixed is not None:
            pl.update(mode="fixed", fixed=fixed[b, h].astype(np.float64))
        payloads.append(pl)
    results, bad = check_payloads(payloads)
    assert not bad, bad[:3]
    for r in results:
        assert "score_rel" in r and "out_err" in r, r


def test_one_wave_blocks_cache_filling():
    # 1,024 bf16 units on the one-wave blocks with a prompt shorter than the
    # budget: new tokens take free slots until the cache is full, then evict
    w = scaled(get("opt6.7b-layer-b16"), layers=1, batch=32, heads=32, prompt_len=100, decode_steps=140,
               heavy_budget=100, recent_budget=100, n_anchors=4)
    g = _run(w, [(0, 0), (9, 21), (31, 31)], 140)
    ev = g["evicted"]
    assert (ev[: 200 - 100] == -1).all() and (ev[200 - 100:] >= 0).all()


@pytest.mark.parametrize("batch,heads,L,T,heavy,recent", [
    (1, 8, 1500, 40, 512, 512),   # 8 units: 16 slices of 64 slots per unit
    (1, 8, 700, 60, 512, 512),    # the cache fills during decode: 10 slices of 70-76 slots
    (4, 64, 600, 30, 256, 256),   # 256 units: 4 slices of 128 slots, the longest on one-wave blocks
])
def test_one_wave_split_blocks(batch, heads, L, T, heavy, recent):
    # the split path's partial blocks for bf16 d=128 with short slices run one wave each
    w = scaled(get("opt6.7b-layer-b16"), layers=1, batch=batch, heads=heads, prompt_len=L, decode_steps=T,
               heavy_budget=heavy, recent_budget=recent, n_anchors=6)
    rng = np.random.default_rng(L + heads)
    idx = rng.choice(w.batch * w.heads, size=2, replace=False)
    _run(w, [(int(i) // w.heads, int(i) % w.heads) for i in sorted(idx)], T)
