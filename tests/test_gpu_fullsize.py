"""GPU ↔ oracle parity at the full workload shapes, in the launch configuration
the benchmark times (needs an MI355X): every unit of the 32-layer stack's
2048-unit launch (plain, with position rolling, with a sparse pattern and
under the global-score comparator) and
of the 32-head stream; 2048 of the 7168 units of each
OPT-30B budget (1024 at 100 %); four heads of the stream's deep replay.

Inputs come from the device-side generator; the oracle reads the units'
inputs back from those tensors (generator output, not GPU-path output) and runs
each unit in full.  Properties that hold for every unit (budget, recent window,
candidate bound, no re-entry) are checked on all units.
"""
import numpy as np
import pytest
import torch

from workload import get, scaled, synth

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)

from gpu_harness import check_payloads, log, run_gpu, run_gpu_scored, unit_payload  # noqa: E402

DEV = torch.device("cuda", 0)


def _sample(w, n, seed):
    g = np.random.default_rng(seed)
    idx = g.choice(w.batch * w.heads, size=min(n, w.batch * w.heads), replace=False)
    return [(int(i) // w.heads, int(i) % w.heads) for i in sorted(idx)]


def _every(w):
    return [(b, h) for b in range(w.batch) for h in range(w.heads)]


def _host_unit(q, k, v, b, h):
    return tuple(x[b, h].to(torch.float32).cpu().numpy() for x in (q, k, v))


def _check_properties(w, g, L, T):
    """Budget, recent window, candidate bound and no re-entry, for every unit."""
    k = w.k
    kept = g["kept"]["pos"]
    ev = g["evicted"]  # [T, B, H]
    fin = g["final"]["pos"]
    n_kept = (kept >= 0).sum(-1)
    assert (n_kept == min(L, k)).all()
    assert ((fin >= 0).sum(-1) == min(L + T, k)).all()
    for t in range(T):
        i = L + t
        e = ev[t]
        if min(L, k) + t < k:
            assert (e == -1).all(), t
        else:
            assert (e >= 0).all() and (e <= i - w.recent_budget).all(), t
    # final set = kept + new tokens - evicted, and the recent window is resident
    for b in range(w.batch):
        for h in range(w.heads):
            s = set(kept[b, h][kept[b, h] >= 0].tolist()) | set(range(L, L + T))
            s -= set(ev[:, b, h][ev[:, b, h] >= 0].tolist())
            assert s == set(fin[b, h][fin[b, h] >= 0].tolist()), (b, h)
            assert set(range(max(0, L + T - w.recent_budget), L + T)) <= s


def _run_units(w, layer, units, T=None, check_props=True, rope=0.0, pattern=None):
    L = w.prompt_len
    T = w.decode_steps if T is None else T
    q, k, v = synth.torch_qkv(w, layer, 0, L + T, DEV)
    log(f"case {w.name} layer {layer}: B={w.batch} H={w.heads} L={L} T={T} k={w.k} rope={rope}; "
        f"{len(units)} units checked")
    g = run_gpu(q, k, v, L, w.heavy_budget, w.recent_budget, w.dtype, out_units=units, rope_base=rope,
                pattern=pattern)
    if check_props:
        _check_properties(w, g, L, T)
    payloads = []
    for n, (b, h) in enumerate(units):
        Q, K, V = _host_unit(q, k, v, b, h)
        pl = unit_payload(g, b, h, Q, K, V, L, w.heavy_budget, w.recent_budget, out_index=n,
                          tag=f"{w.name}/L{layer}/b{b}h{h}")
        if rope:
            pl.update(rope=(rope,))
        if pattern is not None:
            pl.update(pattern=pattern)
        payloads.append(pl)
    del q, k, v
    torch.cuda.empty_cache()
    results, bad = check_payloads(payloads)
    assert not bad, bad[:3]
    for r in results:
        assert "score_rel" in r and "out_err" in r and "colsum_rel" in r, r
    return g, results


@pytest.mark.parametrize("layer", [0, 15, 31])
def test_opt67b_32layer_b64_full_shape(layer):
    # the benchmark's launch configuration: 2048 units, prompt 2048, 1024 decode
    # steps, k = 410; every unit of the launch, on three layers of the stack
    w = get("opt6.7b-32L-b64")
    _, results = _run_units(w, layer, _every(w))
    assert len(results) == w.batch * w.heads


def test_opt67b_full_shape_with_rolling():
    # position rolling in the benchmark's launch configuration (2048 units,
    # prompt 2048, k = 410: the two-wave rolling blocks), 200 decode steps, every
    # unit
    w = get("opt6.7b-32L-b64")
    _run_units(w, 3, _every(w), T=200, rope=10000.0)


def test_opt67b_full_shape_with_pattern():
    # heavy hitters on top of a strided pattern (period 64, the bench's
    # --pattern strided:64) in the benchmark's launch configuration, 256 decode
    # steps, every unit
    w = get("opt6.7b-32L-b64")
    _run_units(w, 5, _every(w), T=256, pattern=("strided", 64, 1))


def test_opt67b_full_shape_global_comparator():
    # the global-score comparator (bench --variant global) in the benchmark's
    # launch configuration: column scores of the whole 2304-token sequence,
    # scored prefill, 256 fixed-score decode steps; every unit
    w = get("opt6.7b-32L-b64")
    L, T = w.prompt_len, 256
    q, k, v = synth.torch_qkv(w, 9, 0, L + T, DEV)
    log(f"case {w.name} layer 9 global comparator: B={w.batch} H={w.heads} L={L} T={T} k={w.k}; every unit")
    g = run_gpu_scored(q, k, v, L, w.heavy_budget, w.recent_budget, w.dtype)
    _check_properties(w, g, L, T)
    payloads = []
    for b, h in _every(w):
        Q, K, V = _host_unit(q, k, v, b, h)
        pl = unit_payload(g, b, h, Q, K, V, L, w.heavy_budget, w.recent_budget, tag=f"{w.name}/global/b{b}h{h}")
        pl.update(mode="global", gscores=g["gscores"][b, h].astype(np.float64))
        payloads.append(pl)
    del q, k, v, g
    torch.cuda.empty_cache()
    results, bad = check_payloads(payloads)
    assert not bad, bad[:3]
    assert len(results) == w.batch * w.heads


@pytest.mark.parametrize("budget", ["4pct", "10pct", "20pct"])
def test_opt30b_b128_full_shape(budget):
    # 7,168 units, prompt 1024, 1024 decode steps, k = 42 / 104 / 206; 2048
    # sampled units each (every unit passed too, 32-37 s of oracle work per
    # budget: more than the suite's time allows for each)
    w = get(f"opt30b-b128-{budget}")
    _run_units(w, 0, _sample(w, 2048, int(budget[:-3])))


def test_opt30b_b128_100pct_is_full_attention():
    # k = N: nothing is ever evicted and every output is full causal attention;
    # 1024 of the 7168 units (a full-attention unit costs the oracle four times
    # one at 20 %), the no-eviction property on every unit
    w = get("opt30b-b128-100pct")
    g, _ = _run_units(w, 0, _sample(w, 1024, 100))
    assert (g["evicted"] == -1).all()


def test_llama7b_stream_split_path():
    # one head per unit, 32 units: the slots of each unit are split over blocks;
    # the first eviction happens at step k - L = 1536; every head, 6000 steps
    w = get("llama7b-stream-4m")
    _run_units(w, 0, _every(w), T=6000)


def test_llama7b_stream_deep_replay():
    # the stream well past its first evictions: 100,000 steps (98,464 of them
    # evicting) replayed in full by the oracle for four heads, so the compensated
    # scores and every eviction are checked far into the stream
    w = get("llama7b-stream-4m")
    _run_units(w, 0, [(0, 5), (0, 12), (0, 19), (0, 26)], T=100000)
