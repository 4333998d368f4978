"""h2o_decode_steps (several decode steps whose tokens are known in advance) through
the C ABI (needs an MI355X): bit-identical to the same number of h2o_decode_step
calls, on every decode path (small budgets, the split path for few units, the
one-wave blocks, position rolling, a sparse pattern, and the launches that hold
each unit's rows in shared memory over all the steps, and the split path's one
launch per step that finishes the previous step), on listed cases and on 48
seeded random shapes spread over calls of random lengths, outputs of every step
kept or only the last, one-step calls interleaved with multi-step calls, a
second prefill after decoding, and its argument checks."""
import numpy as np
import pytest
import torch

from workload import get, scaled, synth

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)

from gpu_harness import log  # noqa: E402
from kv_cache_eviction_prefill_amd import H2OCache, h2o  # noqa: E402

DEV = torch.device("cuda", 0)


def _cache(w, q, k, v, L, rope, pattern):
    c = H2OCache(w.batch, w.heads, w.head_dim, w.heavy_budget, w.recent_budget, dtype=w.dtype, max_prompt=L,
                 rope_base=rope)
    if pattern is not None:
        c.set_pattern(*pattern)
    c.prefill(*(x[:, :, :L].contiguous() for x in (q, k, v)))
    return c


def _same(a, b, what):
    a, b = np.asarray(a), np.asarray(b)
    assert a.shape == b.shape and np.array_equal(a.view(np.uint8), b.view(np.uint8)), what


@pytest.mark.parametrize("wl,B,H,d,L,T,heavy,recent,rope,pattern", [
    ("opt6.7b-layer-b16", 2, 4, 128, 100, 150, 20, 20, 0.0, None),        # single block per unit
    ("opt6.7b-layer-b16", 1, 4, 128, 400, 200, 150, 150, 0.0, None),      # split path (few units, k = 300)
    ("opt6.7b-layer-b16", 8, 128, 128, 300, 40, 100, 100, 0.0, None),     # one-wave blocks (1024 units, k > 128)
    ("opt6.7b-layer-b16", 2, 3, 128, 120, 100, 30, 10, 10000.0, None),    # position rolling
    ("opt6.7b-layer-b16", 32, 32, 128, 330, 20, 90, 70, 10000.0, None),   # rolling on the two-wave blocks
    ("opt6.7b-layer-b16", 2, 3, 64, 120, 100, 30, 10, 0.0, ("strided", 8, 1)),  # sparse pattern
    ("tiny-fp32", 1, 2, 64, 256, 64, 26, 26, 0.0, None),                  # fp32 storage
    # rows held in shared memory over the steps (one launch for all of them)
    ("opt6.7b-layer-b16", 16, 32, 128, 512, 64, 52, 52, 0.0, None),      # the 512-token layer: 512 units, k = 104
    ("opt6.7b-layer-b16", 8, 128, 128, 300, 40, 21, 21, 0.0, None),      # 1024 units, small budget
    ("opt6.7b-layer-b16", 8, 128, 64, 300, 40, 100, 100, 0.0, None),     # 1024 units, d = 64, k = 200
    ("opt6.7b-layer-b16", 2, 4, 128, 20, 60, 20, 20, 0.0, None),         # the cache fills during the steps
    ("opt6.7b-layer-b16", 2, 4, 128, 100, 80, 40, 0, 0.0, None),         # K_r = 0: the new token may be the victim
    # split path, one launch per step (each finishing the previous step)
    ("opt6.7b-layer-b16", 1, 32, 128, 512, 3000, 1024, 1024, 0.0, None),  # the stream's shape: fills, then splits
    ("opt6.7b-layer-b16", 2, 1, 128, 60, 301, 200, 200, 0.0, None),       # from one block per unit into the split
    ("opt6.7b-layer-b16", 2, 1, 64, 700, 150, 300, 300, 0.0, None),       # d = 64: 256-thread slices
    ("opt6.7b-layer-b16", 1, 16, 128, 2400, 120, 1152, 1152, 0.0, None),  # 36 two-wave slices per unit: more
                                                                          # partials than the staged launch holds
    # slices of 64 slots staged in shared memory: one, two or four slices per block
    ("opt6.7b-layer-b16", 2, 1, 128, 600, 80, 256, 256, 0.0, ("fixed", 16, 4)),  # one per block, a pattern
    ("opt6.7b-layer-b16", 1, 32, 128, 1100, 60, 512, 512, 0.0, ("strided", 8, 1)),  # two per block, a pattern
    ("opt6.7b-layer-b16", 1, 32, 128, 1100, 60, 1024, 0, 0.0, None),     # two per block, K_r = 0
    ("opt6.7b-layer-b16", 1, 32, 128, 2100, 60, 1024, 1024, 0.0, ("strided", 8, 1)),  # four per block, a pattern
    ("opt6.7b-layer-b16", 1, 32, 128, 2100, 60, 2048, 0, 0.0, None),     # four per block, K_r = 0
    ("opt6.7b-layer-b16", 1, 64, 128, 1100, 30, 512, 512, 0.0, None),    # four per block, 64 units
    # position rolling on the split path: each launch also moves the slots' places
    ("opt6.7b-layer-b16", 2, 1, 128, 600, 150, 256, 256, 10000.0, None),  # slices of 64, staged
    ("opt6.7b-layer-b16", 1, 4, 128, 400, 200, 150, 150, 10000.0, None),  # slices of 75, from global memory
    ("opt6.7b-layer-b16", 2, 1, 128, 600, 100, 512, 0, 10000.0, None),    # K_r = 0: the new token may leave
    ("opt6.7b-layer-b16", 2, 1, 128, 60, 301, 200, 200, 10000.0, None),   # fills, then splits
    ("opt6.7b-layer-b16", 1, 32, 128, 2100, 40, 1024, 1024, 10000.0, None),  # staged, four slices per block
    ("opt6.7b-layer-b16", 1, 32, 128, 2100, 40, 1024, 1024, 10000.0, ("strided", 8, 1)),  # and a pattern
    ("opt6.7b-layer-b16", 32, 32, 128, 330, 20, 90, 70, 10000.0, ("fixed", 16, 4)),  # two-wave rolling, a pattern
    ("opt6.7b-layer-b16", 8, 32, 128, 2100, 41, 1024, 1024, 0.0, None),   # slices of 512 slots: 256-thread blocks
    ("opt6.7b-layer-b16", 4, 1, 128, 400, 101, 300, 0, 0.0, None),        # K_r = 0 on the split path
    ("opt6.7b-layer-b16", 2, 2, 128, 400, 120, 150, 150, 0.0, ("fixed", 16, 4)),  # a pattern on the split path
    ("tiny-fp32", 2, 1, 128, 400, 90, 150, 150, 0.0, None),               # fp32 on the split path
])
def test_steps_match_single_steps(wl, B, H, d, L, T, heavy, recent, rope, pattern):
    w = scaled(get(wl), batch=B, heads=H, head_dim=d, prompt_len=L, decode_steps=T, heavy_budget=heavy,
               recent_budget=recent, n_anchors=max(1, (L + T) // 50))
    log(f"case steps {w.dtype} B={B} H={H} d={d} L={L} T={T} k={heavy}+{recent} rope={rope} pattern={pattern}")
    _compare(w, L, T, rope, pattern, [T // 2])


def test_steps_random_sweep():
    # seeded random shapes over every decode path, the steps split over three calls
    g = np.random.default_rng(20240611)
    patterns = [None, None, ("strided", 8, 1), ("fixed", 16, 4)]
    for case in range(48):
        B = int(g.choice([1, 2, 4, 8]))
        H = int(g.choice([1, 2, 8, 16, 32, 64, 128]))
        d = int(g.choice([64, 128]))
        if case % 3 == 0:  # any budget
            heavy = int(g.integers(0, 1200))
            recent = int(g.integers(0 if heavy > 0 else 1, 1200))
        elif case % 3 == 1:  # a multiple of 64 slots: slices of exactly 64 once full
            kk = 64 * int(g.integers(2, 33))
            recent = int(g.integers(0, kk))
            heavy = kk - recent
        else:  # small budgets: one block per unit
            heavy = int(g.integers(0, 100))
            recent = int(g.integers(0 if heavy > 0 else 1, 100))
        L = int(g.integers(1, heavy + recent + 300))
        T = int(g.integers(2, 200))
        rope = float(g.choice([0.0, 10000.0]))
        pattern = patterns[int(g.integers(0, 4))]
        wl = "tiny-fp32" if case % 5 == 4 else "opt6.7b-layer-b16"
        w = scaled(get(wl), batch=B, heads=H, head_dim=d, prompt_len=L, decode_steps=T, heavy_budget=heavy,
                   recent_budget=recent, n_anchors=max(1, (L + T) // 50))
        cuts = sorted(int(c) for c in g.integers(1, T, size=2))
        log(f"sweep {case}: {w.dtype} B={B} H={H} d={d} L={L} T={T} k={heavy}+{recent} rope={rope} "
            f"pattern={pattern} calls at {cuts}")
        _compare(w, L, T, rope, pattern, cuts)


def _compare(w, L, T, rope, pattern, cuts):
    """h2o_decode_steps over calls split at `cuts` against one h2o_decode_step per
    step: outputs, evictions, scores, positions, K/V rows and counters bit for bit."""
    B, H, d = w.batch, w.heads, w.head_dim
    q, k, v = synth.torch_qkv(w, 0, 0, L + T, DEV)
    qd, kd, vd = (x[:, :, L:].permute(2, 0, 1, 3).contiguous() for x in (q, k, v))
    one = _cache(w, q, k, v, L, rope, pattern)
    o1 = torch.empty((T, B, H, d), dtype=torch.float32, device=DEV)
    e1 = torch.empty((T, B, H), dtype=torch.int32, device=DEV)
    for t in range(T):
        one.decode_step(qd[t], kd[t], vd[t], o1[t], e1[t])
    many = _cache(w, q, k, v, L, rope, pattern)
    o2 = torch.full((T, B, H, d), float("nan"), dtype=torch.float32, device=DEV)
    e2 = torch.full((T, B, H), -7, dtype=torch.int32, device=DEV)
    bounds = [0] + list(cuts) + [T]  # several calls: each continues from the previous one's state
    for t0, t1 in zip(bounds[:-1], bounds[1:]):
        many.decode_steps(qd[t0:t1], kd[t0:t1], vd[t0:t1], o2[t0:t1], e2[t0:t1])
    torch.cuda.synchronize()
    _same(o1.cpu().numpy(), o2.cpu().numpy(), "outputs")
    _same(e1.cpu().numpy(), e2.cpu().numpy(), "evictions")
    r1, r2 = one.read(), many.read()
    for key in ("pos", "score"):
        _same(r1[key], r2[key], key)
    occupied = r1["pos"] >= 0  # rows of empty slots were never written
    for key in ("k", "v"):
        _same(r1[key][occupied], r2[key][occupied], key)
    assert one.info() == many.info()
    # only the last output kept
    last = _cache(w, q, k, v, L, rope, pattern)
    o3 = torch.empty((B, H, d), dtype=torch.float32, device=DEV)
    last.decode_steps(qd, kd, vd, o3, keep_all=False)
    torch.cuda.synchronize()
    _same(o3.cpu().numpy(), o1[-1].cpu().numpy(), "last output")
    for c in (one, many, last):
        c.close()


@pytest.mark.parametrize("wl,B,H,d,L,T,heavy,recent,rope", [
    ("opt6.7b-layer-b16", 1, 32, 128, 2100, 90, 1024, 1024, 0.0),     # four slices per staged block
    ("opt6.7b-layer-b16", 1, 32, 128, 2100, 90, 1024, 1024, 10000.0),  # the same with rolling
    ("opt6.7b-layer-b16", 32, 32, 128, 330, 40, 90, 70, 10000.0),      # two-wave rolling blocks
])
def test_steps_and_single_steps_interleaved(wl, B, H, d, L, T, heavy, recent, rope):
    # one-step calls between multi-step calls continue the same run: each call
    # finds the state the previous one left, whichever path wrote it
    w = scaled(get(wl), batch=B, heads=H, head_dim=d, prompt_len=L, decode_steps=T, heavy_budget=heavy,
               recent_budget=recent, n_anchors=max(1, (L + T) // 50))
    log(f"case interleaved {w.dtype} B={B} H={H} L={L} T={T} k={heavy}+{recent} rope={rope}")
    q, k, v = synth.torch_qkv(w, 0, 0, L + T, DEV)
    qd, kd, vd = (x[:, :, L:].permute(2, 0, 1, 3).contiguous() for x in (q, k, v))
    one = _cache(w, q, k, v, L, rope, None)
    o1 = torch.empty((T, B, H, d), dtype=torch.float32, device=DEV)
    e1 = torch.empty((T, B, H), dtype=torch.int32, device=DEV)
    for t in range(T):
        one.decode_step(qd[t], kd[t], vd[t], o1[t], e1[t])
    mix = _cache(w, q, k, v, L, rope, None)
    o2 = torch.full((T, B, H, d), float("nan"), dtype=torch.float32, device=DEV)
    e2 = torch.full((T, B, H), -7, dtype=torch.int32, device=DEV)
    t = 0
    for n in (1, 7, 1, 1, 20, 1, 13):
        if n == 1:
            mix.decode_step(qd[t], kd[t], vd[t], o2[t], e2[t])
        else:
            mix.decode_steps(qd[t:t + n], kd[t:t + n], vd[t:t + n], o2[t:t + n], e2[t:t + n])
        t += n
    mix.decode_steps(qd[t:], kd[t:], vd[t:], o2[t:], e2[t:])
    torch.cuda.synchronize()
    _same(o1.cpu().numpy(), o2.cpu().numpy(), "outputs")
    _same(e1.cpu().numpy(), e2.cpu().numpy(), "evictions")
    r1, r2 = one.read(), mix.read()
    for key in ("pos", "score"):
        _same(r1[key], r2[key], key)
    occupied = r1["pos"] >= 0
    for key in ("k", "v"):
        _same(r1[key][occupied], r2[key][occupied], key)
    assert one.info() == mix.info()
    one.close()
    mix.close()


@pytest.mark.parametrize("B,H,L1,L2,heavy,recent,rope", [
    (1, 32, 2100, 300, 1024, 1024, 0.0),    # split path, then a prompt shorter than the budget
    (1, 32, 2100, 300, 1024, 1024, 10000.0),
    (2, 4, 100, 10, 20, 20, 0.0),          # one block per unit
])
def test_second_prefill_starts_over(B, H, L1, L2, heavy, recent, rope):
    # a prefill after decoding re-initialises the cache: the run that follows is
    # the run of a fresh cache given the same prompt
    T1, T2 = 60, 80
    w = scaled(get("opt6.7b-layer-b16"), batch=B, heads=H, head_dim=128, prompt_len=L1, decode_steps=T1,
               heavy_budget=heavy, recent_budget=recent, n_anchors=max(1, (L1 + T1) // 50))
    log(f"case second prefill B={B} H={H} L={L1} then {L2} k={heavy}+{recent} rope={rope}")
    q, k, v = synth.torch_qkv(w, 0, 0, L1 + T1, DEV)
    q2, k2, v2 = synth.torch_qkv(w, 1, 0, L2 + T2, DEV)
    qd, kd, vd = (x[:, :, L1:].permute(2, 0, 1, 3).contiguous() for x in (q, k, v))
    qd2, kd2, vd2 = (x[:, :, L2:].permute(2, 0, 1, 3).contiguous() for x in (q2, k2, v2))
    used = H2OCache(B, H, 128, heavy, recent, dtype="bf16", max_prompt=L1, rope_base=rope)
    used.prefill(*(x[:, :, :L1].contiguous() for x in (q, k, v)))
    junk = torch.empty((T1, B, H, 128), dtype=torch.float32, device=DEV)
    used.decode_steps(qd[:T1 - 3], kd[:T1 - 3], vd[:T1 - 3], junk[:T1 - 3])
    for t in range(T1 - 3, T1):
        used.decode_step(qd[t], kd[t], vd[t], junk[t])
    fresh = H2OCache(B, H, 128, heavy, recent, dtype="bf16", max_prompt=L1, rope_base=rope)
    outs, evs = [], []
    for c in (used, fresh):
        c.prefill(*(x[:, :, :L2].contiguous() for x in (q2, k2, v2)))
        o = torch.empty((T2, B, H, 128), dtype=torch.float32, device=DEV)
        e = torch.empty((T2, B, H), dtype=torch.int32, device=DEV)
        c.decode_steps(qd2, kd2, vd2, o, e)
        outs.append(o)
        evs.append(e)
    torch.cuda.synchronize()
    _same(outs[0].cpu().numpy(), outs[1].cpu().numpy(), "outputs")
    _same(evs[0].cpu().numpy(), evs[1].cpu().numpy(), "evictions")
    r1, r2 = used.read(), fresh.read()
    for key in ("pos", "score"):
        _same(r1[key], r2[key], key)
    occupied = r2["pos"] >= 0
    for key in ("k", "v"):
        _same(r1[key][occupied], r2[key][occupied], key)
    assert used.info() == fresh.info()
    used.close()
    fresh.close()


def test_steps_argument_checks():
    c = H2OCache(1, 2, 128, 4, 4, dtype="bf16", max_prompt=8)
    buf = torch.zeros((4, 1, 2, 128), dtype=torch.bfloat16, device=DEV)
    out = torch.zeros((4, 1, 2, 128), dtype=torch.float32, device=DEV)
    p, o = buf.data_ptr(), out.data_ptr()
    # before any prefill
    assert h2o.h2o_decode_steps(c.handle, p, p, p, 4, o, 256, None, None) == h2o.H2O_ERR_STATE
    prompt = torch.zeros((1, 2, 8, 128), dtype=torch.bfloat16, device=DEV)
    c.prefill(prompt, prompt, prompt)
    assert h2o.h2o_decode_steps(c.handle, p, p, p, -1, o, 256, None, None) == h2o.H2O_ERR_INVALID_ARG
    assert h2o.h2o_decode_steps(c.handle, p, p, p, 4, o, 3, None, None) == h2o.H2O_ERR_INVALID_ARG
    assert h2o.h2o_decode_steps(c.handle, p + 2, p, p, 4, o, 256, None, None) == h2o.H2O_ERR_INVALID_ARG
    assert h2o.h2o_decode_steps(c.handle, None, p, p, 4, o, 256, None, None) == h2o.H2O_ERR_INVALID_ARG
    assert h2o.h2o_decode_steps(c.handle, p, p, p, 0, None, 0, None, None) == h2o.H2O_OK
    assert c.info()[1] == 8  # rejected calls left the step counter alone
    assert h2o.h2o_decode_steps(c.handle, p, p, p, 4, o, 256, None, None) == h2o.H2O_OK
    torch.cuda.synchronize()
    assert c.info()[1] == 12
    c.close()
