"""GPU ↔ oracle parity through the C ABI (needs an MI355X)."""
import numpy as np
import pytest
import torch

from workload import get, scaled, synth

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():  # the whole module needs the GPU
    pytest.skip("no GPU", allow_module_level=True)

from gpu_harness import check_payloads, log, run_gpu, unit_payload  # noqa: E402

DEV = torch.device("cuda", 0)


def _numpy_inputs(w, layer=0):
    Q, K, V = synth.batch_qkv(w, layer)
    return Q, K, V, tuple(synth.to_torch(w, x, DEV) for x in (Q, K, V))


def _check_all(w, Q, K, V, g, units=None, heavy=None, recent=None):
    heavy = w.heavy_budget if heavy is None else heavy
    recent = w.recent_budget if recent is None else recent
    units = units or [(b, h) for b in range(w.batch) for h in range(w.heads)]
    payloads = [unit_payload(g, b, h, Q[b, h], K[b, h], V[b, h], w.prompt_len, heavy, recent) for b, h in units]
    results, bad = check_payloads(payloads)
    assert not bad, bad[:3]
    assert len(results) == len(units)
    for r in results:  # every comparison actually ran
        assert "score_rel" in r and (w.decode_steps == 0 or "out_err" in r), r
        assert w.prompt_len == 0 or "colsum_rel" in r, r
    return results


def test_tiny_fp32_full():
    w = get("tiny-fp32")
    log(f"case {w.name}: B={w.batch} H={w.heads} d={w.head_dim} L={w.prompt_len} T={w.decode_steps} k={w.k}")
    Q, K, V, (q, k, v) = _numpy_inputs(w)
    g = run_gpu(q, k, v, w.prompt_len, w.heavy_budget, w.recent_budget, w.dtype)
    _check_all(w, Q, K, V, g)
    assert g["info"] == (w.k, w.n_positions, w.prompt_len)


def test_tiny_fp32_from_empty_cache():
    # no prompt: the cache fills for k steps, then evicts every step
    w = scaled(get("tiny-fp32"), prompt_len=0, decode_steps=320)
    Q, K, V, (q, k, v) = _numpy_inputs(w)
    g = run_gpu(q, k, v, 0, w.heavy_budget, w.recent_budget, w.dtype)
    assert (g["evicted"][: w.k] == -1).all() and (g["evicted"][w.k:] >= 0).all()
    _check_all(w, Q, K, V, g)


@pytest.mark.parametrize("d,L,T,heavy,recent,B,H", [
    (128, 77, 40, 6, 5, 2, 3),        # ragged prompt, several MFMA tiles
    (128, 200, 33, 20, 0, 1, 4),      # no recent window: the new token can be evicted
    (64, 150, 60, 0, 9, 2, 2),        # no heavy hitters: sliding window
    (64, 31, 50, 41, 41, 1, 3),       # budget covers everything: full attention
    (128, 300, 20, 1, 0, 1, 2),       # k = 1
    (128, 1, 30, 3, 2, 2, 2),         # one-token prompt
    (64, 513, 40, 37, 64, 1, 2),      # prompt crossing 4 row blocks + ragged tail
])
def test_bf16_shapes(d, L, T, heavy, recent, B, H):
    w = scaled(get("opt6.7b-layer-b16"), batch=B, heads=H, head_dim=d, prompt_len=L, decode_steps=T,
               heavy_budget=heavy, recent_budget=recent, n_anchors=max(1, (L + T) // 50))
    log(f"case bf16 d={d} L={L} T={T} K_h={heavy} K_r={recent} B={B} H={H}")
    Q, K, V, (q, k, v) = _numpy_inputs(w)
    g = run_gpu(q, k, v, L, heavy, recent, "bf16")
    _check_all(w, Q, K, V, g)


def test_split_path_matches_oracle():
    # few units and a large budget: each unit's slots are spread over several blocks
    w = scaled(get("opt6.7b-layer-b16"), batch=1, heads=4, prompt_len=700, decode_steps=80,
               heavy_budget=150, recent_budget=150, n_anchors=8)
    log(f"case split path: units={w.units_per_layer} k={w.k}")
    Q, K, V, (q, k, v) = _numpy_inputs(w)
    g = run_gpu(q, k, v, w.prompt_len, w.heavy_budget, w.recent_budget, "bf16")
    _check_all(w, Q, K, V, g)


def test_identical_keys_closed_form_on_gpu():
    # all keys equal: uniform weights; heavy hitters stay {0..K_h-1}; every step evicts i - K_r
    B, H, d, L, T, kh, kr = 2, 2, 128, 100, 40, 10, 6
    w = scaled(get("opt6.7b-layer-b16"), batch=B, heads=H, prompt_len=L, decode_steps=T,
               heavy_budget=kh, recent_budget=kr)
    Q, K, V = synth.batch_qkv(w, 0)
    K[:] = K[:, :, :1].copy()
    q, k, v = (synth.to_torch(w, x, DEV) for x in (Q, K, V))
    g = run_gpu(q, k, v, L, kh, kr, "bf16")
    for t in range(T):
        i = L + t
        assert (g["evicted"][t] == i - kr).all(), t
        G = list(range(kh)) + list(range(i - kr, i + 1))
        np.testing.assert_allclose(g["out"][t], V[:, :, G].astype(np.float64).mean(axis=2), atol=2e-3)
    pos = np.sort(g["final"]["pos"], axis=-1)
    assert (pos == np.array(list(range(kh)) + list(range(L + T - kr, L + T)))).all()


def test_deterministic_bitwise():
    w = scaled(get("opt6.7b-layer-b16"), batch=2, heads=4, prompt_len=300, decode_steps=60,
               heavy_budget=30, recent_budget=30)
    _, _, _, (q, k, v) = _numpy_inputs(w)
    a = run_gpu(q, k, v, w.prompt_len, 30, 30, "bf16")
    b = run_gpu(q, k, v, w.prompt_len, 30, 30, "bf16")
    assert np.array_equal(a["out"].view(np.uint32), b["out"].view(np.uint32))
    assert np.array_equal(a["evicted"], b["evicted"])
    assert np.array_equal(a["final"]["score"].view(np.uint32), b["final"]["score"].view(np.uint32))
    for s in range(len(a["stats"])):
        assert np.array_equal(a["stats"][s].view(np.uint32), b["stats"][s].view(np.uint32))


def test_opt67b_layer_b16_full():
    w = get("opt6.7b-layer-b16")
    log(f"case {w.name}: every unit, {w.prompt_len}+{w.decode_steps}, k={w.k}")
    Q, K, V, (q, k, v) = _numpy_inputs(w)
    g = run_gpu(q, k, v, w.prompt_len, w.heavy_budget, w.recent_budget, w.dtype)
    res = _check_all(w, Q, K, V, g)
    log(f"{w.name}: near-ties adopted {sum(r.get('ties', 0) for r in res)}")


def test_custom_scale_matches_oracle():
    # a caller-chosen logit scale instead of 1/sqrt(d), both dtypes
    for wl, d, scale in (("tiny-fp32", 64, 0.05), ("opt6.7b-layer-b16", 128, 0.2)):
        w = scaled(get(wl), batch=2, heads=2, head_dim=d, prompt_len=150, decode_steps=60, heavy_budget=20,
                   recent_budget=10, n_anchors=3)
        Q, K, V, (q, k, v) = _numpy_inputs(w)
        log(f"case custom scale {scale} {w.dtype} d={d}")
        g = run_gpu(q, k, v, w.prompt_len, 20, 10, w.dtype, scale=scale)
        payloads = []
        for b in range(w.batch):
            for h in range(w.heads):
                pl = unit_payload(g, b, h, Q[b, h], K[b, h], V[b, h], w.prompt_len, 20, 10)
                pl["scale"] = scale
                payloads.append(pl)
        results, bad = check_payloads(payloads)
        assert not bad, bad[:3]


@pytest.mark.parametrize("d,L,T,heavy,recent,B,H", [
    (128, 300, 100, 30, 12, 2, 2),   # fp32 caches beyond the tiny workload
    (64, 97, 140, 0, 16, 1, 3),      # fp32 sliding window, ragged prompt
    (128, 700, 40, 150, 150, 1, 2),  # fp32 split path
])
def test_fp32_shapes(d, L, T, heavy, recent, B, H):
    w = scaled(get("tiny-fp32"), batch=B, heads=H, head_dim=d, prompt_len=L, decode_steps=T,
               heavy_budget=heavy, recent_budget=recent, n_anchors=max(1, (L + T) // 50))
    log(f"case fp32 d={d} L={L} T={T} K_h={heavy} K_r={recent} B={B} H={H}")
    Q, K, V, (q, k, v) = _numpy_inputs(w)
    g = run_gpu(q, k, v, L, heavy, recent, "f32")
    _check_all(w, Q, K, V, g)


def test_interleaved_caches_are_independent():
    # three caches with different shapes and paths (single-block bf16, split-path
    # bf16 with a pattern, fp32) driven step by step in turn on one stream and on
    # a second stream: each ends bit-identical to a run of that cache alone, so no
    # state is shared between caches and nothing depends on the call order
    from kv_cache_eviction_prefill_amd import H2OCache

    specs = [
        (scaled(get("opt6.7b-layer-b16"), batch=2, heads=4, prompt_len=300, decode_steps=40, heavy_budget=30,
                recent_budget=30), None),
        (scaled(get("opt6.7b-layer-b16"), batch=1, heads=2, prompt_len=700, decode_steps=40, heavy_budget=150,
                recent_budget=150), ("strided", 8, 1)),
        (scaled(get("tiny-fp32"), batch=2, heads=3, prompt_len=100, decode_steps=40, heavy_budget=12,
                recent_budget=8), None),
    ]
    inputs = []
    for w, pat in specs:
        _, _, _, (q, k, v) = _numpy_inputs(w)
        inputs.append((w, pat, q, k, v))
    alone = [run_gpu(q, k, v, w.prompt_len, w.heavy_budget, w.recent_budget, w.dtype, pattern=pat)
             for w, pat, q, k, v in inputs]

    side = torch.cuda.Stream()
    caches, outs, evs = [], [], []
    for n, (w, pat, q, k, v) in enumerate(inputs):
        c = H2OCache(w.batch, w.heads, w.head_dim, w.heavy_budget, w.recent_budget, dtype=w.dtype,
                     max_prompt=w.prompt_len)
        if pat is not None:
            c.set_pattern(*pat)
        L = w.prompt_len
        c.prefill(*(x[:, :, :L].contiguous() for x in (q, k, v)))
        caches.append(c)
        outs.append([])
        evs.append([])
    T = specs[0][0].decode_steps
    for t in range(T):
        for n, (w, pat, q, k, v) in enumerate(inputs):
            L = w.prompt_len
            st = side if (t + n) % 2 else torch.cuda.current_stream()
            qd, kd, vd = (x[:, :, L + t].contiguous() for x in (q, k, v))
            ev = torch.empty((w.batch, w.heads), dtype=torch.int32, device=q.device)
            # the side stream waits for the inputs made on the current stream
            st.wait_stream(torch.cuda.current_stream())
            with torch.cuda.stream(st):
                o, _ = caches[n].decode_step(qd, kd, vd, evicted=ev, stream=st)
            torch.cuda.current_stream().wait_stream(st)
            outs[n].append(o)
            evs[n].append(ev)
    torch.cuda.synchronize()
    for n, (w, pat, q, k, v) in enumerate(inputs):
        ref = alone[n]
        out = torch.stack(outs[n]).cpu().numpy()
        ev = torch.stack(evs[n]).cpu().numpy()
        fin = caches[n].read()
        caches[n].close()
        assert np.array_equal(out.view(np.uint32), ref["out"].view(np.uint32)), n
        assert np.array_equal(ev, ref["evicted"]), n
        assert np.array_equal(fin["pos"], ref["final"]["pos"]), n
        assert np.array_equal(fin["score"].view(np.uint32), ref["final"]["score"].view(np.uint32)), n
