"""Benchmark of the H2O hot path on one MI355X.

One *step* is the whole hot path over one batch of synthetic input: prefill of
every layer's prompt (row statistics, column sums, select + fill), then every
decode step of every layer (attention over the budgeted cache, score
accumulation, eviction and in-place overwrite), in model order (all layers of
token t before token t + 1).

Default workload: an OPT-6.7B-shaped 32-layer stack of independent attention
layers (32 heads, head_dim 128, bf16 K/V, fp32 arithmetic), batch 64, prompt
2048, 1024 generated tokens, 20% budget (205 heavy hitters + 205 recent).
Inputs are generated on the GPU before timing and stay resident in HBM.

Prints ONE JSON line.  ``value`` is generated tokens per second over the whole
step (prefill included); the line also carries decode-only and prefill rates,
the dominant kernel's roofline and the CPU oracle's rate on a bounded sample.
"""
from __future__ import annotations

import argparse
import ctypes
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "H2O decode tokens/s + achieved HBM GB/s (% peak) at OPT-6.7B shape, 20% budget"
HBM_PEAK_GBS = 8000.0
BF16_MFMA_PEAK_TFLOPS = 2500.0
MALL_BYTES = 256 * 2 ** 20


def decode_bytes_per_unit(c: int, d: int, s: int, fixed: bool = False) -> int:
    """Algorithmic HBM bytes of one decode step of one unit with c cached slots:
    K and V slot reads (2cds), score read+write (8c), position read (4c), the new
    token's q/k/v reads (3ds), its K/V slot write (2ds), fp32 output (4d).  With
    fixed scores (the global comparator) scores are only read (4c) and the new
    token's score is read (4)."""
    if fixed:
        return c * (2 * d * s + 8) + d * (5 * s + 4) + 4
    return c * (2 * d * s + 12) + d * (5 * s + 4)


def prefill_flops_per_unit(L: int, d: int, with_out: bool = False) -> int:
    """MFMA flops of the two causal QK^T passes over the L(L+1)/2 pairs; with the
    prompt's attention output, the first pass adds a PV product over the pairs."""
    return L * (L + 1) * d * (3 if with_out else 2)


def prefill_bytes_per_unit(L: int, k: int, d: int, s: int, with_out: bool = False) -> int:
    """Q and K read once (2Lds); kept V rows gathered, K/V slots written (3 min(L,k) ds); meta.
    With the prompt's attention output: V read once (Lds) and the fp32 output written (4Ld)."""
    kept = min(L, k)
    extra = L * d * s + 4 * L * d if with_out else 0
    return 2 * L * d * s + 3 * kept * d * s + 12 * kept + extra


TRAFFIC_PROFILE = os.path.join(ROOT, "profiles", "hbm_traffic-opt6.7b-32L-b64.md")


def measured_traffic(workload: str):
    """Decode HBM bytes per launch from the committed rocprofv3 counter summary,
    or None when the workload differs or the kernel sources changed since."""
    import hashlib

    if workload != "opt6.7b-32L-b64" or not os.path.exists(TRAFFIC_PROFILE):
        return None
    fields = {}
    for line in open(TRAFFIC_PROFILE):
        if ":" in line and line.split(":", 1)[0] in ("decode_traffic_bytes_per_launch", "decode_source_sha256",
                                                      "decode_source_files"):
            k, v = line.split(":", 1)
            fields[k] = v.strip()
    if len(fields) != 3:
        return None
    h = hashlib.sha256()
    for f in fields["decode_source_files"].split():
        h.update(open(os.path.join(ROOT, f), "rb").read())
    return float(fields["decode_traffic_bytes_per_launch"]) if h.hexdigest() == fields["decode_source_sha256"] else None


def parse():
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=2)
    ap.add_argument("--warmup", type=int, default=1)
    ap.add_argument("--workload", default="opt6.7b-32L-b64")
    ap.add_argument("--layers", type=int, default=None, help="override the layer count (profiling runs)")
    ap.add_argument("--decode-steps", type=int, default=None, help="override decode steps (profiling runs)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--variant", choices=("h2o", "global"), default="h2o",
                    help="h2o: the method; global: the global-score comparator (column scores of all "
                         "prompt + generated tokens, then the same keep/evict rule with fixed scores)")
    ap.add_argument("--rope", type=float, default=0.0,
                    help="> 0: rotary embedding at positions inside the cache (position rolling) with this base")
    ap.add_argument("--pattern", default="none",
                    help="sparse pattern kept before heavy hitters: none, strided:PERIOD or fixed:PERIOD:WIDTH")
    ap.add_argument("--prefill-out", action="store_true",
                    help="prefill also writes the prompt's attention output (fp32 [B, H, L, d])")
    ap.add_argument("--no-parity", action="store_true",
                    help="skip the untimed re-run that records the sampled units' results for the oracle")
    ap.add_argument("--cpu-max-steps", type=int, default=20000,
                    help="the CPU leg (and its parity re-run) covers at most this many decode steps per unit, "
                         "extrapolated linearly to the whole decode (the 4 M-token stream)")
    ap.add_argument("--cpu-units", type=int, default=96,
                    help="units in the CPU-oracle sample (about 15 s of CPU work at this shape)")
    ap.add_argument("--per-step", action="store_true",
                    help="single-layer workloads: decode through one h2o_decode_step call per step (the call of "
                         "ordinary generation) instead of one h2o_decode_steps call for all steps")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="accepted for older profiling commands: the 1 GiB copy and read that calibrate the "
                         "HBM byte counters and give the measured bandwidth ceilings now always run")
    return ap.parse_args()


def _warm(_):
    import oracle  # noqa: F401 - import before timing
    return 0


def _cpu_unit(args):
    """Worker: the oracle on one unit (prefill + every decode step), timed; then,
    when the GPU's results for the unit are given, their comparison (the oracle
    adopts the GPU's decision only at near-ties, as in the parity tests)."""
    import time as _t

    import numpy as _np

    from oracle import ParityMismatch, Pattern, Rope, run_unit, run_unit_global

    Q, K, V, L, kh, kr, variant, pattern, rope, gpu = args
    rope = Rope(*rope) if rope else None
    replay = {} if gpu is None else {"replay_kept": gpu["kept"], "replay_evicted": gpu["evicted"]}
    t0 = _t.perf_counter()
    try:
        if variant == "global":
            res = run_unit_global(Q, K, V, L, kh, kr, rope=rope, **replay)
        else:
            res = run_unit(Q, K, V, L, kh, kr, pattern=Pattern(*pattern), rope=rope, **replay)
    except ParityMismatch as e:
        return _t.perf_counter() - t0, {"ok": False, "msg": f"decision mismatch: {e}"}
    dt = _t.perf_counter() - t0
    if gpu is None:
        return dt, None
    out_err = float(_np.max(_np.abs(gpu["out"] - res["out"]))) if len(res["out"]) else 0.0
    pos, score, _, _ = res["cache"].snapshot()
    gp, gs = gpu["pos"], gpu["score"]
    valid = gp >= 0
    order = _np.argsort(gp[valid])
    same_pos = _np.array_equal(gp[valid][order], pos)
    score_rel = float(_np.max(_np.abs(gs[valid][order] - score) / score)) if same_pos and len(pos) else 0.0
    ok = same_pos and out_err <= 2e-3 and score_rel <= 1e-4
    return dt, {"ok": ok, "out_err": out_err, "score_rel": score_rel, "same_positions": same_pos,
                "ties": int(res["decode_ties_adopted"]) + int(res["prefill_tie_adopted"])}


def host_info(procs):
    """What the CPU baseline ran on: CPU model, core counts, library versions."""
    import platform

    import numpy as np

    model = platform.processor() or "unknown"
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                model = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    blas = "unknown"
    try:
        cfg = np.show_config(mode="dicts")
        b = cfg.get("Build Dependencies", {}).get("blas", {})
        blas = f"{b.get('name', '?')} {b.get('version', '')}".strip()
    except Exception:  # noqa: BLE001 - older numpy: no dict form
        pass
    import torch

    return {"cpu_model": model, "cores_visible": len(os.sched_getaffinity(0)), "cores_used": procs,
            "core_cap": "at most 16 worker processes: the GPU host's CPU share per GPU",
            "python": platform.python_version(), "numpy": np.__version__, "blas": blas,
            "torch": torch.__version__, "hip": getattr(torch.version, "hip", None)}


def cpu_baseline(w, samples, procs, steps_run):
    import multiprocessing as mp

    ctx = mp.get_context("spawn")
    pool = ctx.Pool(procs)
    try:
        pool.map(_warm, range(procs), chunksize=1)  # start every worker before timing
        t0 = time.perf_counter()
        results = pool.map(_cpu_unit, samples, chunksize=1)
        wall = time.perf_counter() - t0
    finally:
        # close + join lets the workers exit on their own (terminate() would
        # signal them, which profilers that trap signals report as aborts)
        pool.close()
        pool.join()
    per_unit = [r[0] for r in results]
    units_total = w.layers * w.batch * w.heads
    # units are independent and equally sized: whole-job time = mean unit time x units / cores
    # (x the decode steps not run, for a decode longer than the sample covers: the
    # cost per step is flat once the cache is full)
    stretch = w.decode_steps / steps_run
    job_seconds = (sum(per_unit) / len(per_unit)) * stretch * units_total / procs
    part = (f"the first {steps_run} of {w.decode_steps} decode steps, extrapolated linearly"
            if steps_run < w.decode_steps else f"{w.decode_steps} decode steps")
    base = {"value": w.batch * w.decode_steps / job_seconds, "unit": "tokens/s", "cores": procs,
            "kind": "oracle",
            "sample": f"{len(samples)} of {units_total} (layer, batch, head) units, each a full prefill of "
                      f"{w.prompt_len} tokens plus {part} (float64 NumPy, one unit per "
                      f"process, {procs} processes); mean {sum(per_unit) / len(per_unit):.3f} s per unit, "
                      f"whole job extrapolated to {job_seconds:.0f} s; sample wall {wall:.2f} s",
            "host": host_info(procs)}
    checks = [r[1] for r in results if r[1] is not None]
    parity = None
    if checks:
        bad = [c for c in checks if not c["ok"]]
        parity = {"units": len(checks), "ok": not bad,
                  "max_out_err": max((c.get("out_err", 0.0) for c in checks), default=0.0),
                  "max_score_rel": max((c.get("score_rel", 0.0) for c in checks), default=0.0),
                  "near_ties_adopted": sum(c.get("ties", 0) for c in checks),
                  "failures": [c.get("msg", c) for c in bad[:3]],
                  "what": "the sampled units' decode outputs at every step (2e-3 abs), final positions "
                          "(exact) and final scores (1e-4 rel) against the oracle, from an untimed "
                          "run of the same launch sequence after the timed steps"}
    return base, parity


def ceilings(torch, dev, lib, sp, launch_bytes):
    """Measured HBM ceilings on this GPU, best of 5 timed with events: the
    library's streaming-read probe over 4 GiB (reads only), the same probe over
    one decode launch's byte count (each run on a window of the 4 GiB buffer
    that the run before did not touch, so nothing is served from the 256 MB
    Infinity Cache: the ramp and tail of a launch of that size included) and a
    1 GiB device-to-device copy (read + write)."""
    src = torch.empty(1 << 28, dtype=torch.float32, device=dev).fill_(1.0)
    dst = torch.empty_like(src)
    big = torch.ones(1 << 30, dtype=torch.float32, device=dev)
    sink = torch.zeros(4, dtype=torch.int32, device=dev)

    def probe(off=0, nbytes=big.numel() * 4):
        st = lib.h2o_probe_read(big.data_ptr() + off, nbytes, sink.data_ptr(), sp)
        if st:
            raise RuntimeError(f"h2o_probe_read failed with status {st}")

    # launch-sized windows: 256-byte multiples, cycled through the 4 GiB buffer
    nb = min(big.numel() * 4, max(256, int(launch_bytes) // 256 * 256))
    nwin = (big.numel() * 4) // nb
    turn = [0]

    def probe_window():
        probe((turn[0] % nwin) * nb, nb)
        turn[0] += 1

    out = {}
    for name, fn, nbytes in (("read", probe, big.numel() * 4),
                             ("read_launch_size", probe_window, nb),
                             ("copy", lambda: dst.copy_(src), 2 * src.numel() * 4)):
        fn()
        best = None
        for _ in range(5):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            fn()
            e1.record()
            e1.synchronize()
            t = e0.elapsed_time(e1) / 1e3
            best = t if best is None else min(best, t)
        out[f"{name}_GBps"] = nbytes / best / 1e9
    torch.cuda.synchronize()
    del src, dst, big, sink
    out["launch_size_bytes"] = nb
    out["note"] = ("read: h2o_probe_read over 4 GiB (a plain stream of 16-byte non-temporal loads); "
                   "read_launch_size: the same probe over one decode launch's algorithmic bytes, a fresh window "
                   "of the 4 GiB buffer each run; "
                   "copy: torch's 1 GiB device copy (read + write bytes), which also calibrates the rocprofv3 "
                   "byte counters")
    return out


def compute_ceilings(torch, dev, lib, sp):
    """Measured rates of the prefill scoring passes' arithmetic on this GPU, best
    of 3 timed with events: h2o_probe_mix runs, from registers alone, 16 MFMAs
    32x32x16 bf16 per wave and iteration (mode 0), the same with 32 fma + exp2 +
    add per lane beside them (mode 1: the passes' mix, the vector work
    independent of the matrix results), and the vector work alone (mode 2),
    at 4 waves per SIMD."""
    cus = torch.cuda.get_device_properties(dev).multi_processor_count
    iters = 4000
    flops = cus * 16 * iters * 16 * 2.0 * 32 * 32 * 16  # 16 waves per CU
    sink = torch.zeros(4, dtype=torch.int32, device=dev)

    def run(mode, n):
        st = lib.h2o_probe_mix(mode, n, sink.data_ptr(), sp)
        if st:
            raise RuntimeError(f"h2o_probe_mix failed with status {st}")

    out = {}
    for mode, name in ((0, "mfma_only_TFs"), (1, "mix_TFs"), (2, "vector_only_TFs")):
        run(mode, 64)
        best = None
        for _ in range(3):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            run(mode, iters)
            e1.record()
            e1.synchronize()
            t = e0.elapsed_time(e1) / 1e3
            best = t if best is None else min(best, t)
        # mode 2 executes no MFMA: its figure is the MFMA rate the vector work alone would allow
        out[name] = flops / best / 1e12
    out["note"] = ("h2o_probe_mix: 16 MFMAs 32x32x16 bf16 (one 64 x 32 logit tile at d = 128) and, per lane, "
                   "32 x (fma, exp2, add) per wave-iteration, from registers, 4 waves per SIMD; TFLOP/s of the "
                   "MFMA work (vector_only: the MFMA rate the vector work alone would allow)")
    return out


def main():
    a = parse()
    if a.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: units are independent and the path has no cross-GPU step, "
              "so only --gpus 1 is supported.", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    from kv_cache_eviction_prefill_amd import H2OCache, h2o
    from workload import get, scaled, synth

    w = get(a.workload)
    if a.layers is not None or a.decode_steps is not None:
        w = scaled(w, layers=a.layers or w.layers, decode_steps=a.decode_steps or w.decode_steps)
    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
    B, H, d, L, T, NL = w.batch, w.heads, w.head_dim, w.prompt_len, w.decode_steps, w.layers
    s = w.elem_bytes
    lib = h2o.load()
    stream = torch.cuda.current_stream(dev)
    sp = stream.cuda_stream

    glob = a.variant == "global"
    if glob and a.prefill_out:
        print("--prefill-out applies to the h2o variant only", file=sys.stderr)
        sys.exit(2)
    N = L + T

    # ---------------------------------------------------------------- inputs (untimed)
    t_gen = time.time()
    pre, dec, seq, gsc = [], [], [], []
    tdt = torch.bfloat16 if w.dtype == "bf16" else torch.float32
    gen_chunk = 1 << 18  # decode positions generated per call (the 4 M-token stream in 16 pieces)
    for layer in range(NL):
        if glob:  # the comparator reads the whole sequence: column scores over q, k; prompt rows of k, v
            q, k, v = synth.torch_qkv(w, layer, 0, N, dev)
            seq.append((q, k, v))
            gsc.append(torch.empty((B, H, N), dtype=torch.float32, device=dev))
            pre.append(None)
            dec.append(tuple(x[:, :, L:].permute(2, 0, 1, 3).contiguous() for x in (q, k, v)))
            del q, k, v
            continue
        pre.append(synth.torch_qkv(w, layer, 0, L, dev))
        dq = tuple(torch.empty((T, B, H, d), dtype=tdt, device=dev) for _ in range(3))
        for c0 in range(0, T, gen_chunk):
            c1 = min(T, c0 + gen_chunk)
            for x, y in zip(dq, synth.torch_qkv(w, layer, L + c0, L + c1, dev)):
                x[c0:c1] = y.permute(2, 0, 1, 3)
            del y
        dec.append(dq)
    caches = [H2OCache(B, H, d, w.heavy_budget, w.recent_budget, dtype=w.dtype, max_prompt=N if glob else L,
                       rope_base=a.rope) for _ in range(NL)]
    pat = a.pattern.split(":")
    pattern = (pat[0], int(pat[1]) if len(pat) > 1 else 1, int(pat[2]) if len(pat) > 2 else 1)
    for cch in caches:
        cch.set_pattern(*pattern)
    out = torch.empty((NL, B, H, d), dtype=torch.float32, device=dev)
    # the prompt attention output, when asked for: one buffer shared by the layers
    pout = torch.empty((B, H, L, d), dtype=torch.float32, device=dev) if a.prefill_out else None
    pout_ptr = pout.data_ptr() if pout is not None else None
    ev = torch.empty((NL, B, H), dtype=torch.int32, device=dev)
    torch.cuda.synchronize()
    gen_s = time.time() - t_gen

    # raw pointers: the timed loop only marshals integers into the C entry points
    handles = [c.handle for c in caches]
    pre_ptr = [tuple(x.data_ptr() for x in p) if p is not None else None for p in pre]
    seq_ptr = [tuple(x.data_ptr() for x in p) for p in seq]
    gsc_ptr = [g.data_ptr() for g in gsc]
    tok = B * H * d * s  # bytes of one step's q, k or v; decode inputs are [T, B, H, d]
    dec_base = [tuple(x.data_ptr() for x in dq) for dq in dec]
    out_ptr = [out[l].data_ptr() for l in range(NL)]
    ev_ptr = [ev[l].data_ptr() for l in range(NL)]
    prefill_c, decode_c, steps_c = lib.h2o_prefill, lib.h2o_decode_step, lib.h2o_decode_steps
    # one layer: the whole decode is one h2o_decode_steps call (each step's evicted
    # positions kept in a [T, B, H] log, the last step's output in `out`), unless
    # asked for one h2o_decode_step call per step
    use_steps = NL == 1 and not glob and not a.per_step
    ev_log = torch.empty((T, B, H), dtype=torch.int32, device=dev) if use_steps else None
    colsc_c, prefill_sc_c, decode_sc_c = lib.h2o_column_scores, lib.h2o_prefill_scored, lib.h2o_decode_step_scored

    def _ok(st, where):
        if st:
            raise h2o.H2OError(st, where, h2o.h2o_last_error())

    def one_step(evs=None):
        if evs is not None:
            evs[0].record(stream)
        for l in range(NL):
            if glob:
                qf, kf, vf = seq_ptr[l]
                _ok(colsc_c(handles[l], qf, kf, N, gsc_ptr[l], sp), "h2o_column_scores")
                _ok(prefill_sc_c(handles[l], kf, vf, L, N, gsc_ptr[l], sp), "h2o_prefill_scored")
            else:
                _ok(prefill_c(handles[l], *pre_ptr[l], L, pout_ptr, sp), "h2o_prefill")
        if evs is not None:
            evs[1].record(stream)
        if use_steps:
            _ok(steps_c(handles[0], *dec_base[0], T, out_ptr[0], 0, ev_log.data_ptr(), sp), "h2o_decode_steps")
            if evs is not None:
                evs[2].record(stream)
            return
        for t in range(T):
            for l in range(NL):
                qp, kp, vp = (x + t * tok for x in dec_base[l])
                if glob:
                    _ok(decode_sc_c(handles[l], qp, kp, vp, gsc_ptr[l] + 4 * (L + t), N, out_ptr[l], ev_ptr[l], sp),
                        "h2o_decode_step_scored")
                else:
                    _ok(decode_c(handles[l], qp, kp, vp, out_ptr[l], ev_ptr[l], sp), "h2o_decode_step")
        if evs is not None:
            evs[2].record(stream)

    # slots read by decode step t: the cached count before it, min(k, L + t)
    dec_bytes_launch = B * H * sum(decode_bytes_per_unit(min(w.k, L + t), d, s, glob) for t in range(T)) / T
    # untimed: bandwidth references and the counters' calibration copy
    ceil = ceilings(torch, dev, lib, sp, dec_bytes_launch)
    cceil = compute_ceilings(torch, dev, lib, sp)  # untimed: the scoring passes' arithmetic alone

    for _ in range(a.warmup):
        one_step()
    torch.cuda.synchronize()

    events = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(a.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(a.steps):
        one_step(events[i])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    t_pre = sum(e[0].elapsed_time(e[1]) for e in events) / 1e3
    t_dec = sum(e[1].elapsed_time(e[2]) for e in events) / 1e3
    t_all = sum(e[0].elapsed_time(e[2]) for e in events) / 1e3

    # sanity: the caches hold min(k, L + T) entries and advanced by T
    cnt, nxt, pl = caches[0].info()
    assert (cnt, nxt, pl) == (min(L + T, w.k), L + T, L), (cnt, nxt, pl)
    # every eviction written is a position or -1 (a run through h2o_decode_steps writes ev_log, not ev)
    assert bool((ev_log >= -1).all()) if use_steps else bool((ev >= -1).all())

    K = a.steps
    tokens = B * T * K
    launches = NL * T * K
    avg_dec_s = t_dec / launches
    achieved = dec_bytes_launch / avg_dec_s / 1e9
    kv_cache_bytes = B * H * w.k * (2 * d * s + 12)
    if glob:  # the two score passes run over all N tokens; the select reads the prompt's scores
        pf_flops = NL * B * H * prefill_flops_per_unit(N, d) * K
        pf_bytes = NL * B * H * (prefill_bytes_per_unit(N, w.k, d, s) + 8 * N) * K
    else:
        pf_flops = NL * B * H * prefill_flops_per_unit(L, d, a.prefill_out) * K
        pf_bytes = NL * B * H * prefill_bytes_per_unit(L, w.k, d, s, a.prefill_out) * K
    res = {
        "metric": METRIC,
        "value": tokens / t_all,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": a.warmup,
        "ms_per_step": 1e3 * t_all / K,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if w.dtype == "bf16" else "f32",
        "data": "synthetic",
        "config": {"workload": w.name, "layers": NL, "batch": B, "heads": H, "head_dim": d,
                   "prompt_len": L, "decode_steps": T, "heavy_budget": w.heavy_budget,
                   "recent_budget": w.recent_budget, "storage": w.dtype, "accumulate": "fp32",
                   "prefill_out": bool(a.prefill_out), "variant": a.variant, "pattern": a.pattern,
                   "rope_base": a.rope,
                   "decode_call": "h2o_decode_steps" if use_steps else "h2o_decode_step"},
        "roofline": {"kernel": (f"h2o_decode_steps<{w.dtype},{d}> (decode_resident, decode_fused or decode_kernel "
                                f"by cache shape; figures per decode step)" if use_steps
                                else f"h2o_decode_step<{w.dtype},{d}> (decode_kernel, with decode_finish on the split "
                                f"path; figures per decode step)" if a.per_step
                                else f"decode_kernel<{w.dtype},{d}>"),
                     "bound": "hbm", "achieved": achieved,
                     "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": achieved / HBM_PEAK_GBS, "traffic": (measured_traffic(w.name)
                                 if a.layers is None and not glob and a.pattern == "none" and not a.rope else None),
                     "traffic_unit": "HBM bytes per launch (rocprofv3 FETCH_SIZE + WRITE_SIZE, copy-calibrated)",
                     "bytes_per_launch": dec_bytes_launch, "avg_launch_us": 1e6 * avg_dec_s,
                     "launches": launches, "measured_ceilings": ceil,
                     "frac_of_measured_read": achieved / ceil["read_GBps"],
                     "frac_of_measured_read_launch_size": achieved / ceil["read_launch_size_GBps"]},
        "decode": {"tokens_per_s": tokens / t_dec, "ms_per_token_step": 1e3 * t_dec / (T * K),
                   "GBps": achieved, "hbm_frac": achieved / HBM_PEAK_GBS,
                   # a cache that fits the 256 MB Infinity Cache is read from there, not HBM:
                   # its GB/s is an effective rate
                   "mall_resident": kv_cache_bytes <= MALL_BYTES, "cache_bytes_per_layer": kv_cache_bytes},
        "prefill": {"tokens_per_s": B * L * K / t_pre, "ms": 1e3 * t_pre / K,
                    "mfma_tflops": pf_flops / t_pre / 1e12,
                    "mfma_frac": pf_flops / t_pre / 1e12 / BF16_MFMA_PEAK_TFLOPS,
                    "alg_GBps": pf_bytes / t_pre / 1e9,
                    "measured_ceilings": cceil,
                    "frac_of_measured_mix": pf_flops / t_pre / 1e12 / cceil["mix_TFs"]},
        "timing": {"wall_s": wall, "event_s": t_all, "input_gen_s": gen_s},
    }

    def verify_pass(picks):
        """Untimed re-run of one step in the same launch sequence, recording for
        the sampled units the prefill's kept positions, every step's eviction and
        output, and the final positions and scores."""
        by_layer = {}
        for i, (l, b, h) in enumerate(picks):
            by_layer.setdefault(l, []).append((i, b * H + h))
        sel = {l: (torch.tensor([i for i, _ in v], device=dev), torch.tensor([u for _, u in v], device=dev))
               for l, v in by_layer.items()}
        outs = torch.empty((Tc, len(picks), d), dtype=torch.float32, device=dev)
        vlog = torch.empty((Tc, NL, B, H), dtype=torch.int32, device=dev)
        for l in range(NL):
            if glob:
                qf, kf, vf = seq_ptr[l]
                _ok(colsc_c(handles[l], qf, kf, N, gsc_ptr[l], sp), "h2o_column_scores")
                _ok(prefill_sc_c(handles[l], kf, vf, L, N, gsc_ptr[l], sp), "h2o_prefill_scored")
            else:
                _ok(prefill_c(handles[l], *pre_ptr[l], L, pout_ptr, sp), "h2o_prefill")
        kept = {}
        pos = np.empty((B, H, w.k), np.int32)
        for l in by_layer:
            _ok(lib.h2o_cache_read(handles[l], pos.ctypes.data, None, None, None, None, sp), "h2o_cache_read")
            kept[l] = pos.copy()
        for t in range(Tc):
            for l in range(NL):
                qp, kp, vp = (x + t * tok for x in dec_base[l])
                ep = vlog[t, l].data_ptr()
                if glob:
                    _ok(decode_sc_c(handles[l], qp, kp, vp, gsc_ptr[l] + 4 * (L + t), N, out_ptr[l], ep, sp),
                        "h2o_decode_step_scored")
                else:
                    _ok(decode_c(handles[l], qp, kp, vp, out_ptr[l], ep, sp), "h2o_decode_step")
                if l in sel:
                    outs[t].index_copy_(0, sel[l][0], out[l].view(B * H, d).index_select(0, sel[l][1]))
        final = {}
        score = np.empty((B, H, w.k), np.float32)
        for l in by_layer:
            _ok(lib.h2o_cache_read(handles[l], pos.ctypes.data, score.ctypes.data, None, None, None, sp),
                "h2o_cache_read")
            final[l] = (pos.copy(), score.copy())
        outs_h, ev_h = outs.cpu().numpy(), vlog.cpu().numpy()
        res_units = []
        for i, (l, b, h) in enumerate(picks):
            kp_ = kept[l][b, h]
            res_units.append({"kept": sorted(int(x) for x in kp_[kp_ >= 0]),
                              "evicted": ev_h[:, l, b, h].astype(np.int64), "out": outs_h[:, i].astype(np.float64),
                              "pos": final[l][0][b, h], "score": final[l][1][b, h].astype(np.float64)})
        return res_units

    Tc = T if glob else min(T, a.cpu_max_steps)  # decode steps the CPU leg and its parity re-run cover
    if not a.no_cpu_baseline:
        g = np.random.default_rng(7)
        picks = [(int(g.integers(NL)), int(g.integers(B)), int(g.integers(H))) for _ in range(a.cpu_units)]
        gpu_units = verify_pass(picks) if not a.no_parity else [None] * len(picks)
        samples = []
        for n_pick, (l, b, h) in enumerate(picks):
            if glob:
                qf, kf, vf = (x[b, h].float().cpu().numpy() for x in seq[l])
            else:
                qf, kf, vf = (torch.cat([pre[l][i][b, h], dec[l][i][:Tc, b, h]]).float().cpu().numpy()
                              for i in range(3))
            samples.append((qf, kf, vf, L, w.heavy_budget, w.recent_budget, a.variant, pattern,
                            (a.rope,) if a.rope else None, gpu_units[n_pick]))
        procs = min(len(os.sched_getaffinity(0)), 16, len(samples))
        os.environ.setdefault("OMP_NUM_THREADS", "1")
        os.environ.setdefault("OPENBLAS_NUM_THREADS", "1")
        res["cpu_baseline"], res["parity"] = cpu_baseline(w, samples, procs, Tc)
    else:
        res["cpu_baseline"], res["parity"] = None, None

    for cch in caches:
        cch.close()
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
