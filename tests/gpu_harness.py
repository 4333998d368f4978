"""Drive the HIP library through its C ABI for parity tests and hand the results
to the CPU oracle, one unit per worker process."""
from __future__ import annotations

import multiprocessing as mp
import os
import sys
import time

import numpy as np
import torch

from kv_cache_eviction_prefill_amd import H2OCache

HERE = os.path.dirname(os.path.abspath(__file__))


def log(msg: str) -> None:
    print(f"[parity {time.strftime('%H:%M:%S')}] {msg}", flush=True)


def widen(t: torch.Tensor) -> np.ndarray:
    return t.detach().to("cpu", torch.float32).numpy()


def run_gpu(q, k, v, L, heavy, recent, dtype, collect_out=True, out_units=None, scale=0.0, pattern=None,
            rope_base=0.0):
    """Prefill + decode on the GPU.  ``q, k, v``: device tensors [B, H, N, d] in the
    storage dtype; ``pattern``: (kind, period, width) kept before heavy hitters,
    or None; ``rope_base`` > 0: rotary embedding at positions inside the cache.
    Returns host arrays: kept [B, H] lists, stats, evicted [T, B, H],
    out [T, B, H, d] (or [T, n, d] for ``out_units``), final cache."""
    B, H, N, d = q.shape
    T = N - L
    cache = H2OCache(B, H, d, heavy, recent, dtype=dtype, scale=scale, max_prompt=max(L, 1), rope_base=rope_base)
    if pattern is not None:
        cache.set_pattern(*pattern)
    qp, kp, vp = (x[:, :, :L].contiguous() for x in (q, k, v))
    cache.prefill(qp, kp, vp)
    after = cache.read()
    stats = cache.prefill_stats() if L > 0 else None
    del qp, kp, vp
    qd, kd, vd = (x[:, :, L:].permute(2, 0, 1, 3).contiguous() for x in (q, k, v))
    ev = torch.empty((T, B, H), dtype=torch.int32, device=q.device)
    o_step = torch.empty((B, H, d), dtype=torch.float32, device=q.device)
    sel = None
    if out_units is not None:
        sel = torch.tensor([b * H + h for b, h in out_units], device=q.device)
        outs = torch.empty((T, len(out_units), d), dtype=torch.float32, device=q.device)
    elif collect_out:
        outs = torch.empty((T, B, H, d), dtype=torch.float32, device=q.device)
    for t in range(T):
        if sel is None and collect_out:
            cache.decode_step(qd[t], kd[t], vd[t], outs[t], ev[t])
        else:
            cache.decode_step(qd[t], kd[t], vd[t], o_step, ev[t])
            if sel is not None:
                outs[t] = o_step.view(B * H, d).index_select(0, sel)
    final = cache.read()
    torch.cuda.synchronize()
    res = {"kept": after, "stats": stats, "evicted": ev.cpu().numpy(), "final": final,
           "out": outs.cpu().numpy() if (collect_out or sel is not None) else None, "info": cache.info()}
    cache.close()
    return res


def run_gpu_scored(q, k, v, L, heavy, recent, dtype, scores=None, pattern=None, rope_base=0.0):
    """Scored prefill + decode on the GPU.  ``scores``: device float32 [B, H, N]
    fixed scores, or None to compute the global column scores of the whole
    sequence first (the global comparator)."""
    import pytest

    B, H, N, d = q.shape
    T = N - L
    dev = q.device
    cache = H2OCache(B, H, d, heavy, recent, dtype=dtype, max_prompt=N, rope_base=rope_base)
    if pattern is not None:
        cache.set_pattern(*pattern)
    gs = None
    if scores is None:
        scores = cache.column_scores(q, k)
        gs = scores.cpu().numpy()
    # the prompt is read in place from the whole sequence's K/V and scores, and
    # each step's score is a strided column of the [B, H, N] scores
    cache.prefill_scored(k, v, scores, prompt_len=L)
    kept = cache.read()
    qd, kd, vd = (x[:, :, L:].permute(2, 0, 1, 3).contiguous() for x in (q, k, v))
    ev = torch.empty((T, B, H), dtype=torch.int32, device=dev)
    outs = torch.empty((T, B, H, d), dtype=torch.float32, device=dev)
    for t in range(T):
        cache.decode_step_scored(qd[t], kd[t], vd[t], scores[:, :, L + t], outs[t], ev[t])
    final = cache.read()
    with pytest.raises(Exception):
        cache.prefill_stats()  # no statistics after a scored prefill
    torch.cuda.synchronize()
    res = {"kept": kept, "stats": None, "evicted": ev.cpu().numpy(), "final": final, "out": outs.cpu().numpy(),
           "gscores": gs}
    cache.close()
    return res


def unit_payload(g, b, h, Q, K, V, L, heavy, recent, out_index=None, tag=None):
    """Pack one unit's inputs (float32 host arrays [N, d]) and GPU results."""
    kept_pos = g["kept"]["pos"][b, h]
    st = None
    if g["stats"] is not None:
        st = (g["stats"][0][b, h].astype(np.float64), g["stats"][1][b, h].astype(np.float64))
    fin = g["final"]
    if g["out"] is None:
        out = np.zeros((0, Q.shape[1]))
    elif out_index is None:
        out = g["out"][:, b, h]
    else:
        out = g["out"][:, out_index]
    return {"tag": tag or f"b{b}h{h}", "Q": Q, "K": K, "V": V, "L": L, "heavy": heavy, "recent": recent,
            "kept": sorted(int(x) for x in kept_pos[kept_pos >= 0]),
            "evicted": g["evicted"][:, b, h].astype(np.int64), "out": out.astype(np.float64),
            "stats": st, "final": (fin["pos"][b, h], fin["score"][b, h].astype(np.float64),
                                   fin["k"][b, h], fin["v"][b, h])}


def parallel_map(fn, items, procs=None):
    """``fn`` over ``items`` in spawned worker processes (at most 16: the host's
    CPU share per GPU); ``fn`` must live in a module the workers can import."""
    if HERE not in sys.path:
        sys.path.insert(0, HERE)
    procs = procs or min(16, len(os.sched_getaffinity(0)), max(1, len(items)))
    if procs <= 1 or len(items) <= 1:
        return [fn(x) for x in items]
    pool = mp.get_context("spawn").Pool(procs)
    try:
        return pool.map(fn, items, chunksize=1)
    finally:
        pool.close()
        pool.join()


def check_payloads(payloads, procs=None):
    """Run the oracle comparison for every payload (spawned workers)."""
    if HERE not in sys.path:
        sys.path.insert(0, HERE)
    import _oracle_worker

    procs = procs or min(16, len(os.sched_getaffinity(0)), max(1, len(payloads)))
    t0 = time.time()
    if procs <= 1 or len(payloads) <= 2:
        results = [_oracle_worker.check_unit(p) for p in payloads]
    else:
        ctx = mp.get_context("spawn")
        pool = ctx.Pool(procs)
        try:
            results, step = [], max(1, len(payloads) // 8)
            for r in pool.imap(_oracle_worker.check_unit, payloads, chunksize=max(1, len(payloads) // (16 * procs))):
                results.append(r)
                if len(payloads) >= 256 and len(results) % step == 0:  # progress of a long check
                    log(f"oracle: {len(results)} of {len(payloads)} units checked")
        finally:  # let the workers exit on their own (terminate() would signal them)
            pool.close()
            pool.join()
    bad = [r for r in results if not r["ok"]]
    worst = {key: max((r.get(key, 0.0) for r in results), default=0.0)
             for key in ("out_err", "score_rel", "colsum_rel", "lse_err")}
    ties = sum(r.get("ties", 0) for r in results)
    log(f"oracle checked {len(results)} units in {time.time() - t0:.1f}s on {procs} procs; "
        f"worst {worst}; near-ties adopted {ties}; failures {len(bad)}")
    return results, bad
