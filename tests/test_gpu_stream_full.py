"""The LLaMA-7B-shaped stream run end to end: a 512-token prompt, then all
4,000,000 decode steps at k = 1024 + 1024 on 32 heads (Report §4.4 Q1: H2O with
position rolling streams 4 million tokens; here without the rotation), through
h2o_decode_steps (needs an MI355X).  Checked on every head from the GPU's own
eviction log: the budget (no eviction while the cache fills, one per step
after), the candidate bound (the recent window is never evicted), no position
evicted twice, and the final cache holding exactly the positions never
evicted.  Late in the stream the oracle takes over from the GPU's own state:
at steps 1 M, 2 M, 3 M and 10,000 before the end the cache of every head
(positions, scores, K/V rows) is read, the oracle runs the next 10,000 steps from
it, and its outputs (2e-3 absolute), evictions (exact, near-ties adopted) and
the cache after the steps (positions and K/V rows exact, scores 1e-4 relative)
must match the GPU's.  The oracle replays the first 100,000
steps of four heads from the prompt in ``test_gpu_fullsize.py``; the accuracy of
the compensated scores over 4 M increments is bounded in
``test_kahan_drift.py``."""
import numpy as np
import pytest
import torch

from workload import get, synth

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)

import _oracle_worker  # noqa: E402
from gpu_harness import log, parallel_map  # noqa: E402
from kv_cache_eviction_prefill_amd import H2OCache  # noqa: E402

DEV = torch.device("cuda", 0)
CHUNK = 1 << 18   # positions generated per call
CALL = 1_000_000  # decode steps per h2o_decode_steps call
REPLAY = 10_000   # steps the oracle runs from each snapshot
HEADS = tuple(range(32))  # every head of the stream


def _window(w, snap, after, start, dec, out, ev):
    """Payloads of one snapshot window for the sampled heads (host arrays)."""
    q, k, v = (x[start:start + REPLAY, 0].to(torch.float32).cpu().numpy() for x in dec)  # [REPLAY, H, d]
    return [{"tag": f"h{h}@{start}", "heavy": w.heavy_budget, "recent": w.recent_budget,
             "next_pos": w.prompt_len + start,
             "snap": (snap["pos"][0, h], snap["score"][0, h], snap["k"][0, h], snap["v"][0, h]),
             "after": (after["pos"][0, h], after["score"][0, h].astype(np.float64), after["k"][0, h],
                       after["v"][0, h]),
             "q": q[:, h], "k": k[:, h], "v": v[:, h], "out": out[:, h].astype(np.float64), "evicted": ev[:, h]}
            for h in HEADS]


def test_llama7b_stream_four_million_steps():
    w = get("llama7b-stream-4m")
    B, H, d, L, T, k, kr = w.batch, w.heads, w.head_dim, w.prompt_len, w.decode_steps, w.k, w.recent_budget
    assert (B, L, T, k) == (1, 512, 4_000_000, 2048)
    log(f"case stream: generating {T} decode tokens for {H} heads")
    pq, pk, pv = synth.torch_qkv(w, 0, 0, L, DEV)
    dec = tuple(torch.empty((T, B, H, d), dtype=torch.bfloat16, device=DEV) for _ in range(3))
    for c0 in range(0, T, CHUNK):
        c1 = min(T, c0 + CHUNK)
        for x, y in zip(dec, synth.torch_qkv(w, 0, L + c0, L + c1, DEV)):
            x[c0:c1] = y.permute(2, 0, 1, 3)
    cache = H2OCache(B, H, d, w.heavy_budget, kr, dtype="bf16", max_prompt=L)
    cache.prefill(pq, pk, pv)
    kept = cache.read()["pos"][0]
    assert ((kept >= 0).sum(-1) == L).all()  # the prompt fits the budget: everything kept
    ev = torch.empty((T, B, H), dtype=torch.int32, device=DEV)
    out = torch.empty((B, H, d), dtype=torch.float32, device=DEV)
    outs = torch.empty((REPLAY, B, H, d), dtype=torch.float32, device=DEV)
    checks = (1_000_000, 2_000_000, 3_000_000, T - REPLAY)
    cuts = sorted(set(range(0, T, CALL)) | set(checks) | {c + REPLAY for c in checks} | {T})
    windows = []
    for s0, s1 in zip(cuts[:-1], cuts[1:]):
        if s0 in checks:  # the oracle takes over from the GPU's state for REPLAY steps (checked below)
            assert s1 == s0 + REPLAY
            snap = cache.read()
            cache.decode_steps(*(x[s0:s1] for x in dec), out=outs, evicted=ev[s0:s1])
            after = cache.read()
            windows += _window(w, snap, after, s0, dec, outs[:, 0].cpu().numpy(), ev[s0:s1, 0].cpu().numpy())
            out.copy_(outs[-1])
        else:
            cache.decode_steps(*(x[s0:s1] for x in dec), out=out, evicted=ev[s0:s1], keep_all=False)
        torch.cuda.synchronize()
        log(f"stream: {s1} of {T} steps done")
    fin = cache.read()
    assert cache.info() == (k, L + T, L)
    assert torch.isfinite(out).all()
    del dec
    ev = ev[:, 0].cpu().numpy()  # [T, H]
    fill = k - L  # steps until the cache is full
    assert (ev[:fill] == -1).all(), "an eviction while the cache was filling"
    i = L + np.arange(T)
    assert (ev[fill:] >= 0).all(), "a full cache skipped an eviction"
    assert (ev[fill:] <= (i[fill:] - kr)[:, None]).all(), "the recent window was evicted"
    for h in range(H):
        e = np.sort(ev[fill:, h])
        assert (np.diff(e) > 0).all(), f"head {h}: a position evicted twice"
        alive = np.setdiff1d(np.arange(L + T), e, assume_unique=True)
        got = np.sort(fin["pos"][0, h])
        assert np.array_equal(got, alive), f"head {h}: final positions differ from the log"
    sc = fin["score"][0]
    assert np.isfinite(sc).all() and (sc > 0).all()
    log(f"stream: {T} steps x {H} heads: budget, window, candidate bound, no re-entry and final "
        f"positions hold; final score range {sc.min():.4g}..{sc.max():.4g}")
    cache.close()
    res = parallel_map(_oracle_worker.continue_unit, windows)
    bad = [r for r in res if not r["ok"]]
    log(f"stream: oracle from the GPU's state at {checks}, {REPLAY} steps x {len(HEADS)} heads each: worst "
        f"output error {max(r.get('out_err', 0) for r in res):.3g}, score error "
        f"{max(r.get('score_rel', 0) for r in res):.3g}, near-ties adopted {sum(r.get('ties', 0) for r in res)}")
    assert not bad, "; ".join(f"{r['tag']}: {r['msg']}" for r in bad)
