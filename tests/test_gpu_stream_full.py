"""The LLaMA-7B-shaped stream run end to end: a 512-token prompt, then all
4,000,000 decode steps at k = 1024 + 1024 on 32 heads (Report §4.4 Q1: H2O with
position rolling streams 4 million tokens; here without the rotation), through
h2o_decode_steps (needs an MI355X).  Checked on every head from the GPU's own
eviction log: the budget (no eviction while the cache fills, one per step
after), the candidate bound (the recent window is never evicted), no position
evicted twice, and the final cache holding exactly the positions never
evicted.  The oracle replays the first 100,000 steps of four heads in
``test_gpu_fullsize.py``; the accuracy of the compensated scores over 4 M
increments is bounded in ``test_kahan_drift.py``."""
import numpy as np
import pytest
import torch

from workload import get, synth

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)

from gpu_harness import log  # noqa: E402
from kv_cache_eviction_prefill_amd import H2OCache  # noqa: E402

DEV = torch.device("cuda", 0)
CHUNK = 1 << 18   # positions generated per call
CALL = 1_000_000  # decode steps per h2o_decode_steps call


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
    for s0 in range(0, T, CALL):
        s1 = min(T, s0 + CALL)
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
