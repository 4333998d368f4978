"""h2o_column_scores_noalloc, the column scores of a whole sequence with its
scratch in a file-scope device array (for callers that cannot allocate), through
the C ABI (needs an MI355X): two calls in a row, the second with a smaller
input, each bit-identical to h2o_column_scores on a cache and within the score
tolerance (1e-4 relative) of the oracle; the argument checks that guard the
static scratch."""
import ctypes

import numpy as np
import pytest
import torch

from workload import get, scaled, synth

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)

from gpu_harness import log  # noqa: E402
from kv_cache_eviction_prefill_amd import H2OCache  # noqa: E402
from kv_cache_eviction_prefill_amd import h2o as H  # noqa: E402
from oracle import global_scores  # noqa: E402

DEV = torch.device("cuda", 0)
SCORE_RTOL = 1e-4


def _noalloc(w, q, k, n):
    B, Hh, d = w.batch, w.heads, w.head_dim
    params = H.make_params(B, Hh, d, 1, 1, w.dtype, 0.0, 0, 0.0)
    out = torch.full((B, Hh, n), float("nan"), dtype=torch.float32, device=DEV)
    st = H.h2o_column_scores_noalloc(ctypes.byref(params), q.data_ptr(), k.data_ptr(), n, out.data_ptr(),
                                     torch.cuda.current_stream(DEV).cuda_stream)
    assert st == H.H2O_OK, H.h2o_last_error()
    return out


def _with_cache(w, q, k, n):
    cache = H2OCache(w.batch, w.heads, w.head_dim, 1, 1, dtype=w.dtype, max_prompt=n)
    s = cache.column_scores(q, k)
    torch.cuda.synchronize()
    cache.close()
    return s


def _case(base, B, Hh, d, n):
    w = scaled(get(base), batch=B, heads=Hh, head_dim=d, prompt_len=n, decode_steps=0, n_anchors=max(1, n // 50))
    Q, K, _ = synth.batch_qkv(w, 0, 0, n)
    q, k = (synth.to_torch(w, x, DEV) for x in (Q, K))
    return w, Q, K, q, k


def _check(w, Q, K, got, ref, tag):
    g, r = got.cpu().numpy(), ref.cpu().numpy()
    assert np.isfinite(g).all(), f"{tag}: scores not fully written"
    assert np.array_equal(g.view(np.uint32), r.view(np.uint32)), f"{tag}: differs from h2o_column_scores"
    worst = 0.0
    for b in range(w.batch):
        for h in range(w.heads):
            o = global_scores(Q[b, h], K[b, h], 1.0 / np.sqrt(w.head_dim))
            worst = max(worst, float(np.max(np.abs(g[b, h] - o) / o)))
    assert worst <= SCORE_RTOL, f"{tag}: worst relative error {worst:.3g} against the oracle"
    log(f"no-alloc column scores {tag}: bit-identical to the cache call, worst rel err vs oracle {worst:.2e}")


@pytest.mark.parametrize("first,second", [
    (("opt6.7b-layer-b16", 2, 3, 128, 700), ("opt6.7b-layer-b16", 1, 2, 128, 97)),
    (("tiny-fp32", 2, 2, 64, 300), ("tiny-fp32", 1, 1, 64, 33)),
])
def test_two_calls_match_cache_call(first, second):
    for tag, spec in (("first", first), ("second, smaller", second)):
        w, Q, K, q, k = _case(*spec)
        log(f"case no-alloc {tag}: {w.dtype} B={w.batch} H={w.heads} d={w.head_dim} n={spec[-1]}")
        got = _noalloc(w, q, k, spec[-1])
        torch.cuda.synchronize()
        _check(w, Q, K, got, _with_cache(w, q, k, spec[-1]), tag)


def test_limits_and_arguments():
    # checks run on the host before any launch
    p = H.make_params(64, 32, 128, 1, 1, "bf16", 0.0, 0, 0.0)  # 2048 units x 1024 rows x 8 B = 16 MiB: fits
    st = H.h2o_column_scores_noalloc(ctypes.byref(p), None, None, 1024, None, None)
    assert st == H.H2O_ERR_INVALID_ARG and "non-NULL" in H.h2o_last_error()
    buf = torch.empty(16, dtype=torch.float32, device=DEV)
    ptr = buf.data_ptr()
    st = H.h2o_column_scores_noalloc(ctypes.byref(p), ptr, ptr, 1025, ptr, None)
    assert st == H.H2O_ERR_INVALID_ARG and "static scratch" in H.h2o_last_error()
    pr = H.make_params(1, 1, 128, 1, 1, "bf16", 0.0, 0, 10000.0)
    assert H.h2o_column_scores_noalloc(ctypes.byref(pr), ptr, ptr, 4, ptr, None) == H.H2O_ERR_UNSUPPORTED
    assert H.h2o_column_scores_noalloc(None, ptr, ptr, 4, ptr, None) == H.H2O_ERR_INVALID_ARG
    assert H.h2o_column_scores_noalloc(ctypes.byref(p), None, None, 0, None, None) == H.H2O_OK
