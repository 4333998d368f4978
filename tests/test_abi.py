"""The C ABI on the CPU: the library loads, exports every function the header
declares, and rejects bad arguments before any GPU call."""
import ctypes
import json
import math
import os

import pytest

from kv_cache_eviction_prefill_amd import h2o as H

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


@pytest.fixture(scope="module", autouse=True)
def built_library():
    """The in-tree library, compiled here (hipcc cross-compiles for gfx950 without
    a GPU) when nothing has been built yet."""
    if not os.path.exists(H.LIB_PATH):
        from kv_cache_eviction_prefill_amd import build

        build.build()
    return H.load()


def test_every_declared_symbol_is_exported():
    lib = H.load()
    names = H.declared_entry_points()
    assert {"h2o_cache_create", "h2o_cache_destroy", "h2o_prefill", "h2o_decode_step",
            "h2o_cache_read", "h2o_column_scores", "h2o_prefill_scored", "h2o_decode_step_scored"} <= set(names)
    for n in names:
        assert hasattr(lib, n), n
        assert n in H._SIGNATURES, f"binding has no signature for {n}"
        assert callable(getattr(H, n)), f"binding has no same-name wrapper for {n}"


def test_status_strings():
    for code in range(6):
        assert H.h2o_status_str(code) not in ("", "unknown status")
    assert H.h2o_status_str(42) == "unknown status"


def _bytes(**kw):
    base = dict(batch=2, heads=3, head_dim=128, heavy=4, recent=4, dtype="bf16", scale=0.0, max_prompt=64,
                rope_base=0.0)
    base.update(kw)
    p = H.make_params(base["batch"], base["heads"], base["head_dim"], base["heavy"], base["recent"],
                      base["dtype"], base["scale"], base["max_prompt"], base["rope_base"])
    kv, tot = ctypes.c_size_t(), ctypes.c_size_t()
    st = H.h2o_cache_bytes(ctypes.byref(p), ctypes.byref(kv), ctypes.byref(tot))
    return st, kv.value, tot.value


@pytest.mark.parametrize("kw,status", [
    (dict(batch=0), H.H2O_ERR_INVALID_ARG), (dict(heads=-1), H.H2O_ERR_INVALID_ARG),
    (dict(head_dim=0), H.H2O_ERR_INVALID_ARG), (dict(head_dim=96), H.H2O_ERR_UNSUPPORTED),
    (dict(heavy=0, recent=0), H.H2O_ERR_INVALID_ARG), (dict(heavy=-1), H.H2O_ERR_INVALID_ARG),
    (dict(heavy=10000, recent=5000), H.H2O_ERR_UNSUPPORTED), (dict(dtype=7), H.H2O_ERR_INVALID_ARG),
    (dict(scale=float("nan")), H.H2O_ERR_INVALID_ARG), (dict(max_prompt=-1), H.H2O_ERR_INVALID_ARG),
    (dict(rope_base=-1.0), H.H2O_ERR_INVALID_ARG), (dict(rope_base=float("inf")), H.H2O_ERR_INVALID_ARG),
    (dict(rope_base=10000.0), H.H2O_OK),
    (dict(batch=1 << 16, heads=1 << 10, max_prompt=4096), H.H2O_ERR_INVALID_ARG),
    # one unit's [max_prompt, d] bf16 prompt matrix must stay below 2^32 bytes
    (dict(batch=1, heads=1, max_prompt=1 << 24), H.H2O_ERR_INVALID_ARG),
    (dict(batch=1, heads=1, max_prompt=(1 << 24) - 32), H.H2O_OK),
    (dict(), H.H2O_OK), (dict(heavy=0, recent=1), H.H2O_OK), (dict(head_dim=64, dtype="f32"), H.H2O_OK),
])
def test_param_validation(kw, status):
    assert _bytes(**kw)[0] == status
    if status != H.H2O_OK:
        assert H.h2o_last_error() != ""


def test_cache_bytes_accounting():
    st, kv, tot = _bytes(batch=2, heads=3, head_dim=128, heavy=4, recent=4, dtype="bf16", max_prompt=64)
    assert st == 0 and kv == 2 * 6 * 8 * 128 * 2
    # + scores, compensation, positions (12 B / slot, rows padded to 32 slots)
    # + split scratch (few units: partials and logits, twice, and a second score,
    #   compensation and position array) + 2 prefill rows (row normaliser, column sum)
    assert tot == kv + 6 * 32 * 12 + (2 * (6 * 64 * 130 * 4 + 6 * 9 * 4) + 6 * 32 * 12) + 2 * 6 * 64 * 4
    st, kv32, _ = _bytes(dtype="f32")
    assert kv32 == 2 * kv
    # position rolling adds slot ranks (a second buffer of them on the split path),
    # the rotated prompt of a chunk of units (8 bytes per element: bf16 hi and lo
    # of q and of k) and the rotary tables
    st, _, tot_r = _bytes(batch=2, heads=3, head_dim=128, heavy=4, recent=4, dtype="bf16", max_prompt=64,
                          rope_base=10000.0)
    assert st == 0 and tot_r == tot + 2 * 6 * 32 * 4 + 6 * 64 * 128 * 8 + 64 * 64 * 8 + 64 * 8
    # the chunk is capped at 512 MiB of scratch: 256 units of a 2048-token prompt at d = 128
    kw = dict(batch=64, heads=32, head_dim=128, heavy=205, recent=205, dtype="bf16", max_prompt=2048)
    st, _, big = _bytes(**kw)
    st_r, _, big_r = _bytes(rope_base=10000.0, **kw)
    assert st == st_r == 0 and big_r == big + 2048 * 416 * 4 + (512 << 20) + 2048 * 64 * 8 + 64 * 8


def test_kv_size_matches_reported_example():
    with open(os.path.join(GOLDEN, "kv_size.json")) as f:
        g = json.load(f)
    heads = g["hidden"] // 128
    st, kv, _ = _bytes(batch=g["batch"], heads=heads, head_dim=128, heavy=g["seq_len"] // 2,
                       recent=g["seq_len"] // 2, dtype="bf16", max_prompt=0)
    assert st == 0
    total_gb = kv * g["layers"] / 1e9
    assert math.isclose(total_gb, g["reported_gb"], rel_tol=g["rel_tol"])


def test_null_and_state_checks_make_no_gpu_call():
    lib = H.load()
    assert H.h2o_cache_destroy(None) == H.H2O_OK
    assert H.h2o_prefill(None, None, None, None, 0, None, None) == H.H2O_ERR_INVALID_ARG
    assert H.h2o_decode_step(None, None, None, None, None, None, None) == H.H2O_ERR_INVALID_ARG
    assert H.h2o_decode_steps(None, None, None, None, 1, None, 0, None, None) == H.H2O_ERR_INVALID_ARG
    assert H.h2o_cache_read(None, None, None, None, None, None, None) == H.H2O_ERR_INVALID_ARG
    assert H.h2o_prefill_stats_read(None, None, None, None) == H.H2O_ERR_INVALID_ARG
    assert H.h2o_cache_info(None, None, None, None) == H.H2O_ERR_INVALID_ARG
    assert H.h2o_column_scores(None, None, None, 4, None, None) == H.H2O_ERR_INVALID_ARG
    assert H.h2o_cache_set_pattern(None, 1, 4, 1) == H.H2O_ERR_INVALID_ARG
    assert H.h2o_prefill_scored(None, None, None, 4, 4, None, None) == H.H2O_ERR_INVALID_ARG
    assert H.h2o_decode_step_scored(None, None, None, None, None, 1, None, None, None) == H.H2O_ERR_INVALID_ARG
    p = H.make_params(1, 1, 64, 2, 2, "f32")
    assert H.h2o_cache_create(ctypes.byref(p), -1, None) == H.H2O_ERR_INVALID_ARG
    out = ctypes.c_void_p(1234)
    bad = H.make_params(1, 1, 96, 2, 2, "f32")
    assert H.h2o_cache_create(ctypes.byref(bad), -1, ctypes.byref(out)) == H.H2O_ERR_UNSUPPORTED
    assert out.value is None  # *out is cleared on failure
    assert H.h2o_cache_create(ctypes.byref(p), -5, ctypes.byref(out)) == H.H2O_ERR_INVALID_ARG
    assert lib is H.load()


def test_create_without_gpu_reports_hip_error(gpu_available):
    if gpu_available:
        pytest.skip("a GPU is present")
    p = H.make_params(1, 1, 64, 2, 2, "f32")
    out = ctypes.c_void_p()
    st = H.h2o_cache_create(ctypes.byref(p), -1, ctypes.byref(out))
    assert st in (H.H2O_ERR_HIP, H.H2O_ERR_OOM) and out.value is None
    assert H.h2o_last_error() != ""


@pytest.mark.parametrize("mode,iters,sink", [(3, 10, 16), (-1, 10, 16), (0, 0, 16), (1, -5, 16), (2, 10, None)])
def test_probe_mix_rejects_bad_arguments(mode, iters, sink):
    """The compute-ceiling probe checks its arguments before touching the GPU
    (`sink` is never dereferenced on the host: any non-NULL value passes)."""
    assert H.h2o_probe_mix(mode, iters, sink, None) == H.H2O_ERR_INVALID_ARG


def test_probe_read_rejects_bad_arguments():
    assert H.h2o_probe_read(None, 16, 16, None) == H.H2O_ERR_INVALID_ARG
    assert H.h2o_probe_read(16, 16, None, None) == H.H2O_ERR_INVALID_ARG
    assert H.h2o_probe_read(17, 16, 16, None) == H.H2O_ERR_INVALID_ARG
    assert H.h2o_probe_read(16, 15, 16, None) == H.H2O_ERR_INVALID_ARG
