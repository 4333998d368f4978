"""Thin ctypes binding of ``libh2o.so`` (the C ABI in ``include/h2o.h``).

Argument marshalling only: every step of prefill and decode runs in the HIP
kernels behind the C entry points.  PyTorch supplies device memory (tensor
``data_ptr()``) and the stream (``torch.cuda.current_stream().cuda_stream``).
The module fails loudly when the library has not been built; there is no other
implementation to fall back on.

The functions named like the C entry points (``h2o_cache_create``, ...) return
the C status code unchanged; ``H2OCache`` wraps them for torch tensors and
raises ``H2OError`` on any non-zero status.
"""
from __future__ import annotations

import ctypes
import os
import re

import numpy as np

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libh2o.so")
HEADER_PATH = os.path.join(os.path.dirname(_PKG), "include", "h2o.h")

H2O_F32, H2O_BF16 = 0, 1
H2O_PATTERN_NONE, H2O_PATTERN_STRIDED, H2O_PATTERN_FIXED = 0, 1, 2
STATUS = {0: "H2O_OK", 1: "H2O_ERR_INVALID_ARG", 2: "H2O_ERR_STATE", 3: "H2O_ERR_OOM",
          4: "H2O_ERR_HIP", 5: "H2O_ERR_UNSUPPORTED"}
H2O_OK, H2O_ERR_INVALID_ARG, H2O_ERR_STATE, H2O_ERR_OOM, H2O_ERR_HIP, H2O_ERR_UNSUPPORTED = range(6)


class h2o_params(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int32), ("heads", ctypes.c_int32), ("head_dim", ctypes.c_int32),
                ("heavy_budget", ctypes.c_int32), ("recent_budget", ctypes.c_int32),
                ("dtype", ctypes.c_int32), ("scale", ctypes.c_float), ("max_prompt", ctypes.c_int32),
                ("rope_base", ctypes.c_float)]


class H2OError(RuntimeError):
    def __init__(self, status: int, where: str, detail: str = ""):
        self.status = status
        super().__init__(f"{where}: {STATUS.get(status, status)} ({detail})")


_vp, _i32, _p32 = ctypes.c_void_p, ctypes.c_int32, ctypes.POINTER(ctypes.c_int32)
_SIGNATURES = {
    "h2o_cache_bytes": (_i32, [ctypes.POINTER(h2o_params), ctypes.POINTER(ctypes.c_size_t),
                               ctypes.POINTER(ctypes.c_size_t)]),
    "h2o_cache_create": (_i32, [ctypes.POINTER(h2o_params), ctypes.c_int, ctypes.POINTER(_vp)]),
    "h2o_cache_destroy": (_i32, [_vp]),
    "h2o_prefill": (_i32, [_vp, _vp, _vp, _vp, _i32, _vp, _vp]),
    "h2o_decode_step": (_i32, [_vp, _vp, _vp, _vp, _vp, _vp, _vp]),
    "h2o_decode_steps": (_i32, [_vp, _vp, _vp, _vp, _i32, _vp, ctypes.c_int64, _vp, _vp]),
    "h2o_cache_read": (_i32, [_vp, _vp, _vp, _vp, _vp, _vp, _vp]),
    "h2o_prefill_stats_read": (_i32, [_vp, _vp, _vp, _vp]),
    "h2o_cache_info": (_i32, [_vp, _p32, _p32, _p32]),
    "h2o_column_scores": (_i32, [_vp, _vp, _vp, _i32, _vp, _vp]),
    "h2o_column_scores_noalloc": (_i32, [ctypes.POINTER(h2o_params), _vp, _vp, _i32, _vp, _vp]),
    "h2o_cache_set_pattern": (_i32, [_vp, _i32, _i32, _i32]),
    "h2o_prefill_scored": (_i32, [_vp, _vp, _vp, _i32, _i32, _vp, _vp]),
    "h2o_decode_step_scored": (_i32, [_vp, _vp, _vp, _vp, _vp, _i32, _vp, _vp, _vp]),
    "h2o_probe_read": (_i32, [_vp, ctypes.c_size_t, _vp, _vp]),
    "h2o_probe_mix": (_i32, [_i32, _i32, _vp, _vp]),
    "h2o_status_str": (ctypes.c_char_p, [_i32]),
    "h2o_last_error": (ctypes.c_char_p, []),
}

_lib = None


def load() -> ctypes.CDLL:
    """Load ``libh2o.so`` (once) and declare every entry point's signature."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it first (__graft_entry__.build() or "
                               f"python kv_cache_eviction_prefill_amd/build.py)")
        lib = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in _SIGNATURES.items():
            fn = getattr(lib, name)
            fn.restype, fn.argtypes = res, args
        _lib = lib
    return _lib


def declared_entry_points() -> list[str]:
    """Names of the functions ``include/h2o.h`` declares."""
    text = open(HEADER_PATH).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(h2o_\w+)\s*\(", text)))


# ------------------------------------------------------------------ raw entry points (same names as C)
def h2o_cache_bytes(params, kv_bytes=None, total_bytes=None):
    return load().h2o_cache_bytes(params, kv_bytes, total_bytes)


def h2o_cache_create(params, device, out):
    return load().h2o_cache_create(params, device, out)


def h2o_cache_destroy(cache):
    return load().h2o_cache_destroy(cache)


def h2o_prefill(cache, q, k, v, prompt_len, out, stream):
    return load().h2o_prefill(cache, q, k, v, prompt_len, out, stream)


def h2o_decode_step(cache, q, k, v, out, evicted, stream):
    return load().h2o_decode_step(cache, q, k, v, out, evicted, stream)


def h2o_decode_steps(cache, q, k, v, steps, out, out_step, evicted, stream):
    return load().h2o_decode_steps(cache, q, k, v, steps, out, out_step, evicted, stream)


def h2o_cache_read(cache, pos, score, k_slots, v_slots, meta, stream):
    return load().h2o_cache_read(cache, pos, score, k_slots, v_slots, meta, stream)


def h2o_prefill_stats_read(cache, row_lse, col_sum, stream):
    return load().h2o_prefill_stats_read(cache, row_lse, col_sum, stream)


def h2o_cache_info(cache, count, next_pos, prompt_len):
    return load().h2o_cache_info(cache, count, next_pos, prompt_len)


def h2o_column_scores(cache, q, k, n, scores, stream):
    return load().h2o_column_scores(cache, q, k, n, scores, stream)


def h2o_probe_read(buf, nbytes, sink, stream):
    return load().h2o_probe_read(buf, nbytes, sink, stream)


def h2o_probe_mix(mode, iters, sink, stream):
    return load().h2o_probe_mix(mode, iters, sink, stream)


def h2o_column_scores_noalloc(params, q, k, n, scores, stream):
    return load().h2o_column_scores_noalloc(params, q, k, n, scores, stream)


def h2o_prefill_scored(cache, k, v, prompt_len, seq_rows, scores, stream):
    return load().h2o_prefill_scored(cache, k, v, prompt_len, seq_rows, scores, stream)


def h2o_decode_step_scored(cache, q, k, v, new_score, score_stride, out, evicted, stream):
    return load().h2o_decode_step_scored(cache, q, k, v, new_score, score_stride, out, evicted, stream)


def h2o_cache_set_pattern(cache, kind, period, width):
    return load().h2o_cache_set_pattern(cache, kind, period, width)


def h2o_status_str(status):
    return load().h2o_status_str(status).decode()


def h2o_last_error():
    return load().h2o_last_error().decode()


def check(status: int, where: str) -> None:
    if status != H2O_OK:
        raise H2OError(status, where, h2o_last_error())


def make_params(batch, heads, head_dim, heavy, recent, dtype="bf16", scale=0.0, max_prompt=0,
                rope_base=0.0) -> h2o_params:
    dt = {"f32": H2O_F32, "bf16": H2O_BF16}[dtype] if isinstance(dtype, str) else int(dtype)
    return h2o_params(batch, heads, head_dim, heavy, recent, dt, float(scale), max_prompt, float(rope_base))


def _np_ptr(a) -> int | None:
    return None if a is None else a.ctypes.data


# ------------------------------------------------------------------ torch-facing wrapper
class H2OCache:
    """One budgeted cache (one attention layer) on one GPU."""

    def __init__(self, batch, heads, head_dim, heavy, recent, dtype="bf16", scale=0.0, max_prompt=0,
                 device=None, rope_base=0.0):
        import torch

        self.torch = torch
        self.params = make_params(batch, heads, head_dim, heavy, recent, dtype, scale, max_prompt, rope_base)
        self.dtype = dtype
        self.tdtype = torch.float32 if dtype == "f32" else torch.bfloat16
        self.B, self.H, self.d = batch, heads, head_dim
        self.k = heavy + recent
        self.device = torch.device("cuda", torch.cuda.current_device() if device is None else device)
        handle = _vp()
        check(h2o_cache_create(ctypes.byref(self.params), self.device.index, ctypes.byref(handle)),
              "h2o_cache_create")
        self.handle = handle

    # -- helpers
    def _stream(self, stream):
        if stream is None:
            stream = self.torch.cuda.current_stream(self.device)
        return stream.cuda_stream

    def _check_t(self, t, shape, dtype, name):
        if t.device != self.device or t.dtype != dtype or tuple(t.shape) != tuple(shape) or not t.is_contiguous():
            raise ValueError(f"{name}: expected contiguous {dtype} {tuple(shape)} on {self.device}, "
                             f"got {t.dtype} {tuple(t.shape)} on {t.device}")
        return t.data_ptr()

    # -- entry points
    def prefill(self, q, k, v, out=None, stream=None):
        """``out``: optional float32 [B, H, L, d] tensor for the prompt's attention output."""
        L = q.shape[2] if q is not None else 0
        shape = (self.B, self.H, L, self.d)
        ptrs = [self._check_t(t, shape, self.tdtype, n) if L > 0 else None for t, n in ((q, "q"), (k, "k"), (v, "v"))]
        op = self._check_t(out, shape, self.torch.float32, "out") if (out is not None and L > 0) else None
        check(h2o_prefill(self.handle, *ptrs, L, op, self._stream(stream)), "h2o_prefill")

    def decode_step(self, q, k, v, out=None, evicted=None, stream=None):
        torch = self.torch
        shape = (self.B, self.H, self.d)
        qp = self._check_t(q, shape, self.tdtype, "q")
        kp = self._check_t(k, shape, self.tdtype, "k")
        vp = self._check_t(v, shape, self.tdtype, "v")
        if out is None:
            out = torch.empty(shape, dtype=torch.float32, device=self.device)
        op = self._check_t(out, shape, torch.float32, "out")
        ep = None
        if evicted is not None:
            ep = self._check_t(evicted, (self.B, self.H), torch.int32, "evicted")
        check(h2o_decode_step(self.handle, qp, kp, vp, op, ep, self._stream(stream)), "h2o_decode_step")
        return out, evicted

    def decode_steps(self, q, k, v, out=None, evicted=None, keep_all=True, stream=None):
        """``q, k, v``: [T, B, H, d], token t of step t.  ``out``: float32
        [T, B, H, d] (every step's output) or, with ``keep_all=False``,
        [B, H, d] (the last step's); ``evicted``: optional int32 [T, B, H]."""
        torch = self.torch
        T = q.shape[0]
        shape = (T, self.B, self.H, self.d)
        qp = self._check_t(q, shape, self.tdtype, "q")
        kp = self._check_t(k, shape, self.tdtype, "k")
        vp = self._check_t(v, shape, self.tdtype, "v")
        oshape = shape if keep_all else shape[1:]
        if out is None:
            out = torch.empty(oshape, dtype=torch.float32, device=self.device)
        op = self._check_t(out, oshape, torch.float32, "out")
        ep = self._check_t(evicted, shape[:3], torch.int32, "evicted") if evicted is not None else None
        step = self.B * self.H * self.d if keep_all else 0
        check(h2o_decode_steps(self.handle, qp, kp, vp, T, op, step, ep, self._stream(stream)), "h2o_decode_steps")
        return out, evicted

    def read(self, stream=None):
        """Host copy of the cache: dict of numpy arrays (pos, score, k, v) and meta."""
        n = self.B * self.H * self.k
        pos = np.empty((self.B, self.H, self.k), np.int32)
        score = np.empty((self.B, self.H, self.k), np.float32)
        kv_dt = np.float32 if self.dtype == "f32" else np.uint16
        ks = np.empty((self.B, self.H, self.k, self.d), kv_dt)
        vs = np.empty_like(ks)
        meta = np.empty(2, np.int32)
        check(h2o_cache_read(self.handle, _np_ptr(pos), _np_ptr(score), _np_ptr(ks), _np_ptr(vs), _np_ptr(meta),
                             self._stream(stream)), "h2o_cache_read")
        if self.dtype == "bf16":  # widen the bf16 bit patterns to float32 values
            ks = (ks.astype(np.uint32) << 16).view(np.float32)
            vs = (vs.astype(np.uint32) << 16).view(np.float32)
        assert pos.size == n
        return {"pos": pos, "score": score, "k": ks, "v": vs, "count": int(meta[0]), "next_pos": int(meta[1])}

    # -- sparse pattern kept before heavy hitters
    def set_pattern(self, kind="none", period=1, width=1):
        """``kind``: "none", "strided" or "fixed" (see ``h2o_cache_set_pattern``)."""
        k = {"none": H2O_PATTERN_NONE, "strided": H2O_PATTERN_STRIDED, "fixed": H2O_PATTERN_FIXED}[kind]
        check(h2o_cache_set_pattern(self.handle, k, period, width), "h2o_cache_set_pattern")

    # -- global-score comparator
    def column_scores(self, q, k, out=None, stream=None):
        """Column sums of the causal softmax of a whole sequence [B, H, n, d]:
        float32 [B, H, n] (written into ``out`` when given)."""
        n = q.shape[2]
        shape = (self.B, self.H, n, self.d)
        qp, kp = self._check_t(q, shape, self.tdtype, "q"), self._check_t(k, shape, self.tdtype, "k")
        if out is None:
            out = self.torch.empty((self.B, self.H, n), dtype=self.torch.float32, device=self.device)
        op = self._check_t(out, (self.B, self.H, n), self.torch.float32, "out")
        check(h2o_column_scores(self.handle, qp, kp, n, op, self._stream(stream)), "h2o_column_scores")
        return out

    def prefill_scored(self, k, v, scores, prompt_len=None, stream=None):
        """Keep the prompt's recent window and best-scored tokens by ``scores``
        [B, H, n]; ``k, v``: [B, H, n, d]; the prompt is their first ``prompt_len``
        rows (all n by default)."""
        n = k.shape[2]
        L = n if prompt_len is None else prompt_len
        shape = (self.B, self.H, n, self.d)
        kp, vp = self._check_t(k, shape, self.tdtype, "k"), self._check_t(v, shape, self.tdtype, "v")
        sp = self._check_t(scores, (self.B, self.H, n), self.torch.float32, "scores")
        check(h2o_prefill_scored(self.handle, kp, vp, L, n, sp, self._stream(stream)), "h2o_prefill_scored")

    def decode_step_scored(self, q, k, v, new_score, out=None, evicted=None, stream=None):
        """A decode step with fixed scores; ``new_score``: float32 [B, H] (any
        strides along H and B that form one uniform unit stride, e.g. a column of
        a [B, H, n] score tensor)."""
        torch = self.torch
        shape = (self.B, self.H, self.d)
        qp = self._check_t(q, shape, self.tdtype, "q")
        kp = self._check_t(k, shape, self.tdtype, "k")
        vp = self._check_t(v, shape, self.tdtype, "v")
        if (new_score.device != self.device or new_score.dtype != torch.float32
                or tuple(new_score.shape) != (self.B, self.H)
                or new_score.stride(0) != self.H * new_score.stride(1)):
            raise ValueError("new_score: expected float32 [B, H] with one uniform unit stride on the cache device")
        np_, stride = new_score.data_ptr(), new_score.stride(1)
        if out is None:
            out = torch.empty(shape, dtype=torch.float32, device=self.device)
        op = self._check_t(out, shape, torch.float32, "out")
        ep = None
        if evicted is not None:
            ep = self._check_t(evicted, (self.B, self.H), torch.int32, "evicted")
        check(h2o_decode_step_scored(self.handle, qp, kp, vp, np_, stride, op, ep, self._stream(stream)),
              "h2o_decode_step_scored")
        return out, evicted

    def prefill_stats(self, stream=None):
        L = self.info()[2]
        arrs = [np.empty((self.B, self.H, max(L, 0)), np.float32) for _ in range(2)]
        check(h2o_prefill_stats_read(self.handle, *(_np_ptr(a) for a in arrs), self._stream(stream)),
              "h2o_prefill_stats_read")
        return tuple(arrs)

    def info(self):
        c, n, p = ctypes.c_int32(), ctypes.c_int32(), ctypes.c_int32()
        check(h2o_cache_info(self.handle, ctypes.byref(c), ctypes.byref(n), ctypes.byref(p)), "h2o_cache_info")
        return c.value, n.value, p.value

    def close(self):
        if getattr(self, "handle", None):
            check(h2o_cache_destroy(self.handle), "h2o_cache_destroy")
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:  # noqa: BLE001 - interpreter shutdown
            pass
