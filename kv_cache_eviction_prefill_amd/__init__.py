"""H2O budgeted-KV attention for AMD MI355X (gfx950).

The compute path is ``libh2o.so`` (hand-written HIP kernels behind the C ABI in
``include/h2o.h``); ``h2o`` is its ctypes binding.
"""
from .h2o import (  # noqa: F401
    H2OCache, H2OError, h2o_params, load, make_params, declared_entry_points,
    h2o_cache_bytes, h2o_cache_create, h2o_cache_destroy, h2o_prefill, h2o_decode_step,
    h2o_cache_read, h2o_prefill_stats_read, h2o_cache_info, h2o_status_str, h2o_last_error,
)
