"""MI355X-native Heavy-Hitter Oracle (H2O) KV-cache path: HIP kernels behind a C ABI.

The compute lives in ``libh2o.so`` (kernels in ``csrc/``, ABI in
``include/h2o.h``); ``binding`` is a thin ctypes layer over it.
"""
from .binding import (H2OCache, H2OError, h2o_cache, h2o_cache_init, h2o_cache_restore,
                      h2o_cache_state, h2o_decode_step, h2o_fullcache_decode, h2o_last_error,
                      h2o_prefill_select, h2o_prefill_workspace_bytes, h2o_state, load_library)

__all__ = ["H2OCache", "H2OError", "h2o_cache", "h2o_cache_init", "h2o_cache_restore",
           "h2o_cache_state", "h2o_decode_step", "h2o_fullcache_decode", "h2o_last_error",
           "h2o_prefill_select", "h2o_prefill_workspace_bytes", "h2o_state", "load_library"]
