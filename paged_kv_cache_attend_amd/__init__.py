"""Paged KV-cache attention for AMD MI355X (gfx950).

The compute lives in ``libpa.so`` (hand-written HIP kernels behind a C ABI,
declared in ``include/pa.h``).  This package is a thin ctypes binding over
that library (``_lib``) plus the seeded input generator used by tests and
benchmarks (``inputs``).  The library is loaded on first use; if it has not
been built, every entry point raises instead of falling back to any other
implementation.
"""

_BINDING = ("PaError", "Shape", "Status", "attend", "combine", "gather_kv", "validate",
            "lib_path", "load", "make_shape", "plan", "status_string", "workspace_size",
            "EXPORTS", "PreparedAttend", "workspace_init", "write_kv", "copy_blocks", "Pool",
            "PoolStats", "KVCache", "QuantCache", "attend_kv", "write_kv_cache", "KV_BF16",
            "KV_FP8_E4M3", "KV_Q8_0", "KV_Q4_0", "PrefixGroups", "attend_prefix", "attend_noalloc",
            "NOALLOC_SCRATCH_BYTES", "measure_read_tiles", "measure_mfma_bf16")


def __getattr__(name):
    if name in _BINDING:
        from . import _lib
        return getattr(_lib, name)
    raise AttributeError(name)
