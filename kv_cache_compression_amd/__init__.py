"""kv_cache_compression_amd -- SnapKV prefill-time KV-cache compression on AMD MI355X.

The work runs in libsnapkv (HIP kernels for gfx950 behind the C ABI in
include/snapkv.h).  This package holds the thin ctypes binding (``_lib``), the
in-tree build step (``build``) and the seeded synthetic workloads (``synth``).
"""

__version__ = "0.1.0"


def __getattr__(name):
    # The binding (and torch) load on first use, so `synth` stays importable alone.
    if name in ("compress", "scores", "select", "gather", "decode", "hit_rate_counts", "make_spec", "workspace",
                "load", "SnapKVError", "Spec", "Problem", "DecodeProblem"):
        from . import _lib
        return getattr(_lib, name)
    raise AttributeError(name)
