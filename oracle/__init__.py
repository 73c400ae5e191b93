"""CPU oracle for SnapKV prefill-time KV-cache compression -- TEST INFRASTRUCTURE.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  The product path (the HIP library and
its Python binding) never imports it and shares no code with it.

The arithmetic lives in ``snapkv_oracle.c`` (plain C, fp64); ``ref.py`` is the
NumPy-facing wrapper that builds and loads it.
"""
from .ref import (  # noqa: F401
    build,
    votes,
    row_lse,
    lse_all,
    decode,
    decode_all,
    pool,
    k_of,
    select,
    gather,
    hit_rate,
    compress_head,
    compress,
    run_jobs_timed,
)
