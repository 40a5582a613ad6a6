"""kv_cache_vector_amd -- the TurboQuant KV-cache codec on AMD Instinct MI355X (gfx950).

The compute lives in ``libtq.so`` (hand-written HIP kernels behind a C ABI,
declared in ``include/tq.h``).  This package holds the ctypes binding
(``_lib``), thin torch-facing wrappers (``TurboQuant``, ``TQPagedAttention``)
and the seeded synthetic workloads used by the tests and the benchmark.
Nothing is loaded at import time; the library is opened on first use and a
missing library raises instead of falling back to any other code path.
"""

__all__ = ["TurboQuant", "TQPagedAttention"]


def __getattr__(name):
    if name in ("TurboQuant", "TQPagedAttention"):
        from . import turboquant
        return getattr(turboquant, name)
    raise AttributeError(name)
