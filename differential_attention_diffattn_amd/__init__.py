"""MI355X-native differential attention (DIFF V1 / DIFF V2 forward).

The compute lives in ``libdiffattn.so`` (hand-written HIP for gfx950, built
from ``csrc/``).  This package is a thin ctypes binding over its C ABI plus
the seeded synthetic workloads used by the tests and the benchmark.  The
binding is imported lazily so that ``workloads`` can be used on machines
without a GPU.
"""
from __future__ import annotations

__all__ = ["v1_fwd", "v2_fwd", "v2_decode", "v2_decode_workspace_bytes", "lambda_init",
           "DiffAttnError", "library_path", "load_library"]


def __getattr__(name):
    if name in __all__:
        from . import binding
        return getattr(binding, name)
    raise AttributeError(name)
