"""Row-major FP32 GEMM (C = A x B) for AMD MI355X (gfx950).

The product is computed by hand-written HIP kernels behind the C-ABI library
``libgemm_f32.so`` (declared in ``include/gemm_f32.h``).  ``binding`` is the
thin ctypes layer over it; importing this package does not load the library,
so the seeded input generators in ``workloads`` stay usable without a GPU.
"""

from __future__ import annotations

__all__ = ["gemm", "gemm_f32", "gemm_f32_variant", "gemm_f32_strerror", "workloads"]


def __getattr__(name):
    if name in ("gemm", "gemm_f32", "gemm_f32_variant", "gemm_f32_strerror"):
        from . import binding

        return getattr(binding, name)
    if name == "workloads":
        from . import workloads

        return workloads
    raise AttributeError(name)
