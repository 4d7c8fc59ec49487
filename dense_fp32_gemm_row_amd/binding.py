"""ctypes binding of libgemm_f32.so (declared in include/gemm_f32.h).

Argument marshalling only: every step of the product runs in the HIP
kernels behind the C ABI.  PyTorch provides device memory and streams; it
computes nothing here.  There is no fallback: if the library is missing the
calls raise.

Functions with the C names take raw integers (sizes, device addresses,
leading dimensions, a hipStream_t address) and return the C status code.
``gemm`` is the tensor-level convenience used by tests and the benchmark.
"""

from __future__ import annotations

import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIBRARY = os.path.join(HERE, "libgemm_f32.so")

GEMM_F32_OK = 0
GEMM_F32_EINVAL = -1
GEMM_F32_EHIP = -2
GEMM_F32_ENOKERNEL = -3

VARIANT_NAIVE = 0
VARIANT_LDS = 1
VARIANT_REGBLOCK = 2
VARIANT_MFMA = 3
VARIANTS = {"naive": VARIANT_NAIVE, "lds": VARIANT_LDS, "regblock": VARIANT_REGBLOCK,
            "mfma": VARIANT_MFMA}

_i64 = ctypes.c_int64
_vp = ctypes.c_void_p
_int = ctypes.c_int

_LIB: ctypes.CDLL | None = None


class GemmError(RuntimeError):
    def __init__(self, code: int, detail: str):
        self.code = code
        super().__init__(f"{gemm_f32_strerror(code)} ({code}): {detail}")


def load(path: str = LIBRARY) -> ctypes.CDLL:
    """Loads the library (once).  Raises if it has not been built."""
    global _LIB
    if _LIB is not None:
        return _LIB
    if not os.path.exists(path):
        raise RuntimeError(
            f"{path} is missing: build it with `python -c 'import __graft_entry__ as g; g.build()'`")
    # torch ships its own HIP runtime.  Loading torch first makes the
    # library's libamdhip64.so.7 dependency resolve (by soname) to that copy,
    # so the library launches into the same runtime that owns torch's memory
    # and streams.  Loaded the other way round, the process would hold two
    # HIP runtimes and torch's stream handles would be foreign to ours.
    import torch  # noqa: F401

    lib = ctypes.CDLL(path)
    lib.gemm_f32.restype = _int
    lib.gemm_f32.argtypes = [_i64, _i64, _i64, _vp, _i64, _vp, _i64, _vp, _i64, _vp]
    lib.gemm_f32_variant.restype = _int
    lib.gemm_f32_variant.argtypes = [_int, _int, _i64, _i64, _i64, _vp, _i64, _vp, _i64, _vp,
                                     _i64, _vp]
    lib.gemm_f32_strided_batched.restype = _int
    lib.gemm_f32_strided_batched.argtypes = [_i64, _i64, _i64, _i64, _vp, _i64, _i64, _vp, _i64,
                                             _i64, _vp, _i64, _i64, _vp]
    lib.gemm_f32_strided_batched_variant.restype = _int
    lib.gemm_f32_strided_batched_variant.argtypes = [_int, _int, _i64, _i64, _i64, _i64, _vp, _i64,
                                                     _i64, _vp, _i64, _i64, _vp, _i64, _i64, _vp]
    lib.gemm_f32_strerror.restype = ctypes.c_char_p
    lib.gemm_f32_strerror.argtypes = [_int]
    lib.gemm_f32_last_error.restype = ctypes.c_char_p
    lib.gemm_f32_last_error.argtypes = []
    lib.gemm_f32_config_count.restype = _int
    lib.gemm_f32_config_count.argtypes = [_int]
    lib.gemm_f32_config_name.restype = ctypes.c_char_p
    lib.gemm_f32_config_name.argtypes = [_int, _int]
    lib.gemm_f32_select.restype = _int
    lib.gemm_f32_select.argtypes = [_i64, _i64, _i64, _i64, _i64, _i64,
                                    ctypes.POINTER(_int), ctypes.POINTER(_int)]
    lib.gemm_f32_abi_version.restype = _int
    lib.gemm_f32_abi_version.argtypes = []
    _LIB = lib
    return lib


# ---- the C entry points, same names, raw arguments -------------------------

def gemm_f32(M, N, K, A, lda, B, ldb, C, ldc, stream=None) -> int:
    return load().gemm_f32(M, N, K, A, lda, B, ldb, C, ldc, stream)


def gemm_f32_variant(variant, config_id, M, N, K, A, lda, B, ldb, C, ldc, stream=None) -> int:
    return load().gemm_f32_variant(variant, config_id, M, N, K, A, lda, B, ldb, C, ldc, stream)


def gemm_f32_strided_batched(batch, M, N, K, A, lda, sA, B, ldb, sB, C, ldc, sC,
                             stream=None) -> int:
    return load().gemm_f32_strided_batched(batch, M, N, K, A, lda, sA, B, ldb, sB, C, ldc, sC,
                                           stream)


def gemm_f32_strided_batched_variant(variant, config_id, batch, M, N, K, A, lda, sA, B, ldb, sB,
                                     C, ldc, sC, stream=None) -> int:
    return load().gemm_f32_strided_batched_variant(variant, config_id, batch, M, N, K, A, lda, sA,
                                                   B, ldb, sB, C, ldc, sC, stream)


def gemm_f32_strerror(code: int) -> str:
    return load().gemm_f32_strerror(code).decode()


def gemm_f32_last_error() -> str:
    return load().gemm_f32_last_error().decode()


def gemm_f32_config_count(variant: int) -> int:
    return load().gemm_f32_config_count(variant)


def gemm_f32_config_name(variant: int, config_id: int) -> str | None:
    name = load().gemm_f32_config_name(variant, config_id)
    return None if name is None else name.decode()


def gemm_f32_select(M, N, K, lda, ldb, ldc) -> tuple[int, int]:
    v, c = _int(), _int()
    rc = load().gemm_f32_select(M, N, K, lda, ldb, ldc, ctypes.byref(v), ctypes.byref(c))
    if rc != GEMM_F32_OK:
        raise GemmError(rc, gemm_f32_last_error())
    return v.value, c.value


def gemm_f32_abi_version() -> int:
    return load().gemm_f32_abi_version()


def config_names(variant: int) -> list[str]:
    return [gemm_f32_config_name(variant, i) for i in range(gemm_f32_config_count(variant))]


def config_id(variant: int, name: str) -> int:
    names = config_names(variant)
    if name not in names:
        raise KeyError(f"variant {variant} has no configuration {name!r}; have {names}")
    return names.index(name)


# ---- tensor-level convenience ----------------------------------------------

def _row_major_ld(t, name: str) -> int:
    import torch

    if t.dtype != torch.float32 or t.dim() != 2 or not t.is_cuda:
        raise TypeError(f"{name} must be a 2-D float32 GPU tensor")
    rows, cols = t.shape
    if cols > 1 and t.stride(1) != 1:
        raise ValueError(f"{name} must have unit column stride (row-major)")
    if rows <= 1:
        return max(cols, 1)
    return t.stride(0)


def _batch_layout(t, name: str) -> tuple[int, int]:
    """(leading dimension, batch stride) of a 3-D float32 GPU tensor whose
    matrices are row-major; a batch stride of 0 (expanded tensor) is allowed."""
    import torch

    if t.dtype != torch.float32 or t.dim() != 3 or not t.is_cuda:
        raise TypeError(f"{name} must be a 3-D float32 GPU tensor")
    _, rows, cols = t.shape
    if cols > 1 and t.stride(2) != 1:
        raise ValueError(f"{name} must have unit column stride (row-major)")
    ld = t.stride(1) if rows > 1 else max(cols, 1)
    return ld, t.stride(0)


def gemm_batched(A, B, out=None, *, variant: int | str | None = None, config: int | str = -1,
                 stream=None):
    """``out[b] = A[b] @ B[b]`` for 3-D float32 GPU tensors through
    gemm_f32_strided_batched (or its _variant form).  A or B may be an
    expanded tensor (batch stride 0)."""
    import torch

    nb, M, K = A.shape
    nb2, K2, N = B.shape
    if nb != nb2 or K != K2:
        raise ValueError(f"shape mismatch {tuple(A.shape)} x {tuple(B.shape)}")
    lda, sa = _batch_layout(A, "A")
    ldb, sb = _batch_layout(B, "B")
    if out is None:
        out = torch.empty((nb, M, N), dtype=torch.float32, device=A.device)
    ldc, sc = _batch_layout(out, "out")
    if tuple(out.shape) != (nb, M, N):
        raise ValueError(f"out has shape {tuple(out.shape)}, expected {(nb, M, N)}")
    s = stream if stream is not None else torch.cuda.current_stream(A.device)
    if variant is None:
        rc = gemm_f32_strided_batched(nb, M, N, K, A.data_ptr(), lda, sa, B.data_ptr(), ldb, sb,
                                      out.data_ptr(), ldc, sc, s.cuda_stream)
    else:
        v = VARIANTS[variant] if isinstance(variant, str) else int(variant)
        c = config_id(v, config) if isinstance(config, str) else int(config)
        rc = gemm_f32_strided_batched_variant(v, c, nb, M, N, K, A.data_ptr(), lda, sa,
                                              B.data_ptr(), ldb, sb, out.data_ptr(), ldc, sc,
                                              s.cuda_stream)
    if rc != GEMM_F32_OK:
        raise GemmError(rc, gemm_f32_last_error())
    return out


def gemm(A, B, out=None, *, variant: int | str | None = None, config: int | str = -1,
         stream=None):
    """``out = A @ B`` for row-major float32 GPU tensors through the C ABI.

    ``variant`` None lets the library choose (gemm_f32); otherwise a variant
    id or name with an optional configuration id or name (gemm_f32_variant).
    Enqueued on ``stream`` (a torch.cuda.Stream), default torch's current
    stream; returns ``out`` without synchronising.
    """
    import torch

    M, K = A.shape
    K2, N = B.shape
    if K != K2:
        raise ValueError(f"shape mismatch {tuple(A.shape)} x {tuple(B.shape)}")
    lda = _row_major_ld(A, "A")
    ldb = _row_major_ld(B, "B")
    if out is None:
        out = torch.empty((M, N), dtype=torch.float32, device=A.device)
    ldc = _row_major_ld(out, "out")
    if tuple(out.shape) != (M, N):
        raise ValueError(f"out has shape {tuple(out.shape)}, expected {(M, N)}")
    s = stream if stream is not None else torch.cuda.current_stream(A.device)
    sp = s.cuda_stream
    if variant is None:
        rc = gemm_f32(M, N, K, A.data_ptr(), lda, B.data_ptr(), ldb, out.data_ptr(), ldc, sp)
    else:
        v = VARIANTS[variant] if isinstance(variant, str) else int(variant)
        c = config_id(v, config) if isinstance(config, str) else int(config)
        rc = gemm_f32_variant(v, c, M, N, K, A.data_ptr(), lda, B.data_ptr(), ldb,
                              out.data_ptr(), ldc, sp)
    if rc != GEMM_F32_OK:
        raise GemmError(rc, gemm_f32_last_error())
    return out
