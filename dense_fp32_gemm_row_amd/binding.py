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

OP_N = 0  # operand as stored
OP_T = 1  # operand transposed

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
    lib.gemm_f32_ex.restype = _int
    lib.gemm_f32_ex.argtypes = [_int, _int, _int, _int, _i64, _i64, _i64, _i64, _vp, _i64, _i64,
                                _vp, _i64, _i64, _vp, _i64, _i64, _vp]
    lib.gemm_f32_splitk.restype = _int
    lib.gemm_f32_splitk.argtypes = [_int, _int, _i64, _i64, _i64, _i64, _vp, _i64, _vp, _i64, _vp,
                                    _i64, _vp, _i64, _vp]
    lib.gemm_f32_splitk_noalloc.restype = _int
    lib.gemm_f32_splitk_noalloc.argtypes = [_int, _int, _i64, _i64, _i64, _i64, _vp, _i64, _vp,
                                            _i64, _vp, _i64, _vp]
    lib.gemm_f32_splitk_workspace_size.restype = _i64
    lib.gemm_f32_splitk_workspace_size.argtypes = [_i64, _i64, _i64, _i64]
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
    lib.gemm_f32_plan.restype = _int
    lib.gemm_f32_plan.argtypes = [_i64, _i64, _i64, _i64, _i64, _i64, ctypes.POINTER(_int),
                                  ctypes.POINTER(_int), ctypes.POINTER(_i64),
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


def gemm_f32_ex(variant, config_id, opA, opB, batch, M, N, K, A, lda, sA, B, ldb, sB, C, ldc,
                sC, stream=None) -> int:
    return load().gemm_f32_ex(variant, config_id, opA, opB, batch, M, N, K, A, lda, sA, B, ldb,
                              sB, C, ldc, sC, stream)


def gemm_f32_splitk(variant, config_id, splits, M, N, K, A, lda, B, ldb, C, ldc, workspace,
                    workspace_bytes, stream=None) -> int:
    return load().gemm_f32_splitk(variant, config_id, splits, M, N, K, A, lda, B, ldb, C, ldc,
                                  workspace, workspace_bytes, stream)


def gemm_f32_splitk_noalloc(variant, config_id, splits, M, N, K, A, lda, B, ldb, C, ldc,
                            stream=None) -> int:
    return load().gemm_f32_splitk_noalloc(variant, config_id, splits, M, N, K, A, lda, B, ldb, C,
                                          ldc, stream)


SPLITK_SCRATCH_BYTES = 33554432  # GEMM_F32_SPLITK_SCRATCH_BYTES


def gemm_f32_splitk_workspace_size(M, N, K, splits) -> int:
    return load().gemm_f32_splitk_workspace_size(M, N, K, splits)


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


def gemm_f32_plan(M, N, K, lda, ldb, ldc) -> dict:
    """How gemm_f32 runs one product: {"parts", "axis", "split", "configs": [(variant,
    config_id), ...]} with one entry per launch."""
    parts, axis, split = _int(), _int(), _i64()
    v, c = (_int * 2)(), (_int * 2)()
    rc = load().gemm_f32_plan(M, N, K, lda, ldb, ldc, ctypes.byref(parts), ctypes.byref(axis),
                              ctypes.byref(split), v, c)
    if rc != GEMM_F32_OK:
        raise GemmError(rc, gemm_f32_last_error())
    return {"parts": parts.value, "axis": axis.value, "split": split.value,
            "configs": [(v[i], c[i]) for i in range(parts.value)]}


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

def _operand(t, name: str, dims: int) -> tuple[int, int, int]:
    """(op, leading dimension, batch stride) of a float32 GPU tensor holding
    one (dims = 2) or a batch (dims = 3) of matrices.  A row-major matrix is
    OP_N with ld = stride of its rows; a transposed view of a row-major
    matrix (unit stride down the columns, e.g. ``X.T``) is OP_T with ld = the
    stored row stride.  A batch stride of 0 (expanded tensor) is allowed."""
    import torch

    if t.dtype != torch.float32 or t.dim() != dims or not t.is_cuda:
        raise TypeError(f"{name} must be a {dims}-D float32 GPU tensor")
    rows, cols = t.shape[-2], t.shape[-1]
    rs, cs = t.stride(-2), t.stride(-1)
    bs = t.stride(0) if dims == 3 else 0
    if cols <= 1 or cs == 1:
        return OP_N, (rs if rows > 1 else max(cols, 1)), bs
    if rows <= 1 or rs == 1:
        return OP_T, (cs if cols > 1 else max(rows, 1)), bs
    raise ValueError(f"{name} must be row-major or a transposed view of a row-major matrix")


def _marshal(A, B, out, variant, config, stream, batched: bool):
    """Checks the operands and returns (C entry point name, its arguments,
    out) for out = A @ B."""
    import torch

    dims = 3 if batched else 2
    nb = A.shape[0] if batched else 1
    M, K = A.shape[-2], A.shape[-1]
    K2, N = B.shape[-2], B.shape[-1]
    if K != K2 or (batched and B.shape[0] != nb):
        raise ValueError(f"shape mismatch {tuple(A.shape)} x {tuple(B.shape)}")
    opa, lda, sa = _operand(A, "A", dims)
    opb, ldb, sb = _operand(B, "B", dims)
    shape = (nb, M, N) if batched else (M, N)
    if out is None:
        out = torch.empty(shape, dtype=torch.float32, device=A.device)
    if tuple(out.shape) != shape:
        raise ValueError(f"out has shape {tuple(out.shape)}, expected {shape}")
    opc, ldc, sc = _operand(out, "out", dims)
    if opc != OP_N:
        raise ValueError("out must be row-major")
    sp = (stream if stream is not None else torch.cuda.current_stream(A.device)).cuda_stream
    if variant is None:
        v, c = -1, -1
    else:
        v = VARIANTS[variant] if isinstance(variant, str) else int(variant)
        c = config_id(v, config) if isinstance(config, str) else int(config)
    a, b, cp = A.data_ptr(), B.data_ptr(), out.data_ptr()
    if opa == OP_N and opb == OP_N and not batched:
        if v == -1:
            return "gemm_f32", (M, N, K, a, lda, b, ldb, cp, ldc, sp), out
        return "gemm_f32_variant", (v, c, M, N, K, a, lda, b, ldb, cp, ldc, sp), out
    if opa == OP_N and opb == OP_N:
        if v == -1:
            return ("gemm_f32_strided_batched",
                    (nb, M, N, K, a, lda, sa, b, ldb, sb, cp, ldc, sc, sp), out)
        return ("gemm_f32_strided_batched_variant",
                (v, c, nb, M, N, K, a, lda, sa, b, ldb, sb, cp, ldc, sc, sp), out)
    return ("gemm_f32_ex",
            (v, c, opa, opb, nb, M, N, K, a, lda, sa, b, ldb, sb, cp, ldc, sc, sp), out)


def _call(A, B, out, variant, config, stream, batched: bool):
    name, args, out = _marshal(A, B, out, variant, config, stream, batched)
    rc = getattr(load(), name)(*args)
    if rc != GEMM_F32_OK:
        raise GemmError(rc, gemm_f32_last_error())
    return out


def prepare(A, B, out, *, variant: int | str | None = None, config: int | str = -1,
            stream=None, batched: bool = False):
    """A callable with no arguments that enqueues ``out = A @ B`` (as gemm,
    or gemm_batched when ``batched``), with the operands checked and the C
    arguments built once: for launch loops, where the per-call checks of
    gemm would cost more host time than a small product takes on the GPU.
    The callable holds references to A, B and out, so their memory stays
    allocated while it exists; they must not be resized or re-strided."""
    name, args, _ = _marshal(A, B, out, variant, config, stream, batched)
    fn = getattr(load(), name)

    def launch():
        rc = fn(*args)
        if rc != GEMM_F32_OK:
            raise GemmError(rc, gemm_f32_last_error())

    launch.operands = (A, B, out)  # the raw addresses in args point into these
    return launch


def gemm(A, B, out=None, *, variant: int | str | None = None, config: int | str = -1,
         stream=None):
    """``out = A @ B`` for 2-D float32 GPU tensors through the C ABI.

    A and B may be row-major or transposed views of row-major matrices
    (``X.T``); ``out`` is row-major.  ``variant`` None lets the library
    choose; otherwise a variant id or name with an optional configuration
    id or name.  Enqueued on ``stream`` (a torch.cuda.Stream), default
    torch's current stream; returns ``out`` without synchronising.
    """
    return _call(A, B, out, variant, config, stream, batched=False)


def gemm_splitk(A, B, splits: int, out=None, workspace=None, *, variant: int | str | None = None,
                config: int | str = -1, stream=None, noalloc: bool = False):
    """``out = A @ B`` as `splits` partial products over K plus a fixed-order
    reduction (gemm_f32_splitk).  ``workspace`` is a float32 GPU tensor of at
    least gemm_f32_splitk_workspace_size bytes; allocated here when None.
    With ``noalloc`` the call goes to gemm_f32_splitk_noalloc, whose partial
    products use the library's static scratch (no workspace; ``out`` must be
    given, so that nothing is allocated)."""
    import torch

    if noalloc and (workspace is not None or out is None):
        raise ValueError("noalloc takes an out tensor and no workspace")

    M, K = A.shape
    K2, N = B.shape
    if K != K2:
        raise ValueError(f"shape mismatch {tuple(A.shape)} x {tuple(B.shape)}")
    opa, lda, _ = _operand(A, "A", 2)
    opb, ldb, _ = _operand(B, "B", 2)
    if opa != OP_N or opb != OP_N:
        raise ValueError("gemm_splitk takes row-major operands")
    if out is None:
        out = torch.empty((M, N), dtype=torch.float32, device=A.device)
    opc, ldc, _ = _operand(out, "out", 2)
    need = 0 if noalloc else gemm_f32_splitk_workspace_size(M, N, K, splits)
    if workspace is None and need:
        workspace = torch.empty(need // 4, dtype=torch.float32, device=A.device)
    wptr = workspace.data_ptr() if workspace is not None else None
    wbytes = workspace.numel() * 4 if workspace is not None else 0
    sp = (stream if stream is not None else torch.cuda.current_stream(A.device)).cuda_stream
    if variant is None:
        v, c = -1, -1
    else:
        v = VARIANTS[variant] if isinstance(variant, str) else int(variant)
        c = config_id(v, config) if isinstance(config, str) else int(config)
    if noalloc:
        rc = gemm_f32_splitk_noalloc(v, c, splits, M, N, K, A.data_ptr(), lda, B.data_ptr(), ldb,
                                     out.data_ptr(), ldc, sp)
    else:
        rc = gemm_f32_splitk(v, c, splits, M, N, K, A.data_ptr(), lda, B.data_ptr(), ldb,
                             out.data_ptr(), ldc, wptr, wbytes, sp)
    if rc != GEMM_F32_OK:
        raise GemmError(rc, gemm_f32_last_error())
    return out


def gemm_batched(A, B, out=None, *, variant: int | str | None = None, config: int | str = -1,
                 stream=None):
    """``out[b] = A[b] @ B[b]`` for 3-D float32 GPU tensors (strided batch;
    A or B may be an expanded tensor with batch stride 0, and either may be
    a batch of transposed views)."""
    return _call(A, B, out, variant, config, stream, batched=True)
