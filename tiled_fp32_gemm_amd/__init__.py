"""Python binding of the gfx950 SGEMM library (``include/sgemm.h``).

The functions ``sgemm``, ``sgemm_ex``, ``sgemm_ws``, ``sgemm_ws_noalloc``,
``sgemm_workspace_bytes``, ``sgemm_plan_query``, ``sgemm_plan_query_ws``,
``sgemm_transpose``, ``sgemm_transpose_ex``, ``sgemm_ladder*``,
``sgemm_status_string`` and ``sgemm_version`` have the C names and arguments
(device pointers as integers, a HIP stream handle as an integer) and only
marshal arguments: every step of the product runs in the HIP kernels.
``matmul`` is a convenience over torch tensors that derives the leading
dimensions and the stream and calls ``sgemm_ex``.

There is no fallback: if ``libsgemm.so`` has not been built, or does not load,
importing the binding's functions raises.  Build it with
``python -m tiled_fp32_gemm_amd.build``.

torch is imported before the library is loaded so that both bind to the one
HIP runtime torch ships (same SONAME), and torch's stream handles are valid in
the library.
"""
from __future__ import annotations

import ctypes
import os

__all__ = ["sgemm", "sgemm_ex", "sgemm_plan_query", "sgemm_status_string",
           "sgemm_version", "matmul", "library_path", "load", "SgemmPlan",
           "SgemmError", "ALGOS", "OK", "ERR_INVALID_ARG", "ERR_UNSUPPORTED",
           "ERR_LAUNCH", "EXPORTED_SYMBOLS", "sgemm_transpose",
           "sgemm_transpose_ex", "transpose", "TRANSPOSE_LAYOUTS",
           "sgemm_ladder", "sgemm_ladder_steps", "sgemm_ladder_name",
           "ladder_steps", "sgemm_ws", "sgemm_workspace_bytes",
           "sgemm_plan_query_ws", "sgemm_ws_noalloc", "ERR_SCRATCH_LIMIT",
           "NOALLOC_MAX_BYTES"]

OK, ERR_INVALID_ARG, ERR_UNSUPPORTED, ERR_LAUNCH, ERR_SCRATCH_LIMIT = 0, 1, 2, 3, 4
NOALLOC_MAX_BYTES = 32 << 20   # SGEMM_NOALLOC_MAX_BYTES
ALGOS = {"auto": 0, "simple": 1, "fma": 2, "mfma": 3, "mfma_direct": 4}
EXPORTED_SYMBOLS = ("sgemm", "sgemm_ex", "sgemm_plan_query",
                    "sgemm_transpose", "sgemm_transpose_ex",
                    "sgemm_status_string", "sgemm_version",
                    "sgemm_ladder_steps", "sgemm_ladder_name", "sgemm_ladder",
                    "sgemm_ws", "sgemm_workspace_bytes", "sgemm_plan_query_ws",
                    "sgemm_ws_noalloc")
TRANSPOSE_LAYOUTS = {"auto": 0, "naive": 1, "padded": 2, "swizzled": 3}

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "libsgemm.so")
_lib = None


class SgemmError(RuntimeError):
    def __init__(self, status: int, what: str = ""):
        self.status = status
        msg = sgemm_status_string(status)
        super().__init__(f"{what}: {msg} (status {status})" if what else msg)


class SgemmPlan(ctypes.Structure):
    _fields_ = [("algo", ctypes.c_int), ("tile_m", ctypes.c_int),
                ("tile_n", ctypes.c_int), ("tile_k", ctypes.c_int),
                ("threads", ctypes.c_int), ("vec_a", ctypes.c_int),
                ("vec_b", ctypes.c_int), ("workgroups", ctypes.c_int64),
                ("lds_bytes", ctypes.c_int), ("wg_per_cu", ctypes.c_int),
                ("splits", ctypes.c_int), ("workspace_bytes", ctypes.c_int64),
                ("kernel", ctypes.c_char * 64)]

    def as_dict(self) -> dict:
        d = {f: getattr(self, f) for f, _ in self._fields_}
        d["kernel"] = self.kernel.decode()
        return d


def library_path() -> str:
    return _LIB_PATH


def load():
    """The ctypes handle on ``libsgemm.so`` (loaded once, prototypes set)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        raise ImportError(
            f"{_LIB_PATH} is missing: build the HIP library with "
            "`python -m tiled_fp32_gemm_amd.build` (there is no CPU fallback)")
    import torch  # noqa: F401  (binds the HIP runtime first; see module doc)
    lib = ctypes.CDLL(_LIB_PATH)
    i64, fp, i32 = ctypes.c_int64, ctypes.c_void_p, ctypes.c_int
    common = [i64, i64, i64, fp, i64, fp, i64, fp, i64]
    lib.sgemm.argtypes = common + [fp]
    lib.sgemm.restype = i32
    lib.sgemm_ex.argtypes = common + [fp, i32]
    lib.sgemm_ex.restype = i32
    lib.sgemm_plan_query.argtypes = common + [i32, ctypes.POINTER(SgemmPlan)]
    lib.sgemm_plan_query.restype = i32
    tr = [i64, i64, fp, i64, fp, i64, fp]
    lib.sgemm_transpose.argtypes = tr
    lib.sgemm_transpose.restype = i32
    lib.sgemm_transpose_ex.argtypes = tr + [i32]
    lib.sgemm_transpose_ex.restype = i32
    lib.sgemm_status_string.argtypes = [i32]
    lib.sgemm_status_string.restype = ctypes.c_char_p
    lib.sgemm_version.argtypes = []
    lib.sgemm_version.restype = i32
    lib.sgemm_ladder_steps.argtypes = []
    lib.sgemm_ladder_steps.restype = i32
    lib.sgemm_ladder_name.argtypes = [i32]
    lib.sgemm_ladder_name.restype = ctypes.c_char_p
    lib.sgemm_ladder.argtypes = [i32] + common + [fp]
    lib.sgemm_ladder.restype = i32
    lib.sgemm_ws.argtypes = common + [fp, fp, i64]
    lib.sgemm_ws.restype = i32
    lib.sgemm_ws_noalloc.argtypes = common + [fp, i64]
    lib.sgemm_ws_noalloc.restype = i32
    lib.sgemm_workspace_bytes.argtypes = [i64, i64, i64]
    lib.sgemm_workspace_bytes.restype = i64
    lib.sgemm_plan_query_ws.argtypes = common + [i64, ctypes.POINTER(SgemmPlan)]
    lib.sgemm_plan_query_ws.restype = i32
    _lib = lib
    return lib


def sgemm(M, N, K, A, lda, B, ldb, C, ldc, stream=0) -> int:
    """C = A·B on ``stream``; returns the status code (see the C header)."""
    return load().sgemm(M, N, K, A, lda, B, ldb, C, ldc, stream)


def sgemm_ex(M, N, K, A, lda, B, ldb, C, ldc, stream=0, algo=0) -> int:
    """``sgemm`` with an explicit kernel family (``ALGOS`` value)."""
    return load().sgemm_ex(M, N, K, A, lda, B, ldb, C, ldc, stream, algo)


def sgemm_plan_query(M, N, K, A, lda, B, ldb, C, ldc, algo=0):
    """``(status, SgemmPlan)`` for what a call would launch."""
    plan = SgemmPlan()
    st = load().sgemm_plan_query(M, N, K, A, lda, B, ldb, C, ldc, algo,
                                 ctypes.byref(plan))
    return st, plan


def sgemm_ws(M, N, K, A, lda, B, ldb, C, ldc, stream=0, workspace=0,
             workspace_bytes=0) -> int:
    """``sgemm`` that may split K across workgroups into ``workspace``."""
    return load().sgemm_ws(M, N, K, A, lda, B, ldb, C, ldc, stream, workspace,
                           workspace_bytes)


def sgemm_ws_noalloc(M, N, K, A, lda, B, ldb, C, ldc, stream=0,
                     workspace_bytes=0) -> int:
    """``sgemm_ws`` over the library's static scratch (no allocation)."""
    return load().sgemm_ws_noalloc(M, N, K, A, lda, B, ldb, C, ldc, stream,
                                   workspace_bytes)


def sgemm_workspace_bytes(M, N, K) -> int:
    """Workspace bytes for ``sgemm_ws``'s fastest plan (0: no split)."""
    return load().sgemm_workspace_bytes(M, N, K)


def sgemm_plan_query_ws(M, N, K, A, lda, B, ldb, C, ldc, workspace_bytes=0):
    """``(status, SgemmPlan)`` for what ``sgemm_ws`` would launch."""
    plan = SgemmPlan()
    st = load().sgemm_plan_query_ws(M, N, K, A, lda, B, ldb, C, ldc,
                                    workspace_bytes, ctypes.byref(plan))
    return st, plan


def sgemm_transpose(rows, cols, inp, ldi, out, ldo, stream=0) -> int:
    """out = inp^T (rows x cols -> cols x rows); returns the status code."""
    return load().sgemm_transpose(rows, cols, inp, ldi, out, ldo, stream)


def sgemm_transpose_ex(rows, cols, inp, ldi, out, ldo, stream=0, layout=0) -> int:
    """``sgemm_transpose`` with an explicit LDS layout (``TRANSPOSE_LAYOUTS``)."""
    return load().sgemm_transpose_ex(rows, cols, inp, ldi, out, ldo, stream,
                                     layout)


def transpose(A, out=None, layout: str | int = "auto", stream=None):
    """``out = A.T`` for a float32 GPU tensor (row-major, any row stride)."""
    import torch
    if A.dtype != torch.float32 or A.device.type != "cuda" or A.dim() != 2:
        raise ValueError("A must be a 2-D float32 GPU tensor")
    rows, cols = A.shape
    if out is None:
        out = torch.empty((cols, rows), dtype=torch.float32, device=A.device)
    if tuple(out.shape) != (cols, rows) or out.dtype != torch.float32:
        raise ValueError("out must be a float32 tensor of shape A.T")
    code = TRANSPOSE_LAYOUTS[layout] if isinstance(layout, str) else int(layout)
    s = torch.cuda.current_stream(A.device) if stream is None else stream
    st = sgemm_transpose_ex(rows, cols, A.data_ptr(), _ld(A, "A"),
                            out.data_ptr(), _ld(out, "out"), s.cuda_stream, code)
    if st != OK:
        raise SgemmError(st, "sgemm_transpose_ex")
    return out


def sgemm_ladder_steps() -> int:
    return load().sgemm_ladder_steps()


def sgemm_ladder_name(step: int) -> str | None:
    name = load().sgemm_ladder_name(step)
    return None if name is None else name.decode()


def sgemm_ladder(step, M, N, K, A, lda, B, ldb, C, ldc, stream=0) -> int:
    """Ablation ladder step ``step`` of C = A·B; returns the status code."""
    return load().sgemm_ladder(step, M, N, K, A, lda, B, ldb, C, ldc, stream)


def ladder_steps() -> list[str]:
    """Names of the ablation ladder's steps, in order."""
    return [sgemm_ladder_name(i) for i in range(sgemm_ladder_steps())]


def sgemm_status_string(status: int) -> str:
    return load().sgemm_status_string(status).decode()


def sgemm_version() -> int:
    return load().sgemm_version()


def _ld(t, name: str) -> int:
    if t.dim() != 2:
        raise ValueError(f"{name} must be 2-D")
    if t.size(1) > 1 and t.stride(1) != 1:
        raise ValueError(f"{name} must have unit column stride (row-major)")
    return t.stride(0) if t.size(0) > 1 else max(t.size(1), 1)


def _args(A, B, out):
    import torch
    for name, t in (("A", A), ("B", B), ("out", out)):
        if t.dtype != torch.float32:
            raise ValueError(f"{name} must be float32")
        if t.device.type != "cuda":
            raise ValueError(f"{name} must be on a GPU")
    if not (A.device == B.device == out.device):
        raise ValueError("A, B and out must be on the same device")
    M, K = A.shape
    K2, N = B.shape
    if K2 != K or tuple(out.shape) != (M, N):
        raise ValueError(f"shape mismatch: {tuple(A.shape)} x {tuple(B.shape)}"
                         f" -> {tuple(out.shape)}")
    return M, N, K, _ld(A, "A"), _ld(B, "B"), _ld(out, "out")


def matmul(A, B, out=None, algo: str | int = "auto", stream=None, workspace=None):
    """``out = A @ B`` for float32 GPU tensors (row-major, any row stride).

    The product runs in the library's kernels on ``stream`` (a
    ``torch.cuda.Stream``; default: the current stream).  With
    ``workspace`` (a GPU tensor on the same device, contiguous; its bytes
    are the room given, see ``sgemm_workspace_bytes``) the call goes through
    ``sgemm_ws`` and may split K across workgroups; ``algo`` must then be
    "auto".  Raises ``ValueError`` on bad tensors and ``SgemmError`` on a
    library error.
    """
    import torch
    if out is None:
        out = torch.empty((A.shape[0], B.shape[1]), dtype=torch.float32,
                          device=A.device)
    M, N, K, lda, ldb, ldc = _args(A, B, out)
    code = ALGOS[algo] if isinstance(algo, str) else int(algo)
    s = torch.cuda.current_stream(A.device) if stream is None else stream
    if workspace is not None:
        if code != ALGOS["auto"]:
            raise ValueError("a workspace is used by the auto plan only")
        if not workspace.is_cuda or workspace.device != A.device or not workspace.is_contiguous():
            raise ValueError("workspace must be a contiguous tensor on A's device")
        nbytes = workspace.numel() * workspace.element_size()
        with torch.cuda.device(A.device):
            st = sgemm_ws(M, N, K, A.data_ptr(), lda, B.data_ptr(), ldb,
                          out.data_ptr(), ldc, s.cuda_stream, workspace.data_ptr(), nbytes)
        if st != OK:
            raise SgemmError(st, "sgemm_ws")
        return out
    with torch.cuda.device(A.device):
        st = sgemm_ex(M, N, K, A.data_ptr(), lda, B.data_ptr(), ldb,
                      out.data_ptr(), ldc, s.cuda_stream, code)
    if st != OK:
        raise SgemmError(st, "sgemm_ex")
    return out


def plan(A, B, out=None, algo: str | int = "auto") -> dict:
    """The launch ``matmul`` would make for these tensors, as a dict."""
    import torch
    if out is None:
        out = torch.empty((A.shape[0], B.shape[1]), dtype=torch.float32,
                          device=A.device)
    M, N, K, lda, ldb, ldc = _args(A, B, out)
    code = ALGOS[algo] if isinstance(algo, str) else int(algo)
    st, p = sgemm_plan_query(M, N, K, A.data_ptr(), lda, B.data_ptr(), ldb,
                             out.data_ptr(), ldc, code)
    if st != OK:
        raise SgemmError(st, "sgemm_plan_query")
    return p.as_dict()
