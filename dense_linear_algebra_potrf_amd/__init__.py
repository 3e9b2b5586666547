"""Python binding for libbatchlas (batched Cholesky potrf / posv on MI355X).

Argument marshalling only: every step of the computation runs in the HIP
kernels of libbatchlas.so, called through its C ABI (include/batchlas.h).
PyTorch provides device memory and the current stream.  There is no fallback:
if the library has not been built, or a call fails, an exception is raised.

Tensor convention: a batch of column-major matrices is a contiguous device
tensor of shape (batch, n, n) whose element [b, c, i] is A_b(i, c) (so t[b]
holds A_b transposed in row-major order), or any contiguous 1-D buffer together
with explicit n / lda / stride / batch.
"""
from __future__ import annotations

import ctypes
import os
import threading

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "_lib", "libbatchlas.so")

DTYPES = {"f32": 0, "f64": 1, "c64": 2, "c128": 3}
UPLO = {"L": 0, "U": 1}
FAMILIES = {"auto": 0, "tiny": 1, "lds": 2, "blocked": 3, "posv_tiny": 4, "posv_split": 5}
FAMILY_NAMES = {v: k for k, v in FAMILIES.items()}
STATUS = {0: "OK", 1: "INVALID_VALUE", 2: "NULL_POINTER", 3: "NOT_SUPPORTED",
          4: "HIP_ERROR", 5: "INTERNAL"}

# every entry point the header declares
EXPORTS = [
    "batchlas_potrf", "batchlas_posv", "batchlas_potrf_family", "batchlas_posv_family",
    "batchlas_spotrf", "batchlas_dpotrf", "batchlas_cpotrf", "batchlas_zpotrf",
    "batchlas_sposv", "batchlas_dposv", "batchlas_cposv", "batchlas_zposv",
    "batchlas_route", "batchlas_status_string", "batchlas_last_error", "batchlas_version",
]


class BatchlasError(RuntimeError):
    def __init__(self, status: int, message: str):
        self.status = status
        self.status_name = STATUS.get(status, str(status))
        super().__init__(f"{self.status_name}: {message}")


class RouteInfo(ctypes.Structure):
    _fields_ = [("family", ctypes.c_int32), ("lanes_per_matrix", ctypes.c_int32),
                ("rows_per_lane", ctypes.c_int32), ("matrices_per_wave", ctypes.c_int32),
                ("block_threads", ctypes.c_int32), ("panel", ctypes.c_int32),
                ("grid", ctypes.c_int64), ("lds_bytes", ctypes.c_int64)]

    def as_dict(self) -> dict:
        d = {f: getattr(self, f) for f, _ in self._fields_}
        d["family"] = FAMILY_NAMES.get(d["family"], d["family"])
        return d


_lib = None
_lock = threading.Lock()


def library_path() -> str:
    return LIB_PATH


def load_library():
    """Load libbatchlas.so (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    with _lock:
        if _lib is not None:
            return _lib
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(
                f"{LIB_PATH} is missing: build it with "
                "`python -m dense_linear_algebra_potrf_amd.build` (or __graft_entry__.build())")
        try:   # share the HIP runtime torch already loaded, if torch is in use
            import torch  # noqa: F401
        except Exception:
            pass
        lib = ctypes.CDLL(LIB_PATH)
        i32, i64, vp = ctypes.c_int32, ctypes.c_int64, ctypes.c_void_p
        lib.batchlas_potrf.argtypes = [i32, i32, i64, vp, i64, i64, i64, vp, vp]
        lib.batchlas_posv.argtypes = [i32, i32, i64, i64, vp, i64, i64, vp, i64, i64, i64, vp, vp]
        lib.batchlas_potrf_family.argtypes = [i32, i32, i32, i64, vp, i64, i64, i64, vp, vp]
        lib.batchlas_posv_family.argtypes = [i32, i32, i32, i64, i64, vp, i64, i64, vp, i64, i64,
                                             i64, vp, vp]
        lib.batchlas_route.argtypes = [i32, i32, i32, i64, i64, i64, i64, i64,
                                       ctypes.POINTER(RouteInfo)]
        for name in ("batchlas_potrf", "batchlas_posv", "batchlas_potrf_family",
                     "batchlas_posv_family", "batchlas_route"):
            getattr(lib, name).restype = i32
        lib.batchlas_status_string.argtypes = [i32]
        lib.batchlas_status_string.restype = ctypes.c_char_p
        lib.batchlas_last_error.argtypes = []
        lib.batchlas_last_error.restype = ctypes.c_char_p
        lib.batchlas_version.argtypes = []
        lib.batchlas_version.restype = i32
        _lib = lib
    return _lib


def _check(status: int):
    if status != 0:
        msg = load_library().batchlas_last_error().decode()
        raise BatchlasError(status, msg)


def _dtype_key(t) -> str:
    import torch
    m = {torch.float32: "f32", torch.float64: "f64", torch.complex64: "c64",
         torch.complex128: "c128"}
    if t.dtype not in m:
        raise TypeError(f"unsupported dtype {t.dtype}")
    return m[t.dtype]


def _stream_ptr(stream) -> int:
    import torch
    s = stream if stream is not None else torch.cuda.current_stream()
    return int(s.cuda_stream)


def _layout(t, n, ld, stride, batch, ncols):
    """Resolve (n, ld, stride, batch) from a tensor and optional overrides."""
    if not t.is_cuda:
        raise ValueError("tensors must live on the GPU")
    if not t.is_contiguous():
        raise ValueError("tensors must be contiguous")
    if t.dim() == 3 and n is None:
        b_, c_, r_ = t.shape
        if ncols is not None and c_ != ncols:
            raise ValueError("shape does not match nrhs")
        n = r_
        ld = r_ if ld is None else ld
        stride = c_ * r_ if stride is None else stride
        batch = b_ if batch is None else batch
    else:
        if n is None or batch is None:
            raise ValueError("a flat buffer needs explicit n and batch")
        cols = n if ncols is None else ncols
        ld = n if ld is None else ld
        stride = ld * cols if stride is None else stride
        if t.numel() < stride * (batch - 1) + ld * (cols - 1) + n:
            raise ValueError("buffer too small for the layout")
    return n, ld, stride, batch


def potrf(A, uplo: str = "L", info=None, *, n=None, lda=None, stride=None, batch=None,
          family: str = "auto", stream=None):
    """Factor a batch in place.  Returns the info tensor (int32[batch], device).

    Pass info=False to request no info output.
    """
    import torch
    lib = load_library()
    dt = _dtype_key(A)
    n, lda, stride, batch = _layout(A, n, lda, stride, batch, None)
    if info is None:
        info = torch.empty(batch, dtype=torch.int32, device=A.device)
    info_ptr = None if info is False else info.data_ptr()
    if info is not False and (info.dtype != torch.int32 or info.numel() < batch or not info.is_cuda):
        raise ValueError("info must be a device int32 tensor with batch entries")
    st = lib.batchlas_potrf_family(FAMILIES[family], DTYPES[dt], UPLO[uplo.upper()[0]], n,
                                   A.data_ptr(), lda, stride, batch, info_ptr, _stream_ptr(stream))
    _check(st)
    return None if info is False else info


def posv(A, B, uplo: str = "L", info=None, *, n=None, nrhs=None, lda=None, strideA=None,
         ldb=None, strideB=None, batch=None, family: str = "auto", stream=None):
    """Factor A and solve A X = B in place (B becomes X).  Returns info."""
    import torch
    lib = load_library()
    dt = _dtype_key(A)
    if _dtype_key(B) != dt:
        raise TypeError("A and B must share a dtype")
    n, lda, strideA, batch = _layout(A, n, lda, strideA, batch, None)
    if nrhs is None:
        if B.dim() != 3:
            raise ValueError("a flat B needs explicit nrhs")
        nrhs = B.shape[1]
    _, ldb, strideB, _ = _layout(B, n if B.dim() != 3 else None, ldb, strideB,
                                 batch if B.dim() != 3 else None, nrhs)
    if info is None:
        info = torch.empty(batch, dtype=torch.int32, device=A.device)
    info_ptr = None if info is False else info.data_ptr()
    st = lib.batchlas_posv_family(FAMILIES[family], DTYPES[dt], UPLO[uplo.upper()[0]], n, nrhs,
                                  A.data_ptr(), lda, strideA, B.data_ptr(), ldb, strideB, batch,
                                  info_ptr, _stream_ptr(stream))
    _check(st)
    return None if info is False else info


def route(dtype: str, uplo: str, n: int, batch: int, nrhs: int = 0, family: str = "auto",
          lda: int | None = None, stride: int | None = None) -> dict:
    """Family and launch geometry a call would use (host-only, no GPU needed)."""
    lib = load_library()
    out = RouteInfo()
    lda = n if lda is None else lda
    stride = lda * n if stride is None else stride
    st = lib.batchlas_route(FAMILIES[family], DTYPES[dtype], UPLO[uplo.upper()[0]], n, nrhs, lda,
                            stride, batch, ctypes.byref(out))
    _check(st)
    return out.as_dict()


def version() -> int:
    return load_library().batchlas_version()
