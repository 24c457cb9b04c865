"""Python binding of the gfx950 dense GEMM library (libdense_gemm.so).

The functions mirror the C ABI in include/dense_gemm.h one to one and only
marshal arguments; every step of the GEMM runs in the library's HIP kernels.
``run_tensors`` is a convenience that reads shapes, leading dimensions, device
pointers and the current stream from torch tensors (torch supplies device
memory and streams only).

Importing this package loads the library; if it has not been built the import
fails loudly (there is no fallback implementation).

One HIP runtime per process: PyTorch's ROCm wheels ship their own copy of
libamdhip64 (same soname as the system one).  Device pointers and streams
only mean something to the runtime that created them, so torch is imported
before the library is loaded; the dynamic linker then binds the library to
the runtime torch already loaded instead of loading a second one.
"""
from __future__ import annotations

import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libdense_gemm.so")

GEMM_OP_N = 0
GEMM_OP_T = 1
GEMM_DTYPE_F32 = 0
GEMM_DTYPE_BF16_F32 = 1
GEMM_DTYPE_BF16_BF16 = 2
GEMM_OK = 0
GEMM_ERR_INVALID_VALUE = 1
GEMM_ERR_NOT_SUPPORTED = 2
GEMM_ERR_HIP = 3
GEMM_ERR_ALLOC = 4
GEMM_ERR_STREAM_K = 5
# bytes of the static stream-K array gemm_run_no_alloc uses on each GPU
GEMM_NO_ALLOC_SCRATCH_BYTES = 16640 + (16 << 20)
GEMM_ACT_NONE = 0
GEMM_ACT_RELU = 1
GEMM_ACT_GELU = 2

# Every function declared in include/dense_gemm.h.
EXPORTS = ("gemm_create", "gemm_destroy", "gemm_run", "gemm_status_string",
           "gemm_variant_count", "gemm_variant_name", "gemm_variant_dtype",
           "gemm_variant_tile", "gemm_set_variant", "gemm_last_variant",
           "gemm_select_variant", "gemm_stream_k_workspace_bytes", "gemm_set_workspace",
           "gemm_set_stream_k", "gemm_last_stream_k", "gemm_run_epilogue",
           "gemm_variant_pipeline", "gemm_variant_occupancy", "gemm_stream_k_status",
           "gemm_set_stream_k_poll_limit", "gemm_run_no_alloc", "gemm_set_planning_model")


class GemmEpilogue(ctypes.Structure):
    """gemm_epilogue_t: bias pointer (0/None for none), activation, clamp flag
    and bounds."""
    _fields_ = [("bias", ctypes.c_void_p), ("activation", ctypes.c_int),
                ("clamp", ctypes.c_int), ("clamp_lo", ctypes.c_float),
                ("clamp_hi", ctypes.c_float)]


class GemmError(RuntimeError):
    def __init__(self, status: int, what: str = "gemm_run"):
        self.status = status
        super().__init__(f"{what} failed: {gemm_status_string(status)}")


def hip_runtimes_loaded():
    """Distinct libamdhip64 files mapped into this process (Linux)."""
    try:
        with open("/proc/self/maps") as f:
            paths = {line.split()[-1] for line in f if "libamdhip64" in line}
    except OSError:
        return []
    return sorted({os.path.realpath(p) for p in paths})


def _load():
    try:  # bind to torch's HIP runtime when torch is present (see module docstring)
        import torch  # noqa: F401
    except ImportError:
        pass
    if not os.path.exists(LIB_PATH):
        raise ImportError(
            f"{LIB_PATH} is missing: build the HIP library first "
            "(python dense_gemm_11_amd/build.py)")
    lib = ctypes.CDLL(LIB_PATH)
    runtimes = hip_runtimes_loaded()
    if len(runtimes) > 1:
        raise ImportError("two HIP runtimes are loaded in this process (" + ", ".join(runtimes)
                          + "); import torch before anything that loads libamdhip64")
    vp, i64, i32, f32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_float
    lib.gemm_create.argtypes = [ctypes.POINTER(vp)]
    lib.gemm_create.restype = i32
    lib.gemm_destroy.argtypes = [vp]
    lib.gemm_destroy.restype = i32
    lib.gemm_run.argtypes = [vp, i32, i32, i64, i64, i64, f32, vp, i64, vp, i64, f32, vp, i64,
                             vp, i64, i32, vp]
    lib.gemm_run.restype = i32
    lib.gemm_run_no_alloc.argtypes = [vp, i32, i32, i64, i64, i64, f32, vp, i64, vp, i64, f32,
                                      vp, i64, vp, i64, i32, vp]
    lib.gemm_run_no_alloc.restype = i32
    lib.gemm_run_epilogue.argtypes = [vp, i32, i32, i64, i64, i64, f32, vp, i64, vp, i64, f32,
                                      vp, i64, vp, i64, i32, ctypes.POINTER(GemmEpilogue), vp]
    lib.gemm_run_epilogue.restype = i32
    lib.gemm_status_string.argtypes = [i32]
    lib.gemm_status_string.restype = ctypes.c_char_p
    lib.gemm_variant_count.argtypes = []
    lib.gemm_variant_count.restype = i32
    lib.gemm_variant_name.argtypes = [i32]
    lib.gemm_variant_name.restype = ctypes.c_char_p
    lib.gemm_variant_dtype.argtypes = [i32]
    lib.gemm_variant_dtype.restype = i32
    lib.gemm_variant_tile.argtypes = [i32, ctypes.POINTER(i32), ctypes.POINTER(i32),
                                      ctypes.POINTER(i32)]
    lib.gemm_variant_tile.restype = i32
    lib.gemm_variant_pipeline.argtypes = [i32, ctypes.POINTER(i32), ctypes.POINTER(i32)]
    lib.gemm_variant_pipeline.restype = i32
    lib.gemm_variant_occupancy.argtypes = [i32]
    lib.gemm_variant_occupancy.restype = i32
    lib.gemm_set_planning_model.argtypes = [i32, ctypes.POINTER(i32), i32]
    lib.gemm_set_planning_model.restype = i32
    lib.gemm_set_variant.argtypes = [vp, i32]
    lib.gemm_set_variant.restype = i32
    lib.gemm_last_variant.argtypes = [vp]
    lib.gemm_last_variant.restype = i32
    lib.gemm_select_variant.argtypes = [i32, i32, i32, i64, i64, i64]
    lib.gemm_select_variant.restype = i32
    lib.gemm_stream_k_workspace_bytes.argtypes = []
    lib.gemm_stream_k_workspace_bytes.restype = ctypes.c_size_t
    lib.gemm_set_workspace.argtypes = [vp, vp, ctypes.c_size_t, vp]
    lib.gemm_set_workspace.restype = i32
    lib.gemm_set_stream_k.argtypes = [vp, i32]
    lib.gemm_set_stream_k.restype = i32
    lib.gemm_last_stream_k.argtypes = [vp]
    lib.gemm_last_stream_k.restype = i32
    lib.gemm_stream_k_status.argtypes = [vp, vp]
    lib.gemm_stream_k_status.restype = i32
    lib.gemm_set_stream_k_poll_limit.argtypes = [vp, i32]
    lib.gemm_set_stream_k_poll_limit.restype = i32
    return lib


lib = _load()


def gemm_create() -> int:
    h = ctypes.c_void_p()
    s = lib.gemm_create(ctypes.byref(h))
    if s != GEMM_OK:
        raise GemmError(s, "gemm_create")
    return h.value


def gemm_destroy(h) -> int:
    return lib.gemm_destroy(h)


def gemm_run(h, transA, transB, M, N, K, alpha, A, lda, B, ldb, beta, C, ldc, D, ldd,
             dtype, stream) -> int:
    """Raw call: pointers and the stream are integers (0/None for NULL)."""
    return lib.gemm_run(h, transA, transB, M, N, K, alpha, A, lda, B, ldb, beta, C, ldc,
                        D, ldd, dtype, stream)


def gemm_run_no_alloc(h, transA, transB, M, N, K, alpha, A, lda, B, ldb, beta, C, ldc, D,
                      ldd, dtype, stream) -> int:
    """Raw call: pointers and the stream are integers (0/None for NULL)."""
    return lib.gemm_run_no_alloc(h, transA, transB, M, N, K, alpha, A, lda, B, ldb, beta, C,
                                 ldc, D, ldd, dtype, stream)


def gemm_run_epilogue(h, transA, transB, M, N, K, alpha, A, lda, B, ldb, beta, C, ldc, D, ldd,
                      dtype, epilogue, stream) -> int:
    """Raw call: pointers and the stream are integers (0/None for NULL);
    epilogue is a GemmEpilogue or None."""
    ep = None if epilogue is None else ctypes.byref(epilogue)
    return lib.gemm_run_epilogue(h, transA, transB, M, N, K, alpha, A, lda, B, ldb, beta, C,
                                 ldc, D, ldd, dtype, ep, stream)


def gemm_status_string(s: int) -> str:
    return lib.gemm_status_string(s).decode()


def gemm_variant_count() -> int:
    return lib.gemm_variant_count()


def gemm_variant_name(i: int):
    n = lib.gemm_variant_name(i)
    return None if n is None else n.decode()


def gemm_variant_dtype(i: int) -> int:
    return lib.gemm_variant_dtype(i)


def gemm_variant_tile(i: int):
    bm, bn, bk = ctypes.c_int(), ctypes.c_int(), ctypes.c_int()
    s = lib.gemm_variant_tile(i, ctypes.byref(bm), ctypes.byref(bn), ctypes.byref(bk))
    if s != GEMM_OK:
        raise GemmError(s, "gemm_variant_tile")
    return bm.value, bn.value, bk.value


def gemm_variant_pipeline(i: int):
    """(stages, ahead) of variant i."""
    st, ah = ctypes.c_int(), ctypes.c_int()
    s = lib.gemm_variant_pipeline(i, ctypes.byref(st), ctypes.byref(ah))
    if s != GEMM_OK:
        raise GemmError(s, "gemm_variant_pipeline")
    return st.value, ah.value


def gemm_variant_occupancy(i: int) -> int:
    return lib.gemm_variant_occupancy(i)


def gemm_set_planning_model(cus: int, occupancy=None) -> int:
    """gemm_set_planning_model: `occupancy` is a sequence of
    gemm_variant_count() workgroups-per-unit figures (0: keep the device
    query), or None (with cus = 0) to clear the model."""
    if occupancy is None:
        return lib.gemm_set_planning_model(cus, None, 0)
    arr = (ctypes.c_int32 * len(occupancy))(*occupancy)
    return lib.gemm_set_planning_model(cus, arr, len(occupancy))


def gemm_set_variant(h, i: int) -> int:
    return lib.gemm_set_variant(h, i)


def gemm_last_variant(h) -> int:
    return lib.gemm_last_variant(h)


def gemm_select_variant(dtype, transA, transB, M, N, K) -> int:
    return lib.gemm_select_variant(dtype, transA, transB, M, N, K)


def gemm_stream_k_workspace_bytes() -> int:
    return lib.gemm_stream_k_workspace_bytes()


def gemm_set_workspace(h, ws, nbytes: int, stream) -> int:
    """Raw call: ws and stream are integers (0/None for NULL)."""
    return lib.gemm_set_workspace(h, ws, nbytes, stream)


def gemm_set_stream_k(h, mode: int) -> int:
    return lib.gemm_set_stream_k(h, mode)


def gemm_last_stream_k(h) -> int:
    return lib.gemm_last_stream_k(h)


def gemm_stream_k_status(h, stream) -> int:
    """Raw call: stream is an integer (0/None for the default stream)."""
    return lib.gemm_stream_k_status(h, stream)


def gemm_set_stream_k_poll_limit(h, polls: int) -> int:
    return lib.gemm_set_stream_k_poll_limit(h, polls)


def attach_workspace(h, nbytes=None, device=None):
    """Allocate a stream-K workspace as a torch uint8 tensor on `device` (the
    current device by default), hand it to h and return it; the caller keeps
    the tensor alive as long as h may use it."""
    import torch

    nbytes = gemm_stream_k_workspace_bytes() if nbytes is None else int(nbytes)
    ws = torch.empty(nbytes, dtype=torch.uint8, device=device or "cuda")
    stream = torch.cuda.current_stream(ws.device).cuda_stream
    s = gemm_set_workspace(h, ws.data_ptr(), nbytes, stream)
    if s != GEMM_OK:
        raise GemmError(s, "gemm_set_workspace")
    return ws


def variants():
    """[(id, name, dtype, (bm, bn, bk))] for every kernel variant."""
    return [(i, gemm_variant_name(i), gemm_variant_dtype(i), gemm_variant_tile(i))
            for i in range(gemm_variant_count())]


def _marshal(h, A, B, D, C, transA, transB, alpha, beta, stream, bias, activation, clamp,
             no_alloc):
    """Check torch tensors and turn them into (C function, argument tuple)."""
    import torch

    def ld(t):
        if t.dim() != 2 or t.stride(1) != 1:
            raise ValueError("expected a 2-D tensor with unit column stride")
        return t.stride(0)

    if A.dtype == torch.float32 and B.dtype == torch.float32:
        dtype = GEMM_DTYPE_F32
    elif A.dtype == torch.bfloat16 and B.dtype == torch.bfloat16:
        dtype = GEMM_DTYPE_BF16_BF16 if D.dtype == torch.bfloat16 else GEMM_DTYPE_BF16_F32
    else:
        raise TypeError("A and B must both be float32 or both bfloat16")
    out = torch.bfloat16 if dtype == GEMM_DTYPE_BF16_BF16 else torch.float32
    if D.dtype != out or (C is not None and C.dtype != out):
        raise TypeError("C and D must be float32, or both bfloat16 with bfloat16 operands")
    M, K = (A.shape[0], A.shape[1]) if transA == "N" else (A.shape[1], A.shape[0])
    Kb, N = (B.shape[0], B.shape[1]) if transB == "N" else (B.shape[1], B.shape[0])
    if Kb != K or tuple(D.shape) != (M, N) or (C is not None and tuple(C.shape) != (M, N)):
        raise ValueError("inconsistent GEMM shapes")
    if bias is not None and (bias.dtype != out or bias.dim() != 1 or bias.shape[0] != N
                             or (N > 1 and bias.stride(0) != 1)):
        raise ValueError("bias must be a contiguous length-N tensor of D's dtype")
    if stream is None:
        stream = torch.cuda.current_stream(D.device).cuda_stream
    args = (h, GEMM_OP_N if transA == "N" else GEMM_OP_T,
            GEMM_OP_N if transB == "N" else GEMM_OP_T, M, N, K, float(alpha),
            A.data_ptr(), ld(A), B.data_ptr(), ld(B), float(beta),
            None if C is None else C.data_ptr(), ld(C) if C is not None else N,
            D.data_ptr(), ld(D), dtype)
    plain = bias is None and activation == GEMM_ACT_NONE and clamp is None
    if no_alloc:
        if not plain:
            raise ValueError("gemm_run_no_alloc has no fused epilogue")
        return lib.gemm_run_no_alloc, args + (stream,)
    if plain:
        return lib.gemm_run, args + (stream,)
    lo, hi = (0.0, 0.0) if clamp is None else clamp
    ep = GemmEpilogue(None if bias is None else bias.data_ptr(), int(activation),
                      int(clamp is not None), float(lo), float(hi))
    return lib.gemm_run_epilogue, args + (ctypes.byref(ep), stream)


def run_tensors(h, A, B, D, C=None, transA="N", transB="N", alpha=1.0, beta=0.0,
                stream=None, check=True, bias=None, activation=GEMM_ACT_NONE,
                clamp=None, no_alloc=False) -> int:
    """gemm_run on torch tensors (row-major 2-D views with unit column stride).

    A: op(A) is M x K (A stored M x K for "N", K x M for "T"); B likewise;
    C, D: M x N.  A and B are float32 (fp32 GEMM) or bfloat16; with bfloat16
    operands, C and D are float32 (GEMM_DTYPE_BF16_F32) or both bfloat16
    (GEMM_DTYPE_BF16_BF16).  bias (a length-N tensor of D's dtype),
    activation (GEMM_ACT_*) and clamp ((lo, hi)) select gemm_run_epilogue;
    no_alloc selects gemm_run_no_alloc.
    """
    fn, args = _marshal(h, A, B, D, C, transA, transB, alpha, beta, stream, bias, activation,
                        clamp, no_alloc)
    s = fn(*args)
    if check and s != GEMM_OK:
        raise GemmError(s)
    return s


def bind_tensors(h, A, B, D, C=None, transA="N", transB="N", alpha=1.0, beta=0.0,
                 stream=None, bias=None, activation=GEMM_ACT_NONE, clamp=None,
                 no_alloc=False):
    """run_tensors' C call with its arguments marshalled once: returns a
    function that makes the same call again and returns its status (for
    timing loops; the tensors must stay alive while it is used)."""
    fn, args = _marshal(h, A, B, D, C, transA, transB, alpha, beta, stream, bias, activation,
                        clamp, no_alloc)
    return lambda: fn(*args)
