"""ctypes binding of ``libdense_gemm.so`` (the C ABI in include/dense_gemm.h).

Argument marshalling only: every step of the product runs in the library's
HIP kernels.  Tensors are passed as raw device pointers with their leading
dimensions, on the caller's current HIP stream (``torch.cuda`` is HIP on
ROCm builds of PyTorch).  There is no fallback: if the library is missing or a
call fails, a :class:`DenseGemmError` is raised.
"""
from __future__ import annotations

import ctypes
import enum
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIBNAME = "libdense_gemm.so"


class Status(enum.IntEnum):
    OK = 0
    INVALID_DIM = 1
    NULL_PTR = 2
    BAD_LD = 3
    MISALIGNED = 4
    TOO_LARGE = 5
    LAUNCH_FAILED = 6
    NO_DEVICE = 7
    BAD_ARG = 8
    NO_MEMORY = 9
    WORKSPACE_TOO_SMALL = 10
    SCRATCH_TOO_SMALL = 11


# dense_gemm_op: the type and layout pairings of dense_gemm_ex
OPS = {("nt", "f16"): 0, ("nn", "bf16"): 1, ("nt", "bf16"): 2, ("nn", "f16"): 3}


class Options(ctypes.Structure):
    """dense_gemm_options: split_k (0 = the library's choice, 1 = none,
    n = n parts) and tile_n (0 = the library's choice, 128 or 256)."""
    _fields_ = [("split_k", ctypes.c_int32), ("tile_n", ctypes.c_int32)]


class DenseGemmError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = Status(status) if status in Status._value2member_map_ else status
        super().__init__("%s failed: %s (%d)" % (where, _status_string(status), int(status)))


_lib = None

# Every symbol the header declares, with its ctypes signature.
_i64 = ctypes.c_int64
_i32 = ctypes.c_int
_vp = ctypes.c_void_p
_GEMM_ARGS = [_i64, _i64, _i64, _vp, _i64, _vp, _i64, _vp, _i64, _vp]
SIGNATURES = {
    "gemm_nt_f16": (_GEMM_ARGS, _i32),
    "gemm_nn_bf16": (_GEMM_ARGS, _i32),
    "gemm_nt_bf16": (_GEMM_ARGS, _i32),
    "gemm_nn_f16": (_GEMM_ARGS, _i32),
    "gemm_nt_f16_ladder": ([_i32] + _GEMM_ARGS, _i32),
    "gemm_nt_e4m3_mx": ([_i64, _i64, _i64, _vp, _i64, _vp, _i64, _vp, _i64, _vp, _i64, _vp, _i64,
                         _vp], _i32),
    "dense_gemm_status_string": ([_i32], ctypes.c_char_p),
    "dense_gemm_validate": ([_i32, _i64, _i64, _i64, _vp, _i64, _vp, _i64, _vp, _i64], _i32),
    "dense_gemm_tile_of_task": ([_i64, _i64, _i64, _i64, ctypes.POINTER(_i64),
                                 ctypes.POINTER(_i64)], _i32),
    "dense_gemm_xcd_slot": ([_i64, _i64, _i64], _i64),
    "dense_gemm_plan": ([_i32, _i64, _i64, _i64, _i64, ctypes.POINTER(_i64)], _i32),
    "dense_gemm_workspace_size": ([_i32, _i64, _i64, _i64, _vp, _i64, _vp, _i64, _i64,
                                   ctypes.POINTER(Options), ctypes.POINTER(ctypes.c_size_t)], _i32),
    "dense_gemm_ex": ([_i32] + _GEMM_ARGS[:-1] + [ctypes.POINTER(Options), _vp, ctypes.c_size_t,
                                                 _vp], _i32),
    "gemm_nt_f16_noalloc": (_GEMM_ARGS, _i32),
    "gemm_nt_e4m3_mx_workspace_size": ([_i64, _i64, _i64, _i64, ctypes.POINTER(ctypes.c_size_t)],
                                       _i32),
    "gemm_nt_e4m3_mx_plan": ([_i64, _i64, _i64, _i64, ctypes.POINTER(_i64)], _i32),
    "gemm_nt_e4m3_mx_ex": ([_i64, _i64, _i64, _vp, _i64, _vp, _i64, _vp, _i64, _vp, _i64, _vp,
                            _i64, _vp, ctypes.c_size_t, _vp], _i32),
}


def library_path() -> str:
    return os.environ.get("DENSE_GEMM_LIB", os.path.join(_HERE, _LIBNAME))


def load_library():
    """Load the HIP library once; raise if it has not been built.

    PyTorch is imported first when it is installed: it carries its own copy
    of the HIP runtime (and of the HSA runtime below it) under the same
    soname the library links against (libamdhip64.so.7), so with torch
    loaded the dynamic linker binds the library to that copy, and tensors,
    streams and the library's launches share one runtime.  Loaded the other
    way round, the process would map two HIP runtimes, and the library's
    calls would not see the device state torch set up (measured: the first
    call then fails with DENSE_GEMM_NO_DEVICE)."""
    global _lib
    if _lib is not None:
        return _lib
    try:
        import torch  # noqa: F401  (the runtime the library must bind to)
    except ImportError:
        pass
    path = library_path()
    if not os.path.exists(path):
        raise FileNotFoundError(
            "HIP library %s is not built; run `python -c 'import __graft_entry__ as g; g.build()'`"
            % path)
    lib = ctypes.CDLL(path)
    for name, (args, res) in SIGNATURES.items():
        fn = getattr(lib, name)
        fn.argtypes = args
        fn.restype = res
    _lib = lib
    return lib


def _status_string(status: int) -> str:
    try:
        return load_library().dense_gemm_status_string(int(status)).decode()
    except Exception:  # library unavailable: fall back to the enum name
        try:
            return Status(status).name
        except ValueError:
            return "unknown status"


def _stream_handle(stream, device) -> int:
    """The HIP stream handle: ``stream`` itself, or the current stream of
    ``device`` when it is None."""
    if stream is None:
        import torch
        return torch.cuda.current_stream(device).cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _stream_object(stream, device):
    """The torch stream object of a launch stream given as a torch stream or
    a raw HIP stream handle."""
    import torch
    if isinstance(stream, int):
        return torch.cuda.ExternalStream(stream, device=device)
    return stream


def _used_by(t, stream, device):
    """Mark a tensor from torch's caching allocator as in use by the launch
    stream when that is not the current stream (an explicit ``stream``):
    torch ties each block to the stream it was allocated on, so without the
    mark a block dropped (or freed by the caller) while the call's kernels
    still run on the other stream could be handed to a new allocation on
    the current stream and overwritten under them."""
    if stream is not None:
        t.record_stream(_stream_object(stream, device))
    return t


def _ld(t) -> int:
    """Leading dimension (elements between rows) of a 2-D tensor with unit
    column stride.  A single row may carry any row stride (a transposed
    column, an expanded view): its leading dimension is then its width."""
    return t.stride(0) if t.shape[0] > 1 else max(t.shape[1], 1)


def _same_device(*ts):
    dev = ts[0].device
    for t in ts[1:]:
        if t.device != dev:
            raise ValueError("operands on different devices: %s and %s" % (dev, t.device))
    return dev


def _check_tensor(t, dtype_name: str, what: str):
    import torch
    want = torch.float16 if dtype_name == "f16" else torch.bfloat16
    if t.dtype != want:
        raise TypeError("%s must be %s, got %s" % (what, want, t.dtype))
    if not t.is_cuda:
        raise ValueError("%s must be a device tensor" % what)
    if t.dim() != 2 or (t.stride(1) != 1 and t.shape[1] > 1):
        raise ValueError("%s must be 2-D with unit column stride" % what)


def workspace_size(layout: str, fmt: str, M: int, N: int, K: int, A_ptr: int, lda: int,
                   B_ptr: int, ldb: int, options: Options | None = None, num_cus: int = 0) -> int:
    """Bytes of workspace dense_gemm_ex needs (dense_gemm_workspace_size)."""
    lib = load_library()
    out = ctypes.c_size_t()
    st = lib.dense_gemm_workspace_size(OPS[(layout, fmt)], M, N, K, A_ptr, lda, B_ptr, ldb,
                                       num_cus, ctypes.byref(options) if options else None,
                                       ctypes.byref(out))
    if st != Status.OK:
        raise DenseGemmError(st, "dense_gemm_workspace_size")
    return out.value


def _call(name: str, layout: str, fmt: str, A, B, D=None, stream=None, workspace=None):
    """D = A @ B.T (layout "nt", B is N x K) or D = A @ B ("nn", B is K x N).
    With ``workspace`` (a device tensor, or True to take one from torch's
    allocator), the call goes through dense_gemm_ex with that workspace.
    The call is asynchronous on ``stream`` (None: the current stream).  A
    workspace or D passed in stays the caller's to keep alive until the
    call's kernels finish; the ones this function allocates are marked as in
    use by ``stream``."""
    import torch
    lib = load_library()
    _check_tensor(A, fmt, "A")
    _check_tensor(B, fmt, "B")
    M, K = A.shape
    if layout == "nt":
        N, Kb = B.shape
    else:
        Kb, N = B.shape
    if Kb != K:
        raise ValueError("inner dimensions differ: A is %s, B is %s" % (tuple(A.shape), tuple(B.shape)))
    own_d = D is None
    if own_d:
        D = torch.empty((M, N), dtype=A.dtype, device=A.device)
    else:
        _check_tensor(D, fmt, "D")
        if D.shape[0] != M or D.shape[1] != N:
            raise ValueError("D has shape %s, expected (%d, %d)" % (tuple(D.shape), M, N))
    dev = _same_device(A, B, D)
    if own_d:
        _used_by(D, stream, dev)
    # the library launches on the current device
    with torch.cuda.device(dev):
        if workspace is None:
            st = getattr(lib, name)(M, N, K, A.data_ptr(), _ld(A), B.data_ptr(), _ld(B),
                                    D.data_ptr(), _ld(D), _stream_handle(stream, dev))
        else:
            if workspace is True:
                need = workspace_size(layout, fmt, M, N, K, A.data_ptr(), _ld(A), B.data_ptr(),
                                      _ld(B))
                workspace = _used_by(torch.empty(max(need, 1), dtype=torch.uint8, device=dev),
                                     stream, dev)
            if not workspace.is_cuda or workspace.device != dev:
                raise ValueError("workspace must be a device tensor on %s" % dev)
            st = lib.dense_gemm_ex(OPS[(layout, fmt)], M, N, K, A.data_ptr(), _ld(A),
                                   B.data_ptr(), _ld(B), D.data_ptr(), _ld(D), None,
                                   workspace.data_ptr(), workspace.numel() * workspace.element_size(),
                                   _stream_handle(stream, dev))
            name = "dense_gemm_ex"
    if st != Status.OK:
        raise DenseGemmError(st, name)
    return D


def gemm_nt_f16(A, B, D=None, stream=None, workspace=None):
    """D = A @ B.T in FP16 (FP32 accumulation); A is M x K, B is N x K.
    ``workspace``: see :func:`_call`."""
    return _call("gemm_nt_f16", "nt", "f16", A, B, D, stream, workspace)


def gemm_nn_bf16(A, B, D=None, stream=None, workspace=None):
    """D = A @ B in BF16 (FP32 accumulation); A is M x K, B is K x N.
    ``workspace``: see :func:`_call`."""
    return _call("gemm_nn_bf16", "nn", "bf16", A, B, D, stream, workspace)


def gemm_nt_bf16(A, B, D=None, stream=None, workspace=None):
    """D = A @ B.T in BF16 (FP32 accumulation); A is M x K, B is N x K.
    ``workspace``: see :func:`_call`."""
    return _call("gemm_nt_bf16", "nt", "bf16", A, B, D, stream, workspace)


def gemm_nn_f16(A, B, D=None, stream=None, workspace=None):
    """D = A @ B in FP16 (FP32 accumulation); A is M x K, B is K x N.
    ``workspace``: see :func:`_call`."""
    return _call("gemm_nn_f16", "nn", "f16", A, B, D, stream, workspace)


def raw(name: str):
    """The raw ctypes function ``name`` (for calls with explicit pointers)."""
    return getattr(load_library(), name)


def mx_workspace_size(M: int, N: int, K: int, num_cus: int = 0) -> int:
    """Bytes of workspace gemm_nt_e4m3_mx_ex needs (gemm_nt_e4m3_mx_workspace_size;
    num_cus 0: the current device's)."""
    out = ctypes.c_size_t()
    st = load_library().gemm_nt_e4m3_mx_workspace_size(M, N, K, num_cus, ctypes.byref(out))
    if st != Status.OK:
        raise DenseGemmError(st, "gemm_nt_e4m3_mx_workspace_size")
    return out.value


def gemm_nt_e4m3_mx(A, SA, B, SB, D=None, stream=None, workspace=None):
    """D = A @ B.T with E4M3 A (M x K), B (N x K) and E8M0 block scales SA
    (M x K/32), SB (N x K/32), FP32 accumulation, BF16 out.  A and B are
    uint8 or float8_e4m3fn device tensors, SA and SB uint8 device tensors,
    all 2-D with unit column stride.  With ``workspace`` (a device tensor, or
    True to take one from torch's allocator), the call goes through
    gemm_nt_e4m3_mx_ex with that workspace."""
    import torch
    lib = load_library()
    for t, what in ((A, "A"), (SA, "SA"), (B, "B"), (SB, "SB")):
        if t.element_size() != 1 or not t.is_cuda or t.dim() != 2 or (t.stride(1) != 1 and t.shape[1] > 1):
            raise ValueError("%s must be a 2-D byte device tensor with unit column stride" % what)
    M, K = A.shape
    N = B.shape[0]
    if B.shape[1] != K or tuple(SA.shape) != (M, K // 32) or tuple(SB.shape) != (N, K // 32):
        raise ValueError("inconsistent shapes: A %s, SA %s, B %s, SB %s"
                         % (tuple(A.shape), tuple(SA.shape), tuple(B.shape), tuple(SB.shape)))
    own_d = D is None
    if own_d:
        D = torch.empty((M, N), dtype=torch.bfloat16, device=A.device)
    else:
        _check_tensor(D, "bf16", "D")
        if D.shape[0] != M or D.shape[1] != N:
            raise ValueError("D has shape %s, expected (%d, %d)" % (tuple(D.shape), M, N))
    dev = _same_device(A, SA, B, SB, D)
    if own_d:
        _used_by(D, stream, dev)
    name = "gemm_nt_e4m3_mx"
    with torch.cuda.device(dev):
        args = (M, N, K, A.data_ptr(), _ld(A), SA.data_ptr(), _ld(SA), B.data_ptr(), _ld(B),
                SB.data_ptr(), _ld(SB), D.data_ptr(), _ld(D))
        if workspace is None:
            st = lib.gemm_nt_e4m3_mx(*args, _stream_handle(stream, dev))
        else:
            if workspace is True:
                workspace = _used_by(torch.empty(max(mx_workspace_size(M, N, K), 1),
                                                 dtype=torch.uint8, device=dev), stream, dev)
            if not workspace.is_cuda or workspace.device != dev:
                raise ValueError("workspace must be a device tensor on %s" % dev)
            st = lib.gemm_nt_e4m3_mx_ex(*args, workspace.data_ptr(),
                                        workspace.numel() * workspace.element_size(),
                                        _stream_handle(stream, dev))
            name = "gemm_nt_e4m3_mx_ex"
    if st != Status.OK:
        raise DenseGemmError(st, name)
    return D
