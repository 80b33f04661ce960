"""Helpers for the GPU tests: device buffers and raw C-ABI calls.

torch provides device memory and the stream; every GEMM runs in the HIP
library through its C entry points (``include/dense_gemm.h``).
"""
from __future__ import annotations

import numpy as np

from dense_gemm_08_amd import binding

ENTRY = {("nt", "f16"): "gemm_nt_f16", ("nn", "bf16"): "gemm_nn_bf16",
         ("nt", "bf16"): "gemm_nt_bf16", ("nn", "f16"): "gemm_nn_f16"}
CANARY = 0x7E5A  # a NaN pattern in both formats: any write over it shows


def torch():
    import torch as _t
    return _t


def to_dev(bits: np.ndarray, rows: int, cols: int, ld: int | None = None, fill: int = CANARY):
    """A rows x ld int16 device buffer holding ``bits`` in its first cols
    columns and ``fill`` in the padding.  Returns the tensor."""
    t = torch()
    ld = cols if ld is None else ld
    host = np.full((rows, ld), fill, dtype=np.uint16)
    if rows and cols:
        host[:, :cols] = bits.reshape(rows, cols)
    return t.from_numpy(host.view(np.int16)).to("cuda")


def empty_out(rows: int, ld: int, fill: int = CANARY):
    t = torch()
    return t.full((max(rows, 1), max(ld, 1)), np.uint16(fill).view(np.int16).item(),
                  dtype=t.int16, device="cuda")


def from_dev(t_dev) -> np.ndarray:
    return t_dev.cpu().numpy().view(np.uint16)


def workspace(nbytes: int):
    """A device workspace of ``nbytes`` (256-byte aligned) from torch."""
    t = torch()
    ws = t.empty(max(nbytes, 1) + 256, dtype=t.uint8, device="cuda")
    off = (-ws.data_ptr()) % 256
    return ws[off:off + max(nbytes, 1)]


def call(layout, fmt, M, N, K, A, lda, B, ldb, D, ldd, stream=None, offsets=(0, 0, 0),
         opts=None):
    """Run the entry point for (layout, fmt) on device tensors; returns the
    status.  ``offsets`` are byte offsets added to the A, B and D pointers.
    With ``opts`` = (split_k, tile_n) the call goes through dense_gemm_ex
    with those plan overrides and a workspace of the size the library's query
    reports, allocated here and held in _KEEP until the next gemm() has
    synchronised."""
    t = torch()
    st = t.cuda.current_stream() if stream is None else stream
    ptr = lambda x, o: 0 if x is None else x.data_ptr() + o  # noqa: E731
    oa, ob, od = offsets
    if opts is None:
        fn = binding.raw(ENTRY[(layout, fmt)])
        return binding.Status(fn(M, N, K, ptr(A, oa), lda, ptr(B, ob), ldb, ptr(D, od), ldd,
                                 st.cuda_stream))
    lib = binding.load_library()
    o = binding.Options(*opts)
    import ctypes
    need = ctypes.c_size_t()
    rc = binding.Status(lib.dense_gemm_workspace_size(binding.OPS[(layout, fmt)], M, N, K,
                                                      ptr(A, oa), lda, ptr(B, ob), ldb, 0,
                                                      ctypes.byref(o), ctypes.byref(need)))
    if rc != binding.Status.OK:
        return rc
    ws = workspace(need.value)
    _KEEP.append(ws)
    return binding.Status(lib.dense_gemm_ex(binding.OPS[(layout, fmt)], M, N, K, ptr(A, oa), lda,
                                            ptr(B, ob), ldb, ptr(D, od), ldd, ctypes.byref(o),
                                            ws.data_ptr(), need.value, st.cuda_stream))


# workspaces of calls made through call(..., opts=...): released at the next
# gemm() (after its synchronisation), so none is freed while in use
_KEEP = []


def to_dev_at(bits: np.ndarray, rows: int, cols: int, ld: int, off: int, fill: int = CANARY):
    """Like to_dev, with the matrix starting ``off`` elements into the buffer."""
    t = torch()
    host = np.full(rows * ld + off + 8, fill, dtype=np.uint16)
    if rows and cols:
        host[off:off + rows * ld].reshape(rows, ld)[:, :cols] = bits.reshape(rows, cols)
    return t.from_numpy(host.view(np.int16)).to("cuda")


def gemm(layout, fmt, Abits, Bbits, M, N, K, lda=None, ldb=None, ldd=None, stream=None,
         a_off=0, b_off=0, d_off=0, opts=None):
    """Upload, run, download.  Returns (D bits M x ldd, status).  ``*_off``
    place a matrix that many elements into its buffer (misaligned pointers).
    ``opts`` = (split_k, tile_n): through dense_gemm_ex (see call)."""
    t = torch()
    lda = K if lda is None else lda
    ldb = (K if layout == "nt" else N) if ldb is None else ldb
    ldd = N if ldd is None else ldd
    A = to_dev_at(Abits, M, K, lda, a_off)
    if layout == "nt":
        B = to_dev_at(Bbits, N, K, ldb, b_off)
    else:
        B = to_dev_at(Bbits, K, N, ldb, b_off)
    D = to_dev_at(np.zeros(0, np.uint16), M, 0, ldd, d_off)
    st = call(layout, fmt, M, N, K, A, lda, B, ldb, D, ldd, stream,
              offsets=(2 * a_off, 2 * b_off, 2 * d_off), opts=opts)
    t.cuda.synchronize()
    _KEEP.clear()
    out = from_dev(D)[d_off:d_off + M * ldd].reshape(M, ldd) if M else np.zeros((0, ldd), np.uint16)
    assert (from_dev(D)[:d_off] == CANARY).all() and (from_dev(D)[d_off + M * ldd:] == CANARY).all()
    return out, st


def ladder(level, Abits, Bbits, M, N, K):
    """D = A @ B.T (FP16) by optimisation-step kernel `level` (tight leading
    dimensions).  Returns (D bits M x N, status)."""
    t = torch()
    A = to_dev(Abits, M, K)
    B = to_dev(Bbits, N, K)
    D = empty_out(M, N)
    fn = binding.raw("gemm_nt_f16_ladder")
    st = binding.Status(fn(level, M, N, K, A.data_ptr(), K, B.data_ptr(), K, D.data_ptr(), N,
                           t.cuda.current_stream().cuda_stream))
    t.cuda.synchronize()
    return from_dev(D)[:M], st
