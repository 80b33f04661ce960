"""The entry point that allocates nothing (gemm_nt_f16_noalloc), on the GPU.

It must give gemm_nt_f16's result bit for bit (same plan and kernels, its
scratch memory a fixed per-device array instead of a stream-ordered
allocation), which passes the oracle, on calls in a row that reuse the
array: a larger call, then a smaller one; and it must reject, before any
launch, a call that needs more scratch than the array holds.
"""
import numpy as np
import pytest

import oracle
from dense_gemm_08_amd import binding, inputs
from tests import _gpu

pytestmark = pytest.mark.gpu

S = binding.Status


def _noalloc(M, N, K, A, lda, B, ldb, D, ldd):
    t = _gpu.torch()
    fn = binding.raw("gemm_nt_f16_noalloc")
    return S(fn(M, N, K, A.data_ptr(), lda, B.data_ptr(), ldb, D.data_ptr(), ldd,
                t.cuda.current_stream().cuda_stream))


CASES = [
    # (M, N, K, lda, what takes the scratch): a larger call, then a smaller one
    (4252, 4088, 1000, 1000, "the last wave's 16 tiles in 4 K parts (16 MiB of partials)"),
    (256, 128, 4096, 4096, "one 256 x 128 tile in 16 K parts (2 MiB of partials)"),
    (128, 128, 4096, 4096, "the small-output kernel (no scratch)"),
    (300, 264, 1000, 1001, "A repacked (odd leading dimension)"),
]


def test_noalloc_equals_plain_call_on_calls_in_a_row():
    t = _gpu.torch()
    w = inputs.WORKLOADS["ragged_nt"]
    for M, N, K, lda, what in CASES:
        print("gemm_nt_f16_noalloc %dx%dx%d lda=%d: %s" % (M, N, K, lda, what), flush=True)
        A, B = inputs.make_operands(w, seed=M + N + K, M=M, N=N, K=K)
        Ad, Bd = _gpu.to_dev(A, M, K, ld=lda), _gpu.to_dev(B, N, K)
        D1, D2 = _gpu.empty_out(M, N), _gpu.empty_out(M, N)
        assert _gpu.call("nt", "f16", M, N, K, Ad, lda, Bd, K, D1, N) == S.OK
        assert _noalloc(M, N, K, Ad, lda, Bd, K, D2, N) == S.OK
        t.cuda.synchronize()
        g1, g2 = _gpu.from_dev(D1), _gpu.from_dev(D2)
        assert (g1 == g2).all(), what
        d, s = oracle.gemm("nt", "f16", A, B)
        res = oracle.check("f16", d, s, g2)
        assert res.ok, (what, res)


def test_noalloc_rejects_a_call_beyond_its_scratch():
    # K odd: both operands are repacked (4104 x 4096 + 4096 x 4096 FP16), and
    # the last wave's 16 tiles split in 16 parts: 128 MiB > 64 MiB; every
    # buffer is sized for the call
    t = _gpu.torch()
    M, N, K = 4104, 4096, 4095
    Ad = t.zeros((M, K), dtype=t.int16, device="cuda")
    Bd = t.zeros((N, K), dtype=t.int16, device="cuda")
    D = _gpu.empty_out(M, N)
    assert _noalloc(M, N, K, Ad, K, Bd, K, D, N) == S.SCRATCH_TOO_SMALL
    t.cuda.synchronize()
    assert (_gpu.from_dev(D) == _gpu.CANARY).all()
    # the same call with a workspace of its own runs
    assert _gpu.call("nt", "f16", M, N, K, Ad, K, Bd, K, D, N) == S.OK
    t.cuda.synchronize()
    assert (_gpu.from_dev(D) == 0).all()


def test_noalloc_call_captured_in_a_graph():
    # the callers this entry point is for: a HIP graph captured once and
    # replayed.  One 256 x 128 tile in 16 K parts (two kernels, the split
    # partials in the fixed scratch), captured, then replayed three times
    # with new operands copied in eagerly between replays; every replay must
    # give the plain entry point's bits for its operands
    t = _gpu.torch()
    M, N, K = 256, 128, 4096
    w = inputs.WORKLOADS["k_loop"]
    Ad = t.empty((M, K), dtype=t.int16, device="cuda")
    Bd = t.empty((N, K), dtype=t.int16, device="cuda")
    D = t.empty((M, N), dtype=t.int16, device="cuda")
    A0, B0 = inputs.make_operands(w, seed=900, M=M, N=N, K=K)
    Ad.copy_(t.from_numpy(A0.view(np.int16)))
    Bd.copy_(t.from_numpy(B0.view(np.int16)))
    t.cuda.synchronize()
    fn = binding.raw("gemm_nt_f16_noalloc")
    s = t.cuda.Stream()
    s.wait_stream(t.cuda.current_stream())
    with t.cuda.stream(s):  # one eager call first (sets up the scratch address)
        assert S(fn(M, N, K, Ad.data_ptr(), K, Bd.data_ptr(), K, D.data_ptr(), N,
                    s.cuda_stream)) == S.OK
    t.cuda.current_stream().wait_stream(s)
    t.cuda.synchronize()
    g = t.cuda.CUDAGraph()
    with t.cuda.graph(g, stream=s):
        st = fn(M, N, K, Ad.data_ptr(), K, Bd.data_ptr(), K, D.data_ptr(), N, s.cuda_stream)
    assert S(st) == S.OK
    for rep in range(3):
        A, B = inputs.make_operands(w, seed=901 + rep, M=M, N=N, K=K)
        Ad.copy_(t.from_numpy(A.view(np.int16)))
        Bd.copy_(t.from_numpy(B.view(np.int16)))
        D.fill_(-1)
        t.cuda.synchronize()
        g.replay()
        t.cuda.synchronize()
        got = _gpu.from_dev(D)
        Dp = _gpu.empty_out(M, N)
        assert _gpu.call("nt", "f16", M, N, K, Ad, K, Bd, K, Dp, N) == S.OK
        t.cuda.synchronize()
        assert (got == _gpu.from_dev(Dp)).all(), rep
        d, s_ = oracle.gemm("nt", "f16", A, B)
        assert oracle.check("f16", d, s_, got).ok, rep
