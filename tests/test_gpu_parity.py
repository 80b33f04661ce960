"""GPU parity tests: the HIP path (through the C ABI) against the CPU oracle.

Acceptance (per element): |d_gpu - d| <= ulp_out(|d|) + 2^-11 * sum_k |a*b|,
with d the oracle's FP64 value.  Where the FP32 sum is exact (small-integer,
identity and all-ones inputs) the result must equal the oracle's correctly
rounded value bit for bit.  Shapes: every workload at a reduced size checked
element by element (several tiles and a ragged tail in M, N and K), and at its
full size in the launch configuration the benchmark times, on sampled entries.
"""
import numpy as np
import pytest

import oracle
from dense_gemm_08_amd import inputs
from tests import _gpu

pytestmark = pytest.mark.gpu

S = None  # binding.Status, imported lazily


def status():
    from dense_gemm_08_amd.binding import Status
    return Status


def check_full(layout, fmt, A, B, M, N, K, D):
    d, s = oracle.gemm(layout, fmt, A, B, M=M, N=N, K=K)
    res = oracle.check(fmt, d, s, D[:, :N])
    assert res.ok, (res, np.unravel_index(max(res.worst_idx, 0), (M, N)))
    return d


def check_sampled(layout, fmt, A, B, M, N, K, D, n=3000, seed=0):
    rows, cols = inputs.sample_indices(M, N, n, seed)
    ldb = K if layout == "nt" else N
    d, s = oracle.gemm_entries(layout, fmt, A, B, K=K, lda=K, ldb=ldb, rows=rows, cols=cols)
    res = oracle.check(fmt, d, s, D[rows, cols])
    assert res.ok, (res, rows[max(res.worst_idx, 0)], cols[max(res.worst_idx, 0)])


# --------------------------------------------------- workloads, reduced --

REDUCED = [
    # (workload, M, N, K): each spans several 256 x 256 tiles and a ragged tail
    ("single_tile", 128, 128, 64),
    ("k_loop", 128, 128, 4096),
    ("square_nt", 600, 520, 712),
    ("large_nn", 520, 776, 328),
    ("ragged_nt", 300, 500, 400),
]


@pytest.fixture(params=["auto", "off"])
def splitk(request, monkeypatch):
    """Run with the library's own split-K choice, and with split-K disabled."""
    if request.param == "off":
        monkeypatch.setenv("DENSE_GEMM_SPLITK", "off")
    else:
        monkeypatch.delenv("DENSE_GEMM_SPLITK", raising=False)
    return request.param


@pytest.mark.parametrize("name,M,N,K", REDUCED)
def test_workload_reduced_full_check(name, M, N, K, splitk):
    w = inputs.WORKLOADS[name]
    A, B = inputs.make_operands(w, M=M, N=N, K=K)
    D, st = _gpu.gemm(w.layout, w.fmt, A, B, M, N, K)
    assert st == status().OK
    check_full(w.layout, w.fmt, A, B, M, N, K, D)


@pytest.mark.parametrize("layout,fmt", [("nt", "bf16"), ("nn", "f16")])
def test_other_type_layout_pairs(layout, fmt):
    w = inputs.Workload("x", layout, fmt, 0, 0, 0, "uniform", 0.0, 17)
    M, N, K = 300, 264, 200
    A, B = inputs.make_operands(w, M=M, N=N, K=K)
    D, st = _gpu.gemm(layout, fmt, A, B, M, N, K)
    assert st == status().OK
    check_full(layout, fmt, A, B, M, N, K, D)


# ------------------------------------------------ workloads, full size --

@pytest.mark.parametrize("name", ["single_tile", "k_loop", "square_nt", "large_nn", "ragged_nt"])
def test_workload_full_size_sampled(name):
    w = inputs.WORKLOADS[name]
    A, B = inputs.make_operands(w)
    D, st = _gpu.gemm(w.layout, w.fmt, A, B, w.M, w.N, w.K)
    assert st == status().OK
    if w.M * w.N * w.K <= 128 * 128 * 4096:
        check_full(w.layout, w.fmt, A, B, w.M, w.N, w.K, D)
    else:
        check_sampled(w.layout, w.fmt, A, B, w.M, w.N, w.K, D, n=3000, seed=w.seed)
        assert np.isfinite(oracle.decode(w.fmt, D[:: max(w.M // 64, 1), :: max(w.N // 64, 1)])).all()


# ------------------------------------------------- bitwise special cases --

@pytest.mark.parametrize("M,N,K", [(8192, 16384 + 128, 4096), (8192, 4096, 16384 + 40),
                                   (8192, 1024, 1024), (8192, 1024, 16384)])
def test_m8192_sweep_shapes_sampled(M, N, K):
    # extreme shapes of the benchmark's M = 8192 sweep (FP16 A.B^T, N(0,1)/8):
    # the widest N with a ragged last tile column, the deepest K with a partial
    # last step, and the narrowest N (128-wide tiles; split-K at K = 16384);
    # sampled against the oracle
    w = inputs.WORKLOADS["square_nt"]
    A, B = inputs.make_operands(w, seed=M + N + K, M=M, N=N, K=K)
    D, st = _gpu.gemm("nt", "f16", A, B, M, N, K)
    assert st == status().OK
    check_sampled("nt", "f16", A, B, M, N, K, D, n=2000, seed=N + K)


@pytest.mark.parametrize("layout,fmt", [("nt", "f16"), ("nn", "bf16"), ("nt", "bf16"), ("nn", "f16")])
def test_small_integers_exact(layout, fmt, splitk):
    # entries in {-3..3}: every FP32 partial sum is an exact integer, so the
    # result is the exactly rounded integer sum (sums up to 9K exceed the
    # FP16/BF16 integer range, so this pins round-to-nearest-even)
    M, N, K = 264, 392, 1032
    sa, sb = inputs.operand_shapes(layout, M, N, K)
    A = inputs.small_integers(fmt, sa, seed=31)
    B = inputs.small_integers(fmt, sb, seed=32)
    D, st = _gpu.gemm(layout, fmt, A, B, M, N, K)
    assert st == status().OK
    d, _ = oracle.gemm(layout, fmt, A, B)
    want = oracle.round_to(fmt, d)
    assert (D == want).all()


@pytest.mark.parametrize("layout,fmt", [("nt", "f16"), ("nn", "bf16")])
def test_identity_gives_a(layout, fmt):
    w = inputs.Workload("x", layout, fmt, 0, 0, 0, "uniform", 0.0, 41)
    M, K = 333, 264
    A, _ = inputs.make_operands(w, M=M, N=8, K=K)
    eye = inputs.identity(fmt, K)
    D, st = _gpu.gemm(layout, fmt, A, eye, M, K, K)
    assert st == status().OK
    assert (oracle.decode(fmt, D) == oracle.decode(fmt, A)).all()


@pytest.mark.parametrize("K", [64, 4096, 5120, 4000, 8])
def test_all_ones_give_k(K):
    for layout, fmt in (("nt", "f16"), ("nn", "bf16")):
        M, N = 136, 264
        sa, sb = inputs.operand_shapes(layout, M, N, K)
        D, st = _gpu.gemm(layout, fmt, inputs.ones(fmt, sa), inputs.ones(fmt, sb), M, N, K)
        assert st == status().OK
        assert (D == oracle.round_to(fmt, np.array([float(K)]))[0]).all()


def test_power_of_two_scaling():
    w = inputs.WORKLOADS["square_nt"]
    M, N, K = 300, 300, 256
    A, B = inputs.make_operands(w, M=M, N=N, K=K)
    D1, _ = _gpu.gemm("nt", "f16", A, B, M, N, K)
    A4 = inputs.f16_bits(oracle.decode("f16", A) * 4.0)
    D4, _ = _gpu.gemm("nt", "f16", A4, B, M, N, K)
    d1 = oracle.decode("f16", D1)
    d4 = oracle.decode("f16", D4)
    # scaling one operand by 4 scales every product and partial sum exactly;
    # only outputs in FP16's subnormal range round differently
    normal = np.abs(d1) >= 2.0 ** -14
    assert normal.mean() > 0.99
    assert (d4[normal] == d1[normal] * 4.0).all()


@pytest.mark.parametrize("layout,fmt", [("nt", "f16"), ("nn", "bf16")])
@pytest.mark.parametrize("parts", ["2", "3", "7", "64"])
def test_forced_split_k(layout, fmt, parts, monkeypatch):
    # split-K forced on shapes of several tiles, a ragged K tail and parts of
    # unequal length; the summation order is fixed, so a rerun is bitwise equal
    monkeypatch.setenv("DENSE_GEMM_SPLITK", parts)
    w = inputs.Workload("x", layout, fmt, 0, 0, 0, "uniform", 0.0, 71)
    M, N, K = 300, 264, 1000
    A, B = inputs.make_operands(w, M=M, N=N, K=K)
    D, st = _gpu.gemm(layout, fmt, A, B, M, N, K)
    assert st == status().OK
    check_full(layout, fmt, A, B, M, N, K, D)
    D2, _ = _gpu.gemm(layout, fmt, A, B, M, N, K)
    assert (D == D2).all()


@pytest.mark.parametrize("layout,fmt", [("nt", "f16"), ("nn", "bf16")])
@pytest.mark.parametrize("parts", ["off", "4"])
def test_k_remainder_equals_leading_zero_padding(layout, fmt, parts, monkeypatch):
    # K = 4000 is not a multiple of the 64-deep K step: the kernel pads its
    # first step in front (k from -32), so the result must equal, bit for bit,
    # the same data with 32 zero columns of A (and zero k-rows or columns of
    # B) put in front, K = 4032, which has the same steps, unsplit or in 4
    # parts of 16 steps
    monkeypatch.setenv("DENSE_GEMM_SPLITK", parts)
    w = inputs.Workload("x", layout, fmt, 0, 0, 0, "uniform", 0.0, 5)
    M, N, K = 272, 264, 4000
    pad = (64 - K % 64) % 64
    Kp = K + pad
    A, B = inputs.make_operands(w, M=M, N=N, K=K)
    Ap = np.zeros((M, Kp), np.uint16)
    Ap[:, pad:] = A
    if layout == "nt":
        Bp = np.zeros((N, Kp), np.uint16)
        Bp[:, pad:] = B
    else:
        Bp = np.zeros((Kp, N), np.uint16)
        Bp[pad:] = B
    D1, _ = _gpu.gemm(layout, fmt, A, B, M, N, K)
    D2, _ = _gpu.gemm(layout, fmt, Ap, Bp, M, N, Kp)
    assert (D1 == D2).all()
    check_full(layout, fmt, A, B, M, N, K, D1)


@pytest.mark.parametrize("layout,fmt", [("nt", "f16"), ("nn", "bf16")])
def test_ragged_block_equals_padded_block(layout, fmt):
    # a ragged M x N result is the top-left block of the zero-padded product
    w = inputs.Workload("x", layout, fmt, 0, 0, 0, "uniform", 0.0, 51)
    M, N, K, Mp, Np = 300, 504, 136, 512, 512
    A, B = inputs.make_operands(w, M=M, N=N, K=K)
    Ap = np.zeros((Mp, K), np.uint16)
    Ap[:M] = A
    if layout == "nt":
        Bp = np.zeros((Np, K), np.uint16)
        Bp[:N] = B
    else:
        Bp = np.zeros((K, Np), np.uint16)
        Bp[:, :N] = B
    D1, _ = _gpu.gemm(layout, fmt, A, B, M, N, K)
    D2, _ = _gpu.gemm(layout, fmt, Ap, Bp, Mp, Np, K)
    assert (D1 == D2[:M, :N]).all()


# ------------------------------------------------------------ edge paths --

SWEEP = [1, 7, 8, 33, 65, 129, 255, 257]


@pytest.mark.parametrize("layout,fmt", [("nt", "f16"), ("nn", "bf16")])
def test_ragged_sweep(layout, fmt):
    rng = np.random.default_rng(5)
    w = inputs.Workload("x", layout, fmt, 0, 0, 0, "uniform", 0.0, 0)
    for M in SWEEP:
        for N in SWEEP:
            K = int(rng.choice([1, 7, 8, 13, 56, 64, 72, 135]))
            A, B = inputs.make_operands(w, seed=M * 1000 + N, M=M, N=N, K=K)
            D, st = _gpu.gemm(layout, fmt, A, B, M, N, K)
            assert st == status().OK, (M, N, K)
            check_full(layout, fmt, A, B, M, N, K, D)


@pytest.mark.parametrize("layout,fmt", [("nt", "f16"), ("nn", "bf16")])
def test_leading_dimensions_and_untouched_padding(layout, fmt):
    w = inputs.Workload("x", layout, fmt, 0, 0, 0, "uniform", 0.0, 61)
    M, N, K = 280, 272, 200
    lda, ldb, ldd = K + 24, (K if layout == "nt" else N) + 40, N + 16
    A, B = inputs.make_operands(w, M=M, N=N, K=K)
    D, st = _gpu.gemm(layout, fmt, A, B, M, N, K, lda=lda, ldb=ldb, ldd=ldd)
    assert st == status().OK
    assert (D[:, N:] == _gpu.CANARY).all()
    check_full(layout, fmt, A, B, M, N, K, D)


# Operands the 16-byte chunk loader cannot read in place (K, a leading
# dimension or the A.B layout's N not a multiple of 8, or a pointer off 16-byte
# alignment) go through the repack kernel; D may sit at any even address.
UNALIGNED = [
    # (M, N, K, lda_extra, ldb_extra, ldd_extra, a_off, b_off, d_off)
    (300, 264, 1, 0, 0, 0, 0, 0, 0),
    (300, 264, 13, 0, 0, 0, 0, 0, 0),
    (264, 300, 1001, 0, 0, 0, 0, 0, 0),
    (280, 272, 200, 3, 0, 0, 0, 0, 0),
    (280, 272, 200, 0, 5, 1, 0, 0, 0),
    (280, 272, 200, 0, 0, 0, 1, 0, 0),
    (280, 272, 200, 0, 0, 0, 0, 3, 0),
    (280, 272, 200, 0, 0, 0, 0, 0, 5),
    (257, 13, 77, 2, 1, 3, 1, 2, 3),
    (300, 1001, 136, 0, 0, 0, 0, 0, 0),
    (128, 128, 4001, 0, 0, 0, 1, 1, 1),  # + split-K
]


@pytest.mark.parametrize("layout,fmt", [("nt", "f16"), ("nn", "bf16"), ("nt", "bf16"), ("nn", "f16")])
@pytest.mark.parametrize("case", UNALIGNED, ids=lambda c: "x".join(map(str, c)))
def test_unaligned_operands(layout, fmt, case):
    M, N, K, xa, xb, xd, oa, ob, od = case
    w = inputs.Workload("x", layout, fmt, 0, 0, 0, "uniform", 0.0, 81)
    A, B = inputs.make_operands(w, seed=M + N + K, M=M, N=N, K=K)
    lda, ldb, ldd = K + xa, (K if layout == "nt" else N) + xb, N + xd
    D, st = _gpu.gemm(layout, fmt, A, B, M, N, K, lda=lda, ldb=ldb, ldd=ldd,
                      a_off=oa, b_off=ob, d_off=od)
    assert st == status().OK
    assert (D[:, N:] == _gpu.CANARY).all()
    check_full(layout, fmt, A, B, M, N, K, D)


@pytest.mark.parametrize("layout,fmt", [("nt", "f16"), ("nn", "bf16")])
def test_repacked_equals_direct(layout, fmt):
    # an operand read through the repack kernel gives bit-identical results to
    # the same operand read in place (same tiles, same accumulation order)
    w = inputs.Workload("x", layout, fmt, 0, 0, 0, "uniform", 0.0, 91)
    M, N, K = 520, 520, 712
    A, B = inputs.make_operands(w, M=M, N=N, K=K)
    D1, _ = _gpu.gemm(layout, fmt, A, B, M, N, K)
    D2, _ = _gpu.gemm(layout, fmt, A, B, M, N, K, lda=K + 1, ldb=(K if layout == "nt" else N) + 1)
    D3, _ = _gpu.gemm(layout, fmt, A, B, M, N, K, a_off=1, b_off=3)
    assert (D1 == D2).all() and (D1 == D3).all()


def test_repack_beyond_one_grid_pass():
    # the repack kernel strides over a capped grid (65536 workgroups of 256
    # threads, one 8-element chunk per thread and pass): an A of 8200 rows
    # with K = 16390 (rows padded to 16392) holds 16,801,800 chunks, so rows
    # 8188 and up are copied by a second pass.  Sampled entries, and every
    # entry of the last 12 rows, against the oracle.
    w = inputs.WORKLOADS["square_nt"]
    M, N, K = 8200, 256, 16390
    A, B = inputs.make_operands(w, seed=77, M=M, N=N, K=K)
    D, st = _gpu.gemm("nt", "f16", A, B, M, N, K)
    assert st == status().OK
    check_sampled("nt", "f16", A, B, M, N, K, D, n=1000, seed=77)
    rows = np.repeat(np.arange(M - 12, M), N)
    cols = np.tile(np.arange(N), 12)
    d, s = oracle.gemm_entries("nt", "f16", A, B, K=K, lda=K, ldb=K, rows=rows, cols=cols)
    res = oracle.check("f16", d, s, D[rows, cols])
    assert res.ok, (res, rows[max(res.worst_idx, 0)], cols[max(res.worst_idx, 0)])


def test_zero_k_writes_zeros_and_empty_is_noop():
    t = _gpu.torch()
    D = _gpu.empty_out(40, 48)
    st = _gpu.call("nt", "f16", 40, 48, 0, None, 0, None, 0, D, 48)
    t.cuda.synchronize()
    assert st == status().OK
    assert (_gpu.from_dev(D) == 0).all()
    D = _gpu.empty_out(40, 48)
    A = _gpu.to_dev(np.zeros((40, 16), np.uint16), 40, 16)
    B = _gpu.to_dev(np.zeros((16, 48), np.uint16), 16, 48)
    assert _gpu.call("nn", "bf16", 0, 48, 16, A, 16, B, 48, D, 48) == status().OK
    assert _gpu.call("nn", "bf16", 40, 0, 16, A, 16, B, 48, D, 48) == status().OK
    t.cuda.synchronize()
    assert (_gpu.from_dev(D) == _gpu.CANARY).all()


def test_errors_launch_nothing():
    t = _gpu.torch()
    D = _gpu.empty_out(64, 64)
    A = _gpu.to_dev(np.zeros((64, 64), np.uint16), 64, 64)
    Sx = status()
    assert _gpu.call("nt", "f16", 64, 64, 60, A, 64, A, 64, D, 64, offsets=(1, 0, 0)) == Sx.MISALIGNED
    assert _gpu.call("nn", "bf16", 64, 64, 64, A, 64, A, 64, D, 64, offsets=(0, 3, 0)) == Sx.MISALIGNED
    assert _gpu.call("nt", "f16", 64, 64, 64, A, 64, A, 64, D, 64, offsets=(0, 0, 1)) == Sx.MISALIGNED
    assert _gpu.call("nt", "f16", 64, 64, 64, A, 32, A, 64, D, 64) == Sx.BAD_LD
    assert _gpu.call("nt", "f16", -1, 64, 64, A, 64, A, 64, D, 64) == Sx.INVALID_DIM
    t.cuda.synchronize()
    assert (_gpu.from_dev(D) == _gpu.CANARY).all()


def test_deterministic_and_stream_ordered():
    t = _gpu.torch()
    w = inputs.WORKLOADS["square_nt"]
    M = N = K = 1024
    A, B = inputs.make_operands(w, M=M, N=N, K=K)
    Ad, Bd = _gpu.to_dev(A, M, K), _gpu.to_dev(B, N, K)
    outs = []
    s = t.cuda.Stream()
    for stream in (None, s, s):
        D = _gpu.empty_out(M, N)
        if stream is not None:
            stream.wait_stream(t.cuda.current_stream())
            with t.cuda.stream(stream):
                assert _gpu.call("nt", "f16", M, N, K, Ad, K, Bd, K, D, N, stream) == status().OK
            t.cuda.current_stream().wait_stream(stream)
        else:
            assert _gpu.call("nt", "f16", M, N, K, Ad, K, Bd, K, D, N) == status().OK
        t.cuda.synchronize()
        outs.append(_gpu.from_dev(D))
    assert (outs[0] == outs[1]).all() and (outs[1] == outs[2]).all()


def test_concurrent_streams_with_workspaces():
    # calls that each take a stream-ordered workspace (split-K partials, a
    # repacked operand, FP8 scale panels), issued back to back on two
    # streams at once, give the same bits as the same calls run alone
    t = _gpu.torch()
    w = inputs.WORKLOADS["square_nt"]
    A1, B1 = inputs.make_operands(w, seed=61, M=128, N=128, K=4096)           # split-K
    wn = inputs.WORKLOADS["large_nn"]
    A2, B2 = inputs.make_operands(wn, seed=62, M=264, N=304, K=1032)          # repacked A
    A1d, B1d = _gpu.to_dev(A1, 128, 4096), _gpu.to_dev(B1, 128, 4096)
    A2d, B2d = _gpu.to_dev(A2, 264, 1032, ld=1033), _gpu.to_dev(B2, 1032, 304)
    XA, XSA, XB, XSB = [t.from_numpy(x).cuda() for x in inputs.mx_operands(280, 300, 160, seed=63)]
    mx = binding_raw("gemm_nt_e4m3_mx")

    def run(kind, D, stream):
        h = stream.cuda_stream
        if kind == 0:
            return _gpu.call("nt", "f16", 128, 128, 4096, A1d, 4096, B1d, 4096, D, 128, stream)
        if kind == 1:
            return _gpu.call("nn", "bf16", 264, 304, 1032, A2d, 1033, B2d, 304, D, 304, stream)
        return status()(mx(280, 300, 160, XA.data_ptr(), 160, XSA.data_ptr(), 5, XB.data_ptr(), 160,
                           XSB.data_ptr(), 5, D.data_ptr(), 300, h))

    shapes = [(128, 128), (264, 304), (280, 300)]
    ref = []
    main = t.cuda.current_stream()
    for kind in range(3):
        D = _gpu.empty_out(*shapes[kind])
        assert run(kind, D, main) == status().OK
        t.cuda.synchronize()
        ref.append(_gpu.from_dev(D))
    streams = [t.cuda.Stream(), t.cuda.Stream()]
    # outputs (canary-filled on the main stream) first; then both streams
    # wait for that work and run without synchronising with each other
    outs = [((it + si) % 3, si, _gpu.empty_out(*shapes[(it + si) % 3]))
            for it in range(12) for si in range(2)]
    for st in streams:
        st.wait_stream(main)
    for kind, si, D in outs:
        with t.cuda.stream(streams[si]):
            assert run(kind, D, streams[si]) == status().OK
    for st in streams:
        main.wait_stream(st)
    t.cuda.synchronize()
    for kind, _, D in outs:
        assert (_gpu.from_dev(D) == ref[kind]).all(), kind


def test_python_binding_roundtrip():
    t = _gpu.torch()
    import dense_gemm_08_amd as dg
    a = t.randn(200, 136, device="cuda").half()
    b = t.randn(72, 136, device="cuda").half()
    d = dg.gemm_nt_f16(a, b)
    t.cuda.synchronize()
    A = a.cpu().numpy().view(np.uint16)
    B = b.cpu().numpy().view(np.uint16)
    check_full("nt", "f16", A, B, 200, 72, 136, d.cpu().numpy().view(np.uint16))
    a2 = t.randn(64, 128, device="cuda").bfloat16()
    b2 = t.randn(128, 96, device="cuda").bfloat16()
    d2 = dg.gemm_nn_bf16(a2, b2)
    t.cuda.synchronize()
    check_full("nn", "bf16", a2.cpu().view(t.int16).numpy().view(np.uint16),
               b2.cpu().view(t.int16).numpy().view(np.uint16), 64, 96, 128,
               d2.cpu().view(t.int16).numpy().view(np.uint16))


def test_python_binding_row_and_column_views():
    # one-row operands whose row stride is not their width (a transposed
    # column), a one-column output, and a row-sliced B: the binding passes
    # valid leading dimensions for each
    t = _gpu.torch()
    import dense_gemm_08_amd as dg
    a = t.randn(72, 1, device="cuda").half().t()          # 1 x 72, strides (1, 1)
    b = t.randn(40, 72, device="cuda").half()
    d = dg.gemm_nt_f16(a, b)
    t.cuda.synchronize()
    to_bits = lambda x: x.contiguous().cpu().view(t.int16).numpy().view(np.uint16)  # noqa: E731
    check_full("nt", "f16", to_bits(a), to_bits(b), 1, 40, 72, to_bits(d))
    a2 = t.randn(33, 64, device="cuda").bfloat16()
    b2 = t.randn(128, 9, device="cuda").bfloat16()[:64, :1]  # 64 x 1, row stride 9
    d2 = dg.gemm_nn_bf16(a2, b2)
    t.cuda.synchronize()
    check_full("nn", "bf16", to_bits(a2), to_bits(b2), 33, 1, 64, to_bits(d2))
    with pytest.raises(ValueError):
        dg.gemm_nt_f16(a, b.cpu())


# ----------------------------------------------- optimisation-step kernels --

LEVELS = [1, 2, 3, 4, 5, 6, 7]


@pytest.mark.parametrize("level", LEVELS)
def test_ladder_level_full_check(level):
    # each step of the optimisation ladder computes the same product (several
    # tiles in M and N, 11 K steps; the shape divides every level's tile)
    w = inputs.WORKLOADS["square_nt"]
    M, N, K = 512, 768, 704
    A, B = inputs.make_operands(w, seed=level, M=M, N=N, K=K)
    D, st = _gpu.ladder(level, A, B, M, N, K)
    assert st == status().OK
    check_full("nt", "f16", A, B, M, N, K, D)


@pytest.mark.parametrize("level", LEVELS)
def test_ladder_level_4096_sampled(level):
    # the benchmark's shape, in the configuration the ladder benchmark times
    w = inputs.WORKLOADS["square_nt"]
    A, B = inputs.make_operands(w)
    D, st = _gpu.ladder(level, A, B, w.M, w.N, w.K)
    assert st == status().OK
    check_sampled("nt", "f16", A, B, w.M, w.N, w.K, D, n=2000, seed=level)


def test_ladder_small_integers_exact():
    # exact FP32 sums: every level must give the correctly rounded result
    M, N, K = 256, 512, 256
    A = inputs.small_integers("f16", (M, K), seed=3)
    B = inputs.small_integers("f16", (N, K), seed=4)
    d, _ = oracle.gemm("nt", "f16", A, B, M=M, N=N, K=K)
    want = oracle.round_to("f16", d)
    for level in LEVELS:
        D, st = _gpu.ladder(level, A, B, M, N, K)
        assert st == status().OK
        assert (D == want).all(), level


@pytest.mark.parametrize("M,N,K", [(128, 128, 64), (128, 256, 128), (384, 128, 192)])
def test_ladder_producer_short_k(M, N, K):
    # the producer-wave level with one, two and three K steps (the prologue
    # load, the last step without a refill) and fewer tiles than CUs
    w = inputs.WORKLOADS["single_tile"]
    A, B = inputs.make_operands(w, seed=M + N + K, M=M, N=N, K=K)
    D, st = _gpu.ladder(7, A, B, M, N, K)
    assert st == status().OK
    check_full("nt", "f16", A, B, M, N, K, D)


def test_ladder_rejects_shapes():
    Sx = status()
    A = _gpu.to_dev(np.zeros((512, 512), np.uint16), 512, 512)
    D = _gpu.empty_out(512, 512)
    fn = binding_raw("gemm_nt_f16_ladder")
    s = _gpu.torch().cuda.current_stream().cuda_stream
    p = A.data_ptr()
    assert Sx(fn(0, 256, 256, 64, p, 512, p, 512, D.data_ptr(), 512, s)) == Sx.BAD_ARG
    assert Sx(fn(8, 256, 256, 64, p, 512, p, 512, D.data_ptr(), 512, s)) == Sx.BAD_ARG
    assert Sx(fn(7, 384, 200, 64, p, 512, p, 512, D.data_ptr(), 512, s)) == Sx.BAD_ARG
    assert Sx(fn(5, 384, 256, 64, p, 512, p, 512, D.data_ptr(), 512, s)) == Sx.BAD_ARG
    assert Sx(fn(1, 256, 256, 100, p, 512, p, 512, D.data_ptr(), 512, s)) == Sx.BAD_ARG
    assert Sx(fn(2, 256, 256, 64, p + 2, 512, p, 512, D.data_ptr(), 512, s)) == Sx.MISALIGNED
    _gpu.torch().cuda.synchronize()
    assert (_gpu.from_dev(D) == _gpu.CANARY).all()


def binding_raw(name):
    from dense_gemm_08_amd import binding
    return binding.raw(name)


# ------------------------------------------------- split last partial wave --

@pytest.mark.parametrize("layout,fmt", [("nt", "f16"), ("nn", "bf16")])
def test_split_last_wave(layout, fmt, monkeypatch):
    # 17 x 16 = 272 tiles on 256 CUs: 256 tiles whole, the 16 of the last wave
    # in 4 parts of 4 K steps, all in one launch; ragged M and N.  Entries are
    # sampled from the whole output and, half of them, from the split tiles;
    # the run with split-K disabled is checked the same way
    import ctypes
    from dense_gemm_08_amd import binding
    t = _gpu.torch()
    cus = t.cuda.get_device_properties(0).multi_processor_count
    M, N, K = 4252, 4088, 1000
    lib = binding.load_library()
    plan = (ctypes.c_int64 * 10)()
    assert lib.dense_gemm_plan(0 if layout == "nt" else 1, M, N, K, cus, plan) == 0
    tiles_m, tiles_n, group_m, splits = plan[3], plan[4], plan[6], plan[8]
    tasks = tiles_m * tiles_n
    if cus == 256:
        assert splits == 4
    split_tiles = []
    if splits > 1:
        for task in range(tasks - tasks % cus, tasks):
            a, b = ctypes.c_int64(), ctypes.c_int64()
            assert lib.dense_gemm_tile_of_task(task, tiles_m, tiles_n, group_m, ctypes.byref(a),
                                               ctypes.byref(b)) == 0
            split_tiles.append((a.value, b.value))
    w = inputs.Workload("x", layout, fmt, 0, 0, 0, "uniform", 0.0, 101)
    A, B = inputs.make_operands(w, M=M, N=N, K=K)
    rng = np.random.default_rng(7)
    rows, cols = inputs.sample_indices(M, N, 2000, 8)
    if split_tiles:
        pick = rng.integers(0, len(split_tiles), 2000)
        tr = np.array([split_tiles[i][0] for i in pick]) * 256 + rng.integers(0, 256, 2000)
        tc = np.array([split_tiles[i][1] for i in pick]) * 256 + rng.integers(0, 256, 2000)
        keep = (tr < M) & (tc < N)
        rows = np.concatenate([rows, tr[keep]]).astype(np.int64)
        cols = np.concatenate([cols, tc[keep]]).astype(np.int64)
    ldb = K if layout == "nt" else N
    d, s_ = oracle.gemm_entries(layout, fmt, A, B, K=K, lda=K, ldb=ldb, rows=rows, cols=cols)
    for mode in ("auto", "off"):
        if mode == "off":
            monkeypatch.setenv("DENSE_GEMM_SPLITK", "off")
        else:
            monkeypatch.delenv("DENSE_GEMM_SPLITK", raising=False)
        D, st = _gpu.gemm(layout, fmt, A, B, M, N, K)
        assert st == status().OK
        res = oracle.check(fmt, d, s_, D[rows, cols])
        assert res.ok, (mode, res)
        D2, _ = _gpu.gemm(layout, fmt, A, B, M, N, K)
        assert (D == D2).all()


# ------------------------------------------------------ 128-wide tiles --

TILE128 = [
    # (M, N, K): ragged M, N (N = 130: a second tile column of 2), K tails
    (300, 500, 400),
    (256, 1024, 1024),
    (1000, 130, 712),
    (512, 384, 4000),
    (96, 700, 64),
]


@pytest.mark.parametrize("fmt", ["f16", "bf16"])
@pytest.mark.parametrize("M,N,K", TILE128)
def test_tile128_full_check(fmt, M, N, K, splitk, monkeypatch):
    monkeypatch.setenv("DENSE_GEMM_TILE_N", "128")
    w = inputs.Workload("x", "nt", fmt, 0, 0, 0, "uniform", 0.0, 301)
    A, B = inputs.make_operands(w, M=M, N=N, K=K)
    D, st = _gpu.gemm("nt", fmt, A, B, M, N, K)
    assert st == status().OK
    check_full("nt", fmt, A, B, M, N, K, D)


@pytest.mark.parametrize("parts", ["3", "16"])
def test_tile128_forced_split(parts, monkeypatch):
    monkeypatch.setenv("DENSE_GEMM_TILE_N", "128")
    monkeypatch.setenv("DENSE_GEMM_SPLITK", parts)
    M, N, K = 520, 300, 2000
    A, B = inputs.make_operands(inputs.WORKLOADS["ragged_nt"], M=M, N=N, K=K)
    D, st = _gpu.gemm("nt", "f16", A, B, M, N, K)
    assert st == status().OK
    check_full("nt", "f16", A, B, M, N, K, D)


def test_tile128_bitwise_equals_tile256(monkeypatch):
    # each output is the same sequence of MFMA accumulations in either tile
    # width, so the results agree bit for bit (split-K off)
    monkeypatch.setenv("DENSE_GEMM_SPLITK", "off")
    M, N, K = 1000, 900, 1500
    A, B = inputs.make_operands(inputs.WORKLOADS["square_nt"], M=M, N=N, K=K)
    out = {}
    for tn in ("128", "256"):
        monkeypatch.setenv("DENSE_GEMM_TILE_N", tn)
        out[tn], st = _gpu.gemm("nt", "f16", A, B, M, N, K)
        assert st == status().OK
    assert np.array_equal(out["128"], out["256"])
