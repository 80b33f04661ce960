"""GPU parity tests of the FP8 block-scaled product (gemm_nt_e4m3_mx) against
the CPU oracle's gemm_mx, through the C ABI.

Acceptance (per element): |d_gpu - d| <= ulp_bf16(|d|) + 2^-11 * s with d the
oracle's exact FP64 value and s = sum_k |SA a SB b| (the products are exact
in FP32, so only the FP32 sum and the final rounding err).  Small-integer
inputs, whose FP32 sums are exact in any order, must give the correctly
rounded BF16 value bit for bit.  Shapes span several 256 x 256 tiles with
ragged M and N, and K values whose remainder modulo the 128-deep stage is 0,
32, 64 and 96; the full-size workloads are checked element by element in
the launch configuration the benchmark times.
"""
import numpy as np
import pytest

import oracle
from dense_gemm_08_amd import inputs
from tests import _gpu

pytestmark = pytest.mark.gpu

BYTE_CANARY = 0x7F  # an E4M3 NaN: a read of padding would show in the result


def status():
    from dense_gemm_08_amd.binding import Status
    return Status


def bytes_dev(codes, rows, cols, ld, off=0, fill=BYTE_CANARY):
    t = _gpu.torch()
    host = np.full(rows * ld + off + 64, fill, dtype=np.uint8)
    if rows and cols:
        host[off:off + rows * ld].reshape(rows, ld)[:, :cols] = codes.reshape(rows, cols)
    return t.from_numpy(host).to("cuda")


def mx_call(M, N, K, A, lda, SA, ldsa, B, ldb, SB, ldsb, D, ldd, offs=(0, 0, 0, 0, 0)):
    from dense_gemm_08_amd import binding
    t = _gpu.torch()
    ptr = lambda x, o: 0 if x is None else x.data_ptr() + o  # noqa: E731
    fn = binding.raw("gemm_nt_e4m3_mx")
    return binding.Status(fn(M, N, K, ptr(A, offs[0]), lda, ptr(SA, offs[1]), ldsa,
                             ptr(B, offs[2]), ldb, ptr(SB, offs[3]), ldsb, ptr(D, offs[4]), ldd,
                             t.cuda.current_stream().cuda_stream))


def run_mx(A, SA, B, SB, lda=None, ldb=None, ldsa=None, ldsb=None, ldd=None):
    """Upload, run, download.  Returns (D bits M x ldd, status)."""
    t = _gpu.torch()
    M, K = A.shape
    N = B.shape[0]
    nb = K // 32
    lda = K if lda is None else lda
    ldb = K if ldb is None else ldb
    ldsa = nb if ldsa is None else ldsa
    ldsb = nb if ldsb is None else ldsb
    ldd = N if ldd is None else ldd
    dA = bytes_dev(A, M, K, lda)
    dB = bytes_dev(B, N, K, ldb)
    dSA = bytes_dev(SA, M, nb, ldsa, fill=0xFF)
    dSB = bytes_dev(SB, N, nb, ldsb, fill=0xFF)
    dD = _gpu.to_dev_at(np.zeros(0, np.uint16), M, 0, ldd, 0)
    st = mx_call(M, N, K, dA, lda, dSA, ldsa, dB, ldb, dSB, ldsb, dD, ldd)
    t.cuda.synchronize()
    host = _gpu.from_dev(dD)
    assert (host[M * ldd:] == _gpu.CANARY).all()
    return host[:M * ldd].reshape(M, ldd), st


def check_full(A, SA, B, SB, D):
    M, N = A.shape[0], B.shape[0]
    d, s = oracle.gemm_mx(A, SA, B, SB)
    res = oracle.check("bf16", d, s, D[:, :N])
    assert res.ok, (res, np.unravel_index(max(res.worst_idx, 0), (M, N)))
    return d


SHAPES = [
    # (M, N, K): K mod 128 = 0, 32, 64, 96; ragged M and N; one tile to many
    (256, 256, 128),
    (300, 200, 96),
    (513, 1000, 416),
    (1024, 768, 1024),
    (64, 1100, 2080),
    (777, 530, 320),
]


@pytest.mark.parametrize("kind", ["quantised", "codes"])
@pytest.mark.parametrize("M,N,K", SHAPES)
def test_mx_full_parity(kind, M, N, K):
    A, SA, B, SB = inputs.mx_operands(M, N, K, seed=M + 7 * N + K, kind=kind)
    D, st = run_mx(A, SA, B, SB)
    assert st == status().OK
    check_full(A, SA, B, SB, D)


@pytest.mark.parametrize("M,N,K", [(520, 300, 2048), (256, 512, 160)])
def test_mx_small_integers_bit_exact(M, N, K):
    A, SA, B, SB = inputs.mx_small_integers(M, N, K, seed=K)
    D, st = run_mx(A, SA, B, SB)
    assert st == status().OK
    d, _ = oracle.gemm_mx(A, SA, B, SB)
    want = oracle.round_to("bf16", d)
    assert np.array_equal(D, want), np.argwhere(D != want)[:5]


def test_mx_leading_dimensions_and_untouched_padding():
    M, N, K = 300, 270, 352
    A, SA, B, SB = inputs.mx_operands(M, N, K, seed=11)
    D, st = run_mx(A, SA, B, SB, lda=K + 48, ldb=K + 16, ldsa=K // 32 + 3, ldsb=K // 32 + 1,
                   ldd=N + 5)
    assert st == status().OK
    assert (D[:, N:] == _gpu.CANARY).all()
    check_full(A, SA, B, SB, D)


def test_mx_repeatable():
    A, SA, B, SB = inputs.mx_operands(700, 600, 1152, seed=12, kind="codes")
    D1, st1 = run_mx(A, SA, B, SB)
    D2, st2 = run_mx(A, SA, B, SB)
    assert st1 == st2 == status().OK
    assert np.array_equal(D1, D2)


def test_mx_k_zero_writes_zeros_and_empty_writes_nothing():
    t = _gpu.torch()
    D = _gpu.empty_out(40, 50)
    st = mx_call(40, 50, 0, None, 0, None, 0, None, 0, None, 0, D, 50)
    t.cuda.synchronize()
    assert st == status().OK
    assert (_gpu.from_dev(D) == 0).all()
    D = _gpu.empty_out(8, 8)
    for M, N in ((0, 8), (8, 0)):
        st = mx_call(M, N, 64, None, 64, None, 2, None, 64, None, 2, D, 8)
        assert st == status().OK
    t.cuda.synchronize()
    assert (_gpu.from_dev(D) == _gpu.CANARY).all()


def test_mx_argument_errors_leave_d_untouched():
    S = status()
    t = _gpu.torch()
    M, N, K = 64, 64, 128
    A, SA, B, SB = inputs.mx_operands(M, N, K, seed=13)
    dA, dB = bytes_dev(A, M, K, K + 32), bytes_dev(B, N, K, K)
    dSA, dSB = bytes_dev(SA, M, 4, 4), bytes_dev(SB, N, 4, 4)
    D = _gpu.empty_out(M + 1, N + 1)
    base = dict(M=M, N=N, K=K, A=dA, lda=K, SA=dSA, ldsa=4, B=dB, ldb=K, SB=dSB, ldsb=4, D=D,
                ldd=N)
    cases = [
        (dict(K=40), S.BAD_ARG),          # K not a multiple of the 32-value block
        (dict(M=-1), S.INVALID_DIM),
        (dict(lda=K - 16), S.BAD_LD),
        (dict(ldsb=3), S.BAD_LD),
        (dict(ldd=N - 1), S.BAD_LD),
        (dict(lda=K + 8), S.MISALIGNED),  # rows not 16-byte aligned
        (dict(A=None), S.NULL_PTR),
        (dict(D=None), S.NULL_PTR),
    ]
    for change, want in cases:
        a = dict(base)
        a.update(change)
        st = mx_call(a["M"], a["N"], a["K"], a["A"], a["lda"], a["SA"], a["ldsa"], a["B"],
                     a["ldb"], a["SB"], a["ldsb"], a["D"], a["ldd"])
        assert st == want, (change, st)
    # misaligned pointers: A 8 bytes in, D at an odd byte address
    st = mx_call(M, N, K, dA, K, dSA, 4, dB, K, dSB, 4, D, N, offs=(8, 0, 0, 0, 0))
    assert st == S.MISALIGNED
    st = mx_call(M, N, K, dA, K, dSA, 4, dB, K, dSB, 4, D, N, offs=(0, 0, 0, 0, 1))
    assert st == S.MISALIGNED
    t.cuda.synchronize()
    assert (_gpu.from_dev(D) == _gpu.CANARY).all()


def test_mx_python_binding_takes_float8_tensors():
    import dense_gemm_08_amd as dg
    t = _gpu.torch()
    M, N, K = 260, 300, 256
    A, SA, B, SB = inputs.mx_operands(M, N, K, seed=14)
    dev = lambda x: t.from_numpy(x).to("cuda")  # noqa: E731
    D = dg.gemm_nt_e4m3_mx(dev(A).view(t.float8_e4m3fn), dev(SA), dev(B), dev(SB))
    t.cuda.synchronize()
    assert D.dtype == t.bfloat16 and tuple(D.shape) == (M, N)
    check_full(A, SA, B, SB, D.cpu().view(t.int16).numpy().view(np.uint16))
    # the workspace-passing form, with a workspace taken by the binding and
    # with the caller's: the same bits
    D2 = dg.gemm_nt_e4m3_mx(dev(A), dev(SA), dev(B), dev(SB), workspace=True)
    from dense_gemm_08_amd import binding
    ws = t.empty(max(binding.mx_workspace_size(M, N, K), 1), dtype=t.uint8, device="cuda")
    D3 = dg.gemm_nt_e4m3_mx(dev(A), dev(SA), dev(B), dev(SB), workspace=ws)
    t.cuda.synchronize()
    assert t.equal(D.view(t.int16), D2.view(t.int16)) and t.equal(D.view(t.int16), D3.view(t.int16))


@pytest.mark.timeout(900)
@pytest.mark.parametrize("name", ["mx_square", "mx_large"])
def test_mx_workload_full_size_every_output(name):
    # the benchmark's FP8 workloads (their seeds and recipe), in its launch
    # configuration, every output against the oracle
    t = _gpu.torch()
    w = inputs.MX_WORKLOADS[name]
    M, N, K = w.M, w.N, w.K
    print("full size %s %dx%dx%d" % (name, M, N, K), flush=True)
    A, SA, B, SB = inputs.mx_operands(M, N, K, w.seed, kind=w.kind)
    nb = K // 32
    dA, dB = t.from_numpy(A).to("cuda"), t.from_numpy(B).to("cuda")
    dSA, dSB = t.from_numpy(SA).to("cuda"), t.from_numpy(SB).to("cuda")
    D = t.empty((M, N), dtype=t.int16, device="cuda")
    st = mx_call(M, N, K, dA, K, dSA, nb, dB, K, dSB, nb, D, N)
    t.cuda.synchronize()
    assert st == status().OK
    del dA, dB, dSA, dSB
    check_full(A, SA, B, SB, D.cpu().numpy().view(np.uint16))


def test_mx_nan_scale_and_nan_element_propagate_like_the_oracle():
    M, N, K = 256, 300, 256
    A, SA, B, SB = inputs.mx_operands(M, N, K, seed=15)
    SA[3, 1] = 255   # E8M0 NaN: row 3 of D is NaN
    SB[7, 6] = 255   # column 7 of D is NaN
    A[5, 100] = 0x7F  # E4M3 NaN: row 5 of D is NaN
    D, st = run_mx(A, SA, B, SB)
    assert st == status().OK
    d, s = oracle.gemm_mx(A, SA, B, SB)
    g = oracle.decode("bf16", D)
    assert np.array_equal(np.isnan(g), np.isnan(d))
    assert np.isnan(d[3]).all() and np.isnan(d[:, 7]).all() and np.isnan(d[5]).all()
    ok = ~np.isnan(d)
    res = oracle.check("bf16", d[ok], s[ok], D[ok])
    assert res.ok, res


# ------------------------------------------------ the ends of the scale range --

def _check_in_fp32_range(A, SA, B, SB, D):
    """The acceptance bound on every output whose sum of |products| S stays
    below 2^127 (no FP32 partial sum can overflow there, in any order);
    outputs with S >= 2^127 are exempt (an FP32 partial sum may overflow:
    the FP32-accumulating product may return +-Inf or NaN where the FP64
    oracle is finite) but must be non-finite or within the bound.  Returns
    the numbers of checked, exempt and non-finite exempt outputs."""
    d, s = oracle.gemm_mx(A, SA, B, SB)
    inside = s < 2.0 ** 127
    res = oracle.check("bf16", d[inside], s[inside], D[inside])
    assert res.ok, res
    g = D[~inside]
    finite = np.isfinite(oracle.decode("bf16", g))
    res = oracle.check("bf16", d[~inside][finite], s[~inside][finite], g[finite])
    assert res.ok, res
    return int(inside.sum()), int((~inside).sum()), int((~finite).sum())


def _range_operands(case, M, N, K, seed):
    rng = np.random.default_rng(seed)
    nb = K // 32
    A = rng.choice(inputs.E4M3_FINITE, size=(M, K))
    B = rng.choice(inputs.E4M3_FINITE, size=(N, K))
    if case == "compensated":
        # every 32-wide block of A at scale 2^t, of B at 2^-t (plus a little
        # jitter), t from -126 to 126 over the blocks: scale codes from the
        # ends of the E8M0 range while the products stay near 1
        t = np.linspace(-126, 126, nb).round().astype(int)
        SA = np.clip(127 + t[None, :] + rng.integers(-3, 4, (M, nb)), 0, 254).astype(np.uint8)
        SB = np.clip(127 - t[None, :] + rng.integers(-3, 4, (N, nb)), 0, 254).astype(np.uint8)
        assert SA.min() <= 3 and SA.max() >= 251 and SB.min() <= 3 and SB.max() >= 251
        return A, SA, B, SB
    e = {"top": 100, "bottom_normal": -140, "bottom_subnormal": -150, "bottom_zero": -254}.get(case)
    if e is not None:
        # every product scaled by 2^e: top, sums near 2^121; bottom, results in
        # BF16's normal range, its subnormal range, and far below it
        SA = np.full((M, nb), max(0, 127 + e // 2), np.uint8)
        SB = np.full((N, nb), max(0, 127 + e - e // 2), np.uint8)
        return A, SA, B, SB
    SA = rng.integers(118, 137, (M, nb)).astype(np.uint8)
    SB = rng.integers(118, 137, (N, nb)).astype(np.uint8)
    if case == "overflow_rows":
        SA[:16] = 254  # rows 0..15: products beyond the FP32 range
    elif case == "cancelling_overflow":
        # rows 0..7: two blocks of +-448 x 448 at scale 2^127 x 2^73 cancel
        # exactly in FP64; an FP32 partial sum overflows on the way
        A[:8, 0:32], A[:8, 32:64] = 0x7E, 0xFE
        B[:, 0:64] = 0x7E
        SA[:8, 0:2], SB[:, 0:2] = 254, 200
    return A, SA, B, SB


@pytest.mark.parametrize("case", ["compensated", "top", "bottom_normal", "bottom_subnormal",
                                  "bottom_zero", "overflow_rows", "cancelling_overflow"])
def test_mx_scale_range_ends(case):
    M, N, K = 256, 272, 512
    A, SA, B, SB = _range_operands(case, M, N, K, seed=len(case))
    D, st = run_mx(A, SA, B, SB)
    assert st == status().OK
    checked, exempt, nonfinite = _check_in_fp32_range(A, SA, B, SB, D)
    print("%s: %d outputs checked, %d exempt (%d of them non-finite)"
          % (case, checked, exempt, nonfinite), flush=True)
    if case in ("compensated", "top") or case.startswith("bottom"):
        assert exempt == 0 and checked == M * N
    else:
        # only the rows built to overflow are exempt; the rest pass the bound
        assert checked >= (M - 16) * N and 0 < exempt <= 16 * N


# ------------------------------------------------ the small-output kernel --

MX_SPLIT = [
    # (M, N, K) planned with split-K on a 256-CU device: one tile in 16
    # parts, ragged tiles with K mod 128 = 32 (the leading pad of the first
    # stage falls in part 0 only), one tile row (partial tiles with row
    # blocks outside D), M <= 128 past the small kernel's K, and a last wave
    # of 33 tiles after a full one
    (256, 256, 8192), (300, 200, 4128), (129, 520, 2080), (100, 72, 8224), (4097, 4097, 1024),
    (600, 520, 3104),
]


def _mx_plan(M, N, K):
    import ctypes
    from dense_gemm_08_amd import binding
    t = _gpu.torch()
    cus = t.cuda.get_device_properties(0).multi_processor_count
    out = (ctypes.c_int64 * 10)()
    assert binding.load_library().gemm_nt_e4m3_mx_plan(M, N, K, cus, out) == 0
    return list(out)


@pytest.mark.parametrize("kind", ["quantised", "codes"])
@pytest.mark.parametrize("M,N,K", MX_SPLIT, ids=lambda v: str(v))
def test_mx_split_k_full_parity(kind, M, N, K):
    plan = _mx_plan(M, N, K)
    if plan[8] == 1:
        pytest.skip("not split on a device with this CU count")
    A, SA, B, SB = inputs.mx_operands(M, N, K, seed=M + 5 * N + K, kind=kind)
    D, st = run_mx(A, SA, B, SB)
    assert st == status().OK
    check_full(A, SA, B, SB, D)
    # the parts are added in a fixed order: a rerun is equal
    D2, _ = run_mx(A, SA, B, SB)
    assert np.array_equal(D, D2)


@pytest.mark.parametrize("M,N,K", [(256, 256, 8192), (300, 200, 4128), (4097, 4097, 1024)],
                         ids=lambda v: str(v))
def test_mx_split_k_small_integers_bit_exact(M, N, K):
    # exact FP32 sums in any order: the split gives the correctly rounded value
    if _mx_plan(M, N, K)[8] == 1:
        pytest.skip("not split on a device with this CU count")
    A, SA, B, SB = inputs.mx_small_integers(M, N, K, seed=K + 1)
    D, st = run_mx(A, SA, B, SB, ldd=N + 3)
    assert st == status().OK
    assert (D[:, N:] == _gpu.CANARY).all()
    d, _ = oracle.gemm_mx(A, SA, B, SB)
    want = oracle.round_to("bf16", d)
    assert np.array_equal(D[:, :N], want), np.argwhere(D[:, :N] != want)[:5]


def test_mx_split_k_workspace_call_equals_plain_call():
    import ctypes
    from dense_gemm_08_amd import binding
    t = _gpu.torch()
    lib = binding.load_library()
    M, N, K = 300, 200, 4128
    if _mx_plan(M, N, K)[8] == 1:
        pytest.skip("not split on a device with this CU count")
    XA, XSA, XB, XSB = [t.from_numpy(x).cuda() for x in inputs.mx_operands(M, N, K, seed=74)]
    nb = K // 32
    need = ctypes.c_size_t()
    assert lib.gemm_nt_e4m3_mx_workspace_size(M, N, K, 0, ctypes.byref(need)) == 0
    panels = (2 + 1) * 33 * 1024
    assert need.value > panels  # the partial tiles follow the scale panels
    ws = _gpu.workspace(need.value)
    h = t.cuda.current_stream().cuda_stream
    args = (M, N, K, XA.data_ptr(), K, XSA.data_ptr(), nb, XB.data_ptr(), K, XSB.data_ptr(), nb)
    D1, D2, D3, D4 = (_gpu.empty_out(M, N) for _ in range(4))
    assert lib.gemm_nt_e4m3_mx(*args, D1.data_ptr(), N, h) == 0
    assert lib.gemm_nt_e4m3_mx_ex(*args, D2.data_ptr(), N, ws.data_ptr(), need.value, h) == 0
    # a workspace with room for the panels only is refused before any launch
    assert status()(lib.gemm_nt_e4m3_mx_ex(*args, D3.data_ptr(), N, ws.data_ptr(), panels,
                                           h)) == status().WORKSPACE_TOO_SMALL
    # the workspace's old contents do not matter: a second call over the
    # first call's partials gives the same result
    assert lib.gemm_nt_e4m3_mx_ex(*args, D4.data_ptr(), N, ws.data_ptr(), need.value, h) == 0
    t.cuda.synchronize()
    assert (_gpu.from_dev(D1) == _gpu.from_dev(D2)).all()
    assert (_gpu.from_dev(D1) == _gpu.from_dev(D4)).all()
    assert (_gpu.from_dev(D3) == _gpu.CANARY).all()


def test_mx_workspace_calls_on_two_streams():
    # split-K calls (and one with scale panels only), each given its own
    # workspace, issued back to back on two streams that do not wait for
    # each other: the bits of the same calls run alone
    import ctypes
    from dense_gemm_08_amd import binding
    t = _gpu.torch()
    lib = binding.load_library()
    shapes = [(300, 200, 4128), (256, 256, 8192), (520, 300, 416)]
    cases = []
    for i, (M, N, K) in enumerate(shapes):
        ops = [t.from_numpy(x).cuda() for x in inputs.mx_operands(M, N, K, seed=90 + i)]
        need = ctypes.c_size_t()
        assert lib.gemm_nt_e4m3_mx_workspace_size(M, N, K, 0, ctypes.byref(need)) == 0
        assert need.value > 0
        cases.append((M, N, K, ops, need.value))

    def call(c, D, ws, stream):
        M, N, K, (A, SA, B, SB), need = c
        nb = K // 32
        return lib.gemm_nt_e4m3_mx_ex(M, N, K, A.data_ptr(), K, SA.data_ptr(), nb, B.data_ptr(), K,
                                      SB.data_ptr(), nb, D.data_ptr(), N, ws.data_ptr(), need,
                                      stream.cuda_stream)
    main = t.cuda.current_stream()
    ref = []
    for c in cases:
        D = _gpu.empty_out(c[0], c[1])
        assert call(c, D, _gpu.workspace(c[4]), main) == 0
        t.cuda.synchronize()
        ref.append(_gpu.from_dev(D))
    streams = [t.cuda.Stream(), t.cuda.Stream()]
    jobs = []
    for it in range(12):
        for si in range(2):
            k = (it + si) % len(cases)
            jobs.append((k, si, _gpu.empty_out(cases[k][0], cases[k][1]),
                         _gpu.workspace(cases[k][4])))
    for st in streams:
        st.wait_stream(main)
    for k, si, D, ws in jobs:
        with t.cuda.stream(streams[si]):
            assert call(cases[k], D, ws, streams[si]) == 0
    for st in streams:
        main.wait_stream(st)
    t.cuda.synchronize()
    for k, _, D, _ in jobs:
        assert (_gpu.from_dev(D) == ref[k]).all(), k


MX_SMALL = [
    # (M, N, K) for the small-output kernel (M <= 128, K <= 8192, and one
    # 16-row tile row, or at most 1024 tiles of 32 x 32, or 1536 with tiles x
    # K <= 2^23): K mod 128 = 0, 32, 64, 96, the longest K, one tile row past
    # 512 tiles, ragged tiles, one block; on 256 CUs, 16 x 16 tiles for the
    # first seven, 32 x 16 for (128, 1024, 96), (64, 2200, 1056), (120,
    # 1536, 4096) and (128, 1100, 1056), 32 x 32 for the last four (ragged
    # in M, N and K; the 1536-tile band)
    (128, 128, 4096), (100, 72, 8192), (1, 4096, 1024), (16, 8200, 480), (5, 300, 224),
    (33, 17, 32), (64, 1000, 2080), (128, 1024, 96), (64, 2200, 1056), (120, 1536, 4096),
    (128, 1100, 1056), (33, 8200, 1056), (100, 2600, 2144), (128, 4096, 8192),
    (96, 16384, 4096),
]


def _mx_small(M, N, K):
    import ctypes
    from dense_gemm_08_amd import binding
    need = ctypes.c_size_t(1)
    assert binding.load_library().gemm_nt_e4m3_mx_workspace_size(M, N, K, 0,
                                                                 ctypes.byref(need)) == 0
    return need.value == 0


@pytest.mark.parametrize("kind", ["quantised", "codes"])
@pytest.mark.parametrize("M,N,K", MX_SMALL, ids=lambda v: str(v))
def test_mx_small_output_full_parity(kind, M, N, K):
    assert _mx_small(M, N, K), "planned for the tiled kernel"
    A, SA, B, SB = inputs.mx_operands(M, N, K, seed=M + 7 * N + K + 1, kind=kind)
    D, st = run_mx(A, SA, B, SB)
    assert st == status().OK
    check_full(A, SA, B, SB, D)
    # the eight waves' sums are added in a fixed order: a rerun is equal
    D2, _ = run_mx(A, SA, B, SB)
    assert np.array_equal(D, D2)


@pytest.mark.timeout(300)
@pytest.mark.parametrize("M,N,K,small", [
    # the ends of the benchmark's small-M FP8 sweep: one row at the widest N,
    # the longest K at M <= 16, the small kernel's 1024 tiles of 32 x 32 at
    # the longest K, and the tiled kernel split at M = 128 past 1536 tiles
    (1, 16384, 4096, True), (16, 8192, 8192, True), (64, 16384, 8192, True),
    (128, 16384, 4096, False)], ids=lambda v: str(v))
def test_mx_small_m_sweep_shapes_every_output(M, N, K, small):
    assert _mx_small(M, N, K) == small
    print("small-M sweep shape %dx%dx%d" % (M, N, K), flush=True)
    A, SA, B, SB = inputs.mx_operands(M, N, K, seed=M + N + K, kind="quantised")
    D, st = run_mx(A, SA, B, SB)
    assert st == status().OK
    check_full(A, SA, B, SB, D)


def test_mx_small_output_tile_shapes_give_the_same_bits():
    # every output's sum is the same sequence of MFMAs in 16 x 16, 32 x 16
    # and 32 x 32 tiles: the products of A with the first rows of one B agree
    # bit for bit on their common columns, whichever tile each runs in
    for M, K, widths in [(64, 1056, (1000, 4200)), (128, 2080, (300, 1100, 4200))]:
        A, SA, B, SB = inputs.mx_operands(M, max(widths), K, seed=M + K)
        tiles = {tuple(_mx_plan(M, n, K)[:2]) for n in widths}
        assert len(tiles) == len(widths), tiles  # distinct shapes (on 256 CUs: all three)
        outs = []
        for n in widths:
            D, st = run_mx(A, SA, B[:n], SB[:n])
            assert st == status().OK
            outs.append(D)
        for D in outs[1:]:
            assert np.array_equal(D[:, :widths[0]], outs[0]), (M, K)
        check_full(A, SA, B[:widths[0]], SB[:widths[0]], outs[0])


@pytest.mark.parametrize("M,N,K", [(120, 200, 2048), (100, 8200, 2080)], ids=lambda v: str(v))
def test_mx_small_output_small_integers_bit_exact_and_leading_dimensions(M, N, K):
    # 16 x 16 tiles, and 32 x 32 (ragged in M, N and K) on 256 CUs
    assert _mx_small(M, N, K)
    A, SA, B, SB = inputs.mx_small_integers(M, N, K, seed=K + 1)
    d, _ = oracle.gemm_mx(A, SA, B, SB)
    want = oracle.round_to("bf16", d)
    D, st = run_mx(A, SA, B, SB)
    assert st == status().OK
    assert np.array_equal(D, want), np.argwhere(D != want)[:5]
    # padded rows (NaN codes in the padding) and an odd-sized D row: the
    # kernel reads only [0, K) of each row and [0, K/32) of each scale row
    D, st = run_mx(A, SA, B, SB, lda=K + 48, ldb=K + 16, ldsa=K // 32 + 3, ldsb=K // 32 + 1,
                   ldd=N + 3)
    assert st == status().OK
    assert np.array_equal(D[:, :N], want)
    assert (D[:, N:] == _gpu.CANARY).all()


@pytest.mark.parametrize("M,N,K", [(64, 80, 256), (64, 4200, 256)], ids=lambda v: str(v))
def test_mx_small_output_nan_propagates_like_the_oracle(M, N, K):
    # 16 x 16 tiles, and 32 x 32 on 256 CUs
    assert _mx_small(M, N, K)
    A, SA, B, SB = inputs.mx_operands(M, N, K, seed=16)
    SA[3, 1] = 255   # E8M0 NaN: row 3 of D is NaN
    SB[7, 6] = 255   # column 7 of D is NaN
    A[5, 100] = 0x7F  # E4M3 NaN: row 5 of D is NaN
    D, st = run_mx(A, SA, B, SB)
    assert st == status().OK
    d, s = oracle.gemm_mx(A, SA, B, SB)
    g = oracle.decode("bf16", D)
    assert np.array_equal(np.isnan(g), np.isnan(d))
    ok = ~np.isnan(d)
    res = oracle.check("bf16", d[ok], s[ok], D[ok])
    assert res.ok, res


@pytest.mark.parametrize("N", [272, 8200])
@pytest.mark.parametrize("case", ["compensated", "top", "bottom_subnormal", "overflow_rows"])
def test_mx_small_output_scale_range_ends(case, N):
    # 16 x 16 tiles, and 32 x 32 on 256 CUs
    M, K = 64, 512
    assert _mx_small(M, N, K)
    A, SA, B, SB = _range_operands(case, M, N, K, seed=len(case) + 1)
    D, st = run_mx(A, SA, B, SB)
    assert st == status().OK
    checked, exempt, nonfinite = _check_in_fp32_range(A, SA, B, SB, D)
    if case == "overflow_rows":
        assert checked >= (M - 16) * N and 0 < exempt <= 16 * N
    else:
        assert exempt == 0 and checked == M * N
