"""GPU parity tests: the HIP path (through the C ABI) against the CPU oracle.

Acceptance (per element): |d_gpu - d| <= ulp_out(|d|) + 2^-11 * sum_k |a*b|,
with d the oracle's FP64 value.  Where the FP32 sum is exact (small-integer,
identity and all-ones inputs) the result must equal the oracle's correctly
rounded value bit for bit.  Shapes: every workload at a reduced size checked
element by element (several tiles and a ragged tail in M, N and K), and every
workload at its full size, in the launch configuration the benchmark times,
element by element as well (the oracle's full product of the largest,
8192 x 17408 x 5120, takes about a minute on 16 host cores).
"""
import functools

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
def splitk(request):
    """Run with the library's own split-K choice (the plain entry point), and
    with split-K disabled (dense_gemm_ex with split_k = 1): the plan
    overrides as _gpu.gemm takes them."""
    return None if request.param == "auto" else (1, 0)


@pytest.mark.parametrize("name,M,N,K", REDUCED)
def test_workload_reduced_full_check(name, M, N, K, splitk):
    w = inputs.WORKLOADS[name]
    A, B = inputs.make_operands(w, M=M, N=N, K=K)
    D, st = _gpu.gemm(w.layout, w.fmt, A, B, M, N, K, opts=splitk)
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

@functools.lru_cache(maxsize=1)
def square_nt_reference():
    """Operands and oracle (d, s) of the 4096^3 FP16 A.B^T workload (shared
    by the tests of the library kernel and of the step ladder at that size)."""
    w = inputs.WORKLOADS["square_nt"]
    A, B = inputs.make_operands(w)
    d, s = oracle.gemm("nt", "f16", A, B)
    return A, B, d, s


def check_against(fmt, d, s, D, what):
    res = oracle.check(fmt, d, s, D[:, :d.shape[1]])
    assert res.ok, (what, res, np.unravel_index(max(res.worst_idx, 0), d.shape))


@pytest.mark.timeout(900)
@pytest.mark.parametrize("name", ["single_tile", "k_loop", "square_nt", "large_nn", "ragged_nt"])
def test_workload_full_size_every_output(name):
    # the benchmark's call (the plain entry point, the library's own plan:
    # 256 x 256 tiles for the three large workloads, the small-output kernel
    # for single_tile and k_loop),
    # every output against the oracle
    w = inputs.WORKLOADS[name]
    print("full size %s %dx%dx%d" % (name, w.M, w.N, w.K), flush=True)
    if name == "square_nt":
        A, B, d, s = square_nt_reference()
    else:
        A, B = inputs.make_operands(w)
        d, s = oracle.gemm(w.layout, w.fmt, A, B)
    D, st = _gpu.gemm(w.layout, w.fmt, A, B, w.M, w.N, w.K)
    assert st == status().OK
    check_against(w.fmt, d, s, D, name)


@pytest.mark.parametrize("layout,fmt,M,N,K", [("nt", "f16", 4096, 8192, 1024),
                                              ("nn", "bf16", 1536, 17408, 1024)])
def test_two_tiles_per_workgroup_every_output(layout, fmt, M, N, K):
    # persistent workgroups that compute a second tile after their first
    # (the ring slot carried across tiles, the first tile's stores draining
    # under the second tile's loads), no split: 512 tiles of 256 x 256 on 256
    # workgroups (A.B^T), and 408 tiles with 152 workgroups doing two (A.B,
    # the large A.B workload's N, layout and distribution); every output
    w = inputs.WORKLOADS["square_nt" if layout == "nt" else "large_nn"]
    A, B = inputs.make_operands(w, seed=M + N + K, M=M, N=N, K=K)
    D, st = _gpu.gemm(layout, fmt, A, B, M, N, K)
    assert st == status().OK
    check_full(layout, fmt, A, B, M, N, K, D)


@pytest.mark.timeout(600)
@pytest.mark.parametrize("name", ["large_nn_rows8", "large_nn_cols8", "large_nn_rows4",
                                  "large_nn_cols4", "large_nn_rows2", "large_nn_cols2"])
def test_shard_of_large_nn_every_output(name):
    # one GPU's share of the 8192 x 17408 x 5120 A.B product split over 8,
    # 4 or 2 GPUs, as the benchmark times it: e.g. 1024 rows (272 tiles on
    # 256 workgroups, the last 16 split 16 ways in K), 2176 columns (288
    # tiles, 32 split 8 ways), 4096 rows (1088 tiles, 64 split 4 ways);
    # every output
    w = inputs.SHARD_WORKLOADS[name]
    print("shard %s %dx%dx%d" % (name, w.M, w.N, w.K), flush=True)
    A, B = inputs.make_operands(w)
    D, st = _gpu.gemm(w.layout, w.fmt, A, B, w.M, w.N, w.K)
    assert st == status().OK
    check_full(w.layout, w.fmt, A, B, w.M, w.N, w.K, D)


# ------------------------------------------------- bitwise special cases --

@pytest.mark.timeout(600)
@pytest.mark.parametrize("M,N,K", [(8192, 16384 + 128, 4096), (8192, 4096, 16384 + 40),
                                   (8192, 1024, 1024), (8192, 1024, 16384)])
def test_m8192_sweep_shapes_every_output(M, N, K):
    # extreme shapes of the benchmark's M = 8192 sweep (FP16 A.B^T, N(0,1)/8):
    # the widest N with a ragged last tile column, the deepest K with a partial
    # last step (both operands repacked), and the narrowest N (128-wide
    # tiles; split-K at K = 16384); every output against the oracle
    w = inputs.WORKLOADS["square_nt"]
    A, B = inputs.make_operands(w, seed=M + N + K, M=M, N=N, K=K)
    D, st = _gpu.gemm("nt", "f16", A, B, M, N, K)
    assert st == status().OK
    check_full("nt", "f16", A, B, M, N, K, D)


@pytest.mark.parametrize("layout,fmt", [("nt", "f16"), ("nn", "bf16"), ("nt", "bf16"), ("nn", "f16")])
def test_small_integers_exact(layout, fmt, splitk):
    # entries in {-3..3}: every FP32 partial sum is an exact integer, so the
    # result is the exactly rounded integer sum (sums up to 9K exceed the
    # FP16/BF16 integer range, so this pins round-to-nearest-even)
    M, N, K = 264, 392, 1032
    sa, sb = inputs.operand_shapes(layout, M, N, K)
    A = inputs.small_integers(fmt, sa, seed=31)
    B = inputs.small_integers(fmt, sb, seed=32)
    D, st = _gpu.gemm(layout, fmt, A, B, M, N, K, opts=splitk)
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
def test_forced_split_k(layout, fmt, parts):
    # split-K forced on shapes of several tiles, a ragged K tail and parts of
    # unequal length; the summation order is fixed, so a rerun is bitwise equal
    opts = (int(parts), 0)
    w = inputs.Workload("x", layout, fmt, 0, 0, 0, "uniform", 0.0, 71)
    M, N, K = 300, 264, 1000
    A, B = inputs.make_operands(w, M=M, N=N, K=K)
    D, st = _gpu.gemm(layout, fmt, A, B, M, N, K, opts=opts)
    assert st == status().OK
    check_full(layout, fmt, A, B, M, N, K, D)
    D2, _ = _gpu.gemm(layout, fmt, A, B, M, N, K, opts=opts)
    assert (D == D2).all()


@pytest.mark.parametrize("layout,fmt", [("nt", "f16"), ("nn", "bf16")])
@pytest.mark.parametrize("parts", ["off", "4"])
def test_k_remainder_equals_leading_zero_padding(layout, fmt, parts):
    # K = 4000 is not a multiple of the 64-deep K step: the kernel pads its
    # first step in front (k from -32), so the result must equal, bit for bit,
    # the same data with 32 zero columns of A (and zero k-rows or columns of
    # B) put in front, K = 4032, which has the same steps, unsplit or in 4
    # parts of 16 steps
    opts = (1, 0) if parts == "off" else (int(parts), 0)
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
    D1, _ = _gpu.gemm(layout, fmt, A, B, M, N, K, opts=opts)
    D2, _ = _gpu.gemm(layout, fmt, Ap, Bp, M, N, Kp, opts=opts)
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


# ---------------------------------------------------- small-output kernel --

SMALL = [
    # (M, N, K) planned for the small-output kernel (A.B^T, M <= 128, K <=
    # 16384, and one tile row, or at most 512 tiles of 16 x 16, or 32 x 32
    # tiles x K at most 2^21): the longest K (32 chunks per wave), ragged
    # tiles with K not a multiple of the 64-deep chunks, the 512-tile limit
    # at one tile row and at eight, one tile row past it, a K below 8
    # (repacked), one chunk shared by fewer than the eight waves; on 256
    # CUs 32 x 16 tiles for (128, 1024, 64), (128, 1100, 1000) and (17, 4112,
    # 4096) (17 of 32 rows), 32 x 32 for the last three (ragged in M, N and
    # K; 32 x 32 tiles x K = 2^21 exactly)
    (128, 128, 16384), (100, 72, 8000), (1, 8192, 520), (128, 1024, 64), (16, 8200, 1000),
    (3, 20000, 72), (5, 3, 7), (17, 130, 1000), (128, 128, 448), (128, 1100, 1000),
    (17, 4112, 4096), (100, 2600, 1000), (64, 4096, 4096), (48, 8192, 4096),
]


@pytest.mark.parametrize("fmt", ["f16", "bf16"])
@pytest.mark.parametrize("M,N,K", SMALL, ids=lambda v: str(v))
def test_small_output_kernel_full_check(fmt, M, N, K):
    import ctypes
    from dense_gemm_08_amd import binding
    out = (ctypes.c_int64 * 10)()
    assert binding.load_library().dense_gemm_plan(0, M, N, K, 256, out) == 0
    assert out[7] == 512, "planned for the tiled kernel"
    w = inputs.Workload("x", "nt", fmt, 0, 0, 0, "uniform", 0.0, 111)
    A, B = inputs.make_operands(w, seed=M + N + K, M=M, N=N, K=K)
    D, st = _gpu.gemm("nt", fmt, A, B, M, N, K)
    assert st == status().OK
    check_full("nt", fmt, A, B, M, N, K, D)
    # the eight waves' blocks are summed in a fixed order: a rerun is equal
    D2, _ = _gpu.gemm("nt", fmt, A, B, M, N, K)
    assert (D == D2).all()


@pytest.mark.parametrize("fmt", ["f16", "bf16"])
def test_small_output_kernel_tile_shapes_give_the_same_bits(fmt):
    # every output's sum is the same sequence of MFMAs in 16 x 16, 32 x 16
    # and 32 x 32 tiles: the products of A with the first rows of one B
    # agree bit for bit on their common columns, whichever tile each runs in
    import ctypes
    from dense_gemm_08_amd import binding
    lib = binding.load_library()
    cus = _gpu.torch().cuda.get_device_properties(0).multi_processor_count
    out = (ctypes.c_int64 * 10)()
    w = inputs.Workload("x", "nt", fmt, 0, 0, 0, "uniform", 0.0, 141)
    for M, K, widths in [(64, 1000, (1000, 4200)), (128, 1000, (300, 1100, 4200))]:
        A, B = inputs.make_operands(w, seed=M + K, M=M, N=max(widths), K=K)
        tiles = set()
        for n in widths:
            assert lib.dense_gemm_plan(0, M, n, K, cus, out) == 0 and out[7] == 512
            tiles.add((out[0], out[1]))
        assert len(tiles) == len(widths), tiles  # distinct shapes (on 256 CUs: all three)
        outs = []
        for n in widths:
            D, st = _gpu.gemm("nt", fmt, A, B[:n], M, n, K)
            assert st == status().OK
            outs.append(D)
        for D in outs[1:]:
            assert (D[:, :widths[0]] == outs[0]).all(), (M, K)
        check_full("nt", fmt, A, B[:widths[0]], M, widths[0], K, outs[0])


@pytest.mark.parametrize("fmt", ["f16", "bf16"])
def test_small_output_kernel_small_integers_exact(fmt):
    # exact integer sums up to 9K: the correctly rounded value bit for bit,
    # equal to the tiled kernel's (an option asks for it) bit for bit
    M, N, K = 120, 100, 3000
    A = inputs.small_integers(fmt, (M, K), seed=33)
    B = inputs.small_integers(fmt, (N, K), seed=34)
    D, st = _gpu.gemm("nt", fmt, A, B, M, N, K)
    assert st == status().OK
    d, _ = oracle.gemm("nt", fmt, A, B)
    assert (D == oracle.round_to(fmt, d)).all()
    Dt, st = _gpu.gemm("nt", fmt, A, B, M, N, K, opts=(1, 0))
    assert st == status().OK
    assert (Dt == D).all()


SMALL_NN = [
    # (M, N, K) of A.B planned for the small-output kernel (also K <= 4096
    # and at most 21 * 2^20 B elements streamed): the longest K, ragged tiles
    # with K not a multiple of the 64-deep chunks, the streamed-elements
    # limit exactly, one tile row past 512 tiles, N not a multiple of 8 (B
    # repacked) at several widths, a K below 8 (A repacked), one chunk
    # shared by fewer than the eight waves
    (128, 128, 4096), (100, 72, 4000), (1, 5376, 4096), (16, 8200, 1000), (3, 20000, 72),
    (5, 3, 7), (17, 130, 1000), (128, 1024, 64), (33, 266, 448),
]


def _nn_small(M, N, K):
    import ctypes
    from dense_gemm_08_amd import binding
    out = (ctypes.c_int64 * 10)()
    assert binding.load_library().dense_gemm_plan(1, M, N, K, 256, out) == 0
    return out[7] == 512


@pytest.mark.parametrize("fmt", ["bf16", "f16"])
@pytest.mark.parametrize("M,N,K", SMALL_NN, ids=lambda v: str(v))
def test_small_output_kernel_nn_full_check(fmt, M, N, K):
    assert _nn_small(M, N, K), "planned for the tiled kernel"
    w = inputs.Workload("x", "nn", fmt, 0, 0, 0, "uniform", 0.0, 113)
    A, B = inputs.make_operands(w, seed=M + 3 * N + K, M=M, N=N, K=K)
    D, st = _gpu.gemm("nn", fmt, A, B, M, N, K)
    assert st == status().OK
    check_full("nn", fmt, A, B, M, N, K, D)
    D2, _ = _gpu.gemm("nn", fmt, A, B, M, N, K)
    assert (D == D2).all()
    # the same chunks, fragments and MFMA order as A @ B.T with B transposed
    # (its B fragments come from LDS rows instead of transposing reads): the
    # two products are equal bit for bit
    Bt = np.ascontiguousarray(B.reshape(K, N).T)
    Dt, st = _gpu.gemm("nt", fmt, A, Bt, M, N, K)
    assert st == status().OK
    assert (Dt == D).all()


@pytest.mark.parametrize("fmt", ["bf16", "f16"])
def test_small_output_kernel_nn_small_integers_exact(fmt):
    # exact integer sums: the correctly rounded value bit for bit, equal to
    # the tiled kernel's (an option asks for it)
    M, N, K = 120, 104, 3000
    assert _nn_small(M, N, K)
    A = inputs.small_integers(fmt, (M, K), seed=35)
    B = inputs.small_integers(fmt, (K, N), seed=36)
    D, st = _gpu.gemm("nn", fmt, A, B, M, N, K)
    assert st == status().OK
    d, _ = oracle.gemm("nn", fmt, A, B)
    assert (D == oracle.round_to(fmt, d)).all()
    Dt, st = _gpu.gemm("nn", fmt, A, B, M, N, K, opts=(1, 0))
    assert st == status().OK
    assert (Dt == D).all()


def test_small_output_kernel_nn_leading_dimensions_and_offsets():
    # padded rows (B read in place: N and ldb multiples of 8), then pointers
    # off 16-byte alignment (both operands repacked); D's padding untouched
    M, N, K = 40, 520, 1000
    assert _nn_small(M, N, K)
    w = inputs.Workload("x", "nn", "bf16", 0, 0, 0, "uniform", 0.0, 117)
    A, B = inputs.make_operands(w, seed=9, M=M, N=N, K=K)
    D, st = _gpu.gemm("nn", "bf16", A, B, M, N, K, lda=K + 24, ldb=N + 40, ldd=N + 3)
    assert st == status().OK
    assert (D[:, N:] == _gpu.CANARY).all()
    check_full("nn", "bf16", A, B, M, N, K, D[:, :N])
    D2, st = _gpu.gemm("nn", "bf16", A, B, M, N, K, lda=K + 1, ldb=N + 5, ldd=N, a_off=1, b_off=3,
                       d_off=1)
    assert st == status().OK
    assert (D2 == D[:, :N]).all()


# ------------------------------------------------------ 128-row tiles --

TALL = [
    # (layout, fmt, M, N, K) for the tiled kernel with 128-row tiles (M <= 128
    # and not a small-output product: K > 16384, or more than 512 tiles of
    # 16 x 16 with M > 16 and, for A.B^T, 32 x 32 tiles x K above 2^21, or
    # A.B with K > 4096 or streaming more than 21 * 2^20 B elements through
    # 16 x 16 tiles): both widths, split and unsplit, ragged edges
    ("nt", "f16", 64, 8200, 8200), ("nt", "bf16", 100, 4200, 6000),
    ("nt", "f16", 128, 128, 20000), ("nn", "bf16", 128, 1000, 4000), ("nn", "f16", 17, 2600, 5000),
    ("nn", "bf16", 1, 6200, 4100),
]


@pytest.mark.parametrize("layout,fmt,M,N,K", TALL, ids=lambda v: str(v))
def test_128_row_tiles_full_check(layout, fmt, M, N, K):
    import ctypes
    from dense_gemm_08_amd import binding
    out = (ctypes.c_int64 * 10)()
    assert binding.load_library().dense_gemm_plan(0 if layout == "nt" else 1, M, N, K, 256,
                                                  out) == 0
    assert out[0] == 128, list(out)
    w = inputs.Workload("x", layout, fmt, 0, 0, 0, "uniform", 0.0, 121)
    A, B = inputs.make_operands(w, seed=M + N + K, M=M, N=N, K=K)
    D, st = _gpu.gemm(layout, fmt, A, B, M, N, K)
    assert st == status().OK
    check_full(layout, fmt, A, B, M, N, K, D)
    D2, _ = _gpu.gemm(layout, fmt, A, B, M, N, K)
    assert (D == D2).all()


@pytest.mark.parametrize("layout,fmt", [("nt", "f16"), ("nn", "bf16")])
def test_128_row_tiles_equal_256_row_tiles(layout, fmt):
    # each output accumulates its K steps in the same order whatever the tile
    # rows: the M = 128 product (128-row tiles) equals rows 0..127 of the
    # M = 129 product (256-row tiles) bit for bit, split-K off
    w = inputs.Workload("x", layout, fmt, 0, 0, 0, "uniform", 0.0, 131)
    N, K = 1000, 1200
    A, B = inputs.make_operands(w, M=129, N=N, K=K)
    D129, st = _gpu.gemm(layout, fmt, A, B, 129, N, K, opts=(1, 0))
    assert st == status().OK
    D128, st = _gpu.gemm(layout, fmt, A[:128], B, 128, N, K, opts=(1, 0))
    assert st == status().OK
    assert (D128 == D129[:128]).all()
    check_full(layout, fmt, A[:128], B, 128, N, K, D128)


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
    (128, 128, 4001, 0, 0, 0, 1, 1, 1),  # the small-output kernel
    (256, 128, 4001, 0, 0, 0, 1, 1, 1),  # + split-K
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
    # 8188 and up are copied by a second pass.  Every output against the
    # oracle.
    w = inputs.WORKLOADS["square_nt"]
    M, N, K = 8200, 256, 16390
    A, B = inputs.make_operands(w, seed=77, M=M, N=N, K=K)
    D, st = _gpu.gemm("nt", "f16", A, B, M, N, K)
    assert st == status().OK
    check_full("nt", "f16", A, B, M, N, K, D)


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
    A1, B1 = inputs.make_operands(w, seed=61, M=256, N=128, K=4096)           # split-K
    wn = inputs.WORKLOADS["large_nn"]
    A2, B2 = inputs.make_operands(wn, seed=62, M=264, N=304, K=1032)          # repacked A
    A1d, B1d = _gpu.to_dev(A1, 256, 4096), _gpu.to_dev(B1, 128, 4096)
    A2d, B2d = _gpu.to_dev(A2, 264, 1032, ld=1033), _gpu.to_dev(B2, 1032, 304)
    XA, XSA, XB, XSB = [t.from_numpy(x).cuda() for x in inputs.mx_operands(280, 300, 160, seed=63)]
    mx = binding_raw("gemm_nt_e4m3_mx")

    def run(kind, D, stream):
        h = stream.cuda_stream
        if kind == 0:
            return _gpu.call("nt", "f16", 256, 128, 4096, A1d, 4096, B1d, 4096, D, 128, stream)
        if kind == 1:
            return _gpu.call("nn", "bf16", 264, 304, 1032, A2d, 1033, B2d, 304, D, 304, stream)
        return status()(mx(280, 300, 160, XA.data_ptr(), 160, XSA.data_ptr(), 5, XB.data_ptr(), 160,
                           XSB.data_ptr(), 5, D.data_ptr(), 300, h))

    shapes = [(256, 128), (264, 304), (280, 300)]
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

LEVELS = [1, 2, 3, 4, 5, 6, 7, 8, 9]


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
def test_ladder_level_4096_every_output(level):
    # the benchmark's shape, in the configuration the ladder benchmark times
    w = inputs.WORKLOADS["square_nt"]
    A, B, d, s = square_nt_reference()
    D, st = _gpu.ladder(level, A, B, w.M, w.N, w.K)
    assert st == status().OK
    check_against("f16", d, s, D, "ladder level %d" % level)


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
    assert Sx(fn(10, 256, 256, 64, p, 512, p, 512, D.data_ptr(), 512, s)) == Sx.BAD_ARG
    assert Sx(fn(8, 384, 256, 64, p, 512, p, 512, D.data_ptr(), 512, s)) == Sx.BAD_ARG
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
def test_split_last_wave(layout, fmt):
    # 17 x 16 = 272 tiles on 256 CUs: 256 tiles whole, the 16 of the last wave
    # in 4 parts of 4 K steps, all in one launch; ragged M and N.  Every
    # output against the oracle, plus entries drawn from the split tiles
    # alone; the run with split-K disabled is checked the same way
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
    dfull, sfull = oracle.gemm(layout, fmt, A, B)
    for mode, opts in (("auto", None), ("off", (1, 0))):
        D, st = _gpu.gemm(layout, fmt, A, B, M, N, K, opts=opts)
        assert st == status().OK
        res = oracle.check(fmt, d, s_, D[rows, cols])
        assert res.ok, (mode, res)
        check_against(fmt, dfull, sfull, D, mode)
        D2, _ = _gpu.gemm(layout, fmt, A, B, M, N, K, opts=opts)
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


@pytest.mark.parametrize("tile_n", [128, 256])
@pytest.mark.parametrize("fmt", ["f16", "bf16"])
@pytest.mark.parametrize("M,N,K", TILE128)
def test_tile_width_full_check(fmt, M, N, K, splitk, tile_n):
    # both tile widths of A.B^T forced on the same shapes (the plan picks 128
    # for most of them), with the library's split-K choice and without
    opts = (0 if splitk is None else 1, tile_n)
    w = inputs.Workload("x", "nt", fmt, 0, 0, 0, "uniform", 0.0, 301)
    A, B = inputs.make_operands(w, M=M, N=N, K=K)
    D, st = _gpu.gemm("nt", fmt, A, B, M, N, K, opts=opts)
    assert st == status().OK
    check_full("nt", fmt, A, B, M, N, K, D)


@pytest.mark.parametrize("parts", ["3", "16"])
def test_tile128_forced_split(parts):
    M, N, K = 520, 300, 2000
    A, B = inputs.make_operands(inputs.WORKLOADS["ragged_nt"], M=M, N=N, K=K)
    D, st = _gpu.gemm("nt", "f16", A, B, M, N, K, opts=(int(parts), 128))
    assert st == status().OK
    check_full("nt", "f16", A, B, M, N, K, D)


def test_tile128_bitwise_equals_tile256():
    # each output is the same sequence of MFMA accumulations in either tile
    # width, so the results agree bit for bit (split-K off)
    M, N, K = 1000, 900, 1500
    A, B = inputs.make_operands(inputs.WORKLOADS["square_nt"], M=M, N=N, K=K)
    out = {}
    for tn in (128, 256):
        out[tn], st = _gpu.gemm("nt", "f16", A, B, M, N, K, opts=(1, tn))
        assert st == status().OK
    assert np.array_equal(out[128], out[256])


# ------------------------------------------------ caller-owned workspace --

def _need(layout, fmt, M, N, K, A, lda, B, ldb, offsets=(0, 0), opts=None):
    import ctypes
    from dense_gemm_08_amd import binding
    lib = binding.load_library()
    out = ctypes.c_size_t()
    o = binding.Options(*opts) if opts else None
    st = lib.dense_gemm_workspace_size(binding.OPS[(layout, fmt)], M, N, K,
                                       A.data_ptr() + offsets[0], lda,
                                       B.data_ptr() + offsets[1], ldb, 0,
                                       ctypes.byref(o) if o else None, ctypes.byref(out))
    assert st == 0
    return out.value


def _ex(layout, fmt, M, N, K, A, lda, B, ldb, D, ldd, ws_ptr, nbytes, stream=None,
        offsets=(0, 0), opts=None):
    import ctypes
    from dense_gemm_08_amd import binding
    t = _gpu.torch()
    lib = binding.load_library()
    st = t.cuda.current_stream() if stream is None else stream
    o = binding.Options(*opts) if opts else None
    return status()(lib.dense_gemm_ex(binding.OPS[(layout, fmt)], M, N, K,
                                      A.data_ptr() + offsets[0], lda, B.data_ptr() + offsets[1],
                                      ldb, D.data_ptr(), ldd, ctypes.byref(o) if o else None,
                                      ws_ptr, nbytes, st.cuda_stream))


WS_CASES = [
    # (layout, fmt, M, N, K, lda_extra, a_off): what takes the workspace
    ("nt", "f16", 256, 128, 4096, 0, 0),    # one 256 x 128 tile in 16 K parts
    ("nn", "bf16", 264, 304, 1032, 1, 0),   # A repacked (odd leading dimension)
    ("nt", "f16", 4252, 4088, 1000, 0, 0),  # the last wave's 16 tiles in 4 parts
    ("nt", "bf16", 280, 272, 200, 0, 3),    # A repacked (pointer off 16-byte alignment)
    ("nn", "f16", 300, 264, 1001, 0, 0),    # both repacked (K odd), then split
]


@pytest.mark.parametrize("case", WS_CASES, ids=lambda c: "%s_%s_%dx%dx%d" % c[:5])
def test_workspace_call_equals_plain_call(case):
    # dense_gemm_ex with exactly the workspace the query reports gives the
    # plain entry point's result bit for bit (same plan and kernels), which
    # passes the oracle; a workspace one byte short, or a null one, is
    # rejected and a misaligned one too, with D untouched
    layout, fmt, M, N, K, xa, oa = case
    t = _gpu.torch()
    w = inputs.Workload("x", layout, fmt, 0, 0, 0, "uniform", 0.0, 401)
    A, B = inputs.make_operands(w, seed=M + N + K, M=M, N=N, K=K)
    lda, ldb = K + xa, (K if layout == "nt" else N)
    Ad = _gpu.to_dev_at(A, M, K, lda, oa)
    Bd = _gpu.to_dev(B, *((N, K) if layout == "nt" else (K, N)))
    need = _need(layout, fmt, M, N, K, Ad, lda, Bd, ldb, offsets=(2 * oa, 0))
    assert need > 0
    D1 = _gpu.empty_out(M, N)
    assert _gpu.call(layout, fmt, M, N, K, Ad, lda, Bd, ldb, D1, N, offsets=(2 * oa, 0, 0)) == \
        status().OK
    ws = _gpu.workspace(need + 512)
    D2 = _gpu.empty_out(M, N)
    assert _ex(layout, fmt, M, N, K, Ad, lda, Bd, ldb, D2, N, ws.data_ptr(), need,
               offsets=(2 * oa, 0)) == status().OK
    D3 = _gpu.empty_out(M, N)
    assert _ex(layout, fmt, M, N, K, Ad, lda, Bd, ldb, D3, N, ws.data_ptr(), need - 1,
               offsets=(2 * oa, 0)) == status().WORKSPACE_TOO_SMALL
    assert _ex(layout, fmt, M, N, K, Ad, lda, Bd, ldb, D3, N, 0, 0,
               offsets=(2 * oa, 0)) == status().WORKSPACE_TOO_SMALL
    assert _ex(layout, fmt, M, N, K, Ad, lda, Bd, ldb, D3, N, ws.data_ptr() + 16, need,
               offsets=(2 * oa, 0)) == status().MISALIGNED
    t.cuda.synchronize()
    g1, g2 = _gpu.from_dev(D1), _gpu.from_dev(D2)
    assert (g1 == g2).all()
    assert (_gpu.from_dev(D3) == _gpu.CANARY).all()
    check_full(layout, fmt, A, B, M, N, K, g2)


def test_workspace_calls_on_two_streams():
    # calls that each need a workspace (split-K partials, a repacked operand),
    # each given its own, issued back to back on two streams that do not
    # wait for each other, give the bits of the same calls run alone
    t = _gpu.torch()
    w = inputs.WORKLOADS["square_nt"]
    A1, B1 = inputs.make_operands(w, seed=71, M=256, N=128, K=4096)
    wn = inputs.WORKLOADS["large_nn"]
    A2, B2 = inputs.make_operands(wn, seed=72, M=264, N=304, K=1032)
    A1d, B1d = _gpu.to_dev(A1, 256, 4096), _gpu.to_dev(B1, 128, 4096)
    A2d, B2d = _gpu.to_dev(A2, 264, 1032, ld=1033), _gpu.to_dev(B2, 1032, 304)
    cases = [("nt", "f16", 256, 128, 4096, A1d, 4096, B1d, 4096),
             ("nn", "bf16", 264, 304, 1032, A2d, 1033, B2d, 304)]
    needs = [_need(c[0], c[1], c[2], c[3], c[4], c[5], c[6], c[7], c[8]) for c in cases]
    ref = []
    for c in cases:
        D = _gpu.empty_out(c[2], c[3])
        assert _gpu.call(c[0], c[1], c[2], c[3], c[4], c[5], c[6], c[7], c[8], D, c[3]) == \
            status().OK
        t.cuda.synchronize()
        ref.append(_gpu.from_dev(D))
    main = t.cuda.current_stream()
    streams = [t.cuda.Stream(), t.cuda.Stream()]
    jobs = []
    for it in range(12):
        for si in range(2):
            k = (it + si) % 2
            c = cases[k]
            jobs.append((k, si, _gpu.empty_out(c[2], c[3]), _gpu.workspace(needs[k])))
    for st in streams:
        st.wait_stream(main)
    for k, si, D, ws in jobs:
        c = cases[k]
        with t.cuda.stream(streams[si]):
            assert _ex(c[0], c[1], c[2], c[3], c[4], c[5], c[6], c[7], c[8], D, c[3],
                       ws.data_ptr(), needs[k], stream=streams[si]) == status().OK
    for st in streams:
        main.wait_stream(st)
    t.cuda.synchronize()
    for k, _, D, _ in jobs:
        assert (_gpu.from_dev(D) == ref[k]).all(), k


def test_mx_workspace_call_equals_plain_call():
    import ctypes
    from dense_gemm_08_amd import binding
    t = _gpu.torch()
    lib = binding.load_library()
    M, N, K = 520, 300, 416
    XA, XSA, XB, XSB = [t.from_numpy(x).cuda() for x in inputs.mx_operands(M, N, K, seed=73)]
    nb = K // 32
    need = ctypes.c_size_t()
    assert lib.gemm_nt_e4m3_mx_workspace_size(M, N, K, 0, ctypes.byref(need)) == 0
    ws = _gpu.workspace(need.value)
    h = t.cuda.current_stream().cuda_stream
    args = (M, N, K, XA.data_ptr(), K, XSA.data_ptr(), nb, XB.data_ptr(), K, XSB.data_ptr(), nb)
    D1, D2, D3 = (_gpu.empty_out(M, N) for _ in range(3))
    assert lib.gemm_nt_e4m3_mx(*args, D1.data_ptr(), N, h) == 0
    assert lib.gemm_nt_e4m3_mx_ex(*args, D2.data_ptr(), N, ws.data_ptr(), need.value, h) == 0
    assert status()(lib.gemm_nt_e4m3_mx_ex(*args, D3.data_ptr(), N, ws.data_ptr(),
                                           need.value - 1, h)) == status().WORKSPACE_TOO_SMALL
    t.cuda.synchronize()
    assert (_gpu.from_dev(D1) == _gpu.from_dev(D2)).all()
    assert (_gpu.from_dev(D3) == _gpu.CANARY).all()


def test_binding_call_on_another_stream_with_its_own_workspace_and_output():
    # the Python binding on a stream other than the current one, taking its
    # workspace (split-K partials) and D from torch's allocator: both are
    # marked as in use by that stream, so the allocations the current stream
    # makes right after the call (filled at once) cannot land on them while
    # the call's kernels run
    import dense_gemm_08_amd as dg
    t = _gpu.torch()
    w = inputs.WORKLOADS["k_loop"]
    M, N, K = 256, 128, 4096  # one 256 x 128 tile: the plan splits K 16 ways
    A, B = inputs.make_operands(w, seed=91, M=M, N=N, K=K)
    Ad = t.from_numpy(A.view(np.int16)).cuda().view(t.float16)
    Bd = t.from_numpy(B.view(np.int16)).cuda().view(t.float16)
    side = t.cuda.Stream()
    side.wait_stream(t.cuda.current_stream())
    outs = []
    for rep in range(8):
        outs.append(dg.gemm_nt_f16(Ad, Bd, stream=side, workspace=True))
        outs.append(dg.gemm_nt_f16(Ad, Bd, stream=side.cuda_stream, workspace=True))
        junk = [t.full((1 << 20,), -1.0, dtype=t.float32, device="cuda") for _ in range(4)]
        del junk
    t.cuda.synchronize()
    d, s = oracle.gemm("nt", "f16", A, B, M=M, N=N, K=K)
    first = _gpu.from_dev(outs[0].view(t.int16))
    for D in outs:
        got = _gpu.from_dev(D.view(t.int16))
        assert (got == first).all()
    check_against("f16", d, s, first, "side stream")
