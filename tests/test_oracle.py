"""Pins for the CPU oracle (no GPU).

The oracle is checked against things other than itself: exact rational
arithmetic on tiny inputs, numpy's own FP16 conversion and float64 matmul,
closed-form invariants, and the worked values printed on the pages.  Each
test is chosen so that a plausible slip in ``oracle.c`` (a dropped term, a
transposed operand, a wrong leading dimension, a wrong rounding direction or
exponent bound) fails it.
"""
import math
import os
from fractions import Fraction

import numpy as np
import pytest

import oracle
from dense_gemm_08_amd import inputs
from tests import _exact

U53 = 2.0 ** -53
GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "page_worked_values.txt")


def golden():
    out = {}
    with open(GOLDEN) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            name, val, cite = [x.strip() for x in line.split("|")]
            assert cite
            out[name] = int(val)
    return out


# ---------------------------------------------------------------- decoding --

def test_decode_all_f16_patterns_match_numpy():
    bits = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    got = oracle.decode("f16", bits)
    want = bits.view(np.float16).astype(np.float64)
    same = (got == want) | (np.isnan(got) & np.isnan(want))
    assert same.all()
    # signed zero kept
    assert math.copysign(1.0, got[0x8000]) == -1.0


@pytest.mark.filterwarnings("ignore::RuntimeWarning")
def test_decode_all_bf16_patterns_match_float32_view():
    bits = np.arange(1 << 16, dtype=np.uint32)
    got = oracle.decode("bf16", bits.astype(np.uint16))
    want = (bits << 16).astype(np.uint32).view(np.float32).astype(np.float64)
    same = (got == want) | (np.isnan(got) & np.isnan(want))
    assert same.all()


def test_decode_matches_exact_fields():
    for fmt in ("f16", "bf16"):
        for b in inputs.random_finite_bits(fmt, (400,), seed=3):
            assert Fraction(float(oracle.decode(fmt, np.array([b], np.uint16))[0])) == \
                _exact.value(fmt, int(b))


# ---------------------------------------------------------------- rounding --

def _f16_grid_midpoints():
    # all finite non-negative FP16 values and every midpoint between neighbours
    vals = np.arange(0, 0x7C00, dtype=np.uint32).astype(np.uint16).view(np.float16)
    v = vals.astype(np.float64)
    mids = (v[:-1] + v[1:]) / 2.0  # exact in float64
    return v, mids


@pytest.mark.filterwarnings("ignore::RuntimeWarning")
def test_round_f16_matches_numpy_cast():
    v, mids = _f16_grid_midpoints()
    rng = np.random.default_rng(5)
    rand = rng.standard_normal(20000) * np.exp2(rng.integers(-30, 18, 20000))
    near_mid = mids * (1.0 + rng.choice([-1, 1], mids.size) * 2.0 ** -40)
    edge = np.array([65504.0, 65519.999, 65520.0, 65520.0001, 1e9, 2.0 ** -24, 2.0 ** -25,
                     2.0 ** -25 * (1 + 2.0 ** -30), 3 * 2.0 ** -26, 2.0 ** -14 - 2.0 ** -26,
                     0.0, -0.0, -65520.0, -2.0 ** -25])
    for x in (v, mids, rand, near_mid, edge, -mids):
        got = oracle.round_to("f16", x)
        want = x.astype(np.float16).view(np.uint16)
        assert (got == want).all(), x[got != want][:5]


def test_round_bf16_matches_exact_rne():
    rng = np.random.default_rng(7)
    cases = []
    # random values over the whole exponent range, including subnormals
    for _ in range(3000):
        cases.append(float(rng.standard_normal()) * 2.0 ** int(rng.integers(-140, 128)))
    # exact midpoints between neighbouring BF16 values
    for b in inputs.random_finite_bits("bf16", (1500,), seed=9):
        b = int(b) & 0x7FFF
        if b >= 0x7F7F:
            continue
        lo, hi = _exact.value("bf16", b), _exact.value("bf16", b + 1)
        cases.append(float((lo + hi) / 2))
    big = 2.0 ** 127 * (2 - 2.0 ** -7)
    cases += [big, big * (1 + 2.0 ** -9), 2.0 ** 127 * (2 - 2.0 ** -8), 2.0 ** -133,
              2.0 ** -134, 2.0 ** -134 * 3, 2.0 ** -126 - 2.0 ** -135, 0.0]
    x = np.array(cases + [-c for c in cases], dtype=np.float64)
    got = oracle.round_to("bf16", x)
    want = np.array([_exact.round_bits("bf16", Fraction(float(c)),
                                       negative_zero=(c == 0 and math.copysign(1, c) < 0))
                     for c in x], dtype=np.uint16)
    bad = np.nonzero(got != want)[0]
    assert bad.size == 0, [(x[i], hex(got[i]), hex(want[i])) for i in bad[:5]]


def test_round_f16_matches_exact_rne():
    rng = np.random.default_rng(8)
    x = rng.standard_normal(2000) * np.exp2(rng.integers(-28, 17, 2000))
    got = oracle.round_to("f16", x)
    want = np.array([_exact.round_bits("f16", Fraction(float(c))) for c in x], dtype=np.uint16)
    assert (got == want).all()


# --------------------------------------------------------------------- ulp --

def test_ulp_f16_matches_numpy_spacing():
    # every positive finite FP16 value: spacing above it within its binade
    vals = np.arange(1, 0x7C00, dtype=np.uint32).astype(np.uint16).view(np.float16)
    for v in vals[::7]:
        want = float(np.spacing(v))
        if int(np.float16(v).view(np.uint16)) == 0x7BFF:
            want = 32.0  # numpy spacing at the largest finite value is inf
        assert oracle.ulp("f16", float(v)) == want
        assert oracle.ulp("f16", -float(v)) == want
    assert oracle.ulp("f16", 0.0) == 2.0 ** -24
    # a double strictly inside a binade takes that binade's spacing
    assert oracle.ulp("f16", 1.999) == 2.0 ** -10
    assert oracle.ulp("f16", 2.0) == 2.0 ** -9


def test_ulp_bf16_matches_float32_spacing():
    rng = np.random.default_rng(4)
    e = rng.integers(-126, 127, 500)
    m = rng.integers(1 << 23, 1 << 24, 500)
    x = (m.astype(np.float64) * np.exp2(e - 23.0)).astype(np.float32)  # exact float32 normals
    for v in x:
        assert oracle.ulp("bf16", float(v)) == float(np.spacing(np.float32(abs(v)))) * 65536.0
    assert oracle.ulp("bf16", 0.0) == 2.0 ** -133
    assert oracle.ulp("bf16", 2.0 ** -130) == 2.0 ** -133


# -------------------------------------------------- exact brute force pins --

@pytest.mark.parametrize("layout", ["nt", "nn"])
@pytest.mark.parametrize("fmt", ["f16", "bf16"])
def test_gemm_matches_exact_rationals_all_tiny_shapes(layout, fmt):
    seed = 100
    for M in range(1, 6):
        for N in range(1, 6):
            for K in range(1, 6):
                seed += 1
                sa, sb = inputs.operand_shapes(layout, M, N, K)
                if seed % 3 == 0:
                    A = inputs.random_finite_bits(fmt, sa, seed)
                    B = inputs.random_finite_bits(fmt, sb, seed + 5000)
                else:
                    rng = np.random.default_rng(seed)
                    A = inputs.to_bits(fmt, rng.uniform(-4, 4, sa))
                    B = inputs.to_bits(fmt, rng.uniform(-4, 4, sb))
                d, s = oracle.gemm(layout, fmt, A, B)
                de, se = _exact.gemm(layout, fmt, A.tolist(), B.tolist())
                for i in range(M):
                    for j in range(N):
                        bound = K * U53 * float(se[i][j])
                        assert abs(Fraction(d[i, j]) - de[i][j]) <= Fraction(bound), (M, N, K, i, j)
                        assert abs(Fraction(s[i, j]) - se[i][j]) <= Fraction(bound)
                        if Fraction(d[i, j]) == de[i][j]:
                            # exact sum: the rounded output is the exact RNE
                            got = int(oracle.round_to(fmt, np.array([d[i, j]]))[0])
                            want = _exact.round_bits(fmt, de[i][j],
                                                     negative_zero=math.copysign(1, d[i, j]) < 0)
                            assert got == want


def test_gemm_special_values():
    # +-0, subnormals, the largest finite value, powers of two: every product
    # is exact; sums spanning 2^-48 .. 2^32 are within the recursive-sum bound.
    vals = [0.0, -0.0, 2.0 ** -24, -(2.0 ** -24), 2.0 ** -14, 65504.0, -65504.0, 1.0, 0.5, 1024.0]
    A = inputs.f16_bits(np.array([vals, vals[::-1]]))              # 2 x 10
    B = inputs.f16_bits(np.array([[1.0] * 10, [2.0 ** -10] * 10, vals]))  # 3 x 10 (NT)
    d, s = oracle.gemm("nt", "f16", A, B)
    de, se = _exact.gemm("nt", "f16", A.tolist(), B.tolist())
    for i in range(2):
        for j in range(3):
            bound = Fraction(10 * U53) * se[i][j]
            assert abs(Fraction(d[i, j]) - de[i][j]) <= bound
            assert abs(Fraction(s[i, j]) - se[i][j]) <= bound
    # a narrower range keeps every partial sum exact: then d is exact
    small = [0.0, -0.0, 2.0 ** -14, -(2.0 ** -13), 1.0, 0.5, -3.0, 1024.0, 2.0 ** -6, 7.0]
    A = inputs.f16_bits(np.array([small, small[::-1]]))
    B = inputs.f16_bits(np.array([[1.0] * 10, [2.0 ** -10] * 10, small]))
    d, s = oracle.gemm("nt", "f16", A, B)
    de, se = _exact.gemm("nt", "f16", A.tolist(), B.tolist())
    for i in range(2):
        for j in range(3):
            assert Fraction(d[i, j]) == de[i][j] and Fraction(s[i, j]) == se[i][j]


# ------------------------------------------------------------- invariants --

@pytest.mark.parametrize("fmt", ["f16", "bf16"])
def test_identity_gives_a(fmt):
    A, _ = inputs.make_operands(inputs.WORKLOADS["ragged_nt"], M=37, N=1, K=53)
    if fmt == "bf16":
        A = inputs.bf16_bits(oracle.decode("f16", A))
    eye = inputs.identity(fmt, 53)
    for layout in ("nt", "nn"):
        d, s = oracle.gemm(layout, fmt, A, eye)
        assert (d == oracle.decode(fmt, A)).all()
        assert (oracle.decode(fmt, oracle.round_to(fmt, d)) == oracle.decode(fmt, A)).all()


@pytest.mark.parametrize("layout", ["nt", "nn"])
def test_all_ones_give_k(layout):
    for K in (1, 7, 64, 4000, 4096, 5120):
        sa, sb = inputs.operand_shapes(layout, 3, 5, K)
        d, s = oracle.gemm(layout, "f16", inputs.ones("f16", sa), inputs.ones("f16", sb))
        assert (d == K).all() and (s == K).all()


def test_transposition_symmetry_bitwise():
    w = inputs.WORKLOADS["ragged_nt"]
    A, B = inputs.make_operands(w, M=29, N=41, K=77)
    d1, s1 = oracle.gemm("nt", "f16", A, B)
    d2, s2 = oracle.gemm("nt", "f16", B, A)
    assert (d1 == d2.T).all() and (s1 == s2.T).all()


@pytest.mark.parametrize("fmt", ["f16", "bf16"])
def test_nn_equals_nt_on_materialised_transpose(fmt):
    w = inputs.WORKLOADS["large_nn"]
    A, B = inputs.make_operands(w, M=19, N=33, K=70)  # B is K x N
    dn, sn = oracle.gemm("nn", fmt, A, B)
    dt, st = oracle.gemm("nt", fmt, A, np.ascontiguousarray(B.T))
    assert (dn == dt).all() and (sn == st).all()


def test_leading_dimensions_are_honoured():
    w = inputs.WORKLOADS["ragged_nt"]
    A, B = inputs.make_operands(w, M=13, N=9, K=24)
    Ap = np.full((13, 40), 0x7C00, np.uint16)  # padding = +inf: must never be read
    Ap[:, :24] = A
    Bp = np.full((9, 32), 0x7C00, np.uint16)
    Bp[:, :24] = B
    d1, _ = oracle.gemm("nt", "f16", A, B)
    d2, _ = oracle.gemm("nt", "f16", Ap, Bp, M=13, N=9, K=24, lda=40, ldb=32)
    assert (d1 == d2).all()
    Bn = np.ascontiguousarray(B.T)  # 24 x 9
    Bnp = np.full((24, 16), 0x7C00, np.uint16)
    Bnp[:, :9] = Bn
    d3, _ = oracle.gemm("nn", "f16", A, Bnp, M=13, N=9, K=24, lda=24, ldb=16)
    assert (d1 == d3).all()


def test_against_numpy_float64_matmul():
    for layout, fmt in (("nt", "f16"), ("nn", "bf16")):
        w = inputs.Workload("t", layout, fmt, 0, 0, 0, "normal", 1.0, 21)
        A, B = inputs.make_operands(w, M=257, N=131, K=1000)
        a = oracle.decode(fmt, A) if fmt == "f16" else \
            (A.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
        b = oracle.decode(fmt, B) if fmt == "f16" else \
            (B.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
        ref = a @ (b.T if layout == "nt" else b)
        refs = np.abs(a) @ np.abs(b.T if layout == "nt" else b)
        d, s = oracle.gemm(layout, fmt, A, B)
        bound = 2 * 1000 * U53 * refs
        assert (np.abs(d - ref) <= bound).all()
        assert (np.abs(s - refs) <= bound).all()


def _padded(X, ld, fill=0x7C00):
    """X in a wider row-major array (leading dimension ld) whose padding
    holds +Inf (FP16) / a huge value (BF16): a read of it shows in the sums."""
    P = np.full((X.shape[0], ld), fill, np.uint16)
    P[:, :X.shape[1]] = X
    return P


@pytest.mark.parametrize("layout", ["nt", "nn"])
@pytest.mark.parametrize("fmt", ["f16", "bf16"])
def test_entries_agree_with_full_product(layout, fmt):
    # non-square (M, N, K all different, so a transposed read of B or a
    # stride taken from the wrong dimension lands elsewhere), with padded
    # leading dimensions on both operands; every entry of a 31 x 47 product
    # plus repeated and out-of-order samples
    M, N, K = 31, 47, 90
    w = inputs.Workload("t", layout, fmt, 0, 0, 0, "uniform", 0.0, 40 + len(layout + fmt))
    A, B = inputs.make_operands(w, M=M, N=N, K=K)
    d, s = oracle.gemm(layout, fmt, A, B)
    lda = K + 13
    ldb = (K + 5) if layout == "nt" else (N + 7)
    Ap, Bp = _padded(A, lda), _padded(B, ldb)
    rows = np.concatenate([np.repeat(np.arange(M), N),
                           inputs.sample_indices(M, N, 64, seed=2)[0]])
    cols = np.concatenate([np.tile(np.arange(N), M),
                           inputs.sample_indices(M, N, 64, seed=2)[1]])
    de, se = oracle.gemm_entries(layout, fmt, Ap, Bp, K=K, lda=lda, ldb=ldb, rows=rows, cols=cols)
    assert (de == d[rows, cols]).all() and (se == s[rows, cols]).all()


@pytest.mark.parametrize("layout", ["nt", "nn"])
def test_entries_match_exact_rationals_with_padding(layout):
    # the sampled-entry path against exact arithmetic on its own (not only
    # against the full product): 3 x 4 x 5 with padded leading dimensions
    M, N, K = 3, 4, 5
    rng = np.random.default_rng(77)
    sa, sb = inputs.operand_shapes(layout, M, N, K)
    A = inputs.to_bits("f16", rng.uniform(-4, 4, sa))
    B = inputs.to_bits("f16", rng.uniform(-4, 4, sb))
    de, se = _exact.gemm(layout, "f16", A.tolist(), B.tolist())
    lda, ldb = K + 3, (K + 2 if layout == "nt" else N + 3)
    rows = np.repeat(np.arange(M), N)
    cols = np.tile(np.arange(N), M)
    d, s = oracle.gemm_entries(layout, "f16", _padded(A, lda), _padded(B, ldb), K=K, lda=lda,
                               ldb=ldb, rows=rows, cols=cols)
    for t in range(M * N):
        bound = Fraction(K * U53) * se[rows[t]][cols[t]]
        assert abs(Fraction(d[t]) - de[rows[t]][cols[t]]) <= bound
        assert abs(Fraction(s[t]) - se[rows[t]][cols[t]]) <= bound


# ------------------------------------------------- worked values on pages --

def test_page_worked_sums():
    g = golden()
    # one sum per thread: thread t holds 2t+1, 2t+2
    vals = np.arange(1, 65, dtype=np.float64)
    A = inputs.f16_bits(vals.reshape(32, 2))
    d, _ = oracle.gemm("nt", "f16", A, inputs.ones("f16", (1, 2)))
    assert d[0, 0] == g["thread_sum_0"] and d[1, 0] == g["thread_sum_1"]
    # one sum for the warp: all 64 values
    d, _ = oracle.gemm("nt", "f16", inputs.f16_bits(vals.reshape(1, 64)), inputs.ones("f16", (1, 64)))
    assert d[0, 0] == g["warp_sum_1_to_64"]
    assert oracle.round_to("f16", d)[0, 0] == inputs.f16_bits(np.array([2080.0]))[0]


@pytest.mark.parametrize("fmt", ["f16", "bf16"])
def test_page_rowmajor_offset(fmt):
    g = golden()
    # A holds its own flat offsets, 8 x 16 row-major; a one-hot B picks column 9
    A = inputs.to_bits(fmt, np.arange(128, dtype=np.float64).reshape(8, 16))
    onehot = np.zeros((1, 16))
    onehot[0, 9] = 1.0
    d, _ = oracle.gemm("nt", fmt, A, inputs.to_bits(fmt, onehot))
    assert d[3, 0] == g["rowmajor_8x16_offset_3_9"]
    # the same through the A.B layout, with B = e_9 as a 16 x 1 column
    d, _ = oracle.gemm("nn", fmt, A, inputs.to_bits(fmt, onehot.T.copy()))
    assert d[3, 0] == g["rowmajor_8x16_offset_3_9"]


# ---------------------------------------------------------- check routine --

def test_check_accepts_within_and_rejects_beyond_tolerance():
    d = np.array([1.0, 1.0, 100.0, 0.0, 70000.0])
    s = np.array([2048.0, 0.0, 100.0, 0.0, 70000.0])
    # element 0: tol = 2^-10 + 1 ; element 1: tol = 2^-10 ; element 2: tol = 2^-4 + 100/2048
    # element 3: tol = 2^-24 ; element 4: d overflows FP16 -> only +inf passes
    ok = np.array([1.0 + 1.0, 1.0 + 2.0 ** -10, 100.0 + 0.0625, 2.0 ** -24, np.inf])
    res = oracle.check("f16", d, s, inputs.f16_bits(ok))
    assert res.ok, res
    bad = np.array([1.0 + 2.0, 1.0 + 2.0 ** -9, 100.25, 2.0 ** -23, 65504.0])
    res = oracle.check("f16", d, s, inputs.f16_bits(bad))
    assert res.n_fail == 5
    nan = inputs.f16_bits(np.array([np.nan] * 5))
    assert oracle.check("f16", d, s, nan).n_fail == 5


def test_check_detects_a_dropped_k_block():
    # the tolerance must not hide a kernel that skips a 64-wide k block
    w = inputs.WORKLOADS["square_nt"]
    A, B = inputs.make_operands(w, M=64, N=64, K=512)
    d, s = oracle.gemm("nt", "f16", A, B)
    A2 = A.copy()
    A2[:, 128:192] = 0
    d2, _ = oracle.gemm("nt", "f16", A2, B)
    res = oracle.check("f16", d, s, oracle.round_to("f16", d2))
    assert res.n_fail > 64 * 64 // 2
    assert oracle.check("f16", d, s, oracle.round_to("f16", d)).ok


# ------------------------------------------------ FP8 block-scaled (MX) --
#
# oracle.gemm_mx: E4M3 elements, one E8M0 scale per 32 consecutive K values
# of a row (the reading of the CMU blog's "FP8 block-scaled matrix
# multiplication" stated in oracle.c).

def _torch_e4m3(codes):
    import torch
    c = np.ascontiguousarray(codes, dtype=np.uint8)
    return torch.from_numpy(c.copy()).view(torch.float8_e4m3fn).float().numpy().astype(np.float64)


def _mx_operands(rng, M, N, K, lo=118, hi=136):
    finite = np.array([c for c in range(256) if (c & 0x7F) != 0x7F], np.uint8)
    A = rng.choice(finite, size=(M, K)).astype(np.uint8)
    B = rng.choice(finite, size=(N, K)).astype(np.uint8)
    nb = (K + 31) // 32
    SA = rng.integers(lo, hi + 1, size=(M, nb)).astype(np.uint8)
    SB = rng.integers(lo, hi + 1, size=(N, nb)).astype(np.uint8)
    return A, SA, B, SB


def test_e4m3_decode_all_codes_match_torch():
    codes = np.arange(256, dtype=np.uint8)
    mine, ref = oracle.decode_e4m3(codes), _torch_e4m3(codes)
    assert np.array_equal(np.isnan(mine), np.isnan(ref))
    assert np.isnan(mine).sum() == 2  # S.1111.111 only
    ok = ~np.isnan(ref)
    assert np.array_equal(mine[ok], ref[ok])
    # the format's landmarks: largest finite, smallest normal and subnormal
    assert oracle.decode_e4m3(np.array([0x7E, 0x08, 0x01, 0x80], np.uint8)).tolist() == \
        [448.0, 2.0 ** -6, 2.0 ** -9, -0.0]


def test_e8m0_decode_matches_float32_exponent_field():
    import struct
    codes = np.arange(256, dtype=np.uint8)
    mine = oracle.decode_e8m0(codes)
    assert np.isnan(mine[255]) and not np.isnan(mine[:255]).any()
    for e in range(1, 255):  # a float32 with exponent field e and no fraction is 2^(e-127)
        assert mine[e] == struct.unpack("<f", struct.pack("<I", e << 23))[0]
    assert mine[0] == 2.0 ** -127


@pytest.mark.parametrize("K", [32, 40, 96])
def test_gemm_mx_matches_exact_rationals(K):
    rng = np.random.default_rng(K)
    M, N = 3, 4
    A, SA, B, SB = _mx_operands(rng, M, N, K)
    d, s = oracle.gemm_mx(A, SA, B, SB)
    va, vb = _torch_e4m3(A), _torch_e4m3(B)
    for i in range(M):
        for j in range(N):
            exact = sum(Fraction(va[i, k]) * Fraction(2) ** (int(SA[i, k // 32]) - 127) *
                        Fraction(vb[j, k]) * Fraction(2) ** (int(SB[j, k // 32]) - 127)
                        for k in range(K))
            absum = sum(abs(Fraction(va[i, k]) * Fraction(vb[j, k])) *
                        Fraction(2) ** (int(SA[i, k // 32]) + int(SB[j, k // 32]) - 254)
                        for k in range(K))
            assert abs(Fraction(d[i, j]) - exact) <= K * Fraction(U53) * absum
            assert Fraction(s[i, j]) == absum or abs(Fraction(s[i, j]) - absum) <= K * Fraction(U53) * absum


def test_gemm_mx_unit_scales_is_the_plain_product():
    rng = np.random.default_rng(11)
    M, N, K = 37, 29, 160
    A, SA, B, SB = _mx_operands(rng, M, N, K, 127, 127)
    d, s = oracle.gemm_mx(A, SA, B, SB)
    ref = _torch_e4m3(A) @ _torch_e4m3(B).T
    assert np.all(np.abs(d - ref) <= 2 * K * U53 * s)


def test_gemm_mx_scale_acts_on_its_block_only():
    # raising one block's scale by one (x2) adds exactly that block's share:
    # a wrong block size, a wrong block index or a scale applied to the wrong
    # operand changes a different share
    rng = np.random.default_rng(12)
    M, N, K = 9, 7, 160
    A, SA, B, SB = _mx_operands(rng, M, N, K)
    d0, s0 = oracle.gemm_mx(A, SA, B, SB)
    for b in range(K // 32):
        SA2 = SA.copy()
        SA2[:, b] += 1
        d1, _ = oracle.gemm_mx(A, SA2, B, SB)
        part, _ = oracle.gemm_mx(np.ascontiguousarray(A[:, 32 * b:32 * b + 32]),
                                 np.ascontiguousarray(SA[:, b:b + 1]),
                                 np.ascontiguousarray(B[:, 32 * b:32 * b + 32]),
                                 np.ascontiguousarray(SB[:, b:b + 1]))
        assert np.all(np.abs((d1 - d0) - part) <= 4 * K * U53 * 2 * s0)
        SB2 = SB.copy()
        SB2[:, b] -= 1
        d2, _ = oracle.gemm_mx(A, SA, B, SB2)
        assert np.all(np.abs((d0 - d2) - part / 2) <= 4 * K * U53 * s0)


def test_gemm_mx_entries_agree_with_full_product():
    rng = np.random.default_rng(13)
    A, SA, B, SB = _mx_operands(rng, 33, 21, 224)
    d, s = oracle.gemm_mx(A, SA, B, SB)
    rows = rng.integers(0, 33, 50)
    cols = rng.integers(0, 21, 50)
    de, se = oracle.gemm_mx_entries(A, SA, B, SB, rows, cols)
    assert np.array_equal(de, d[rows, cols]) and np.array_equal(se, s[rows, cols])


def test_gemm_mx_nan_scale_propagates():
    rng = np.random.default_rng(14)
    A, SA, B, SB = _mx_operands(rng, 4, 4, 64)
    SA[2, 1] = 255
    d, _ = oracle.gemm_mx(A, SA, B, SB)
    assert np.isnan(d[2]).all() and not np.isnan(np.delete(d, 2, axis=0)).any()
