"""Randomised GPU parity: many small products with random shapes, leading
dimensions, pointer offsets, type/layout pairings and plan overrides, each
checked element by element against the oracle (through the C ABI).

Seeded, so a failure names a reproducible case (printed before each call).
Shapes stay small (M, N <= 700, K <= 1500) so the oracle keeps up; they
still span several tiles, ragged edges in M, N and K, K below one step, and
repacked operands.  Each case's padding must stay untouched.
"""
import numpy as np
import pytest

import oracle
from dense_gemm_08_amd import inputs
from tests import _gpu

pytestmark = pytest.mark.gpu

PAIRS = [("nt", "f16"), ("nn", "bf16"), ("nt", "bf16"), ("nn", "f16")]


def _case(rng):
    layout, fmt = PAIRS[rng.integers(0, 4)]
    M = int(rng.choice([1, 2, 7, 16, 100, 255, 256, 257, 300, 511, 700]))
    N = int(rng.choice([1, 3, 8, 64, 128, 129, 200, 256, 384, 500, 700]))
    K = int(rng.choice([1, 5, 8, 31, 64, 65, 127, 500, 1000, 1500]))
    xa, xb, xd = (int(rng.choice([0, 0, 0, 1, 3, 8, 24])) for _ in range(3))
    oa, ob, od = (int(rng.choice([0, 0, 0, 1, 4, 8])) for _ in range(3))
    opts = [None, None, (1, 0), (int(rng.integers(2, 9)), 0),
            (0, 128) if layout == "nt" else (0, 256), (int(rng.integers(2, 5)), 256)][rng.integers(0, 6)]
    return layout, fmt, M, N, K, xa, xb, xd, oa, ob, od, opts


@pytest.mark.parametrize("block", range(4))
def test_random_products_against_the_oracle(block):
    rng = np.random.default_rng(1000 + block)
    for i in range(100):
        layout, fmt, M, N, K, xa, xb, xd, oa, ob, od, opts = _case(rng)
        seed = int(rng.integers(0, 1 << 30))
        what = ("case %d.%d: %s %s M=%d N=%d K=%d ld+(%d,%d,%d) off(%d,%d,%d) opts=%s seed=%d"
                % (block, i, layout, fmt, M, N, K, xa, xb, xd, oa, ob, od, opts, seed))
        print(what, flush=True)
        w = inputs.Workload("x", layout, fmt, 0, 0, 0,
                            "uniform" if seed % 2 else "normal", 0.0 if seed % 2 else 0.5, seed)
        A, B = inputs.make_operands(w, M=M, N=N, K=K)
        lda, ldb, ldd = K + xa, (K if layout == "nt" else N) + xb, N + xd
        D, st = _gpu.gemm(layout, fmt, A, B, M, N, K, lda=lda, ldb=ldb, ldd=ldd,
                          a_off=oa, b_off=ob, d_off=od, opts=opts)
        assert st == 0, what
        assert (D[:, N:] == _gpu.CANARY).all(), what
        d, s = oracle.gemm(layout, fmt, A, B)
        res = oracle.check(fmt, d, s, D[:, :N])
        assert res.ok, (what, res)
