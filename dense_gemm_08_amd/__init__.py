"""MI355X (gfx950) tiled dense GEMM: D = A.B^T (FP16) and D = A.B (BF16), and
the FP8 block-scaled D = A.B^T (E4M3 with E8M0 scales per 32 K values).

The arithmetic runs in the hand-written HIP kernels of ``libdense_gemm.so``
(built from ``csrc/``).  This package only marshals arguments to its C ABI;
importing it does not load the library, and every call fails loudly if the
library is missing.
"""
from .binding import (  # noqa: F401
    Status,
    DenseGemmError,
    gemm_nt_f16,
    gemm_nn_bf16,
    gemm_nt_bf16,
    gemm_nn_f16,
    gemm_nt_e4m3_mx,
    library_path,
    load_library,
)
