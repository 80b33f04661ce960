// tile_config.h -- the tile configurations of the FP16/BF16 GEMM and of the
// FP8 block-scaled GEMM, shared by the kernels (gemm_kernel.h,
// gemm_small_kernel.h, gemm_mx_kernel.h, gemm_mx_small_kernel.h) and the
// host-side planning
// (plan.cpp, which is plain C++ and builds without HIP).
#pragma once

namespace dg {

enum Layout { NT = 0, NN = 1 };

constexpr int BM = 256;              // tile rows (M)
constexpr int BN = 256;              // tile columns (N); A @ B.T also has a 128-wide
                                     // tile for outputs too narrow to fill the CUs
constexpr int BK = 64;               // K depth of one LDS stage (128-byte rows)
constexpr int WAVES = 4;             // 2 x 2 waves
constexpr int THREADS = WAVES * 64;

// The small-output kernel (gemm_small_kernel.h): A @ B.T with M at most
// SMALL_MAX, K at most SMALL_K_MAX, and a single tile row (M <= SMALL_TILE),
// or at most SMALL_MAX_TILES 16 x 16 tiles of D, or tiles of 32 x 32 x K at
// most SMALL_T32_K; each tile (16 x 16, 32 x 16 or 32 x 32) a workgroup of
// eight waves that split K among themselves.
constexpr int SMALL_TILE = 16;
constexpr int SMALL_WAVES = 8;
constexpr int SMALL_THREADS = SMALL_WAVES * 64;
constexpr int SMALL_MAX = 128;
constexpr int SMALL_K_MAX = 16384;
constexpr int SMALL_MAX_TILES = 512;
constexpr long long SMALL_T32_K = 1LL << 21;
// A @ B also needs K at most SMALL_NN_K_MAX and tile rows x N x K, the B
// elements its tiles stream, at most SMALL_NN_ELEMS (plan.cpp: small_output).
constexpr int SMALL_NN_K_MAX = 4096;
constexpr long long SMALL_NN_ELEMS = 21LL << 20;

// The FP8 block-scaled GEMM (gemm_mx_kernel.h): 256 x 256 tiles, 128-deep
// K stages (128 bytes per row), one E8M0 scale per GROUP K values.  Its
// small-output kernel (gemm_mx_small_kernel.h: tiles of 16 x 16, 32 x 16 or
// 32 x 32) takes products with M up to SMALL_MAX and K up to
// MX_SMALL_K_MAX with one 16-row tile row, or at most MX_SMALL_T32 tiles of
// 32 x 32 in D, or at most MX_SMALL_T32_MAX such tiles with tiles x K at
// most MX_SMALL_T32_K (plan.cpp: mx_small_output).
namespace mx {
constexpr int BM = 256, BN = 256;
constexpr int BKE = 128;                   // K elements (= bytes) per stage
constexpr int GROUP = 32;                  // K elements per scale
constexpr int SC_BYTES = 1024;             // packed scale panel per operand per stage
constexpr int MX_SMALL_K_MAX = 8192;
constexpr int MX_SMALL_T32 = 1024;
constexpr int MX_SMALL_T32_MAX = 1536;
constexpr long long MX_SMALL_T32_K = 1LL << 23;
}  // namespace mx

}  // namespace dg
