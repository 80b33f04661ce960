// tile_config.h -- the FP16/BF16 GEMM's tile configuration, shared by the
// kernels (gemm_kernel.h) and the host-side planning (plan.cpp, which is
// plain C++ and builds without HIP).
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
// SMALL_MAX, K at most SMALL_K_MAX, and at most SMALL_MAX_TILES 16 x 16
// tiles of D or a single tile row (M <= SMALL_TILE), each tile a workgroup
// of eight waves that split K among themselves.
constexpr int SMALL_TILE = 16;
constexpr int SMALL_WAVES = 8;
constexpr int SMALL_THREADS = SMALL_WAVES * 64;
constexpr int SMALL_MAX = 128;
constexpr int SMALL_K_MAX = 16384;
constexpr int SMALL_MAX_TILES = 512;

}  // namespace dg
