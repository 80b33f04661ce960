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

}  // namespace dg
