// cdna_ops.h -- gfx950 building blocks shared by the GEMM kernels:
// vector types, the LDS chunk swizzles, buffer descriptors, the LDS-DMA
// load, barriers and fences, the 16 x 16 x 32 MFMA, RNE packing and the
// transposing LDS read.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dg {

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void lds_void;

constexpr uint32_t OOB = 0x80000000u;  // a buffer offset past every range

// LDS layouts.
// K-contiguous tiles (A, and B for NT): row r holds 64 elements = eight
// 16-byte chunks (one 128-byte line of the source row); chunk c is stored at
// slot c ^ swz_k(r).  Eight consecutive rows read at one chunk, or sixteen,
// land in distinct bank groups.
__device__ __forceinline__ int swz_k(int r) { return ((r >> 1) ^ (r << 2)) & 7; }
// N-contiguous B tile (NN): row k holds 256 elements = 32 chunks; chunk c is
// stored at slot c ^ swz_n(k).  One transposing load reads 32 bytes (two
// chunks) from each of 16 rows k = 8 q + 4 h + r (q, r = 0..3, h fixed);
// the XOR of chunk bits 1-4 with r and q puts each of those rows' 32 bytes
// in a different 32-byte group of the 512-byte row, i.e. in distinct banks.
__device__ __forceinline__ int swz_n(int k) { return ((k & 3) | (((k >> 3) & 3) << 2)) << 1; }

__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)(const lds_void*)p;
}

__device__ __forceinline__ i32x4 make_rsrc(uint64_t a, uint32_t bytes) {
  i32x4 r;
  r[0] = (int)(uint32_t)a;
  r[1] = (int)(uint32_t)(a >> 32);  // stride 0
  r[2] = (int)bytes;                // num_records: bytes in range
  r[3] = 0x00020000;
  return r;
}

// 16-byte global -> LDS copy for every lane of the wave: lane L's 16 bytes at
// buffer offset `off` land at LDS address m0 + 16 L.  Offsets at or past the
// descriptor's range write zeros.  The asm sets m0 itself; the clobber tells
// the compiler, which warns that m0 is reserved (it keeps no value in m0
// across these statements in the kernels that use them), hence the pragma.
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
__device__ __forceinline__ void dma16(i32x4 rsrc, uint32_t off, uint32_t m0) {
  asm volatile("s_mov_b32 m0, %2\n\tbuffer_load_dwordx4 %0, %1, 0 offen lds"
               :
               : "v"(off), "s"(rsrc), "s"(m0)
               : "memory", "m0");
}
// The same with the LDS address given as base + imm, where imm must be a
// constant once the caller's loops are unrolled: the sum goes straight into
// m0, so no address register is computed ahead of the load.  (The add sets
// SCC, hence that clobber.)
__device__ __forceinline__ void dma16_at(i32x4 rsrc, uint32_t off, uint32_t base, int imm) {
  asm volatile("s_add_u32 m0, %2, %3\n\tbuffer_load_dwordx4 %0, %1, 0 offen lds"
               :
               : "v"(off), "s"(rsrc), "s"(base), "i"(imm)
               : "memory", "m0", "scc");
}
// 4-byte global -> LDS copy for every lane of the wave: lane L's 4 bytes at
// buffer offset `off` land at LDS address base + imm + 4 L (offsets at or
// past the descriptor's range write zeros).
__device__ __forceinline__ void dma4_at(i32x4 rsrc, uint32_t off, uint32_t base, int imm) {
  asm volatile("s_add_u32 m0, %2, %3\n\tbuffer_load_dword %0, %1, 0 offen lds"
               :
               : "v"(off), "s"(rsrc), "s"(base), "i"(imm)
               : "memory", "m0", "scc");
}
#pragma clang diagnostic pop

// Scheduling fence: the compiler may move no instruction across it.
__device__ __forceinline__ void fence() { __builtin_amdgcn_sched_barrier(0); }

// Wait until at most N vector-memory operations of this wave are in flight and
// its LDS reads are done, then synchronize the workgroup.
template <int N>
__device__ __forceinline__ void wait_vm_barrier() {
  asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" : : "n"(N) : "memory");
}
// Wait for this wave's LDS operations only, then synchronize the workgroup
// (global stores still in flight keep going).
__device__ __forceinline__ void wait_lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" : : : "memory");
}
// c += a-rows x b-columns over 32 k: v_mfma_f32_16x16x32_{f16,bf16}, the
// accumulator updated in place.  Written as asm: for this instruction the
// compiler's builtin picks a form whose result may not overwrite its
// accumulator input, and with all 256 accumulator registers live it then
// copies accumulators through VGPRs around every MFMA.  The compiler does not
// know these are MFMAs, so it adds no wait states for their results: the
// kernel orders the accumulator reset and the reads of results itself.
// (Measured alone on every CU, this MFMA shape sustains about 15% more
// FLOP/s than 32 x 32 x 16 under the chip's power limit.)
template <typename T>
__device__ __forceinline__ void mfma16(f32x4& c, u32x4 a, u32x4 b);
template <>
__device__ __forceinline__ void mfma16<_Float16>(f32x4& c, u32x4 a, u32x4 b) {
  asm("v_mfma_f32_16x16x32_f16 %0, %1, %2, %0" : "+a"(c) : "v"(a), "v"(b));
}
template <>
__device__ __forceinline__ void mfma16<__bf16>(f32x4& c, u32x4 a, u32x4 b) {
  asm("v_mfma_f32_16x16x32_bf16 %0, %1, %2, %0" : "+a"(c) : "v"(a), "v"(b));
}

// c += a-rows x b-columns over 16 k: v_mfma_f32_32x32x16_f16, the 32 x 32
// accumulator (16 registers per lane) updated in place.  Used only by the
// step-ladder kernel that compares this MFMA shape with 16 x 16 x 32 at the
// same tile, loads and schedule; the same wait-state rules apply.
typedef float f32x16 __attribute__((ext_vector_type(16)));
__device__ __forceinline__ void mfma32_f16(f32x16& c, u32x4 a, u32x4 b) {
  asm("v_mfma_f32_32x32x16_f16 %0, %1, %2, %0" : "+a"(c) : "v"(a), "v"(b));
}

// Round two floats to the output type (round-to-nearest-even) and pack them
// (one v_cvt_pk_f16_f32 / v_cvt_pk_bf16_f32).
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
template <typename T>
__device__ __forceinline__ uint32_t pack2(float lo, float hi);
template <>
__device__ __forceinline__ uint32_t pack2<_Float16>(float lo, float hi) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2){lo, hi}, f16x2));
}
template <>
__device__ __forceinline__ uint32_t pack2<__bf16>(float lo, float hi) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2){lo, hi}, bf16x2));
}

// Transposing LDS read: within each 16-lane block, lane i receives element
// i % 4 of the 8 bytes addressed by lanes 4j + i / 4, for j = 0..3.
__device__ __forceinline__ u32x2 read_tr(const char* p) {
  s16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4*)p);
  return __builtin_bit_cast(u32x2, v);
}

// threadIdx.x through an opaque move: values derived from it are recomputed
// where they are used instead of being hoisted and kept live across the whole
// persistent loop (where they would compete with the epilogue for registers).
__device__ __forceinline__ int opaque_tid() {
  int t;
  asm volatile("v_mov_b32 %0, %1" : "=v"(t) : "v"((int)threadIdx.x));
  return t;
}

}  // namespace dg
