// Device-side helpers shared by the gfx950 attention kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace swa {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kNegInf = -__builtin_inff();

// Lazy-rescale threshold (log2 units): the running maximum used to shift the
// exponents is only raised when a new score exceeds it by more than this, so
// unnormalised weights stay below 2^kRescaleTau (exact in bf16 / fp32) and the
// accumulator rescale is skipped for most tiles.
constexpr float kRescaleTau = 8.0f;

__device__ __forceinline__ float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }

// 32x32x16 bf16 MFMA: C[i][j] += sum_k A[i][k] B[k][j].  Lane l supplies
// A[l%32][k in group l/32] and B[k in group l/32][l%32]; both operands must use
// the same (lane group, register) -> k assignment.  C: lane l holds column
// j = l%32, register v holds row 8*(v/4) + 4*(l/32) + v%4.
__device__ __forceinline__ f32x16 mfma32(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// Row of the 32x32 MFMA result held in register v by a lane of half `half`.
__device__ __forceinline__ constexpr int c_row(int v, int half) {
  return 8 * (v >> 2) + 4 * half + (v & 3);
}

// Value of x in lane (l ^ 32).
__device__ __forceinline__ float swap_halves(float x) { return __shfl_xor(x, 32, 64); }

__device__ __forceinline__ bool wave_any(bool p) { return __ballot(p) != 0ull; }

__device__ __forceinline__ uint32_t pack_bf16x2(uint16_t lo, uint16_t hi) {
  return (uint32_t)lo | ((uint32_t)hi << 16);
}

// Wave-local LDS ordering: make this wave's LDS writes visible to its other
// lanes before the reads that follow (and keep reads before later writes).
__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

}  // namespace swa
