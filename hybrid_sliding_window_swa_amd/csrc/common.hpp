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
constexpr float kLn2 = 0.69314718055994531f;
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

// Both halves of the wave combined, lane l with lane l ^ 32, in registers:
// v_permlane32_swap leaves (x_lo, x_lo) in one result and (x_hi, x_hi) in the
// other, so every lane sees both values of its pair without an LDS round trip.
__device__ __forceinline__ float halves_max(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __builtin_elementwise_maximum(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float halves_sum(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Raw buffer resource over [base, base + bytes): a load past the end reads
// zeros and a store past the end is dropped (the buffer range check), so
// ragged tails need no per-lane clamps or branches, and the tile / row
// offset can live in a scalar register.
typedef __amdgpu_buffer_rsrc_t rsrc_t;
__device__ __forceinline__ rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}
// Cache policy of a vector memory access: kCacheNT marks data that is
// touched once (streamed rows, outputs) as non-temporal, so it does not
// displace reused data in the L2 and the Infinity Cache.
constexpr int kCacheDefault = 0, kCacheNT = 2;
template <int POLICY = kCacheDefault>
__device__ __forceinline__ u32x4 buf_load16(rsrc_t r, uint32_t voff, uint32_t soff) {
  return __builtin_amdgcn_raw_buffer_load_b128(r, (int)voff, (int)soff, POLICY);
}
template <int POLICY = kCacheDefault>
__device__ __forceinline__ void buf_store16(u32x4 v, rsrc_t r, uint32_t voff, uint32_t soff) {
  __builtin_amdgcn_raw_buffer_store_b128(v, r, (int)voff, (int)soff, POLICY);
}

// One wave-wide 16-byte-per-lane load from global memory straight into LDS:
// lane l's 16 bytes (voffset bytes past first_row, checked against
// num_records; a lane out of range writes zeros) land at LDS byte address
// lds_byte + 16 l, so one instruction fills a contiguous 1 KiB window.
// Written as asm so that the compiler's wait-count pass, which cannot tell
// one LDS buffer from another, does not make every later LDS read wait for
// these loads: the caller waits for them itself (s_waitcnt vmcnt) before the
// barrier that publishes the window.  vmcnt retires in order, so loads the
// compiler does not count only make its own waits stricter.  The buffer
// descriptor is base, stride 0, num_records and the flags word of make_rsrc;
// lds_byte and the descriptor must be wave-uniform.
__device__ __forceinline__ void lds_dma16(const void* first_row, uint32_t num_records, uint32_t lds_byte,
                                          uint32_t voffset) {
  const uint64_t base = (uint64_t)(uintptr_t)first_row;
  const u32x4 desc = {(uint32_t)base, (uint32_t)(base >> 32) & 0xffffu, num_records, 0x00020000u};
  __asm__ volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds"
                   :
                   : "s"(lds_byte), "v"(voffset), "s"(desc)
                   : "m0");
}

// The descriptor lds_dma16 builds, for callers that keep one across several
// loads: base, stride 0, num_records, the flags word of make_rsrc.
__device__ __forceinline__ u32x4 buffer_desc(const void* base_ptr, uint32_t num_records) {
  const uint64_t base = (uint64_t)(uintptr_t)base_ptr;
  return u32x4{(uint32_t)base, (uint32_t)(base >> 32) & 0xffffu, num_records, 0x00020000u};
}

// lds_dma16 with a prebuilt descriptor and a scalar byte offset soffset
// added to every lane's address (the range check is made on voffset alone,
// so a lane past num_records still writes zeros and reads nothing); desc,
// soffset and lds_byte must be wave-uniform.
__device__ __forceinline__ void lds_dma16_soff(u32x4 desc, uint32_t soffset, uint32_t lds_byte, uint32_t voffset) {
  __asm__ volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, %3 offen lds"
                   :
                   : "s"(lds_byte), "v"(voffset), "s"(desc), "s"(soffset)
                   : "m0");
}

// Plain global accesses with a cache policy (see kCacheNT).
template <bool NT, typename T>
__device__ __forceinline__ T load_pol(const T* p) {
  if constexpr (NT) return __builtin_nontemporal_load(p);
  return *p;
}
template <bool NT, typename T>
__device__ __forceinline__ void store_pol(T v, T* p) {
  if constexpr (NT) {
    __builtin_nontemporal_store(v, p);
  } else {
    *p = v;
  }
}

// Scheduling-group masks of __builtin_amdgcn_sched_group_barrier.
constexpr int kSchedValu = 0x002, kSchedMfma = 0x008, kSchedDsRead = 0x100;

__device__ __forceinline__ bool wave_any(bool p) { return __ballot(p) != 0ull; }

// Index of this wave in its workgroup, as a wave-uniform (scalar) value so
// that everything derived from it stays in SGPRs and branches stay uniform.
__device__ __forceinline__ int wave_index() {
  return __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
}

__device__ __forceinline__ uint32_t pack_bf16x2(uint16_t lo, uint16_t hi) {
  return (uint32_t)lo | ((uint32_t)hi << 16);
}

typedef short i16x4 __attribute__((ext_vector_type(4)));

// A tile of 32 rows x D bf16 in LDS, row-major with a padded row pitch of
// PITCH elements (a multiple of 8).  Every MFMA operand address is a per-lane
// base plus a compile-time offset, so no address arithmetic sits in the tile
// loop.  gfx950's LDS has 64 banks of 4 bytes (256 bytes per clock; measured
// with the SQ_LDS_BANK_CONFLICT counter per access pattern):
//   * K tiles, pitch D + 8: a 16-byte K-operand read serves 16 lanes per
//     clock, rows 0..15 of one chunk, whose 16-byte positions advance by one
//     per row, so all 64 banks are distinct.
//   * V tiles, pitch D + 32: ds_read_b64_tr_b16 serves 32 lanes per clock,
//     rows n0..n0+3 x 64 bytes; the pitch is 16 (D = 128) or 48 (D = 64)
//     dwords modulo 64, so the four rows land on disjoint 16-bank groups.
//     (D + 16 costs two extra clocks per read.)
//   * staging tiles of D/2 columns + 8, as K tiles.
typedef __attribute__((address_space(3))) uint16_t lds_u16;
typedef __attribute__((address_space(3))) bf16x8 lds_bf16x8;
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;

// 32-bit LDS byte address of a pointer into __shared__ memory.
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)p;
}

// tile base + per-lane offset, opaque to the optimizer (an empty asm with a
// register operand; it touches no memory) so that every operand read of the
// tile becomes this one register plus an immediate offset.
__device__ __forceinline__ const lds_u16* lane_base(uint32_t tile_addr, uint32_t lane_off_bytes) {
  uint32_t a = tile_addr + lane_off_bytes;
  __asm__ volatile("" : "+v"(a));
  return (const lds_u16*)(uintptr_t)a;
}

template <int D, int PITCH>
struct PadTile {
  static_assert(PITCH % 8 == 0, "rows must stay 16-byte aligned");
  static constexpr int ELEMS = 32 * PITCH;   // bf16 elements per tile
  static __device__ __forceinline__ int off(int row, int d) { return row * PITCH + d; }

  // K-operand reads: lane (col, half) reads row `col`, d in [16c + 8*half, +8)
  static __device__ __forceinline__ uint32_t k_lane_off(int lane) {
    return 2u * ((lane & 31) * PITCH + 8 * (lane >> 5));
  }
  static __device__ __forceinline__ bf16x8 k_operand(const lds_u16* b, int c) {
    return *(const lds_bf16x8*)(b + 16 * c);
  }

  // V^T-operand reads of O^T += V^T P^T for output rows d in [32db, 32db+32)
  // and keys [16kc, 16kc + 16): lane l receives V[n][32db + l%32] for
  // n = 16kc + 4(l/32) + {0..3} and then n + 8 + {0..3}.  gfx950's
  // ds_read_b64_tr_b16 gives lane j of each 16-lane group element j%4 of the
  // 8-byte chunks addressed by lanes 4e + j/4 (e = 0..3), so source lane s
  // addresses row n0 + s/4, columns d0 + 4(s%4).
  static __device__ __forceinline__ uint32_t vt_lane_off(int lane) {
    const int s = lane & 15;
    return 2u * ((4 * (lane >> 5) + (s >> 2)) * PITCH + 16 * ((lane >> 4) & 1) + 4 * (s & 3));
  }
  static __device__ __forceinline__ bf16x8 vt_operand(const lds_u16* b, int db, int kc) {
    const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(b + 16 * kc * PITCH + 32 * db));
    const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(b + (16 * kc + 8) * PITCH + 32 * db));
    typedef short i16x8 __attribute__((ext_vector_type(8)));
    const i16x8 both = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
    return __builtin_bit_cast(bf16x8, both);
  }
};
template <int D>
using KTile = PadTile<D, D + 8>;
template <int D>
using VTile = PadTile<D, D + 32>;

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

// Two weights rounded to bf16 and packed (a pair of the B operand of P V),
// and their sum added to the row sum t: with ROUNDED the rounded weights
// that enter P V (one v_dot2_f32_bf16), else the fp32 weights before the
// rounding (within 2^-9 of each rounded weight; two VALU adds).  gfx950's
// v_dot2_f32_bf16 issues to the matrix-core pipeline and waits for every
// MFMA in flight (measured: 13 cycles of exclusive matrix-core time each),
// while an add runs beside the MFMAs: kernels that keep the matrix core
// busy take the adds, the others the rounded sum.
template <bool ROUNDED = false>
__device__ __forceinline__ uint32_t pack_sum(float e0, float e1, float& t) {
  const bf16x2 w2 = {(__bf16)e0, (__bf16)e1};
  uint32_t w = __builtin_bit_cast(uint32_t, w2);
  __asm__ volatile("" : "+v"(w));
  if constexpr (ROUNDED) {
    const bf16x2 one = {(__bf16)1.0f, (__bf16)1.0f};
    t = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, w), one, t, false);
  } else {
    t += e0 + e1;
  }
  return w;
}

// Wave-local LDS ordering: make this wave's LDS writes visible to its other
// lanes before the reads that follow (and keep reads before later writes).
__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

}  // namespace swa
