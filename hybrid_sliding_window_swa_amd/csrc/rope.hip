// Partial rotary position embedding, in place, on query or key rows.
//
// The pages give the RoPE bases (technical-report digest, "Pre-training",
// long-context extension: 10000 for the sliding-window layers, 640000 for the
// global layers, 5000000 after the 256K extension) and the fraction of each
// head that rotates (partial_rotary_factor 0.334 in the model card's config
// extract).  The pairing is not on the pages; this library rotates the first
// `rot` dimensions of every head in rot/2 pairs (i, i + rot/2) by the angle
// pos * base^(-2i/rot) and leaves the remaining dimensions untouched.
//
// HBM-bound (each rotated element is read and written once), so the kernel
// touches only the 16-byte vectors that hold the first `rot` dimensions of a
// row, with coalesced vector loads and stores staged through LDS:
//   1. the block's rows (consecutive [position, head] rows) are copied into
//      LDS with a pitch of an odd number of dwords (no bank conflicts when
//      each lane walks its own row);
//   2. the cos / sin of every (position, pair) the block needs are computed
//      once and shared by all heads of that position: the angle is formed in
//      fp64 and reduced modulo 2*pi before fp32 sincosf, so positions up to
//      2^31 keep full fp32 accuracy;
//   3. one lane per row rotates its pairs in LDS in fp32 (bf16 rows are
//      widened exactly and rounded to nearest even on the way back);
//   4. the vectors are stored back.
#include "common.hpp"
#include "launch.hpp"

namespace swa {

namespace {

constexpr int kRopeThreads = 256;
// every rotated vector is read and written once
constexpr bool kRopeNT = false;
constexpr double kTwoPi = 6.283185307179586476925286766559;
constexpr double kInvTwoPi = 0.15915494309189533576888376337251;

__device__ __forceinline__ float load_elem(const uint32_t* row, int e, int esize) {
  if (esize == 4) return __uint_as_float(row[e]);
  const uint32_t w = row[e >> 1];
  return __uint_as_float((e & 1) ? (w & 0xffff0000u) : (w << 16));
}

__device__ __forceinline__ void store_elem(uint32_t* row, int e, float v, int esize) {
  if (esize == 4) {
    row[e] = __float_as_uint(v);
    return;
  }
  const __bf16 h = (__bf16)v;  // round to nearest even
  const uint16_t bits = __builtin_bit_cast(uint16_t, h);
  reinterpret_cast<uint16_t*>(row)[e] = bits;
}

__global__ __launch_bounds__(kRopeThreads) void rope_kernel(RopeArgs a) {
  extern __shared__ uint32_t lds[];
  const int tid = threadIdx.x;
  const long r0 = (long)blockIdx.x * a.rows_blk;
  const int nrows = (int)((a.rows - r0) < a.rows_blk ? (a.rows - r0) : a.rows_blk);
  const long row_bytes = (long)a.D * a.esize;
  uint8_t* gbase = (uint8_t*)a.x + r0 * row_bytes;
  const int nv = a.nv, pitch = a.pitch_dw, half = a.rot / 2;

  for (int q = tid; q < nrows * nv; q += kRopeThreads) {
    const int row = q / nv, v = q - row * nv;
    const u32x4 d = load_pol<kRopeNT>((const u32x4*)(gbase + row * row_bytes + v * 16));
    uint32_t* dst = lds + row * pitch + v * 4;
    dst[0] = d[0];
    dst[1] = d[1];
    dst[2] = d[2];
    dst[3] = d[3];
  }

  // cos / sin of every (position, pair) this block touches
  const long p_first = r0 / a.H;
  const int np = (int)((r0 + nrows - 1) / a.H - p_first + 1);
  float2* tab = reinterpret_cast<float2*>(lds + ((a.rows_blk * pitch + 1) & ~1));  // 8-byte aligned
  for (int q = tid; q < np * half; q += kRopeThreads) {
    const int pl = q / half, i = q - pl * half;
    const long p = p_first + pl;
    const long b = p / a.S, s = p - b * a.S;
    const long pos = (a.pos0 ? (long)a.pos0[b] : 0L) + a.pos_offset + s;
    const double freq = exp2(-2.0 * i / a.rot * a.log2_base);
    const double th = (double)pos * freq;
    const double r = th - rint(th * kInvTwoPi) * kTwoPi;
    float sn, cs;
    sincosf((float)r, &sn, &cs);
    tab[q] = make_float2(cs, sn);
  }
  __syncthreads();

  for (int row = tid; row < nrows; row += kRopeThreads) {
    uint32_t* x = lds + row * pitch;
    const float2* t = tab + (int)((r0 + row) / a.H - p_first) * half;
    for (int i = 0; i < half; ++i) {
      const float u = load_elem(x, i, a.esize), w = load_elem(x, i + half, a.esize);
      const float2 cs = t[i];
      store_elem(x, i, u * cs.x - w * cs.y, a.esize);
      store_elem(x, i + half, w * cs.x + u * cs.y, a.esize);
    }
  }
  __syncthreads();

  for (int q = tid; q < nrows * nv; q += kRopeThreads) {
    const int row = q / nv, v = q - row * nv;
    const uint32_t* src = lds + row * pitch + v * 4;
    store_pol<kRopeNT>(u32x4{src[0], src[1], src[2], src[3]}, (u32x4*)(gbase + row * row_bytes + v * 16));
  }
}

}  // namespace

RopePlan plan_rope(int H, int D, int rot, int esize) {
  RopePlan p = {};
  p.nv = (rot * esize + 15) / 16;
  p.pitch_dw = p.nv * 4 + 1;
  // rows per block: up to one per lane, while rows + table stay within 48 KB
  int rows = kRopeThreads;
  for (;;) {
    const long np = rows / H + 2;
    const long bytes = (long)((rows * p.pitch_dw + 1) & ~1) * 4 + np * (rot / 2) * 8;
    if (bytes <= 48 * 1024 || rows == 1) {
      p.lds_bytes = (size_t)bytes;
      break;
    }
    rows /= 2;
  }
  p.rows_blk = rows;
  return p;
}

hipError_t launch_rope(RopeArgs a, hipStream_t s) {
  const RopePlan p = plan_rope(a.H, a.D, a.rot, a.esize);
  a.nv = p.nv;
  a.pitch_dw = p.pitch_dw;
  a.rows_blk = p.rows_blk;
  const long blocks = (a.rows + p.rows_blk - 1) / p.rows_blk;
  hipLaunchKernelGGL(rope_kernel, dim3((unsigned)blocks), dim3(kRopeThreads), p.lds_bytes, s, a);
  return hipGetLastError();
}

}  // namespace swa
