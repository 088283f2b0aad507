// Greedy acceptance of MTP drafts after a verify pass, and the advance of the
// committed lengths once the accepted rows are in the caches.
//
// Self-speculative decoding (release blog, section "Multi-Token Prediction",
// verify diagram): the main model scores the committed token and the drafts
// in one pass.  Its prediction at each position is the argmax of that
// position's logits; a draft is accepted while it equals the prediction for
// its position and every earlier draft was accepted, the first mismatch is
// rejected (the prediction replaces it) and everything after it is discarded.
// n_append = 1 + accepted rows (the committed token's and the accepted
// drafts') then join the caches.
//
// The argmax is HBM-bound (one pass over B * q_len * vocab logits, nothing
// reused), so it is split for bandwidth rather than arithmetic:
//   * argmax_partial: grid (chunks, rows).  Each workgroup scans one chunk of
//     one row with four independent 16-byte loads in flight per lane and
//     leaves (max, lowest index of the max) in the workspace.  Enough chunks
//     per row are used that a launch holds about 2048 workgroups even for a
//     single request.  The loop does about 2.5 VALU operations per bf16
//     logit, well below what would make it compute-bound.
//   * accept_finish: one wave per request combines the chunk results of its
//     q_len rows and runs the acceptance prefix.
// Measured on 64 x 4 x 152064 bf16 logits (78 MB): 25 us for both kernels,
// against about 17 us for a bare one-pass read of the same bytes.
// Ties resolve to the lowest index everywhere (within a lane by scan order,
// across lanes and chunks by comparing indices), so the result does not
// depend on the chunking.  bf16 logits are widened to fp32 exactly before
// any comparison.
#include <limits.h>

#include "common.hpp"
#include "launch.hpp"

namespace swa {

namespace {

constexpr int kAcceptThreads = 256;
constexpr int kLoadsInFlight = 4;
constexpr long kTargetBlocks = 2048;
constexpr long kChunkQuantum = 1024;  // elements; a multiple of every vector width
constexpr int kMaxAcceptLen = 16;    // largest q_len

// (v, i) replaces (bv, bi) when larger, or equal with a lower index.  A NaN
// never replaces anything.
__device__ __forceinline__ void take(float& bv, int& bi, float v, int i) {
  if (v > bv || (v == bv && i < bi)) {
    bv = v;
    bi = i;
  }
}

__device__ __forceinline__ void wave_best(float& v, int& i) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) {
    const float ov = __shfl_xor(v, off);
    const int oi = __shfl_xor(i, off);
    take(v, i, ov, oi);
  }
}

// the logits are read once
constexpr bool kAcceptNT = false;

__device__ __forceinline__ float widen(float x) { return x; }
__device__ __forceinline__ float widen(uint16_t x) { return __uint_as_float((uint32_t)x << 16); }

// One 16-byte vector of logits: its maximum, and the lowest position inside
// it that holds a given value.  bf16 is widened exactly: the high half of a
// dword is the fp32 value with its low 16 bits cleared, the low half is the
// dword shifted left by 16.
struct VecBf16 {
  static constexpr int E = 8;
  u32x4 x;
  __device__ __forceinline__ float at(int j) const {
    const uint32_t w = x[j >> 1];
    return __uint_as_float((j & 1) ? (w & 0xffff0000u) : (w << 16));
  }
  __device__ __forceinline__ float vmax() const {
    float m = __builtin_fmaxf(__builtin_fmaxf(at(0), at(1)), at(2));
    m = __builtin_fmaxf(__builtin_fmaxf(m, at(3)), at(4));
    m = __builtin_fmaxf(__builtin_fmaxf(m, at(5)), at(6));
    return __builtin_fmaxf(m, at(7));
  }
};
struct VecF32 {
  static constexpr int E = 4;
  u32x4 x;
  __device__ __forceinline__ float at(int j) const { return __uint_as_float(x[j]); }
  __device__ __forceinline__ float vmax() const {
    return __builtin_fmaxf(__builtin_fmaxf(at(0), at(1)), __builtin_fmaxf(at(2), at(3)));
  }
};
template <typename T>
struct VecOf;
template <>
struct VecOf<uint16_t> {
  typedef VecBf16 type;
};
template <>
struct VecOf<float> {
  typedef VecF32 type;
};

// Block-wide (value, lowest index) reduction; thread 0 writes the result.
__device__ __forceinline__ void block_best_store(float bv, int bi, float* out_v, int32_t* out_i) {
  wave_best(bv, bi);
  __shared__ float sv[kAcceptThreads / 64];
  __shared__ int si[kAcceptThreads / 64];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  if (lane == 0) {
    sv[wave] = bv;
    si[wave] = bi;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    for (int w = 1; w < kAcceptThreads / 64; ++w) take(bv, bi, sv[w], si[w]);
    *out_v = bv;
    *out_i = bi;
  }
}

// Vector path: each lane keeps the maximum it has seen and a copy of the
// first vector that reached it (a strictly larger vector maximum replaces it;
// lanes visit their vectors in increasing index order), so the inner loop
// costs one widen and one max per logit plus a compare and five selects per
// vector.  The lowest position of the maximum inside the kept vector is
// resolved once at the end.
template <typename T>
__global__ __launch_bounds__(kAcceptThreads) void argmax_partial_vec_kernel(AcceptArgs a) {
  typedef typename VecOf<T>::type V;
  constexpr int E = V::E;
  const int chunk = blockIdx.x;
  const long row = blockIdx.y;
  const T* lg = (const T*)a.logits + row * a.V;
  const long lo = (long)chunk * a.chunk_len;
  const long hi = lo + a.chunk_len < a.V ? lo + a.chunk_len : a.V;
  // V, lo and hi are multiples of E: every vector is wholly inside or outside.
  constexpr long step = (long)kAcceptThreads * E;
  float best = kNegInf;
  long best_e = -1;
  V keep;
  keep.x = u32x4{0, 0, 0, 0};
  auto consider = [&](const V& x, long e) {
    const float m = x.vmax();
    if (m > best) {
      best = m;
      best_e = e;
      keep = x;
    }
  };
  long e = lo + (long)threadIdx.x * E;
  for (; e + (kLoadsInFlight - 1) * step < hi; e += kLoadsInFlight * step) {
    V x[kLoadsInFlight];
#pragma unroll
    for (int u = 0; u < kLoadsInFlight; ++u) x[u].x = load_pol<kAcceptNT>((const u32x4*)(lg + e + u * step));
#pragma unroll
    for (int u = 0; u < kLoadsInFlight; ++u) consider(x[u], e + u * step);
  }
  for (; e < hi; e += step) {
    V x;
    x.x = load_pol<kAcceptNT>((const u32x4*)(lg + e));
    consider(x, e);
  }
  int bi = INT_MAX;
  if (best_e >= 0) {
#pragma unroll
    for (int j = E - 1; j >= 0; --j)
      if (keep.at(j) == best) bi = (int)(best_e + j);
  }
  const long slot = row * a.nchunk + chunk;
  block_best_store(best, bi, a.ws_v + slot, a.ws_i + slot);
}

// Element path for logits rows that are not 16-byte aligned.
template <typename T>
__global__ __launch_bounds__(kAcceptThreads) void argmax_partial_elem_kernel(AcceptArgs a) {
  const int chunk = blockIdx.x;
  const long row = blockIdx.y;
  const T* lg = (const T*)a.logits + row * a.V;
  const long lo = (long)chunk * a.chunk_len;
  const long hi = lo + a.chunk_len < a.V ? lo + a.chunk_len : a.V;
  float bv = kNegInf;
  int bi = INT_MAX;
  for (long e = lo + threadIdx.x; e < hi; e += kAcceptThreads) take(bv, bi, widen(lg[e]), (int)e);
  const long slot = row * a.nchunk + chunk;
  block_best_store(bv, bi, a.ws_v + slot, a.ws_i + slot);
}

// One wave per request.  The chunk results of all q_len rows and the drafts
// are loaded before any reduction, so the wave waits for memory once.
__global__ __launch_bounds__(64) void accept_finish_kernel(AcceptArgs a) {
  const int b = blockIdx.x, lane = threadIdx.x;
  const int draft_t = lane < a.T - 1 ? a.draft[(long)b * (a.T - 1) + lane] : -1;
  float bv[kMaxAcceptLen];
  int bi[kMaxAcceptLen];
#pragma unroll
  for (int t = 0; t < kMaxAcceptLen; ++t) {
    bv[t] = kNegInf;
    bi[t] = INT_MAX;
    if (t < a.T) {
      const long base = ((long)b * a.T + t) * a.nchunk;
      for (int c = lane; c < a.nchunk; c += 64) take(bv[t], bi[t], a.ws_v[base + c], a.ws_i[base + c]);
    }
  }
  int accepted = 0;
  bool open = true;
#pragma unroll
  for (int t = 0; t < kMaxAcceptLen; ++t) {
    if (t < a.T) {
      wave_best(bv[t], bi[t]);
      const int tok = bi[t] == INT_MAX ? 0 : bi[t];  // a row with no comparable entry (all NaN)
      if (lane == 0) a.target[(long)b * a.T + t] = tok;
      if (t + 1 < a.T && open) {
        if (tok == __shfl(draft_t, t))
          ++accepted;
        else
          open = false;
      }
    }
  }
  if (lane == 0) a.n_append[b] = 1 + accepted;
}

__global__ __launch_bounds__(256) void advance_kernel(int32_t* cache_len, const int32_t* n_append, int B) {
  const int b = blockIdx.x * 256 + threadIdx.x;
  if (b < B) cache_len[b] += n_append[b];
}

}  // namespace

AcceptPlan plan_accept(int B, int T, long V) {
  AcceptPlan p = {};
  const long rows = (long)B * T;
  long want = (kTargetBlocks + rows - 1) / rows;  // chunks per row
  if (want < 1) want = 1;
  long cl = (V + want - 1) / want;
  cl = (cl + kChunkQuantum - 1) / kChunkQuantum * kChunkQuantum;
  p.chunk_len = cl;
  p.nchunk = (int)((V + cl - 1) / cl);
  p.ws_bytes = (size_t)rows * p.nchunk * (sizeof(float) + sizeof(int32_t));
  return p;
}

hipError_t launch_accept(AcceptArgs a, const AcceptPlan& p, hipStream_t s) {
  const long rows = (long)a.B * a.T;
  a.chunk_len = p.chunk_len;
  a.nchunk = p.nchunk;
  a.ws_i = (int32_t*)(a.ws_v + rows * p.nchunk);
  const dim3 grid(p.nchunk, (unsigned)rows);
  const bool vec = ((uintptr_t)a.logits % 16 == 0) && ((a.V * a.elem_bytes) % 16 == 0);
  if (a.elem_bytes == 2) {
    if (vec)
      hipLaunchKernelGGL(argmax_partial_vec_kernel<uint16_t>, grid, dim3(kAcceptThreads), 0, s, a);
    else
      hipLaunchKernelGGL(argmax_partial_elem_kernel<uint16_t>, grid, dim3(kAcceptThreads), 0, s, a);
  } else {
    if (vec)
      hipLaunchKernelGGL(argmax_partial_vec_kernel<float>, grid, dim3(kAcceptThreads), 0, s, a);
    else
      hipLaunchKernelGGL(argmax_partial_elem_kernel<float>, grid, dim3(kAcceptThreads), 0, s, a);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(accept_finish_kernel, dim3(a.B), dim3(64), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_advance(int32_t* cache_len, const int32_t* n_append, int B, hipStream_t s) {
  hipLaunchKernelGGL(advance_kernel, dim3((B + 255) / 256), dim3(256), 0, s, cache_len, n_append, B);
  return hipGetLastError();
}

}  // namespace swa
