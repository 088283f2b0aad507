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
//     single request.
//   * accept_finish: one wave per request combines the chunk results of its
//     q_len rows and runs the acceptance prefix.
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

__device__ __forceinline__ float widen(float x) { return x; }
__device__ __forceinline__ float widen(uint16_t x) { return __uint_as_float((uint32_t)x << 16); }

template <typename T>
struct Vec16;
template <>
struct Vec16<float> {
  static constexpr int E = 4;
  typedef f32x4 type;
};
template <>
struct Vec16<uint16_t> {
  static constexpr int E = 8;
  typedef uint16_t type __attribute__((ext_vector_type(8)));
};

template <typename T, bool VEC>
__global__ __launch_bounds__(kAcceptThreads) void argmax_partial_kernel(AcceptArgs a) {
  const int chunk = blockIdx.x;
  const long row = blockIdx.y;
  const T* lg = (const T*)a.logits + row * a.V;
  const long lo = (long)chunk * a.chunk_len;
  const long hi = lo + a.chunk_len < a.V ? lo + a.chunk_len : a.V;
  float bv = kNegInf;
  int bi = INT_MAX;
  if constexpr (VEC) {
    // V, lo and hi are multiples of E: every vector is wholly inside or outside.
    constexpr int E = Vec16<T>::E;
    typedef typename Vec16<T>::type vec_t;
    constexpr long step = (long)kAcceptThreads * E;
    for (long e = lo + (long)threadIdx.x * E; e < hi; e += kLoadsInFlight * step) {
      vec_t x[kLoadsInFlight];
#pragma unroll
      for (int u = 0; u < kLoadsInFlight; ++u)
        if (e + u * step < hi) x[u] = *(const vec_t*)(lg + e + u * step);
#pragma unroll
      for (int u = 0; u < kLoadsInFlight; ++u)
        if (e + u * step < hi) {
#pragma unroll
          for (int j = 0; j < E; ++j) take(bv, bi, widen(x[u][j]), (int)(e + u * step + j));
        }
    }
  } else {
    for (long e = lo + threadIdx.x; e < hi; e += kAcceptThreads) take(bv, bi, widen(lg[e]), (int)e);
  }
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
    const long slot = row * a.nchunk + chunk;
    a.ws_v[slot] = bv;
    a.ws_i[slot] = bi;
  }
}

__global__ __launch_bounds__(64) void accept_finish_kernel(AcceptArgs a) {
  const int b = blockIdx.x, lane = threadIdx.x;
  int accepted = 0;
  bool open = true;
  for (int t = 0; t < a.T; ++t) {
    const long row = (long)b * a.T + t;
    float bv = kNegInf;
    int bi = INT_MAX;
    for (int c = lane; c < a.nchunk; c += 64) take(bv, bi, a.ws_v[row * a.nchunk + c], a.ws_i[row * a.nchunk + c]);
    wave_best(bv, bi);
    if (bi == INT_MAX) bi = 0;  // a row with no comparable entry (all NaN)
    if (lane == 0) a.target[row] = bi;
    if (t + 1 < a.T && open) {
      if (bi == a.draft[(long)b * (a.T - 1) + t])
        ++accepted;
      else
        open = false;
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
      hipLaunchKernelGGL((argmax_partial_kernel<uint16_t, true>), grid, dim3(kAcceptThreads), 0, s, a);
    else
      hipLaunchKernelGGL((argmax_partial_kernel<uint16_t, false>), grid, dim3(kAcceptThreads), 0, s, a);
  } else {
    if (vec)
      hipLaunchKernelGGL((argmax_partial_kernel<float, true>), grid, dim3(kAcceptThreads), 0, s, a);
    else
      hipLaunchKernelGGL((argmax_partial_kernel<float, false>), grid, dim3(kAcceptThreads), 0, s, a);
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
