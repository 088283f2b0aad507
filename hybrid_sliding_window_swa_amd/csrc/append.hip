// Commit accepted tokens to a KV cache after a verify step.
//
// For request b the first n_append[b] of the q_len rows under verification
// (the committed token plus the accepted drafts; the release blog's
// "Multi-Token Prediction" diagram accepts a prefix, rejects one token and
// discards the rest) are copied to the slots of positions cache_len[b] + t:
// slot p % slots for a ring (the fixed-size sliding-window cache of the
// release blog's section on pushing efficiency), slot p for a linear cache.
// Rejected rows never touch the cache.  A plain 16-byte-vector copy.
#include "common.hpp"
#include "launch.hpp"

namespace swa {

__global__ __launch_bounds__(256) void append_kernel(AppendArgs a) {
  const int b = blockIdx.x, t = blockIdx.y;
  if (t >= a.n_append[b]) return;
  const long pos = (long)a.cache_len[b] + t;
  const long slot = a.ring ? pos % a.slots : pos;
  if (pos < 0 || slot >= a.slots) return;  // outside the cache: dropped
  const long src = ((long)b * a.T + t) * a.row_bytes;
  const long dst = ((long)b * a.slots + slot) * a.row_bytes;
  for (int c = threadIdx.x * 16; c < a.row_bytes; c += blockDim.x * 16) {
    *(u32x4*)(a.k_cache + dst + c) = *(const u32x4*)(a.k_new + src + c);
    *(u32x4*)(a.v_cache + dst + c) = *(const u32x4*)(a.v_new + src + c);
  }
}

hipError_t launch_append(const AppendArgs& a, hipStream_t s) {
  int threads = a.row_bytes / 16;
  if (threads > 256) threads = 256;
  if (threads < 64) threads = 64;
  hipLaunchKernelGGL(append_kernel, dim3(a.B, a.T), dim3(threads), 0, s, a);
  return hipGetLastError();
}

}  // namespace swa
