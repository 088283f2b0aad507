// Allocation-free variant of swa_attn_verify: the split-KV partials (running
// max, running sum and unnormalised output per query row and split) live in a
// file-scope device array instead of a caller-provided workspace, for callers
// that cannot allocate device memory (code under HIP graph capture, tight
// serving loops, harnesses that forbid allocation).
//
// Each GPU the library runs on holds its own copy of `scratch` from module
// load until the process ends.  In host code the array's name is only a
// host-side stand-in for the symbol: its device address is looked up with
// hipGetSymbolAddress once per device (with that device current, on the
// first call there) and only that address is ever passed to the kernels.
// Every call on a GPU shares that GPU's array; nothing in it has to start at
// zero (every partial the combine reads is written by the same call first).
#include <hip/hip_runtime.h>

#include <atomic>
#include <mutex>

#include "swa_attn.h"

namespace {

constexpr size_t kScratchBytes = SWA_VERIFY_NOALLOC_SCRATCH_BYTES;
static_assert(kScratchBytes % 256 == 0, "the scratch size keeps 256-byte alignment");

static __device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::atomic<void*> g_scratch_ptr[kMaxDevices];
std::mutex g_scratch_mu;

// Device address of this device's copy of `scratch`, or nullptr on failure.
void* scratch_for_current_device() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  void* p = g_scratch_ptr[dev].load(std::memory_order_acquire);
  if (p) return p;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  p = g_scratch_ptr[dev].load(std::memory_order_relaxed);
  if (p) return p;
  void* addr = nullptr;
  if (hipGetSymbolAddress(&addr, HIP_SYMBOL(scratch)) != hipSuccess || !addr) return nullptr;
  g_scratch_ptr[dev].store(addr, std::memory_order_release);
  return addr;
}

}  // namespace

extern "C" swa_status_t swa_attn_verify_noalloc(const void* q, const void* k_new, const void* v_new,
                                                const void* k_cache, const void* v_cache,
                                                const int32_t* cache_len, const float* sinks, void* o, int B,
                                                int q_len, int Hq, int Hkv, int D, int cache_slots, int ring,
                                                int window, float sm_scale, swa_dtype_t dtype, void* stream) {
  const size_t need =
      swa_attn_verify_workspace_bytes(B, q_len, Hq, Hkv, D, cache_slots, ring, window, dtype);
  if (need > kScratchBytes) return SWA_ERR_WORKSPACE;
  void* ws = nullptr;
  if (need > 0) {
    ws = scratch_for_current_device();
    if (!ws) return SWA_ERR_LAUNCH;
  }
  // the same validation, plan and kernels as swa_attn_verify
  return swa_attn_verify(q, k_new, v_new, k_cache, v_cache, cache_len, sinks, o, B, q_len, Hq, Hkv, D,
                         cache_slots, ring, window, sm_scale, dtype, ws, need > 0 ? kScratchBytes : 0, stream);
}
