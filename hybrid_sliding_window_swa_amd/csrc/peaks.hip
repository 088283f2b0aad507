// swa_peaks: the ceilings the attention kernels are measured against, taken
// on the GPU itself (the datasheet figures are 8 TB/s HBM and 2.5 PFLOP/s
// dense bf16 MFMA at the peak engine clock).
//
//   * HBM streaming read: a grid-stride read of 8 GiB, four independent
//     16-byte loads in flight per thread, XOR-reduced so nothing is dead code.
//   * HBM copy: the same grid stride reading one 8 GiB buffer and writing
//     another (bytes read + bytes written per second).
//   * Both with default and with non-temporal loads / stores; the faster
//     policy is the ceiling.
//   * bf16 MFMA: v_mfma_f32_32x32x16_bf16 on four independent accumulators,
//     two waves per SIMD, operands in registers (no memory traffic).
//
// Every kernel runs untimed for about half a second first, so the clocks
// are at their sustained-load level, then the mean of several launches is
// timed with HIP events (the streaming kernels: best of five grid sizes and
// two cache policies).
// One JSON line per measurement on stdout.
// All accesses are grid-stride loops bounded by the element count.
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stdio.h>

namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

// NT: non-temporal loads and stores (the data is touched once)
template <bool NT>
__device__ __forceinline__ u32x4 ld(const u32x4* p) {
  if constexpr (NT) return __builtin_nontemporal_load(p);
  return *p;
}

template <bool NT>
__global__ __launch_bounds__(256) void read_kernel(const u32x4* __restrict__ p, long n16, uint32_t* out) {
  u32x4 acc = {0, 0, 0, 0};
  long i = blockIdx.x * 256L + threadIdx.x;
  const long stride = (long)gridDim.x * 256;
  for (; i + 3 * stride < n16; i += 4 * stride) {
    const u32x4 a = ld<NT>(p + i), b = ld<NT>(p + i + stride), c = ld<NT>(p + i + 2 * stride),
                d = ld<NT>(p + i + 3 * stride);
    acc ^= a ^ b ^ c ^ d;
  }
  for (; i < n16; i += stride) acc ^= ld<NT>(p + i);
  if ((acc.x ^ acc.y ^ acc.z ^ acc.w) == 0x9e3779b9u) out[0] = 1;
}

template <bool NT>
__global__ __launch_bounds__(256) void copy_kernel(const u32x4* __restrict__ p, u32x4* __restrict__ q, long n16) {
  long i = blockIdx.x * 256L + threadIdx.x;
  const long stride = (long)gridDim.x * 256;
  for (; i < n16; i += stride) {
    const u32x4 v = ld<NT>(p + i);
    if constexpr (NT) {
      __builtin_nontemporal_store(v, q + i);
    } else {
      q[i] = v;
    }
  }
}

constexpr int kMfmaIter = 8192;

__global__ __launch_bounds__(512) void mfma_kernel(float* out, float seed) {
  bf16x8 a, b;
  for (int i = 0; i < 8; ++i) {
    a[i] = (__bf16)(seed * (float)(threadIdx.x + i));
    b[i] = (__bf16)(seed - (float)i);
  }
  f32x16 acc[4] = {};
  for (int it = 0; it < kMfmaIter; ++it) {
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc[j], 0, 0, 0);
  }
  float r = 0.0f;
  for (int j = 0; j < 4; ++j)
    for (int v = 0; v < 16; ++v) r += acc[j][v];
  out[blockIdx.x * blockDim.x + threadIdx.x] = r;
}

bool ok(hipError_t e, const char* what) {
  if (e != hipSuccess) {
    fprintf(stderr, "swa_peaks: %s failed: %s\n", what, hipGetErrorString(e));
    return false;
  }
  return true;
}

// untimed repetition for `settle_ms`, then the mean of `reps` timed launches
template <typename F>
float time_ms(F launch, float settle_ms, int reps) {
  hipEvent_t s, e;
  (void)hipEventCreate(&s);
  (void)hipEventCreate(&e);
  float elapsed = 0.0f;
  while (elapsed < settle_ms) {
    (void)hipEventRecord(s);
    launch();
    (void)hipEventRecord(e);
    (void)hipEventSynchronize(e);
    float ms = 0.0f;
    (void)hipEventElapsedTime(&ms, s, e);
    elapsed += ms;
  }
  (void)hipEventRecord(s);
  for (int r = 0; r < reps; ++r) launch();
  (void)hipEventRecord(e);
  (void)hipEventSynchronize(e);
  float ms = 0.0f;
  (void)hipEventElapsedTime(&ms, s, e);
  (void)hipEventDestroy(s);
  (void)hipEventDestroy(e);
  return ms / reps;
}

}  // namespace

int main() {
  int dev = 0, cus = 0;
  if (!ok(hipGetDevice(&dev), "hipGetDevice") ||
      !ok(hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev), "CU count"))
    return 1;
  const long bytes = 8L << 30;
  const long n16 = bytes / 16;
  u32x4 *a = nullptr, *b = nullptr;
  uint32_t* flag = nullptr;
  float* sink = nullptr;
  const int mfma_blocks = 2 * cus;  // 512 threads: two waves per SIMD
  if (!ok(hipMalloc(&a, bytes), "hipMalloc") || !ok(hipMalloc(&b, bytes), "hipMalloc") ||
      !ok(hipMalloc(&flag, 4), "hipMalloc") || !ok(hipMalloc(&sink, (size_t)mfma_blocks * 512 * 4), "hipMalloc"))
    return 1;
  if (!ok(hipMemset(a, 1, bytes), "hipMemset") || !ok(hipDeviceSynchronize(), "init")) return 1;

  // streaming kernels: best of several grid sizes and both cache policies
  // (clocks settle on the first)
  float rd = 1e30f, cp = 1e30f;
  int rd_grid = 0, cp_grid = 0;
  bool rd_nt = false, cp_nt = false;
  for (int nt = 0; nt < 2; ++nt) {
    for (int mult : {4, 8, 16, 32, 64}) {
      const int grid = mult * cus;
      const float settle = (mult == 4 && nt == 0) ? 500.0f : 0.0f;
      const float r = time_ms(
          [&] {
            if (nt)
              hipLaunchKernelGGL(read_kernel<true>, dim3(grid), dim3(256), 0, 0, a, n16, flag);
            else
              hipLaunchKernelGGL(read_kernel<false>, dim3(grid), dim3(256), 0, 0, a, n16, flag);
          },
          settle, 10);
      if (r < rd) { rd = r; rd_grid = grid; rd_nt = nt; }
      const float c = time_ms(
          [&] {
            if (nt)
              hipLaunchKernelGGL(copy_kernel<true>, dim3(grid), dim3(256), 0, 0, a, b, n16);
            else
              hipLaunchKernelGGL(copy_kernel<false>, dim3(grid), dim3(256), 0, 0, a, b, n16);
          },
          settle, 10);
      if (c < cp) { cp = c; cp_grid = grid; cp_nt = nt; }
    }
  }
  printf("{\"measure\": \"hbm_read\", \"bytes\": %ld, \"grid\": %d, \"nontemporal\": %s, \"ms\": %.4f, \"GB/s\": %.1f}\n",
         bytes, rd_grid, rd_nt ? "true" : "false", rd, bytes / (rd * 1e-3) / 1e9);
  printf("{\"measure\": \"hbm_copy\", \"bytes_read_plus_written\": %ld, \"grid\": %d, \"nontemporal\": %s, \"ms\": %.4f, "
         "\"GB/s\": %.1f}\n",
         2 * bytes, cp_grid, cp_nt ? "true" : "false", cp, 2.0 * bytes / (cp * 1e-3) / 1e9);
  const float mm = time_ms([&] { hipLaunchKernelGGL(mfma_kernel, dim3(mfma_blocks), dim3(512), 0, 0, sink, 0.001f); },
                           500.0f, 10);
  const double flop = (double)mfma_blocks * 8 * kMfmaIter * 4 * 32768.0;
  printf("{\"measure\": \"mfma_bf16_32x32x16\", \"flop\": %.4e, \"ms\": %.4f, \"TFLOP/s\": %.1f}\n", flop, mm,
         flop / (mm * 1e-3) / 1e12);
  if (!ok(hipDeviceSynchronize(), "kernels")) return 1;
  (void)hipFree(a);
  (void)hipFree(b);
  (void)hipFree(flag);
  (void)hipFree(sink);
  return 0;
}
