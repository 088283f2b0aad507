// swa_peaks: the ceilings the attention kernels are measured against, taken
// on the GPU itself (the datasheet figures are 8 TB/s HBM and 2.5 PFLOP/s
// dense bf16 MFMA at the peak engine clock).
//
//   * HBM streaming read: a read of 8 GiB, grid-stride or one contiguous
//     range per workgroup, four independent 16-byte loads in flight per
//     thread, XOR-reduced so nothing is dead code.
//   * The same 8 GiB read in the global-cache verify's pattern: one KV
//     head's 256-byte rows of a [rows, 8, 128] bf16 cache per workgroup
//     (the other heads' rows in between), the eight heads' workgroups of a
//     row range side by side.
//   * The 8 GiB copy in the sliding-window prefill's pattern: 2 KiB head-group
//     segments of 16 KiB token rows, one head group and token range per
//     workgroup, the eight groups' workgroups of a range side by side.
//   * HBM copy: reading one 8 GiB buffer and writing another (bytes read +
//     bytes written per second), best of 1, 2, 4 or 8 independent loads in
//     flight per thread before their stores, grid-stride or one contiguous
//     range per workgroup.
//   * Both with default and with non-temporal loads / stores; the faster
//     policy is the ceiling.
//   * bf16 MFMA: v_mfma_f32_32x32x16_bf16 on four independent accumulators,
//     two waves per SIMD, operands in registers (no memory traffic).
//   * The same with operands that change every instruction (pseudo-random
//     bf16 values): the rate at the clock the chip holds when the matrix
//     cores switch like they do on attention's data.
//   * Cold small read: the streaming read of 42,729,472 bytes (the bytes one
//     SWA-ring verify of 64 requests moves) right after 512 MiB of other
//     memory was written (so none of it sits in the L2 or the 256 MB
//     Infinity Cache), one launch timed with HIP events, median of 21: the
//     floor for a kernel that has to fetch that much from HBM in one launch.
//
// Every kernel runs untimed for about half a second first, so the clocks
// are at their sustained-load level, then the mean of several launches is
// timed with HIP events (the streaming kernels: best of five grid sizes and
// two cache policies; the copies also of the depths and orders above).
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

// Four independent 16-byte loads in flight per thread.  BLOCKED: workgroup
// b reads one contiguous range; otherwise grid-stride.
template <bool NT, bool BLOCKED = false>
__global__ __launch_bounds__(256) void read_kernel(const u32x4* __restrict__ p, long n16, uint32_t* out) {
  u32x4 acc = {0, 0, 0, 0};
  long i, end, stride;
  if constexpr (BLOCKED) {
    const long per = ((n16 + gridDim.x - 1) / gridDim.x + 1023) / 1024 * 1024;
    i = blockIdx.x * per + threadIdx.x;
    end = blockIdx.x * per + per < n16 ? blockIdx.x * per + per : n16;
    stride = 256;
  } else {
    i = blockIdx.x * 256L + threadIdx.x;
    end = n16;
    stride = (long)gridDim.x * 256;
  }
  for (; i + 3 * stride < end; i += 4 * stride) {
    const u32x4 a = ld<NT>(p + i), b = ld<NT>(p + i + stride), c = ld<NT>(p + i + 2 * stride),
                d = ld<NT>(p + i + 3 * stride);
    acc ^= a ^ b ^ c ^ d;
  }
  for (; i < end; i += stride) acc ^= ld<NT>(p + i);
  if ((acc.x ^ acc.y ^ acc.z ^ acc.w) == 0x9e3779b9u) out[0] = 1;
}

// The global-cache verify's access pattern: the buffer as a [rows, 8, 128]
// bf16 cache, workgroup w = 8 s + h reading the 256-byte rows of KV head h
// in row range s (so the eight heads' workgroups of a range run side by
// side), non-temporal, four 16-byte loads in flight per thread.  rows_per:
// rows per workgroup, a multiple of 64.
__global__ __launch_bounds__(256) void read_head_rows_kernel(const u32x4* __restrict__ p, long rows_per,
                                                             uint32_t* out) {
  u32x4 acc = {0, 0, 0, 0};
  const int t = threadIdx.x, h = blockIdx.x & 7;
  const long r0 = (long)(blockIdx.x >> 3) * rows_per;
  for (long r = r0 + t / 16; r + 48 < r0 + rows_per; r += 64) {
    const u32x4 a = ld<true>(p + (r * 8 + h) * 16 + (t & 15)), b = ld<true>(p + ((r + 16) * 8 + h) * 16 + (t & 15)),
                c = ld<true>(p + ((r + 32) * 8 + h) * 16 + (t & 15)), d = ld<true>(p + ((r + 48) * 8 + h) * 16 + (t & 15));
    acc ^= a ^ b ^ c ^ d;
  }
  if ((acc.x ^ acc.y ^ acc.z ^ acc.w) == 0x9e3779b9u) out[0] = 1;
}

template <bool NT>
__device__ __forceinline__ void st(u32x4 v, u32x4* p) {
  if constexpr (NT) {
    __builtin_nontemporal_store(v, p);
  } else {
    *p = v;
  }
}

// The sliding-window prefill's access pattern as a copy: both buffers as
// [tokens, 64, 128] bf16 (16 KiB token rows), workgroup w = 8 s + g
// copying the 2 KiB segment of head group g (heads 8g .. 8g + 7) of the
// token rows in range s, non-temporal, four 16-byte loads in flight per
// thread before their stores.  tok_per: tokens per workgroup, a multiple
// of 2.
__global__ __launch_bounds__(256) void copy_head_groups_kernel(const u32x4* __restrict__ p, u32x4* __restrict__ q,
                                                               long tok_per) {
  const int t = threadIdx.x, g = blockIdx.x & 7;
  const long t0 = (long)(blockIdx.x >> 3) * tok_per;
  // thread t: token (t / 128) + 2 k, chunk t % 128 of the 2 KiB segment
  for (long k = t0 + t / 128; k + 6 < t0 + tok_per; k += 8) {
    u32x4 v[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) v[j] = ld<true>(p + ((k + 2 * j) * 8 + g) * 128 + (t & 127));
#pragma unroll
    for (int j = 0; j < 4; ++j) st<true>(v[j], q + ((k + 2 * j) * 8 + g) * 128 + (t & 127));
  }
}

// DEPTH independent 16-byte loads in flight per thread, then their DEPTH
// stores.  BLOCKED: workgroup b copies one contiguous range (a stream per
// workgroup, like a strip of the attention kernels); otherwise grid-stride.
template <bool NT, int DEPTH, bool BLOCKED>
__global__ __launch_bounds__(256) void copy_kernel(const u32x4* __restrict__ p, u32x4* __restrict__ q, long n16) {
  long i, end, stride;
  if constexpr (BLOCKED) {
    const long per = ((n16 + gridDim.x - 1) / gridDim.x + 256L * DEPTH - 1) / (256L * DEPTH) * (256L * DEPTH);
    i = blockIdx.x * per + threadIdx.x;
    end = blockIdx.x * per + per < n16 ? blockIdx.x * per + per : n16;
    stride = 256;
  } else {
    i = blockIdx.x * 256L + threadIdx.x;
    end = n16;
    stride = (long)gridDim.x * 256;
  }
  for (; i + (DEPTH - 1) * stride < end; i += DEPTH * stride) {
    u32x4 v[DEPTH];
#pragma unroll
    for (int j = 0; j < DEPTH; ++j) v[j] = ld<NT>(p + i + j * stride);
#pragma unroll
    for (int j = 0; j < DEPTH; ++j) st<NT>(v[j], q + i + j * stride);
  }
  for (; i < end; i += stride) st<NT>(ld<NT>(p + i), q + i);
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

// The same MFMA stream on operands that change from one instruction to the
// next: eight (A, B) pairs per lane of pseudo-random bf16 values in
// [-2, 2) (an integer hash of the thread and pair index), each MFMA of an
// iteration on its own pair.  Attention's operands toggle like this; the
// constant operands above hardly switch the multipliers, and the chip's
// power-limited clock differs between the two.
__device__ __forceinline__ uint32_t hash32(uint32_t x) {
  x ^= x >> 16;
  x *= 0x7feb352dU;
  x ^= x >> 15;
  x *= 0x846ca68bU;
  x ^= x >> 16;
  return x;
}

__global__ __launch_bounds__(512) void mfma_rand_kernel(float* out, uint32_t seed) {
  bf16x8 a[8], b[8];
  const uint32_t t = blockIdx.x * blockDim.x + threadIdx.x;
#pragma unroll
  for (int j = 0; j < 8; ++j)
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      a[j][i] = (__bf16)((float)(hash32(seed ^ (t * 131u + j * 17u + i)) >> 8) * 0x1p-22f - 2.0f);
      b[j][i] = (__bf16)((float)(hash32(~seed ^ (t * 137u + j * 19u + i)) >> 8) * 0x1p-22f - 2.0f);
    }
  f32x16 acc[4] = {};
  for (int it = 0; it < kMfmaIter / 2; ++it) {
#pragma unroll
    for (int j = 0; j < 8; ++j) acc[j & 3] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[j], b[j], acc[j & 3], 0, 0, 0);
  }
  float r = 0.0f;
#pragma unroll
  for (int j = 0; j < 4; ++j)
#pragma unroll
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
  // (clocks settle on the first); copies also over 1, 2, 4 or 8 loads in
  // flight per thread, grid-stride or one contiguous range per workgroup
  float rd = 1e30f, cp = 1e30f;
  int rd_grid = 0, cp_grid = 0, cp_depth = 0;
  bool rd_nt = false, rd_blocked = false, cp_nt = false, cp_blocked = false;
  for (int nt = 0; nt < 2; ++nt) {
    for (int mult : {4, 8, 16, 32, 64}) {
      const int grid = mult * cus;
      const float settle = (mult == 4 && nt == 0) ? 500.0f : 0.0f;
      for (int blocked = 0; blocked < 2; ++blocked) {
        const float r = time_ms(
            [&] {
              if (nt && blocked)
                hipLaunchKernelGGL((read_kernel<true, true>), dim3(grid), dim3(256), 0, 0, a, n16, flag);
              else if (nt)
                hipLaunchKernelGGL((read_kernel<true, false>), dim3(grid), dim3(256), 0, 0, a, n16, flag);
              else if (blocked)
                hipLaunchKernelGGL((read_kernel<false, true>), dim3(grid), dim3(256), 0, 0, a, n16, flag);
              else
                hipLaunchKernelGGL((read_kernel<false, false>), dim3(grid), dim3(256), 0, 0, a, n16, flag);
            },
            blocked ? 0.0f : settle, 10);
        if (r < rd) { rd = r; rd_grid = grid; rd_nt = nt; rd_blocked = blocked; }
      }
      for (int blocked = 0; blocked < 2; ++blocked) {
        for (int depth : {1, 2, 4, 8}) {
          const float c = time_ms(
              [&] {
#define SWA_COPY(NTV, DV, BV) hipLaunchKernelGGL((copy_kernel<NTV, DV, BV>), dim3(grid), dim3(256), 0, 0, a, b, n16)
#define SWA_COPY_D(NTV, BV)       \
  switch (depth) {                \
    case 1: SWA_COPY(NTV, 1, BV); break; \
    case 2: SWA_COPY(NTV, 2, BV); break; \
    case 4: SWA_COPY(NTV, 4, BV); break; \
    default: SWA_COPY(NTV, 8, BV); break; \
  }
                if (nt && blocked) { SWA_COPY_D(true, true) }
                else if (nt) { SWA_COPY_D(true, false) }
                else if (blocked) { SWA_COPY_D(false, true) }
                else { SWA_COPY_D(false, false) }
#undef SWA_COPY_D
#undef SWA_COPY
              },
              0.0f, 10);
          if (c < cp) { cp = c; cp_grid = grid; cp_nt = nt; cp_depth = depth; cp_blocked = blocked; }
        }
      }
    }
  }
  printf("{\"measure\": \"hbm_read\", \"bytes\": %ld, \"grid\": %d, \"nontemporal\": %s, "
         "\"contiguous_per_workgroup\": %s, \"ms\": %.4f, \"GB/s\": %.1f}\n",
         bytes, rd_grid, rd_nt ? "true" : "false", rd_blocked ? "true" : "false", rd, bytes / (rd * 1e-3) / 1e9);
  printf("{\"measure\": \"hbm_copy\", \"bytes_read_plus_written\": %ld, \"grid\": %d, \"nontemporal\": %s, "
         "\"loads_in_flight\": %d, \"contiguous_per_workgroup\": %s, \"ms\": %.4f, \"GB/s\": %.1f}\n",
         2 * bytes, cp_grid, cp_nt ? "true" : "false", cp_depth, cp_blocked ? "true" : "false", cp,
         2.0 * bytes / (cp * 1e-3) / 1e9);
  {
    // rows of 2 KiB (eight heads x 256 bytes); grids that divide them evenly
    const long rows = bytes / 2048;
    float hr = 1e30f;
    int hr_grid = 0;
    for (int mult : {8, 16, 32, 64}) {
      const int grid = mult * cus;
      const long rows_per = rows / (grid / 8);
      if (rows_per % 64 != 0 || rows_per * (grid / 8) != rows) continue;
      const float r = time_ms(
          [&] { hipLaunchKernelGGL(read_head_rows_kernel, dim3(grid), dim3(256), 0, 0, a, rows_per, flag); }, 0.0f,
          10);
      if (r < hr) { hr = r; hr_grid = grid; }
    }
    printf("{\"measure\": \"hbm_read_head_rows\", \"bytes\": %ld, \"grid\": %d, \"ms\": %.4f, \"GB/s\": %.1f}\n",
           bytes, hr_grid, hr, bytes / (hr * 1e-3) / 1e9);
  }
  {
    const long toks = bytes / 16384;
    float hc = 1e30f;
    int hc_grid = 0;
    for (int mult : {1, 2, 4, 8}) {
      const int grid = mult * cus;
      const long tok_per = toks / (grid / 8);
      if (tok_per % 8 != 0 || tok_per * (grid / 8) != toks) continue;
      const float r = time_ms(
          [&] { hipLaunchKernelGGL(copy_head_groups_kernel, dim3(grid), dim3(256), 0, 0, a, b, tok_per); }, 0.0f, 10);
      if (r < hc) { hc = r; hc_grid = grid; }
    }
    printf("{\"measure\": \"hbm_copy_head_groups\", \"bytes_read_plus_written\": %ld, \"grid\": %d, \"ms\": %.4f, "
           "\"GB/s\": %.1f}\n",
           2 * bytes, hc_grid, hc, 2.0 * bytes / (hc * 1e-3) / 1e9);
  }
  const float mm = time_ms([&] { hipLaunchKernelGGL(mfma_kernel, dim3(mfma_blocks), dim3(512), 0, 0, sink, 0.001f); },
                           500.0f, 10);
  const double flop = (double)mfma_blocks * 8 * kMfmaIter * 4 * 32768.0;
  printf("{\"measure\": \"mfma_bf16_32x32x16\", \"flop\": %.4e, \"ms\": %.4f, \"TFLOP/s\": %.1f}\n", flop, mm,
         flop / (mm * 1e-3) / 1e12);
  const float mr = time_ms(
      [&] { hipLaunchKernelGGL(mfma_rand_kernel, dim3(mfma_blocks), dim3(512), 0, 0, sink, 12345u); }, 500.0f, 10);
  printf("{\"measure\": \"mfma_bf16_32x32x16_random_operands\", \"flop\": %.4e, \"ms\": %.4f, \"TFLOP/s\": %.1f}\n",
         flop, mr, flop / (mr * 1e-3) / 1e12);
  {
    const long cold = 42729472L, c16 = cold / 16;
    const int grid = 16 * cus;
    hipEvent_t s0, s1;
    (void)hipEventCreate(&s0);
    (void)hipEventCreate(&s1);
    float t[21];
    for (int r = 0; r < 21; ++r) {
      (void)hipMemsetAsync(b, r & 0xff, 512L << 20);  // evict: 512 MiB written elsewhere
      (void)hipEventRecord(s0);
      hipLaunchKernelGGL((read_kernel<true, false>), dim3(grid), dim3(256), 0, 0, a, c16, flag);
      (void)hipEventRecord(s1);
      (void)hipEventSynchronize(s1);
      (void)hipEventElapsedTime(&t[r], s0, s1);
    }
    for (int i = 1; i < 21; ++i)
      for (int j = i; j > 0 && t[j] < t[j - 1]; --j) {
        const float x = t[j];
        t[j] = t[j - 1];
        t[j - 1] = x;
      }
    printf("{\"measure\": \"hbm_read_cold_small\", \"bytes\": %ld, \"grid\": %d, \"us_median\": %.2f, "
           "\"us_min\": %.2f, \"GB/s\": %.1f}\n",
           cold, grid, t[10] * 1e3, t[0] * 1e3, cold / (t[10] * 1e-3) / 1e9);
    (void)hipEventDestroy(s0);
    (void)hipEventDestroy(s1);
  }
  if (!ok(hipDeviceSynchronize(), "kernels")) return 1;
  (void)hipFree(a);
  (void)hipFree(b);
  (void)hipFree(flag);
  (void)hipFree(sink);
  return 0;
}
