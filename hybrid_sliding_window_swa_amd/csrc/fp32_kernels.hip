// fp32 prefill and verify: plain VALU kernels with no bf16 rounding anywhere.
//
// Same definition as the bf16 MFMA paths (window of W keys including the
// query's own position, or global; gpt-oss-style sink in the softmax
// denominator; MiMo-V2-Flash technical-report digest, section "MiMo-V2-Flash
// Model Architecture"), computed one query row per thread: the K/V rows a
// workgroup needs are staged through LDS 32 at a time and every thread of
// the workgroup (the G heads of one KV head times a run of tokens) reads
// them as broadcasts.  Single-pass online softmax in fp32 with expf, started
// from the sink (m = sink, l = 1).
#include "common.hpp"
#include "launch.hpp"

namespace swa {

namespace {

template <int D>
struct RowState {
  float q[D];
  float o[D];
  float m, l;

  __device__ __forceinline__ void init(const float* qp, const float* sinks, int h, float scale) {
#pragma unroll
    for (int d = 0; d < D; ++d) {
      q[d] = qp ? qp[d] * scale : 0.0f;
      o[d] = 0.0f;
    }
    if (sinks) {
      m = sinks[h];
      l = 1.0f;
    } else {
      m = kNegInf;
      l = 0.0f;
    }
  }

  // Fold in one key: s = <q*scale, k>.
  __device__ __forceinline__ void step(const float* kr, const float* vr) {
    float s = 0.0f;
#pragma unroll
    for (int d = 0; d < D; ++d) s = fmaf(q[d], kr[d], s);
    if (s > m) {
      const float a = expf(m - s);
      l *= a;
#pragma unroll
      for (int d = 0; d < D; ++d) o[d] *= a;
      m = s;
    }
    const float e = expf(s - m);
    l += e;
#pragma unroll
    for (int d = 0; d < D; ++d) o[d] = fmaf(e, vr[d], o[d]);
  }

  __device__ __forceinline__ void store(float* op) const {
    const float inv = 1.0f / l;
#pragma unroll
    for (int d = 0; d < D; ++d) op[d] = o[d] * inv;
  }
};

constexpr int KT32 = 32;

}  // namespace

// grid (token blocks, Hkv, B); block = tokens_per_block * G threads
template <int D>
__global__ __launch_bounds__(128) void prefill_f32_kernel(PrefillArgs p) {
  __shared__ float k_lds[KT32][D];
  __shared__ float v_lds[KT32][D];
  const float* q = (const float*)p.q;
  const float* k = (const float*)p.k;
  const float* v = (const float*)p.v;
  float* o = (float*)p.o;
  const int G = p.Hq / p.Hkv;
  const int tpb = blockDim.x / G;   // tokens per block
  const int tb = blockIdx.x, g = blockIdx.y, b = blockIdx.z;
  const int tid = threadIdx.x;
  const int tok = tb * tpb + tid / G, h = g * G + tid % G;
  const bool valid = tok < p.Sq;
  const long i = (long)p.q_offset + tok;

  RowState<D> st;
  st.init(valid ? q + (((long)b * p.Sq + tok) * p.Hq + h) * D : nullptr, p.sinks, h, p.scale);

  const int t_first = tb * tpb;
  const int t_last = min(t_first + tpb, p.Sq) - 1;
  const int lo = p.window > 0 ? max(0, p.q_offset + t_first - p.window + 1) : 0;
  const int hi = p.q_offset + t_last;
  const long kv_tok = (long)p.Hkv * D;
  const float* kg = k + ((long)b * p.Sk * p.Hkv + g) * D;
  const float* vg = v + ((long)b * p.Sk * p.Hkv + g) * D;
  const long jlo = p.window > 0 ? i - p.window + 1 : 0;

  for (int kb = lo; kb <= hi; kb += KT32) {
    const int n = min(KT32, hi - kb + 1);
    for (int e = tid; e < n * D; e += blockDim.x) {
      const int r = e / D, d = e % D;
      k_lds[r][d] = kg[(long)(kb + r) * kv_tok + d];
      v_lds[r][d] = vg[(long)(kb + r) * kv_tok + d];
    }
    __syncthreads();
    if (valid) {
      for (int r = 0; r < n; ++r) {
        const long j = kb + r;
        if (j <= i && j >= jlo) st.step(k_lds[r], v_lds[r]);
      }
    }
    __syncthreads();
  }
  if (valid) st.store(o + (((long)b * p.Sq + tok) * p.Hq + h) * D);
}

// grid (Hkv, B); block = G * T threads (one query row each)
template <int D>
__global__ __launch_bounds__(256) void verify_f32_kernel(VerifyArgs p) {
  __shared__ float k_lds[KT32][D];
  __shared__ float v_lds[KT32][D];
  const int g = blockIdx.x, b = blockIdx.y;
  const int G = p.Hq / p.Hkv;
  const int tid = threadIdx.x;
  const int t = tid / G, h = g * G + tid % G;
  const bool valid = t < p.T;
  const int L = p.cache_len[b];
  const long kv_tok = (long)p.Hkv * D;
  const float* q = (const float*)p.q;
  const float* kc = (const float*)p.k_cache + ((long)b * p.slots * p.Hkv + g) * D;
  const float* vc = (const float*)p.v_cache + ((long)b * p.slots * p.Hkv + g) * D;
  const float* kn = (const float*)p.k_new + ((long)b * p.T * p.Hkv + g) * D;
  const float* vn = (const float*)p.v_new + ((long)b * p.T * p.Hkv + g) * D;

  RowState<D> st;
  st.init(valid ? q + (((long)b * p.T + t) * p.Hq + h) * D : nullptr, p.sinks, h, p.scale);
  const long qpos = (long)L + t;
  const long jlo = p.window > 0 ? qpos - p.window + 1 : 0;

  // committed rows, as slot indices [c0, c0 + n)
  int c0, n;
  if (p.ring) {
    c0 = 0;
    n = min(L, p.slots);
  } else {
    c0 = p.window > 0 ? max(0, L - p.window + 1) : 0;
    n = L - c0;
  }
  const int ring_n = min(L, p.slots);
  const int base_slot = p.ring ? (L - ring_n) % p.slots : 0;
  for (int kb = 0; kb < n; kb += KT32) {
    const int cnt = min(KT32, n - kb);
    for (int e = tid; e < cnt * D; e += blockDim.x) {
      const int r = e / D, d = e % D;
      k_lds[r][d] = kc[(long)(c0 + kb + r) * kv_tok + d];
      v_lds[r][d] = vc[(long)(c0 + kb + r) * kv_tok + d];
    }
    __syncthreads();
    if (valid) {
      for (int r = 0; r < cnt; ++r) {
        const int ci = c0 + kb + r;
        long pos = ci;
        if (p.ring) {
          const int dd = ci - base_slot;
          pos = (long)L - ring_n + (dd >= 0 ? dd : dd + p.slots);
        }
        if (pos >= jlo) st.step(k_lds[r], v_lds[r]);
      }
    }
    __syncthreads();
  }
  // the new rows under verification: token t sees u <= t (inside its window)
  for (int e = tid; e < p.T * D; e += blockDim.x) {
    const int r = e / D, d = e % D;
    k_lds[r][d] = kn[(long)r * kv_tok + d];
    v_lds[r][d] = vn[(long)r * kv_tok + d];
  }
  __syncthreads();
  if (valid) {
    for (int u = 0; u <= t; ++u)
      if ((long)L + u >= jlo) st.step(k_lds[u], v_lds[u]);
    st.store((float*)p.o + (((long)b * p.T + t) * p.Hq + h) * D);
  }
}

hipError_t launch_prefill_f32(const PrefillArgs& a, hipStream_t s) {
  const int G = a.Hq / a.Hkv;
  const int tpb = G >= 128 ? 1 : 128 / G;
  dim3 grid((a.Sq + tpb - 1) / tpb, a.Hkv, a.B), block(tpb * G);
  if (a.D == 128)
    hipLaunchKernelGGL(prefill_f32_kernel<128>, grid, block, 0, s, a);
  else
    hipLaunchKernelGGL(prefill_f32_kernel<64>, grid, block, 0, s, a);
  return hipGetLastError();
}

hipError_t launch_verify_f32(const VerifyArgs& a, hipStream_t s) {
  const int G = a.Hq / a.Hkv;
  dim3 grid(a.Hkv, a.B), block(G * a.T);
  if (a.D == 128)
    hipLaunchKernelGGL(verify_f32_kernel<128>, grid, block, 0, s, a);
  else
    hipLaunchKernelGGL(verify_f32_kernel<64>, grid, block, 0, s, a);
  return hipGetLastError();
}

}  // namespace swa
