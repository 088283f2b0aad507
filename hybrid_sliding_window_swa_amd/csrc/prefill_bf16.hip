// bf16 causal prefill with a sliding window (or global) and per-head sinks,
// on gfx950 MFMA.
//
// What it computes (MiMo-V2-Flash technical-report digest, section
// "MiMo-V2-Flash Model Architecture" and its "Hybrid Sliding Window Attention
// Architecture" paragraph; release blog, section on pushing efficiency):
// for each query at position i the keys max(0, i-W+1) .. i (all keys <= i
// when W <= 0), softmax over the scaled scores with exp(sink_h) added to the
// denominator, times the values.
//
// Work decomposition
//   * A workgroup owns TB consecutive tokens of one request and ALL G query
//     heads of one KV head g, so every K/V tile it stages in LDS serves G
//     heads (the GQA group) and TB tokens.  Each wave owns 32*NB query rows:
//     row m of a 32-row block is (token m / G, head m % G).
//   * Scores are computed transposed, S^T = K Q^T, with the 32x32x16 bf16
//     MFMA: lane l then holds 16 scores of ONE query (column l%32) and the
//     other 16 live in lane l^32, so the softmax row max needs one half swap
//     and the row sum none until the end.  The exponentiated scores P^T are
//     already laid out as the B operand of O^T += V^T P^T, so P never goes
//     through LDS.
//   * V^T is the A operand of that product; the staging step writes each V
//     tile into LDS transposed ([d][key]) once per workgroup.
//   * Key tiles are 32 keys.  Only tiles that intersect the workgroup's
//     window are loaded; each wave skips tiles outside its own window and
//     applies the causal / window mask only on boundary tiles.
//   * Online softmax in the log2 domain, fp32, started from the sink
//     (m = sink*log2e, l = 1), with a lazy rescale: the running max is only
//     raised when a score exceeds it by more than kRescaleTau.
//   * Workgroup -> work mapping is XCD-aware: workgroups dispatched to the
//     same XCD (blockIdx % 8) take consecutive token blocks of one (b, g), so
//     the K/V rows that neighbouring blocks share stay in that XCD's L2, and
//     the latest (longest, for global attention) blocks go first.
#include "common.hpp"
#include "launch.hpp"

namespace swa {

template <int D, int G, int NB, int NW>
__global__ __launch_bounds__(NW * 64) void prefill_bf16_kernel(PrefillArgs p) {
  constexpr int NT = NW * 64;
  constexpr int TW = 32 * NB / G;   // tokens per wave
  constexpr int TB = TW * NW;       // tokens per workgroup
  constexpr int NC = D / 16;        // 16-wide chunks of the QK^T contraction
  constexpr int ND = D / 32;        // 32-wide blocks of d in the output
  constexpr int KT = 32;            // keys per tile
  constexpr int KROW = D + 8;       // LDS pitch of a K row (bf16 elements)
  constexpr int VROW = KT + 4;      // LDS pitch of a V^T row (bf16 elements)
  constexpr int KCH = KT * D / 8;   // 16-byte chunks of a K tile
  constexpr int VU = (KT / 2) * (D / 8);  // (key pair, 8 d) units of a V tile
  constexpr int K_IT = (KCH + NT - 1) / NT;
  constexpr int V_IT = (VU + NT - 1) / NT;
  static_assert(32 * NB % G == 0, "a 32-row block must hold whole tokens");

  __shared__ __attribute__((aligned(16))) uint16_t k_lds[2][KT * KROW];
  __shared__ __attribute__((aligned(16))) uint16_t vt_lds[2][D * VROW];

  // ---- work item
  const int bid = blockIdx.x;
  const int w = (bid & 7) * p.per_xcd + (bid >> 3);
  if (w >= p.total) return;
  const int bg = w / p.n_tb;
  const int tb = p.n_tb - 1 - (w - bg * p.n_tb);
  const int g = bg % p.Hkv;
  const int b = bg / p.Hkv;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wv = tid >> 6;
  const int half = lane >> 5;
  const int col = lane & 31;
  const int t0 = tb * TB;
  const int tw0 = t0 + wv * TW;
  const long q_tok = (long)p.Hq * D;
  const long kv_tok = (long)p.Hkv * D;
  const uint16_t* __restrict__ kg = p.k + ((long)b * p.Sk * p.Hkv + g) * D;
  const uint16_t* __restrict__ vg = p.v + ((long)b * p.Sk * p.Hkv + g) * D;

  // ---- this lane's queries (one per 32-row block)
  bf16x8 qreg[NB][NC];
  int qpos[NB];
  float m_run[NB], l_run[NB];
  f32x16 acc[NB][ND];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
    const int tok = tw0 + nb * (32 / G) + col / G;
    const int h = g * G + col % G;
    qpos[nb] = p.q_offset + tok;
    if (tok < p.Sq) {
      const uint16_t* qp = p.q + ((long)b * p.Sq + tok) * q_tok + (long)h * D + half * 8;
#pragma unroll
      for (int c = 0; c < NC; ++c) qreg[nb][c] = *(const bf16x8*)(qp + c * 16);
    } else {
#pragma unroll
      for (int c = 0; c < NC; ++c) qreg[nb][c] = bf16x8{};
    }
    if (p.sinks) {
      m_run[nb] = p.sinks[h] * kLog2e;   // start from the sink: exp2(sink - m) = 1
      l_run[nb] = half == 0 ? 1.0f : 0.0f;
    } else {
      m_run[nb] = kNegInf;
      l_run[nb] = 0.0f;
    }
#pragma unroll
    for (int db = 0; db < ND; ++db) acc[nb][db] = f32x16{};
  }

  // ---- key range of the workgroup and of this wave
  const int tlast = min(t0 + TB, p.Sq) - 1;
  const int pos_lo = p.q_offset + t0, pos_hi = p.q_offset + tlast;
  const int key_lo = p.window > 0 ? max(0, pos_lo - p.window + 1) : 0;
  const int kt_begin = key_lo / KT, kt_end = pos_hi / KT;
  const bool wave_active = tw0 < p.Sq;
  const int wpos_lo = p.q_offset + tw0;
  const int wpos_hi = p.q_offset + min(tw0 + TW, p.Sq) - 1;
  const int wkey_lo = p.window > 0 ? max(0, wpos_lo - p.window + 1) : 0;

  // ---- tile staging: global -> registers -> LDS (V transposed)
  u32x4 kpre[K_IT];
  u32x4 vpre[V_IT][2];
  auto load_tile = [&](int kt) {
    const int kb = kt * KT;
#pragma unroll
    for (int i = 0; i < K_IT; ++i) {
      const int c = tid + i * NT;
      kpre[i] = u32x4{};
      if (c < KCH) {
        const int row = c / (D / 8), c8 = c % (D / 8);
        const int key = kb + row;
        if (key < p.Sk) kpre[i] = *(const u32x4*)(kg + (long)key * kv_tok + c8 * 8);
      }
    }
#pragma unroll
    for (int i = 0; i < V_IT; ++i) {
      const int u = tid + i * NT;
      vpre[i][0] = u32x4{};
      vpre[i][1] = u32x4{};
      if (u < VU) {
        const int pr = u % (KT / 2), c8 = u / (KT / 2);
        const int key = kb + 2 * pr;
        if (key < p.Sk) vpre[i][0] = *(const u32x4*)(vg + (long)key * kv_tok + c8 * 8);
        if (key + 1 < p.Sk) vpre[i][1] = *(const u32x4*)(vg + (long)(key + 1) * kv_tok + c8 * 8);
      }
    }
  };
  auto store_tile = [&](int buf) {
#pragma unroll
    for (int i = 0; i < K_IT; ++i) {
      const int c = tid + i * NT;
      if (c < KCH) {
        const int row = c / (D / 8), c8 = c % (D / 8);
        *(u32x4*)&k_lds[buf][row * KROW + c8 * 8] = kpre[i];
      }
    }
#pragma unroll
    for (int i = 0; i < V_IT; ++i) {
      const int u = tid + i * NT;
      if (u < VU) {
        const int pr = u % (KT / 2), c8 = u / (KT / 2);
        uint32_t* dst = (uint32_t*)&vt_lds[buf][(c8 * 8) * VROW + 2 * pr];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const uint32_t w0 = vpre[i][0][e >> 1], w1 = vpre[i][1][e >> 1];
          const uint32_t lo = (e & 1) ? (w0 >> 16) : (w0 & 0xffffu);
          const uint32_t hi = (e & 1) ? (w1 & 0xffff0000u) : (w1 << 16);
          dst[e * (VROW / 2)] = lo | hi;
        }
      }
    }
  };

  load_tile(kt_begin);
  store_tile(0);
  __syncthreads();

  for (int kt = kt_begin; kt <= kt_end; ++kt) {
    const int buf = (kt - kt_begin) & 1;
    const bool more = kt < kt_end;
    if (more) load_tile(kt + 1);
    const int kb = kt * KT;
    if (wave_active && kb + KT - 1 >= wkey_lo && kb <= wpos_hi) {
      const bool need_mask = (kb + KT - 1 > wpos_lo) ||
                             (p.window > 0 && kb < wpos_hi - p.window + 1);
      // S^T = K Q^T for each 32-query block
      f32x16 s[NB];
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) s[nb] = f32x16{};
#pragma unroll
      for (int c = 0; c < NC; ++c) {
        const bf16x8 a = *(const bf16x8*)&k_lds[buf][col * KROW + c * 16 + half * 8];
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) s[nb] = mfma32(a, qreg[nb][c], s[nb]);
      }
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) {
        float mx = kNegInf;
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          float x = s[nb][v] * p.scale_log2;
          if (need_mask) {
            const int kpos = kb + c_row(v, half);
            const bool ok = kpos <= qpos[nb] && (p.window <= 0 || kpos > qpos[nb] - p.window);
            x = ok ? x : kNegInf;
          }
          s[nb][v] = x;
          mx = fmaxf(mx, x);
        }
        mx = fmaxf(mx, swap_halves(mx));
        const float m_new = fmaxf(m_run[nb], mx);
        const bool need = m_new > m_run[nb] + kRescaleTau;
        if (wave_any(need)) {
          const float alpha = need ? exp2_fast(m_run[nb] - m_new) : 1.0f;
          m_run[nb] = need ? m_new : m_run[nb];
          l_run[nb] *= alpha;
#pragma unroll
          for (int db = 0; db < ND; ++db) acc[nb][db] *= alpha;
        }
        const float mu = m_run[nb] == kNegInf ? 0.0f : m_run[nb];
        bf16x8 pb[2];
        float ls = 0.0f;
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const float e = exp2_fast(s[nb][v] - mu);
          ls += e;
          pb[v >> 3][v & 7] = (__bf16)e;
        }
        l_run[nb] += ls;
        // O^T += V^T P^T: keys 16kc .. 16kc+15 per MFMA
#pragma unroll
        for (int kc = 0; kc < 2; ++kc) {
#pragma unroll
          for (int db = 0; db < ND; ++db) {
            const uint16_t* vp = &vt_lds[buf][(db * 32 + col) * VROW + 16 * kc + 4 * half];
            const u32x2 lo = *(const u32x2*)vp;
            const u32x2 hi = *(const u32x2*)(vp + 8);
            const u32x4 av = {lo[0], lo[1], hi[0], hi[1]};
            acc[nb][db] = mfma32(__builtin_bit_cast(bf16x8, av), pb[kc], acc[nb][db]);
          }
        }
      }
    }
    if (more) store_tile(buf ^ 1);
    __syncthreads();
  }

  // ---- epilogue: O = acc / l, bf16, one 8-byte store per 4 consecutive d
  if (!wave_active) return;
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
    const int tok = tw0 + nb * (32 / G) + col / G;
    const int h = g * G + col % G;
    const float lt = l_run[nb] + swap_halves(l_run[nb]);
    if (tok >= p.Sq) continue;
    const float inv = 1.0f / lt;
    uint16_t* op = p.o + ((long)b * p.Sq + tok) * q_tok + (long)h * D;
#pragma unroll
    for (int db = 0; db < ND; ++db) {
#pragma unroll
      for (int a4 = 0; a4 < 4; ++a4) {
        const f32x4 y = {acc[nb][db][4 * a4] * inv, acc[nb][db][4 * a4 + 1] * inv,
                         acc[nb][db][4 * a4 + 2] * inv, acc[nb][db][4 * a4 + 3] * inv};
        const bf16x4 yb = __builtin_convertvector(y, bf16x4);
        *(bf16x4*)(op + db * 32 + 8 * a4 + 4 * half) = yb;
      }
    }
  }
}

template <int D, int G, int NB, int NW>
static hipError_t launch_prefill_t(const PrefillArgs& a0, hipStream_t stream) {
  PrefillArgs a = a0;
  constexpr int TB = (32 * NB / G) * NW;
  a.n_tb = (a.Sq + TB - 1) / TB;
  a.total = a.B * a.Hkv * a.n_tb;
  a.per_xcd = (a.total + 7) / 8;
  dim3 grid(8 * a.per_xcd), block(NW * 64);
  hipLaunchKernelGGL((prefill_bf16_kernel<D, G, NB, NW>), grid, block, 0, stream, a);
  return hipGetLastError();
}

template <int D>
static hipError_t launch_prefill_d(const PrefillArgs& a, int G, hipStream_t s) {
  switch (G) {
    case 1: return launch_prefill_t<D, 1, 1, 8>(a, s);
    case 2: return launch_prefill_t<D, 2, 1, 8>(a, s);
    case 4: return launch_prefill_t<D, 4, 1, 8>(a, s);
    case 8: return launch_prefill_t<D, 8, 1, 8>(a, s);
    case 16: return launch_prefill_t<D, 16, 1, 8>(a, s);
    case 32: return launch_prefill_t<D, 32, 1, 8>(a, s);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_prefill_bf16(const PrefillArgs& a, hipStream_t s) {
  const int G = a.Hq / a.Hkv;
  return a.D == 128 ? launch_prefill_d<128>(a, G, s) : launch_prefill_d<64>(a, G, s);
}

}  // namespace swa
