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
// Shared structure of both kernels in this file
//   * A workgroup owns consecutive tokens of one request and ALL G query heads
//     of one KV head g, so every K/V tile it stages in LDS serves the whole
//     GQA group.  Each wave owns 32*NB query rows: row m of a 32-row block is
//     (token m / G, head m % G).
//   * Scores are computed transposed, S^T = K Q^T, with the 32x32x16 bf16
//     MFMA: lane l then holds 16 scores of ONE query (column l%32) and the
//     other 16 live in lane l^32, so the softmax row max needs one half swap
//     and the row sum none until the end.  The exponentiated scores P^T are
//     already laid out as the B operand of O^T += V^T P^T, so P never goes
//     through LDS.
//   * V^T is the A operand of that product; the staging step writes each V
//     tile into LDS transposed ([d][key]) once per workgroup.
//   * Key tiles are 32 keys.  Each wave skips tiles outside its own window and
//     applies the causal / window mask only on boundary tiles.
//   * Online softmax in the log2 domain, fp32, started from the sink
//     (m = sink*log2e, l = 1), with a lazy rescale: the running max is only
//     raised when a score exceeds it by more than kRescaleTau.
//
// prefill_swa_strip_kernel (sliding window, G in {4, 8}): persistent over a
//   strip of consecutive 32-token blocks of one (request, KV head).  The K/V
//   window lives in an LDS ring of 32-key tiles; each block adds one tile.
//   While a block is computed, the next block's queries and its new K/V tile
//   are already in flight, and the block's output is stored asynchronously,
//   so HBM streams continuously.
// prefill_bf16_kernel (global attention and any other shape): one workgroup
//   per token block, double-buffered K/V tiles, XCD-aware block order with
//   the longest (latest) blocks first.
#include "common.hpp"
#include "launch.hpp"

namespace swa {

namespace {

constexpr int KT = 32;  // keys per tile
constexpr int kMaskHi = 1, kMaskLo = 2;

template <int D>
struct TileGeom {
  static constexpr int NC = D / 16;             // 16-wide chunks of the QK^T contraction
  static constexpr int ND = D / 32;             // 32-wide blocks of d in the output
  static constexpr int K_ELEMS = KTile<D>::ELEMS;  // one K tile in LDS
  static constexpr int V_ELEMS = VTile<D>::ELEMS;  // one V tile in LDS (row-major)
  static constexpr int KCH = KT * D / 8;        // 16-byte chunks of a K (or V) tile
};

// Global -> register half of staging one 32-key tile of K and of V; rows at
// or past Sk are clamped to row Sk - 1 (finite data, always masked out).
template <int D, int NT>
struct Stager {
  using Gm = TileGeom<D>;
  static constexpr int IT = (Gm::KCH + NT - 1) / NT;
  u32x4 kpre[IT];
  u32x4 vpre[IT];

  __device__ __forceinline__ void load(const uint16_t* kg, const uint16_t* vg, long kv_tok, int kb,
                                       int Sk, int tid) {
#pragma unroll
    for (int i = 0; i < IT; ++i) {
      const int c = tid + i * NT;
      if (c < Gm::KCH) {
        const int row = c / (D / 8), c8 = c % (D / 8);
        const long off = (long)min(kb + row, Sk - 1) * kv_tok + c8 * 8;
        kpre[i] = *(const u32x4*)(kg + off);
        vpre[i] = *(const u32x4*)(vg + off);
      }
    }
  }

  // Register -> LDS half: both tiles row-major with padded pitches.
  __device__ __forceinline__ void store(uint16_t* k_dst, uint16_t* v_dst, int tid) const {
#pragma unroll
    for (int i = 0; i < IT; ++i) {
      const int c = tid + i * NT;
      if (c < Gm::KCH) {
        const int row = c / (D / 8), c8 = c % (D / 8);
        *(u32x4*)&k_dst[KTile<D>::off(row, c8 * 8)] = kpre[i];
        *(u32x4*)&v_dst[VTile<D>::off(row, c8 * 8)] = vpre[i];
      }
    }
  }
};

// Per-lane state of NB 32-query blocks.
template <int D, int NB>
struct QState {
  using Gm = TileGeom<D>;
  bf16x8 q[NB][Gm::NC];
  int qpos[NB];
  float m_run[NB], l_run[NB];
  f32x16 acc[NB][Gm::ND];

  // token of block nb for this lane, with G heads per token
  __device__ __forceinline__ void load_q(const uint16_t* qbase, long q_tok, int tw0, int G, int g,
                                         int Sq, int q_offset, int col, int half) {
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      const int tok = tw0 + nb * (32 / G) + col / G;
      const int h = g * G + col % G;
      qpos[nb] = q_offset + tok;
      if (tok < Sq) {
        const uint16_t* qp = qbase + (long)tok * q_tok + (long)h * D + half * 8;
#pragma unroll
        for (int c = 0; c < Gm::NC; ++c) q[nb][c] = *(const bf16x8*)(qp + c * 16);
      } else {
#pragma unroll
        for (int c = 0; c < Gm::NC; ++c) q[nb][c] = bf16x8{};
      }
    }
  }

  // Start every row from its head's sink: m = sink*log2e, l = 1 (counted once,
  // in the lower half of the wave).  sink2 = sink * log2(e), or -inf for none.
  // Every lane's rows share one head set (col % G), so one value serves all
  // blocks.
  __device__ __forceinline__ void reset(float sink2, int half) {
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      m_run[nb] = sink2;
      l_run[nb] = (sink2 != kNegInf && half == 0) ? 1.0f : 0.0f;
#pragma unroll
      for (int db = 0; db < Gm::ND; ++db) acc[nb][db] = f32x16{};
    }
  }

  // Fold one 32-key tile (K and V rows in LDS, first key position kb).
  // mask: kMaskHi if some key of the tile lies after some query of the wave,
  // kMaskLo if some key lies below some query's window.
  __device__ __forceinline__ void attend(const uint16_t* k_t, const uint16_t* v_t, int kb,
                                         int mask, int window, float c2, int lane) {
    const int col = lane & 31, half = lane >> 5;
    f32x16 s[NB];
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) s[nb] = f32x16{};
    const lds_u16* kbase = lane_base(lds_addr(k_t), KTile<D>::k_lane_off(lane));
#pragma unroll
    for (int c = 0; c < Gm::NC; ++c) {
      const bf16x8 a = KTile<D>::k_operand(kbase, c);
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) s[nb] = mfma32(a, q[nb][c], s[nb]);
    }
    if (mask) {
      // Causal / window mask of a boundary tile (masked scores -> -inf).  The
      // key of register v sits at kb + 4*half + cv with cv = 8*(v/4) + v%4, so
      // with a = qpos - kb - 4*half it is valid iff a - W + 1 <= cv <= a: one
      // compare per score when only one bound can bite.
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) {
        const int a = qpos[nb] - kb - 4 * half;
        const int alo = a - window + 1;
        if (mask == kMaskHi) {
#pragma unroll
          for (int v = 0; v < 16; ++v) s[nb][v] = (c_row(v, 0) <= a) ? s[nb][v] : kNegInf;
        } else if (mask == kMaskLo) {
#pragma unroll
          for (int v = 0; v < 16; ++v) s[nb][v] = (c_row(v, 0) >= alo) ? s[nb][v] : kNegInf;
        } else {
#pragma unroll
          for (int v = 0; v < 16; ++v)
            s[nb][v] = (c_row(v, 0) <= a && c_row(v, 0) >= alo) ? s[nb][v] : kNegInf;
        }
      }
    }
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      // raw-score max (scale > 0 commutes with max)
      float mx = kNegInf;
#pragma unroll
      for (int v = 0; v < 16; ++v) mx = fmaxf(mx, s[nb][v]);
      mx = fmaxf(mx, swap_halves(mx)) * c2;
      const float m_new = fmaxf(m_run[nb], mx);
      const bool need = m_new > m_run[nb] + kRescaleTau;
      if (wave_any(need)) {
        const float alpha = need ? exp2_fast(m_run[nb] - m_new) : 1.0f;
        m_run[nb] = need ? m_new : m_run[nb];
        l_run[nb] *= alpha;
#pragma unroll
        for (int db = 0; db < Gm::ND; ++db) acc[nb][db] *= alpha;
      }
      const float mu = m_run[nb] == kNegInf ? 0.0f : m_run[nb];
      bf16x8 pb[2];
#pragma unroll
      for (int v = 0; v < 16; ++v) pb[v >> 3][v & 7] = (__bf16)exp2_fast(fmaf(s[nb][v], c2, -mu));
      l_run[nb] = sum_bf16x16(pb[0], pb[1], l_run[nb]);
      // O^T += V^T P^T: keys 16kc .. 16kc+15 per MFMA
      const lds_u16* vbase = lane_base(lds_addr(v_t), VTile<D>::vt_lane_off(lane));
#pragma unroll
      for (int kc = 0; kc < 2; ++kc) {
#pragma unroll
        for (int db = 0; db < Gm::ND; ++db)
          acc[nb][db] = mfma32(VTile<D>::vt_operand(vbase, db, kc), pb[kc], acc[nb][db]);
      }
    }
  }

  // O = acc / l in bf16, one 8-byte store per 4 consecutive d.
  __device__ __forceinline__ void store_o(uint16_t* obase, long q_tok, int tw0, int G, int g, int Sq,
                                          int col, int half) {
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      const int tok = tw0 + nb * (32 / G) + col / G;
      const int h = g * G + col % G;
      const float lt = l_run[nb] + swap_halves(l_run[nb]);
      if (tok >= Sq) continue;
      const float inv = 1.0f / lt;
      uint16_t* op = obase + (long)tok * q_tok + (long)h * D;
#pragma unroll
      for (int db = 0; db < Gm::ND; ++db) {
#pragma unroll
        for (int a4 = 0; a4 < 4; ++a4) {
          const f32x4 y = {acc[nb][db][4 * a4] * inv, acc[nb][db][4 * a4 + 1] * inv,
                           acc[nb][db][4 * a4 + 2] * inv, acc[nb][db][4 * a4 + 3] * inv};
          *(bf16x4*)(op + db * 32 + 8 * a4 + 4 * half) = __builtin_convertvector(y, bf16x4);
        }
      }
    }
  }
};

// Does the wave whose queries sit at positions [wpos_lo, wpos_hi] need tile
// [kb, kb + 31], and which mask bounds can bite there?
__device__ __forceinline__ bool tile_needed(int kb, int wpos_lo, int wpos_hi, int window,
                                            int& mask) {
  const int wkey_lo = window > 0 ? max(0, wpos_lo - window + 1) : 0;
  mask = ((kb + KT - 1 > wpos_lo) ? kMaskHi : 0) |
         ((window > 0 && kb < wpos_hi - window + 1) ? kMaskLo : 0);
  return kb + KT - 1 >= wkey_lo && kb <= wpos_hi;
}

}  // namespace

// ----------------------------------------------------------------------------
// One workgroup per block of TB tokens (global attention and general shapes).
template <int D, int G, int NB, int NW>
__global__ __launch_bounds__(NW * 64) void prefill_bf16_kernel(PrefillArgs p) {
  using Gm = TileGeom<D>;
  constexpr int NT = NW * 64;
  constexpr int TW = 32 * NB / G;   // tokens per wave
  constexpr int TB = TW * NW;       // tokens per workgroup
  static_assert(32 * NB % G == 0, "a 32-row block must hold whole tokens");

  __shared__ __attribute__((aligned(16))) uint16_t k_lds[2][Gm::K_ELEMS];
  __shared__ __attribute__((aligned(16))) uint16_t v_lds[2][Gm::V_ELEMS];

  // XCD-aware work item: workgroups on one XCD (blockIdx % 8) take consecutive
  // token blocks of one (b, g), latest (longest) first.
  const int bid = blockIdx.x;
  const int w = (bid & 7) * p.per_xcd + (bid >> 3);
  if (w >= p.total) return;
  const int bg = w / p.n_tb;
  const int tb = p.n_tb - 1 - (w - bg * p.n_tb);
  const int g = bg % p.Hkv;
  const int b = bg / p.Hkv;

  const int tid = threadIdx.x, lane = tid & 63, wv = wave_index();
  const int half = lane >> 5, col = lane & 31;
  const int t0 = tb * TB;
  const int tw0 = t0 + wv * TW;
  const long q_tok = (long)p.Hq * D;
  const long kv_tok = (long)p.Hkv * D;
  const uint16_t* kg = p.k + ((long)b * p.Sk * p.Hkv + g) * D;
  const uint16_t* vg = p.v + ((long)b * p.Sk * p.Hkv + g) * D;
  const long qoff = (long)b * p.Sq * q_tok;

  QState<D, NB> st;
  st.load_q(p.q + qoff, q_tok, tw0, G, g, p.Sq, p.q_offset, col, half);
  st.reset(p.sinks ? p.sinks[g * G + col % G] * kLog2e : kNegInf, half);

  const int tlast = min(t0 + TB, p.Sq) - 1;
  const int pos_lo = p.q_offset + t0, pos_hi = p.q_offset + tlast;
  const int key_lo = p.window > 0 ? max(0, pos_lo - p.window + 1) : 0;
  const int kt_begin = key_lo / KT, kt_end = pos_hi / KT;
  const bool wave_active = tw0 < p.Sq;
  const int wpos_lo = p.q_offset + tw0;
  const int wpos_hi = p.q_offset + min(tw0 + TW, p.Sq) - 1;

  Stager<D, NT> sg;
  sg.load(kg, vg, kv_tok, kt_begin * KT, p.Sk, tid);
  sg.store(k_lds[0], v_lds[0], tid);
  // Drain the prologue loads (queries, first tile): inside the loop the only
  // loads in flight are then the next tile's, and no wait for the queries
  // can stall on them.
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();

  for (int kt = kt_begin; kt <= kt_end; ++kt) {
    const int buf = (kt - kt_begin) & 1;
    const bool more = kt < kt_end;
    if (more) sg.load(kg, vg, kv_tok, (kt + 1) * KT, p.Sk, tid);
    int mask;
    if (wave_active && tile_needed(kt * KT, wpos_lo, wpos_hi, p.window, mask))
      st.attend(k_lds[buf], v_lds[buf], kt * KT, mask, p.window, p.scale_log2, lane);
    if (more) sg.store(k_lds[buf ^ 1], v_lds[buf ^ 1], tid);
    __syncthreads();
  }
  if (wave_active) st.store_o(p.o + qoff, q_tok, tw0, G, g, p.Sq, col, half);
}

// ----------------------------------------------------------------------------
// Sliding window: persistent over a strip of 32-token blocks with an LDS ring.
// G waves per workgroup, each wave 32/G tokens x G heads (one 32-row block).
// A wave's 32 query rows are TW runs of G*D contiguous elements in q and o
// (the G heads of one token), so Q is loaded and O stored in whole rows,
// half a head_dim at a time, through a private 32 x D/2 LDS staging tile that
// converts between that layout and the MFMA register layout.
constexpr int kRingTiles = 7;

template <int D, int G>
__global__ __launch_bounds__(G * 64) void prefill_swa_strip_kernel(PrefillArgs p) {
  using Gm = TileGeom<D>;
  constexpr int NW = G;
  constexpr int NT = NW * 64;
  constexpr int TW = 32 / G;   // tokens per wave
  constexpr int TB = 32;       // tokens per block (= one key tile)
  constexpr int NR = kRingTiles;
  constexpr int HD = D / 2;    // staging width: half a head
  constexpr int HC = HD / 8;   // 16-byte chunks per staged row
  constexpr int SIT = 32 * HC / 64;  // 16-byte chunks per lane per staged half
  using Stg = PadTile<HD, HD + 8>;

  __shared__ __attribute__((aligned(16))) uint16_t k_ring[NR][Gm::K_ELEMS];
  __shared__ __attribute__((aligned(16))) uint16_t v_ring[NR][Gm::V_ELEMS];
  __shared__ __attribute__((aligned(16))) uint16_t stage_lds[NW][Stg::ELEMS];

  // strip -> (b, g, block range)
  const int strip = blockIdx.x;
  const int bg = strip / p.per_xcd;          // per_xcd holds strips per (b, g) here
  const int sidx = strip - bg * p.per_xcd;
  const int g = bg % p.Hkv, b = bg / p.Hkv;
  const int blk0 = (int)((long)sidx * p.n_tb / p.per_xcd);
  const int blk1 = (int)((long)(sidx + 1) * p.n_tb / p.per_xcd);
  if (blk0 >= blk1) return;

  const int tid = threadIdx.x, lane = tid & 63, wv = wave_index();
  const int half = lane >> 5, col = lane & 31;
  const long q_tok = (long)p.Hq * D;
  const long kv_tok = (long)p.Hkv * D;
  const uint16_t* kg = p.k + ((long)b * p.Sk * p.Hkv + g) * D;
  const uint16_t* vg = p.v + ((long)b * p.Sk * p.Hkv + g) * D;
  // element offset of query row m (token tw0 + m / G, head g*G + m % G) of this request
  const long qoff = (long)b * p.Sq * q_tok + (long)g * G * D;
  const int W = p.window;
  uint16_t* stg = stage_lds[wv];

  auto kt_lo = [&](int blk) { return max(0, p.q_offset + blk * TB - W + 1) / KT; };
  auto kt_hi = [&](int blk) { return (p.q_offset + min(blk * TB + TB, p.Sq) - 1) / KT; };
  auto row_off = [&](int tw0, int m) {  // rows past Sq read row Sq-1's token (never stored)
    return qoff + (long)min(tw0 + m / G, p.Sq - 1) * q_tok + (long)(m % G) * D;
  };

  // Q of a block in whole-row layout: chunk u = it*64 + lane of half hh is
  // row u / HC, 16-byte chunk u % HC of that half.
  u32x4 qpre[2][SIT];
  auto load_q_rows = [&](int tw0) {
#pragma unroll
    for (int hh = 0; hh < 2; ++hh)
#pragma unroll
      for (int it = 0; it < SIT; ++it) {
        const int u = it * 64 + lane;
        qpre[hh][it] = *(const u32x4*)(p.q + row_off(tw0, u / HC) + hh * HD + (u % HC) * 8);
      }
  };
  QState<D, 1> st;
  // whole rows -> LDS -> MFMA B-operand layout (row col, d = 16c + 8*half)
  auto stage_q = [&]() {
#pragma unroll
    for (int hh = 0; hh < 2; ++hh) {
#pragma unroll
      for (int it = 0; it < SIT; ++it) {
        const int u = it * 64 + lane;
        *(u32x4*)&stg[Stg::off(u / HC, (u % HC) * 8)] = qpre[hh][it];
      }
      wave_lds_sync();
      const lds_u16* sbase = lane_base(lds_addr(stg), Stg::k_lane_off(lane));
#pragma unroll
      for (int c = 0; c < Gm::NC / 2; ++c)
        st.q[0][hh * (Gm::NC / 2) + c] = Stg::k_operand(sbase, c);
      wave_lds_sync();
    }
  };
  // O = acc / l: MFMA layout -> LDS -> whole rows, half a head at a time
  auto store_o_rows = [&](int tw0) {
    const float lt = st.l_run[0] + swap_halves(st.l_run[0]);
    const float inv = 1.0f / lt;
#pragma unroll
    for (int hh = 0; hh < 2; ++hh) {
#pragma unroll
      for (int db2 = 0; db2 < Gm::ND / 2; ++db2) {
        const int db = hh * (Gm::ND / 2) + db2;
#pragma unroll
        for (int a4 = 0; a4 < 4; ++a4) {
          const f32x4 y = {st.acc[0][db][4 * a4] * inv, st.acc[0][db][4 * a4 + 1] * inv,
                           st.acc[0][db][4 * a4 + 2] * inv, st.acc[0][db][4 * a4 + 3] * inv};
          *(bf16x4*)&stg[Stg::off(col, 32 * db2 + 8 * a4 + 4 * half)] = __builtin_convertvector(y, bf16x4);
        }
      }
      wave_lds_sync();
#pragma unroll
      for (int it = 0; it < SIT; ++it) {
        const int u = it * 64 + lane;
        const int m = u / HC;
        if (tw0 + m / G < p.Sq)
          *(u32x4*)(p.o + qoff + (long)(tw0 + m / G) * q_tok + (long)(m % G) * D + hh * HD + (u % HC) * 8) =
              *(const u32x4*)&stg[Stg::off(m, (u % HC) * 8)];
      }
      wave_lds_sync();
    }
  };

  Stager<D, NT> sg;
  const float sink2 = p.sinks ? p.sinks[g * G + col % G] * kLog2e : kNegInf;

  // prologue: the first block's queries and its whole window
  load_q_rows(blk0 * TB + wv * TW);
  int loaded_hi = kt_hi(blk0);
  for (int kt = kt_lo(blk0); kt <= loaded_hi; ++kt) {
    sg.load(kg, vg, kv_tok, kt * KT, p.Sk, tid);
    sg.store(k_ring[kt % NR], v_ring[kt % NR], tid);
  }
  stage_q();
  // Drain every prologue load here, so that inside the loop the only loads in
  // flight are the prefetches and no wait inserted for the current queries
  // can stall on them.
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();

  for (int blk = blk0; blk < blk1; ++blk) {
    const int tw0 = blk * TB + wv * TW;
    const bool nxt = blk + 1 < blk1;
    // prefetch: next block's queries and (at most one) new K/V tile
    const int new_kt = nxt ? kt_hi(blk + 1) : -1;
    const bool have_new = new_kt > loaded_hi;
    if (nxt) load_q_rows(tw0 + TB);
    if (have_new) sg.load(kg, vg, kv_tok, new_kt * KT, p.Sk, tid);

    // compute this block from the ring
    st.qpos[0] = p.q_offset + tw0 + col / G;
    st.reset(sink2, half);
    const bool wave_active = tw0 < p.Sq;
    if (wave_active) {
      const int wpos_lo = p.q_offset + tw0;
      const int wpos_hi = p.q_offset + min(tw0 + TW, p.Sq) - 1;
      const int k1 = kt_hi(blk);
      for (int kt = kt_lo(blk); kt <= k1; ++kt) {
        int mask;
        if (tile_needed(kt * KT, wpos_lo, wpos_hi, W, mask))
          st.attend(k_ring[kt % NR], v_ring[kt % NR], kt * KT, mask, W, p.scale_log2, lane);
      }
      store_o_rows(tw0);
    }
    // the new tile's slot held tile new_kt - NR, older than this block's window
    if (have_new) {
      sg.store(k_ring[new_kt % NR], v_ring[new_kt % NR], tid);
      loaded_hi = new_kt;
    }
    if (nxt) stage_q();
    __syncthreads();
  }
}

// ----------------------------------------------------------------------------
template <int D, int G, int NB, int NW>
static hipError_t launch_generic(const PrefillArgs& a0, hipStream_t stream) {
  PrefillArgs a = a0;
  constexpr int TB = (32 * NB / G) * NW;
  a.n_tb = (a.Sq + TB - 1) / TB;
  a.total = a.B * a.Hkv * a.n_tb;
  a.per_xcd = (a.total + 7) / 8;
  dim3 grid(8 * a.per_xcd), block(NW * 64);
  hipLaunchKernelGGL((prefill_bf16_kernel<D, G, NB, NW>), grid, block, 0, stream, a);
  return hipGetLastError();
}

template <int D, int G>
static hipError_t launch_strip(const PrefillArgs& a0, int num_cu, hipStream_t stream) {
  PrefillArgs a = a0;
  a.n_tb = (a.Sq + 31) / 32;
  const int bgs = a.B * a.Hkv;
  int spb = num_cu / bgs;                 // strips per (b, g): about one workgroup per CU
  if (spb < 1) spb = 1;
  if (spb > a.n_tb) spb = a.n_tb;
  a.per_xcd = spb;
  a.total = bgs * spb;
  hipLaunchKernelGGL((prefill_swa_strip_kernel<D, G>), dim3(a.total), dim3(G * 64), 0, stream, a);
  return hipGetLastError();
}

template <int D>
static hipError_t launch_d(const PrefillArgs& a, int G, hipStream_t s) {
  // the strip kernel's ring must hold a block's window (at most
  // floor((W + 30) / 32) + 2 tiles) plus the next block's new tile
  const bool ring_fits = a.window > 0 && (a.window + 30) / KT + 2 + 1 <= kRingTiles;
  if (ring_fits && (G == 8 || G == 4)) {
    int dev = 0, num_cu = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&num_cu, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        num_cu <= 0)
      num_cu = 256;
    return G == 8 ? launch_strip<D, 8>(a, num_cu, s) : launch_strip<D, 4>(a, num_cu, s);
  }
  switch (G) {
    case 1: return launch_generic<D, 1, 1, 8>(a, s);
    case 2: return launch_generic<D, 2, 1, 8>(a, s);
    case 4: return launch_generic<D, 4, 1, 8>(a, s);
    case 8: return launch_generic<D, 8, 1, 8>(a, s);
    case 16: return launch_generic<D, 16, 1, 8>(a, s);
    case 32: return launch_generic<D, 32, 1, 8>(a, s);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_prefill_bf16(const PrefillArgs& a, hipStream_t s) {
  const int G = a.Hq / a.Hkv;
  return a.D == 128 ? launch_d<128>(a, G, s) : launch_d<64>(a, G, s);
}

}  // namespace swa
