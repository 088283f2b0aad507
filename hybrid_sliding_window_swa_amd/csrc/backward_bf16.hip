// Backward of bf16 sliding-window / global attention with per-head sinks, on
// gfx950 MFMA.
//
// The gradients of L = sum(dO * O) for the forward of prefill_bf16.hip (the
// pages give no training kernel; the report digest's "Model Architecture"
// section motivates MTP for RL training, which needs them).  With the
// forward's log-sum-exp per row (LSE, sink included) saved:
//   P_ij  = exp(s_ij - LSE_i)          s_ij = scale <q_i, k_j>, j in window(i)
//   D_i   = <dO_i, O_i>
//   dS_ij = P_ij (<dO_i, v_j> - D_i)
//   dQ_i  = scale sum_j dS_ij k_j,  dK_j = scale sum_i dS_ij q_i,
//   dV_j  = sum_i P_ij dO_i,        dsink_h = -sum_i exp(sink_h - LSE_i) D_i
// (the sink adds exp(sink) to the denominator and carries no value).
//
// Kernels
//   * bwd_dq (first): besides dQ, D_i = <dO_i, O_i> for its rows (written for
//     bwd_dkdv) and, per workgroup and head, the partial sum of
//     exp(sink - LSE) D in a fixed order; bwd_sink_reduce adds the partials
//     in a fixed order, so dsink is deterministic.
//   * bwd_dkdv: KV-parallel.  A wave owns 32 keys of one KV head and keeps
//     their K and V rows as MFMA B operands in registers; the workgroup's four
//     waves walk the query blocks (32 rows = 32/G tokens x the G heads of the
//     KV head) that see any of their keys, staged through a double-buffered
//     LDS tile.  Scores are computed as S = Q K^T, so a lane holds one key's
//     column and 16 query rows: P and dS are then already the B operands of
//     dV^T += dO^T P and dK^T += Q^T dS, with dO^T and Q^T read transposed
//     from the row-major LDS tiles by ds_read_b64_tr_b16 (the forward's V^T
//     trick, with the query as the contraction index).
//   * bwd_dq: Q-parallel, the forward's structure, launched first.  A wave owns 32 query rows
//     with q and dO in registers; S^T = K Q^T and dP^T = V dO^T give a lane
//     one query's column, dS^T is the B operand of dQ^T += K^T dS^T with K^T
//     read transposed from the K tile.
// P and dS are rounded to bf16 for the MFMAs, as the forward rounds P; every
// accumulation is fp32; dQ, dK, dV are rounded to bf16 (nearest even).
#include "common.hpp"
#include "launch.hpp"

namespace swa {

namespace {

constexpr int BKT = 32;  // keys per tile / rows per query block
constexpr int kDqWaves = 8;      // waves (32-row query blocks) per dQ workgroup
constexpr int kDkdvPrefetch = 1;  // query blocks loaded ahead in the dK/dV kernel (deeper measured slower)

template <int D>
struct BwdGeom {
  static constexpr int NC = D / 16;   // 16-wide chunks of a D contraction
  static constexpr int ND = D / 32;   // 32-row blocks of d in a D x 32 result
  using Tile = VTile<D>;              // pitch D + 32: transposed reads conflict-free
  static constexpr int ELEMS = Tile::ELEMS;
  static constexpr int CH = BKT * D / 8;  // 16-byte chunks of a 32-row tile
};

// Row m of a query block starting at token t0: token t0 + m / G, head g*G + m % G.
__device__ __forceinline__ long qrow_off(int t0, int m, int G, int g, long q_tok, int D) {
  return (long)(t0 + m / G) * q_tok + (long)(g * G + m % G) * D;
}

// Is key j visible from the query at position i?
__device__ __forceinline__ bool visible(int i, int j, int window) {
  return j <= i && (window <= 0 || j > i - window);
}

__global__ __launch_bounds__(256) void bwd_zero_kernel(float* x, int n) {
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i < n) x[i] = 0.0f;
}

// ---------------------------------------------------------------- dsink
// dsink_h = sum of the per-workgroup partials the dQ kernel leaves (one per
// (request, token block) and head): one workgroup per head, each lane adding
// a fixed stride of partials, then a fixed-order tree in LDS (deterministic).
__global__ __launch_bounds__(256) void bwd_sink_reduce_kernel(BwdArgs a) {
  __shared__ float part[256];
  const int h = blockIdx.x, tid = threadIdx.x;
  float s = 0.0f;
  for (int i = tid; i < a.n_sink_parts; i += 256) s += a.sink_part[(long)i * a.Hq + h];
  part[tid] = s;
  __syncthreads();
  for (int w = 128; w >= 1; w >>= 1) {
    if (tid < w) part[tid] += part[tid + w];
    __syncthreads();
  }
  if (tid == 0) a.dsink[h] = part[0];
}

// ---------------------------------------------------------------- dK, dV
// Per-lane MFMA operand of a 32-row, row-major global tile: lane (col, half)
// gets row col, d in [16c + 8 half, +8); rows past `rows` read as zeros.
template <int D>
__device__ __forceinline__ void load_rows_operand(bf16x8 (&x)[D / 16], const uint16_t* base, long row_stride,
                                                  int rows, int col, int half) {
  const rsrc_t r = make_rsrc(base, rows > 0 ? (uint32_t)(((rows - 1) * row_stride + D) * 2) : 0u);
  const uint32_t voff = (uint32_t)((col * row_stride + half * 8) * 2);
#pragma unroll
  for (int c = 0; c < D / 16; ++c) x[c] = __builtin_bit_cast(bf16x8, buf_load16(r, voff + c * 32, 0));
}

template <int D, int G, int PF>
__global__ __launch_bounds__(256) void bwd_dkdv_kernel(BwdArgs a) {
  using Gm = BwdGeom<D>;
  using Tile = typename Gm::Tile;
  constexpr int NW = 4;
  constexpr int TQ = BKT / G;                  // tokens per query block
  __shared__ __attribute__((aligned(16))) uint16_t q_lds[2][Gm::ELEMS];
  __shared__ __attribute__((aligned(16))) uint16_t o_lds[2][Gm::ELEMS];  // dO
  __shared__ float lse_lds[2][BKT];
  __shared__ float del_lds[2][BKT];

  // work item: (b, g, block of NW key tiles).  Workgroups are dealt to the 8
  // XCDs in turn; each XCD takes a contiguous range of work items, i.e.
  // consecutive key blocks of one (b, g), whose query blocks overlap, so the
  // re-read Q / dO rows come from that XCD's L2.
  const int n_kb = (a.Sk + NW * BKT - 1) / (NW * BKT);
  const int total = n_kb * a.B * a.Hkv;
  const int per_xcd = (total + 7) / 8;
  const int w = (int)(blockIdx.x & 7) * per_xcd + (int)(blockIdx.x >> 3);
  if (w >= total) return;
  const int bg = w / n_kb;
  const int kblk = w - bg * n_kb;
  const int g = bg % a.Hkv, b = bg / a.Hkv;

  const int tid = threadIdx.x, lane = tid & 63, wv = wave_index();
  const int half = lane >> 5, col = lane & 31;
  const long q_tok = (long)a.Hq * D, kv_tok = (long)a.Hkv * D;
  const int W = a.window;
  const int kb0 = kblk * NW * BKT;            // first key of the workgroup
  const int kb = kb0 + wv * BKT;              // first key of this wave
  const int key = kb + col;                   // this lane's key column

  // this wave's K and V rows as B operands
  bf16x8 kop[Gm::NC], vop[Gm::NC];
  {
    const long kvbase = ((long)b * a.Sk + kb) * kv_tok + (long)g * D;
    const int rows = min(BKT, a.Sk - kb);
    load_rows_operand<D>(kop, a.k + kvbase, kv_tok, rows, col, half);
    load_rows_operand<D>(vop, a.v + kvbase, kv_tok, rows, col, half);
  }
  f32x16 dk[Gm::ND], dv[Gm::ND];
#pragma unroll
  for (int db = 0; db < Gm::ND; ++db) {
    dk[db] = f32x16{};
    dv[db] = f32x16{};
  }

  // query tokens that see any key of the workgroup: positions kb0 .. kb0 +
  // NW*32 - 1 + W - 1 (or the end), as query rows r = position - q_offset
  const int kend = min(a.Sk, kb0 + NW * BKT) - 1;
  const int r_lo = max(0, kb0 - a.q_offset);
  const int r_hi = W > 0 ? min(a.Sq - 1, kend + W - 1 - a.q_offset) : a.Sq - 1;
  const int qb_lo = r_lo / TQ;                      // query blocks of TQ tokens
  const int qb_hi = r_hi >= r_lo ? r_hi / TQ : qb_lo - 1;

  // staging: the block's 32 Q rows and dO rows (G*D contiguous per token),
  // one 16-byte chunk per thread and step, plus LSE*log2e and D per row.
  // Loads run PF blocks ahead of their use (PF register slots, block m in
  // slot m % PF) so that enough bytes are in flight to cover the memory
  // latency with one workgroup per CU; LDS holds two blocks (the one being
  // computed and the next, stored after the compute and before the barrier).
  constexpr int CPR = D / 8;                   // chunks per row
  constexpr int IT = Gm::CH / 256;
  u32x4 qpre[PF][IT], opre[PF][IT];
  float lpre[PF], dpre[PF];
  const long qbase_b = (long)b * a.Sq * q_tok;
  const long rbase_b = (long)b * a.Sq * a.Hq;
  auto load_block = [&](int qb, int slot) {
    const int t0 = qb * TQ;
#pragma unroll
    for (int i = 0; i < IT; ++i) {
      const int c = tid + i * 256;
      const int m = c / CPR, ch = c % CPR;
      const int tok = t0 + m / G;
      if (tok < a.Sq) {
        const long off = qbase_b + qrow_off(t0, m, G, g, q_tok, D) + ch * 8;
        qpre[slot][i] = *(const u32x4*)(a.q + off);
        opre[slot][i] = *(const u32x4*)(a.dout + off);
      } else {
        qpre[slot][i] = u32x4{0, 0, 0, 0};
        opre[slot][i] = u32x4{0, 0, 0, 0};
      }
    }
    if (tid < BKT) {
      const int tok = t0 + tid / G;
      const long row = rbase_b + (long)tok * a.Hq + g * G + tid % G;
      lpre[slot] = tok < a.Sq ? a.lse[row] * kLog2e : __builtin_inff();
      dpre[slot] = tok < a.Sq ? a.delta[row] : 0.0f;
    }
  };
  auto store_block = [&](int buf, int slot) {
#pragma unroll
    for (int i = 0; i < IT; ++i) {
      const int c = tid + i * 256;
      const int m = c / CPR, ch = c % CPR;
      *(u32x4*)&q_lds[buf][Tile::off(m, ch * 8)] = qpre[slot][i];
      *(u32x4*)&o_lds[buf][Tile::off(m, ch * 8)] = opre[slot][i];
    }
    if (tid < BKT) {
      lse_lds[buf][tid] = lpre[slot];
      del_lds[buf][tid] = dpre[slot];
    }
  };

  const float c2 = a.scale_log2;
  const uint32_t ko = Tile::k_lane_off(lane), vo = Tile::vt_lane_off(lane);
  auto compute_block = [&](int qb, int buf) {
    // does this wave's key tile meet the block's queries?
    const int t0 = qb * TQ;
    const int i_lo = a.q_offset + t0, i_hi = a.q_offset + min(t0 + TQ, a.Sq) - 1;
    const bool need = kb < a.Sk && kb <= i_hi && (W <= 0 || kb + BKT - 1 > i_lo - W);
    if (!need) return;
    const lds_u16* qa = lane_base(lds_addr(q_lds[buf]), ko);
    const lds_u16* oa = lane_base(lds_addr(o_lds[buf]), ko);
    // S = Q K^T and dP = dO V^T: lane (col = key), rows = queries c_row(v, half)
    f32x16 s = {}, dp = {};
#pragma unroll
    for (int c = 0; c < Gm::NC; ++c) {
      s = mfma32(Tile::k_operand(qa, c), kop[c], s);
      dp = mfma32(Tile::k_operand(oa, c), vop[c], dp);
    }
    // P, dS (masked entries exactly zero), rounded to bf16 B operands
    const bool edge = !(kb + BKT - 1 <= i_lo && (W <= 0 || kb > i_hi - W)) || i_hi < a.q_offset + t0 + TQ - 1;
    bf16x8 pb[2], sb[2];
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      const int m = c_row(v, half);
      float p = exp2_fast(fmaf(s[v], c2, -lse_lds[buf][m]));
      if (edge) {
        const int i = a.q_offset + t0 + m / G;
        if (!visible(i, key, W) || key >= a.Sk) p = 0.0f;
      }
      const float ds = p * (dp[v] - del_lds[buf][m]);
      pb[v >> 3][v & 7] = (__bf16)p;
      sb[v >> 3][v & 7] = (__bf16)ds;
    }
    const lds_u16* qt = lane_base(lds_addr(q_lds[buf]), vo);
    const lds_u16* ot = lane_base(lds_addr(o_lds[buf]), vo);
#pragma unroll
    for (int kc = 0; kc < 2; ++kc)
#pragma unroll
      for (int db = 0; db < Gm::ND; ++db) {
        dv[db] = mfma32(Tile::vt_operand(ot, db, kc), pb[kc], dv[db]);
        dk[db] = mfma32(Tile::vt_operand(qt, db, kc), sb[kc], dk[db]);
      }
  };

  const int nblk = qb_hi - qb_lo + 1;
  if (nblk > 0) {
    load_block(qb_lo, 0);
    store_block(0, 0);
#pragma unroll
    for (int u = 0; u < PF; ++u)
      if (1 + u < nblk) load_block(qb_lo + 1 + u, (1 + u) % PF);
  }
  __syncthreads();
  for (int n0 = 0; n0 < nblk; n0 += PF) {
#pragma unroll
    for (int u = 0; u < PF; ++u) {
      const int n = n0 + u;
      if (n < nblk) {
        compute_block(qb_lo + n, n & 1);
        // block n + 1 (slot (u + 1) % PF) into the other LDS buffer, then
        // the load of block n + 1 + PF into the slot it frees
        if (n + 1 < nblk) store_block((n + 1) & 1, (u + 1) % PF);
        if (n + 1 + PF < nblk) load_block(qb_lo + n + 1 + PF, (u + 1) % PF);
        __syncthreads();
      }
    }
  }

  // dK = scale * dK^T, dV = dV^T, transposed back: lane col is key kb + col,
  // register v of block db is d = 32 db + c_row(v, half)
  if (key < a.Sk && kb < a.Sk) {
    uint16_t* dkp = a.dk + ((long)b * a.Sk + key) * kv_tok + (long)g * D;
    uint16_t* dvp = a.dv + ((long)b * a.Sk + key) * kv_tok + (long)g * D;
#pragma unroll
    for (int db = 0; db < Gm::ND; ++db)
#pragma unroll
      for (int a4 = 0; a4 < 4; ++a4) {
        const f32x4 yk = {dk[db][4 * a4] * a.scale, dk[db][4 * a4 + 1] * a.scale, dk[db][4 * a4 + 2] * a.scale,
                          dk[db][4 * a4 + 3] * a.scale};
        const f32x4 yv = {dv[db][4 * a4], dv[db][4 * a4 + 1], dv[db][4 * a4 + 2], dv[db][4 * a4 + 3]};
        *(bf16x4*)(dkp + db * 32 + 8 * a4 + 4 * half) = __builtin_convertvector(yk, bf16x4);
        *(bf16x4*)(dvp + db * 32 + 8 * a4 + 4 * half) = __builtin_convertvector(yv, bf16x4);
      }
  }
}

// ---------------------------------------------------------------- dQ
template <int D, int G, int NW>
__global__ __launch_bounds__(NW * 64) void bwd_dq_kernel(BwdArgs a) {
  using Gm = BwdGeom<D>;
  using KT_ = typename Gm::Tile;     // K tile: row-major reads and transposed reads
  using VT_ = KTile<D>;              // V tile: row-major reads only
  constexpr int NT = NW * 64;
  constexpr int TQ = BKT / G;        // tokens per wave
  constexpr int TB = TQ * NW;        // tokens per workgroup
  __shared__ __attribute__((aligned(16))) uint16_t k_lds[2][KT_::ELEMS];
  __shared__ __attribute__((aligned(16))) uint16_t v_lds[2][VT_::ELEMS];

  // XCD-aware work item, as in the dK/dV kernel: consecutive token blocks of
  // one (b, g) on one XCD share their K / V tiles through its L2; latest
  // (longest, for global attention) blocks first
  const int n_tb = (a.Sq + TB - 1) / TB;
  const int total = n_tb * a.B * a.Hkv;
  const int per_xcd = (total + 7) / 8;
  const int w = (int)(blockIdx.x & 7) * per_xcd + (int)(blockIdx.x >> 3);
  if (w >= total) return;
  const int bg = w / n_tb;
  const int tb = n_tb - 1 - (w - bg * n_tb);
  const int g = bg % a.Hkv, b = bg / a.Hkv;

  const int tid = threadIdx.x, lane = tid & 63, wv = wave_index();
  const int half = lane >> 5, col = lane & 31;
  const long q_tok = (long)a.Hq * D, kv_tok = (long)a.Hkv * D;
  const int W = a.window;
  const int t0 = tb * TB, tw0 = t0 + wv * TQ;
  const int tok = tw0 + col / G, h = g * G + col % G;
  const int qpos = a.q_offset + tok;

  // q and dO of this lane's query row as B operands (d = 16c + 8 half + 0..7);
  // D = <dO, O> from the lane's half of the row and its partner's
  __shared__ float sink_term[NW][32];
  bf16x8 qop[Gm::NC], oop[Gm::NC];
  float lse2 = __builtin_inff(), del = 0.0f;
  {
    const long qoff = ((long)b * a.Sq + tok) * q_tok + (long)h * D + half * 8;
    float part = 0.0f;
#pragma unroll
    for (int c = 0; c < Gm::NC; ++c) {
      qop[c] = tok < a.Sq ? *(const bf16x8*)(a.q + qoff + c * 16) : bf16x8{};
      oop[c] = tok < a.Sq ? *(const bf16x8*)(a.dout + qoff + c * 16) : bf16x8{};
      const bf16x8 ov = tok < a.Sq ? *(const bf16x8*)(a.o + qoff + c * 16) : bf16x8{};
#pragma unroll
      for (int e = 0; e < 8; ++e) part = fmaf((float)oop[c][e], (float)ov[e], part);
    }
    del = halves_sum(part);
    float term = 0.0f;
    if (tok < a.Sq) {
      const long row = ((long)b * a.Sq + tok) * a.Hq + h;
      const float lse = a.lse[row];
      lse2 = lse * kLog2e;
      if (half == 0) a.delta[row] = del;
      if (a.sinks) term = __expf(a.sinks[h] - lse) * del;
    }
    if (half == 0) sink_term[wv][col] = term;
  }
  f32x16 dq[Gm::ND];
#pragma unroll
  for (int db = 0; db < Gm::ND; ++db) dq[db] = f32x16{};

  const int tlast = min(t0 + TB, a.Sq) - 1;
  const int pos_lo = a.q_offset + t0, pos_hi = a.q_offset + tlast;
  const int kt_begin = (W > 0 ? max(0, pos_lo - W + 1) : 0) / BKT, kt_end = pos_hi / BKT;
  const int wpos_lo = a.q_offset + tw0, wpos_hi = a.q_offset + min(tw0 + TQ, a.Sq) - 1;
  const bool wave_live = tw0 < a.Sq;

  constexpr int CPR = D / 8;
  constexpr int IT = (Gm::CH + NT - 1) / NT;
  u32x4 kpre[IT], vpre[IT];
  const long kvb = (long)b * a.Sk * kv_tok + (long)g * D;
  auto load_tile = [&](int kt) {
    const int kb = kt * BKT;
    const rsrc_t rk = make_rsrc(a.k + kvb + (long)kb * kv_tok, (uint32_t)(((min(BKT, a.Sk - kb) - 1) * kv_tok + D) * 2));
    const rsrc_t rv = make_rsrc(a.v + kvb + (long)kb * kv_tok, (uint32_t)(((min(BKT, a.Sk - kb) - 1) * kv_tok + D) * 2));
#pragma unroll
    for (int i = 0; i < IT; ++i) {
      const int c = tid + i * NT;
      if (c < Gm::CH) {
        const uint32_t off = (uint32_t)(((c / CPR) * kv_tok + (c % CPR) * 8) * 2);
        kpre[i] = buf_load16(rk, off, 0);
        vpre[i] = buf_load16(rv, off, 0);
      }
    }
  };
  auto store_tile = [&](int buf) {
#pragma unroll
    for (int i = 0; i < IT; ++i) {
      const int c = tid + i * NT;
      if (c < Gm::CH) {
        *(u32x4*)&k_lds[buf][KT_::off(c / CPR, (c % CPR) * 8)] = kpre[i];
        *(u32x4*)&v_lds[buf][VT_::off(c / CPR, (c % CPR) * 8)] = vpre[i];
      }
    }
  };

  load_tile(kt_begin);
  store_tile(0);
  __syncthreads();
  // this workgroup's share of dsink for the G heads of group g, fixed order
  if (a.sinks && tid < G) {
    float sum = 0.0f;
    for (int wq = 0; wq < NW; ++wq)
      for (int c = tid; c < 32; c += G) sum += sink_term[wq][c];
    a.sink_part[((long)b * n_tb + tb) * a.Hq + g * G + tid] = -sum;
  }
  const float c2 = a.scale_log2;
  for (int kt = kt_begin; kt <= kt_end; ++kt) {
    const int buf = (kt - kt_begin) & 1;
    if (kt < kt_end) load_tile(kt + 1);
    const int kb = kt * BKT;
    const bool need = wave_live && kb <= wpos_hi && (W <= 0 || kb + BKT - 1 > wpos_lo - W);
    if (need) {
      const lds_u16* ka = lane_base(lds_addr(k_lds[buf]), KT_::k_lane_off(lane));
      const lds_u16* va = lane_base(lds_addr(v_lds[buf]), VT_::k_lane_off(lane));
      f32x16 s = {}, dp = {};
#pragma unroll
      for (int c = 0; c < Gm::NC; ++c) s = mfma32(KT_::k_operand(ka, c), qop[c], s);
#pragma unroll
      for (int c = 0; c < Gm::NC; ++c) dp = mfma32(VT_::k_operand(va, c), oop[c], dp);
      // S^T, dP^T: lane = query column, register v = key kb + c_row(v, half)
      const bool edge = !(kb + BKT - 1 <= wpos_lo && (W <= 0 || kb > wpos_hi - W));
      bf16x8 sb[2];
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        float p = exp2_fast(fmaf(s[v], c2, -lse2));
        if (edge) {
          const int j = kb + c_row(v, half);
          if (!visible(qpos, j, W)) p = 0.0f;
        }
        sb[v >> 3][v & 7] = (__bf16)(p * (dp[v] - del));
      }
      const lds_u16* kt_op = lane_base(lds_addr(k_lds[buf]), KT_::vt_lane_off(lane));
#pragma unroll
      for (int kc = 0; kc < 2; ++kc)
#pragma unroll
        for (int db = 0; db < Gm::ND; ++db) dq[db] = mfma32(KT_::vt_operand(kt_op, db, kc), sb[kc], dq[db]);
    }
    if (kt < kt_end) store_tile(buf ^ 1);
    __syncthreads();
  }

  if (wave_live && tok < a.Sq) {
    uint16_t* dqp = a.dq + ((long)b * a.Sq + tok) * q_tok + (long)h * D;
#pragma unroll
    for (int db = 0; db < Gm::ND; ++db)
#pragma unroll
      for (int a4 = 0; a4 < 4; ++a4) {
        const f32x4 y = {dq[db][4 * a4] * a.scale, dq[db][4 * a4 + 1] * a.scale, dq[db][4 * a4 + 2] * a.scale,
                         dq[db][4 * a4 + 3] * a.scale};
        *(bf16x4*)(dqp + db * 32 + 8 * a4 + 4 * half) = __builtin_convertvector(y, bf16x4);
      }
  }
}

template <int D, int G>
hipError_t launch_bwd_dg(BwdArgs a, hipStream_t s) {
  // dQ first: it also leaves D = <dO, O> for dK/dV and the dsink partials
  const int TB = (BKT / G) * kDqWaves;
  const int n_tb = (a.Sq + TB - 1) / TB;
  a.n_sink_parts = a.B * n_tb;
  if (n_tb > 0) {
    const int total = n_tb * a.B * a.Hkv;
    hipLaunchKernelGGL((bwd_dq_kernel<D, G, kDqWaves>), dim3(8 * ((total + 7) / 8)), dim3(kDqWaves * 64), 0, s, a);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (a.dsink) {
    if (a.sinks && n_tb > 0) {
      hipLaunchKernelGGL(bwd_sink_reduce_kernel, dim3(a.Hq), dim3(256), 0, s, a);
    } else {
      hipLaunchKernelGGL(bwd_zero_kernel, dim3((a.Hq + 255) / 256), dim3(256), 0, s, a.dsink, a.Hq);
    }
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  const int n_kb = (a.Sk + 4 * BKT - 1) / (4 * BKT);
  if (n_kb > 0) {
    const int total = n_kb * a.B * a.Hkv;
    hipLaunchKernelGGL((bwd_dkdv_kernel<D, G, kDkdvPrefetch>), dim3(8 * ((total + 7) / 8)), dim3(256), 0, s, a);
    return hipGetLastError();
  }
  return hipSuccess;
}

template <int D>
hipError_t launch_bwd_d(const BwdArgs& a, hipStream_t s) {
  switch (a.Hq / a.Hkv) {
    case 1: return launch_bwd_dg<D, 1>(a, s);
    case 2: return launch_bwd_dg<D, 2>(a, s);
    case 4: return launch_bwd_dg<D, 4>(a, s);
    case 8: return launch_bwd_dg<D, 8>(a, s);
    case 16: return launch_bwd_dg<D, 16>(a, s);
    case 32: return launch_bwd_dg<D, 32>(a, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

BwdPlan plan_backward(int B, int Sq, int Hq) {
  BwdPlan p = {};
  // partials: one per (request, dQ token block) and head; blocks hold at
  // least 8 tokens (G <= 32)
  const long parts = (long)B * ((Sq + 7) / 8);
  const size_t delta_bytes = ((size_t)B * Sq * Hq * 4 + 255) / 256 * 256;
  p.delta_bytes = delta_bytes;
  p.ws_bytes = delta_bytes + (size_t)parts * Hq * 4;
  return p;
}

hipError_t launch_backward_bf16(BwdArgs a, const BwdPlan& p, hipStream_t s) {
  (void)p;
  return a.D == 128 ? launch_bwd_d<128>(a, s) : launch_bwd_d<64>(a, s);
}

}  // namespace swa
