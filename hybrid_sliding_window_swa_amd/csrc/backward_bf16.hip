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
//   * dQ, launched first.  Besides dQ it writes D_i = <dO_i, O_i> for its
//     rows (read by the dK/dV kernel) and, per workgroup or strip and head,
//     the partial sum of exp(sink - LSE) D in a fixed order;
//     bwd_sink_reduce adds the partials in a fixed order, so dsink is
//     deterministic.  Q-parallel: a wave owns 32 query rows (32/G tokens x
//     the G heads of a KV head) with q and dO as MFMA B operands;
//     S^T = K Q^T and dP^T = V dO^T give a lane one query's column, dS^T is
//     the B operand of dQ^T += K^T dS^T with K^T read transposed from the K
//     tile.  Sliding windows with G in {4, 8} use bwd_dq_strip (persistent
//     strips of 16-token blocks, the window's K/V tiles in an LDS ring, rows
//     loaded whole and turned into operands through LDS, the tile loop
//     software-pipelined); other shapes use bwd_dq (one workgroup per block,
//     the forward's structure).
//   * bwd_dkdv: KV-parallel.  A wave owns 32 keys of one KV head and keeps
//     their K and V rows as MFMA B operands in registers; the workgroup's
//     waves walk the query blocks that see any of their keys, staged through
//     a double-buffered LDS tile.  Scores are computed as S = Q K^T, so a
//     lane holds one key's column and 16 query rows: P and dS are then
//     already the B operands of dV^T += dO^T P and dK^T += Q^T dS, with dO^T
//     and Q^T read transposed from the row-major LDS tiles by
//     ds_read_b64_tr_b16 (the forward's V^T trick, with the query as the
//     contraction index).
// P and dS are rounded to bf16 for the MFMAs, as the forward rounds P; every
// accumulation is fp32; dQ, dK, dV are rounded to bf16 (nearest even).
#include "common.hpp"
#include "launch.hpp"

namespace swa {

namespace {

constexpr int BKT = 32;  // keys per tile / rows per query block
constexpr int kDqWaves = 8;      // waves (32-row query blocks) per dQ workgroup
// Cache policies: the strip dQ kernel reads each q, dO and O row once (the
// dK/dV kernel re-reads q and dO, so those stay cacheable there); dq, dk and
// dv are written once.
constexpr int kDqRowPolicy = kCacheDefault;
constexpr bool kBwdOutNT = false;
constexpr int kDkdvWaves = 2;    // 32-key tiles (waves) per dK/dV workgroup (measured: 2 beats 1 and 4)
constexpr int kDkdvPrefetch = 1;  // query blocks loaded ahead in the dK/dV kernel (deeper measured slower)

template <int D>
struct BwdGeom {
  static constexpr int NC = D / 16;   // 16-wide chunks of a D contraction
  static constexpr int ND = D / 32;   // 32-row blocks of d in a D x 32 result
  // Tiles read both ways (16-byte row reads as MFMA operands, and
  // ds_read_b64_tr_b16): pitch D + 24, an odd number of 16-byte slots, keeps
  // the row reads conflict-free (D + 32 puts rows 0, 4, 8, 12 on one bank
  // group) at two-way conflicts on some transposed reads; measured faster.
  using Tile = PadTile<D, D + 24>;
  static constexpr int ELEMS = Tile::ELEMS;
  static constexpr int CH = BKT * D / 8;  // 16-byte chunks of a 32-row tile
};

// Row m of a query block starting at token t0: token t0 + m / G, head g*G + m % G.
__device__ __forceinline__ long qrow_off(int t0, int m, int G, int g, long q_tok, int D) {
  return (long)(t0 + m / G) * q_tok + (long)(g * G + m % G) * D;
}

// <x, y> of bf16 vectors in fp32, two products per v_dot2_f32_bf16.
__device__ __forceinline__ float dot_bf16x8(const bf16x8& x, const bf16x8& y, float acc) {
#define SWA_DOT2_XY(e) \
  acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(x, x, e, e + 1), \
                                        __builtin_shufflevector(y, y, e, e + 1), acc, false)
  SWA_DOT2_XY(0);
  SWA_DOT2_XY(2);
  SWA_DOT2_XY(4);
  SWA_DOT2_XY(6);
#undef SWA_DOT2_XY
  return acc;
}
template <int NC>
__device__ __forceinline__ float dot_bf16(const bf16x8 (&x)[NC], const bf16x8 (&y)[NC]) {
  float acc = 0.0f;
#pragma unroll
  for (int c = 0; c < NC; ++c) acc = dot_bf16x8(x[c], y[c], acc);
  return acc;
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
template <int D, int G, int PF, int NW>
__global__ __launch_bounds__(NW * 64) void bwd_dkdv_kernel(BwdArgs a) {
  using Gm = BwdGeom<D>;
  using Tile = typename Gm::Tile;
  constexpr int NT = NW * 64;
  constexpr int TQ = BKT / G;                  // tokens per query block
  __shared__ __attribute__((aligned(16))) uint16_t q_lds[2][Gm::ELEMS];
  __shared__ __attribute__((aligned(16))) uint16_t o_lds[2][Gm::ELEMS];  // dO
  __shared__ float lse_lds[2][BKT];
  __shared__ float del_lds[2][BKT];
  // each wave's 32 K and V rows, read as MFMA B operands for every query
  // block (held in LDS rather than in 64 registers, which the allocator
  // otherwise shuttles through accumulation registers every block)
  __shared__ __attribute__((aligned(16))) uint16_t kv_lds[NW][2][KTile<D>::ELEMS];

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

  // this wave's K and V rows into its LDS tiles (whole rows; rows past Sk
  // read as zeros), read back as B operands in every query block
  {
    const long kvbase = ((long)b * a.Sk + kb) * kv_tok + (long)g * D;
    const int rows = kb < a.Sk ? min(BKT, a.Sk - kb) : 0;
    const uint32_t bytes = rows > 0 ? (uint32_t)(((rows - 1) * kv_tok + D) * 2) : 0u;
    const rsrc_t rk = make_rsrc(a.k + kvbase, bytes), rv = make_rsrc(a.v + kvbase, bytes);
    constexpr int CPR_ = D / 8, IT_ = BKT * CPR_ / 64;
#pragma unroll
    for (int i = 0; i < IT_; ++i) {
      const int c = lane + 64 * i;
      const uint32_t off = (uint32_t)(((c / CPR_) * kv_tok + (c % CPR_) * 8) * 2);
      const u32x4 kx = buf_load16(rk, off, 0), vx = buf_load16(rv, off, 0);
      *(u32x4*)&kv_lds[wv][0][KTile<D>::off(c / CPR_, (c % CPR_) * 8)] = kx;
      *(u32x4*)&kv_lds[wv][1][KTile<D>::off(c / CPR_, (c % CPR_) * 8)] = vx;
    }
  }
  const lds_u16* kop_base = lane_base(lds_addr(kv_lds[wv][0]), KTile<D>::k_lane_off(lane));
  const lds_u16* vop_base = lane_base(lds_addr(kv_lds[wv][1]), KTile<D>::k_lane_off(lane));
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
  constexpr int IT = Gm::CH / NT;
  u32x4 qpre[PF][IT], opre[PF][IT];
  float lpre[PF], dpre[PF];
  const long qbase_b = (long)b * a.Sq * q_tok;
  const long rbase_b = (long)b * a.Sq * a.Hq;
  // Plain buffer loads only (no branch, no arithmetic on the results until
  // the store to LDS), so the compiler leaves them in flight while a block is
  // computed; rows at or past Sq read as zeros (zero q and dO rows give zero
  // dS and zero dV contributions whatever their P).
  uint32_t ch_voff[IT];
#pragma unroll
  for (int i = 0; i < IT; ++i) {
    const int c = tid + i * NT;
    const int m = c / CPR, ch = c % CPR;
    ch_voff[i] = (uint32_t)((((m / G) * q_tok) + (long)(m % G) * D + ch * 8) * 2);
  }
  const uint32_t row_voff4 = (uint32_t)((((tid & (BKT - 1)) / G) * a.Hq + (tid & (BKT - 1)) % G) * 4);
  auto load_block = [&](int qb, int slot) {
    const int t0 = qb * TQ;
    const int ntok = min(TQ, a.Sq - t0);
    const long base = qbase_b + (long)t0 * q_tok + (long)g * G * D;
    const uint32_t bytes = (uint32_t)(((ntok - 1) * q_tok + (long)G * D) * 2);
    const rsrc_t rq = make_rsrc(a.q + base, bytes), ro = make_rsrc(a.dout + base, bytes);
#pragma unroll
    for (int i = 0; i < IT; ++i) {
      qpre[slot][i] = buf_load16(rq, ch_voff[i], 0);
      opre[slot][i] = buf_load16(ro, ch_voff[i], 0);
    }
    if (tid < BKT) {
      const long rb0 = rbase_b + (long)t0 * a.Hq + g * G;
      const uint32_t rbytes = (uint32_t)(((ntok - 1) * a.Hq + G) * 4);
      const rsrc_t rl = make_rsrc(a.lse + rb0, rbytes), rd = make_rsrc(a.delta + rb0, rbytes);
      lpre[slot] = __uint_as_float((uint32_t)__builtin_amdgcn_raw_buffer_load_b32(rl, (int)row_voff4, 0, 0));
      dpre[slot] = __uint_as_float((uint32_t)__builtin_amdgcn_raw_buffer_load_b32(rd, (int)row_voff4, 0, 0));
    }
  };
  auto store_block = [&](int buf, int slot) {
#pragma unroll
    for (int i = 0; i < IT; ++i) {
      const int c = tid + i * NT;
      const int m = c / CPR, ch = c % CPR;
      *(u32x4*)&q_lds[buf][Tile::off(m, ch * 8)] = qpre[slot][i];
      *(u32x4*)&o_lds[buf][Tile::off(m, ch * 8)] = opre[slot][i];
    }
    if (tid < BKT) {
      lse_lds[buf][tid] = lpre[slot] * kLog2e;
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
      s = mfma32(Tile::k_operand(qa, c), KTile<D>::k_operand(kop_base, c), s);
      dp = mfma32(Tile::k_operand(oa, c), KTile<D>::k_operand(vop_base, c), dp);
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
    // the transposed operands are read two MFMA pairs ahead of their use,
    // so each pair waits for reads issued long before, not for its own
    constexpr int NM = 2 * Gm::ND;
    bf16x8 otop[3], qtop[3];
#pragma unroll
    for (int i = 0; i < 2 && i < NM; ++i) {
      otop[i] = Tile::vt_operand(ot, i % Gm::ND, i / Gm::ND);
      qtop[i] = Tile::vt_operand(qt, i % Gm::ND, i / Gm::ND);
    }
#pragma unroll
    for (int i = 0; i < NM; ++i) {
      if (i + 2 < NM) {
        otop[(i + 2) % 3] = Tile::vt_operand(ot, (i + 2) % Gm::ND, (i + 2) / Gm::ND);
        qtop[(i + 2) % 3] = Tile::vt_operand(qt, (i + 2) % Gm::ND, (i + 2) / Gm::ND);
      }
      const int db = i % Gm::ND, kc = i / Gm::ND;
      dv[db] = mfma32(otop[i % 3], pb[kc], dv[db]);
      dk[db] = mfma32(qtop[i % 3], sb[kc], dk[db]);
      __builtin_amdgcn_sched_barrier(0);
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
  // Everything the prologue loaded (the K/V operands, the first blocks) is
  // drained here, so that inside the loop no wait the compiler derives for
  // those registers can land on a prefetch.
  __builtin_amdgcn_s_waitcnt(0);
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
        store_pol<kBwdOutNT>(__builtin_convertvector(yk, bf16x4), (bf16x4*)(dkp + db * 32 + 8 * a4 + 4 * half));
        store_pol<kBwdOutNT>(__builtin_convertvector(yv, bf16x4), (bf16x4*)(dvp + db * 32 + 8 * a4 + 4 * half));
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
      part = dot_bf16x8(oop[c], ov, part);
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

// ---------------------------------------------------------------- dQ, sliding window
// Persistent over a strip of consecutive TB-token blocks of one (b, g), like
// the forward's strip kernel: the K/V tiles of the window live in an LDS ring
// (each tile is loaded once per strip), and while a block is computed the next
// block's q, dO, O rows and LSE are already loading into a second register
// set (one wave per SIMD, so the register file holds both).  Per lane the
// sink-gradient terms of the whole strip are summed, then reduced in a fixed
// order into one partial per (strip, head).
constexpr int kDqRing = 7;

template <int D>
struct DqRows {
  bf16x8 q[D / 16], o[D / 16], ov[D / 16];  // q, dO, O in B-operand layout
  float lse;
};

template <int D, int G>
__global__ __launch_bounds__(256) void bwd_dq_strip_kernel(BwdArgs a) {
  using Gm = BwdGeom<D>;
  using KT_ = typename Gm::Tile;     // K tile: row-major reads and transposed reads
  using VT_ = KTile<D>;              // V tile: row-major reads only
  constexpr int NW = 4, NT = 256;
  constexpr int TQ = BKT / G;        // tokens per wave
  constexpr int TB = TQ * NW;        // tokens per block
  constexpr int NR = kDqRing;
  __shared__ __attribute__((aligned(16))) uint16_t k_ring[NR][KT_::ELEMS];
  __shared__ __attribute__((aligned(16))) uint16_t v_ring[NR][VT_::ELEMS];
  __shared__ float sink_red[NW][32];
  constexpr int HD = D / 2;           // staging width: half a head
  constexpr int HC = HD / 8;          // 16-byte chunks per staged row
  constexpr int SIT = 32 * HC / 64;   // chunks per lane per staged half
  constexpr int RPI = 64 / HC;        // rows per load instruction
  static_assert(RPI % G == 0, "a load instruction must cover whole tokens");
  static_assert(SIT == Gm::NC / 2, "one register per chunk in both layouts");
  constexpr int TPI = RPI / G;        // tokens per load instruction
  using Stg = PadTile<HD, HD + 8>;
  __shared__ __attribute__((aligned(16))) uint16_t stage_lds[NW][Stg::ELEMS];

  const int n_tb = (a.Sq + TB - 1) / TB;
  const int spb = a.strips_per_bg;
  const int strip = blockIdx.x;
  const int bg = strip / spb, sidx = strip - bg * spb;
  const int g = bg % a.Hkv, b = bg / a.Hkv;
  const int blk0 = (int)((long)sidx * n_tb / spb), blk1 = (int)((long)(sidx + 1) * n_tb / spb);

  const int tid = threadIdx.x, lane = tid & 63, wv = wave_index();
  const int half = lane >> 5, col = lane & 31;
  const long q_tok = (long)a.Hq * D, kv_tok = (long)a.Hkv * D;
  const int W = a.window;
  const int h = g * G + col % G;
  const float c2 = a.scale_log2;
  const float sink = a.sinks ? a.sinks[h] : 0.0f;

  auto kt_lo = [&](int blk) { return max(0, a.q_offset + blk * TB - W + 1) / BKT; };
  auto kt_hi = [&](int blk) { return (a.q_offset + min(blk * TB + TB, a.Sq) - 1) / BKT; };

  // A wave's q, dO and O rows of block blk (tokens blk*TB + wv*TQ ..., heads
  // g*G ...: TQ runs of G*D contiguous elements) are loaded as whole rows,
  // half a head at a time: load instruction it of half hh covers RPI rows
  // (TPI tokens), lane l taking row l / HC, 16-byte chunk l % HC, so every
  // instruction reads whole 128-byte lines.  The raw chunks sit in the
  // DqRows registers (chunk it of half hh in slot hh*SIT + it) until
  // to_operand() turns them, through a per-wave LDS tile, into the MFMA
  // B-operand layout (row col, d = 16c + 8*half).  Plain buffer loads only
  // (no branch, no arithmetic on the results), so the compiler can leave
  // them in flight across the block that is computed meanwhile; rows at or
  // past Sq read as zeros, which makes their dS zero.
  const uint32_t wrow_voff =
      (uint32_t)((((lane / HC) / G) * q_tok + ((lane / HC) % G) * D + (lane % HC) * 8) * 2);
  const uint32_t lse_voff = (uint32_t)(((wv * TQ + col / G) * a.Hq + h) * 4);
  auto load_rows = [&](DqRows<D>& r, int blk) {
    const int tw0 = blk * TB + wv * TQ;
    const int ntok = min(TQ, a.Sq - tw0);
    const long base = ((long)b * a.Sq + tw0) * q_tok + (long)g * G * D;
    const uint32_t bytes = ntok > 0 ? (uint32_t)(((ntok - 1) * q_tok + (long)G * D) * 2) : 0u;
    const rsrc_t rq = make_rsrc(a.q + base, bytes), ro = make_rsrc(a.dout + base, bytes);
    const rsrc_t rv = make_rsrc(a.o + base, bytes);
#pragma unroll
    for (int hh = 0; hh < 2; ++hh)
#pragma unroll
      for (int it = 0; it < SIT; ++it) {
        const uint32_t off = wrow_voff + (uint32_t)((it * TPI * q_tok + hh * HD) * 2);
        r.q[hh * SIT + it] = __builtin_bit_cast(bf16x8, buf_load16<kDqRowPolicy>(rq, off, 0));
        r.o[hh * SIT + it] = __builtin_bit_cast(bf16x8, buf_load16<kDqRowPolicy>(ro, off, 0));
        r.ov[hh * SIT + it] = __builtin_bit_cast(bf16x8, buf_load16<kDqRowPolicy>(rv, off, 0));
      }
    const int t0 = blk * TB;
    const int ntok_b = min(TB, a.Sq - t0);
    const rsrc_t rl = make_rsrc(a.lse + ((long)b * a.Sq + t0) * a.Hq, (uint32_t)(ntok_b * a.Hq * 4));
    r.lse = __uint_as_float((uint32_t)__builtin_amdgcn_raw_buffer_load_b32(rl, (int)lse_voff, 0, 0));
  };
  // whole-row chunks -> LDS -> B-operand layout, in place, half a head at a time
  auto to_operand = [&](bf16x8 (&x)[D / 16]) {
    uint16_t* stg = stage_lds[wv];
    const lds_u16* sbase = lane_base(lds_addr(stg), Stg::k_lane_off(lane));
#pragma unroll
    for (int hh = 0; hh < 2; ++hh) {
#pragma unroll
      for (int it = 0; it < SIT; ++it) {
        const int u = it * 64 + lane;
        *(u32x4*)&stg[Stg::off(u / HC, (u % HC) * 8)] = __builtin_bit_cast(u32x4, x[hh * SIT + it]);
      }
      wave_lds_sync();
#pragma unroll
      for (int c = 0; c < Gm::NC / 2; ++c) x[hh * (Gm::NC / 2) + c] = Stg::k_operand(sbase, c);
      wave_lds_sync();
    }
  };

  // K/V tile staging through registers (two 16-byte chunks per thread and
  // tensor for D = 128); rows at or past Sk read as zeros
  constexpr int CPR = D / 8;
  constexpr int IT = (Gm::CH + NT - 1) / NT;
  u32x4 kpre[IT], vpre[IT];
  const long kvb = (long)b * a.Sk * kv_tok + (long)g * D;
  auto load_tile = [&](int kt) {
    const int kb = kt * BKT;
    const uint32_t bytes = (uint32_t)(((min(BKT, a.Sk - kb) - 1) * kv_tok + D) * 2);
    const rsrc_t rk = make_rsrc(a.k + kvb + (long)kb * kv_tok, bytes);
    const rsrc_t rv = make_rsrc(a.v + kvb + (long)kb * kv_tok, bytes);
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
  auto store_tile = [&](int kt) {
    uint16_t* kd = k_ring[kt % NR];
    uint16_t* vd = v_ring[kt % NR];
#pragma unroll
    for (int i = 0; i < IT; ++i) {
      const int c = tid + i * NT;
      if (c < Gm::CH) {
        *(u32x4*)&kd[KT_::off(c / CPR, (c % CPR) * 8)] = kpre[i];
        *(u32x4*)&vd[VT_::off(c / CPR, (c % CPR) * 8)] = vpre[i];
      }
    }
  };

  float sterm = 0.0f;  // this lane's sink-gradient terms over the strip
  // Per-row scalars of a block's rows, computed when they are first needed,
  // at the end of the step that loaded them: D = <dO, O> (also written for
  // dK/dV), LSE * log2(e), and the row's sink-gradient term.
  auto prep = [&](DqRows<D>& r, int blk, float& del, float& lse2) {
    to_operand(r.q);
    to_operand(r.o);
    to_operand(r.ov);
    const int tok = blk * TB + wv * TQ + col / G;
    del = halves_sum(dot_bf16(r.o, r.ov));
    lse2 = r.lse * kLog2e;
    if (tok < a.Sq) {
      if (half == 0) a.delta[((long)b * a.Sq + tok) * a.Hq + h] = del;
      if (a.sinks) sterm += __expf(sink - r.lse) * del;
    }
  };
  // dQ of one block from the ring, with the rows in r.  Software pipelined:
  // the S^T and dP^T MFMAs of tile kt + 1 are issued between the dS^T
  // elements of tile kt (a pair of MFMAs, then that chunk's share of the
  // exponentials), so the matrix core and the vector ALU of the SIMD work at
  // the same time; then the dQ^T MFMAs of tile kt.
  auto block = [&](const DqRows<D>& r, int blk, float del, float lse2) {
    const int tw0 = blk * TB + wv * TQ;
    const int tok = tw0 + col / G;
    const int qpos = a.q_offset + tok;
    if (tw0 >= a.Sq) return;
    const int wpos_lo = a.q_offset + tw0, wpos_hi = a.q_offset + min(tw0 + TQ, a.Sq) - 1;
    const int wk0 = max(0, wpos_lo - W + 1) / BKT, wk1 = wpos_hi / BKT;
    constexpr int EPC = 16 / Gm::NC;  // dS elements per MFMA pair
    f32x16 dq[Gm::ND];
#pragma unroll
    for (int db = 0; db < Gm::ND; ++db) dq[db] = f32x16{};
    auto edge_of = [&](int kb) { return !(kb + BKT - 1 <= wpos_lo && kb > wpos_hi - W); };
    // dS of elements v, v + 1 of tile kb, packed to bf16
    auto ds_pair = [&](const f32x16& s, const f32x16& dp, int v, bool edge, int kb) {
      float p0 = exp2_fast(fmaf(s[v], c2, -lse2));
      float p1 = exp2_fast(fmaf(s[v + 1], c2, -lse2));
      if (edge) {
        if (!visible(qpos, kb + c_row(v, half), W)) p0 = 0.0f;
        if (!visible(qpos, kb + c_row(v + 1, half), W)) p1 = 0.0f;
      }
      const bf16x2 w2 = {(__bf16)(p0 * (dp[v] - del)), (__bf16)(p1 * (dp[v + 1] - del))};
      return __builtin_bit_cast(uint32_t, w2);
    };
    auto dq_acc = [&](int kt, const uint32_t (&pw)[8]) {
      bf16x8 sb[2];
      sb[0] = __builtin_bit_cast(bf16x8, u32x4{pw[0], pw[1], pw[2], pw[3]});
      sb[1] = __builtin_bit_cast(bf16x8, u32x4{pw[4], pw[5], pw[6], pw[7]});
      const lds_u16* kt_op = lane_base(lds_addr(k_ring[kt % NR]), KT_::vt_lane_off(lane));
#pragma unroll
      for (int kc = 0; kc < 2; ++kc)
#pragma unroll
        for (int db = 0; db < Gm::ND; ++db) dq[db] = mfma32(KT_::vt_operand(kt_op, db, kc), sb[kc], dq[db]);
    };
    f32x16 s = {}, dp = {};
    {
      const lds_u16* ka = lane_base(lds_addr(k_ring[wk0 % NR]), KT_::k_lane_off(lane));
      const lds_u16* va = lane_base(lds_addr(v_ring[wk0 % NR]), VT_::k_lane_off(lane));
      // operand reads run two chunks ahead of their MFMAs
      bf16x8 krd[3], vrd[3];
#pragma unroll
      for (int c = 0; c < 2 && c < Gm::NC; ++c) {
        krd[c] = KT_::k_operand(ka, c);
        vrd[c] = VT_::k_operand(va, c);
      }
#pragma unroll
      for (int c = 0; c < Gm::NC; ++c) {
        if (c + 2 < Gm::NC) {
          krd[(c + 2) % 3] = KT_::k_operand(ka, c + 2);
          vrd[(c + 2) % 3] = VT_::k_operand(va, c + 2);
        }
        s = mfma32(krd[c % 3], r.q[c], s);
        dp = mfma32(vrd[c % 3], r.o[c], dp);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    for (int kt = wk0; kt < wk1; ++kt) {
      const int kb = kt * BKT;
      const bool edge = edge_of(kb);
      const lds_u16* ka = lane_base(lds_addr(k_ring[(kt + 1) % NR]), KT_::k_lane_off(lane));
      const lds_u16* va = lane_base(lds_addr(v_ring[(kt + 1) % NR]), VT_::k_lane_off(lane));
      bf16x8 kop[Gm::NC], vop[Gm::NC];
#pragma unroll
      for (int c = 0; c < Gm::NC; ++c) {
        kop[c] = KT_::k_operand(ka, c);
        vop[c] = VT_::k_operand(va, c);
      }
      __builtin_amdgcn_sched_barrier(0);
      f32x16 sn = {}, dpn = {};
      uint32_t pw[8];
#pragma unroll
      for (int c = 0; c < Gm::NC; ++c) {
        sn = mfma32(kop[c], r.q[c], sn);
        dpn = mfma32(vop[c], r.o[c], dpn);
#pragma unroll
        for (int e = 0; e < EPC; e += 2) {
          uint32_t w = ds_pair(s, dp, c * EPC + e, edge, kb);
          __asm__ volatile("" : "+v"(w));
          pw[(c * EPC + e) >> 1] = w;
        }
        __builtin_amdgcn_sched_barrier(0);
      }
      dq_acc(kt, pw);
      s = sn;
      dp = dpn;
    }
    {
      const int kb = wk1 * BKT;
      const bool edge = edge_of(kb);
      uint32_t pw[8];
#pragma unroll
      for (int v = 0; v < 16; v += 2) pw[v >> 1] = ds_pair(s, dp, v, edge, kb);
      dq_acc(wk1, pw);
    }
    // dQ = scale * dQ^T: MFMA layout -> the wave's LDS tile -> whole rows,
    // half a head at a time (full 128-byte lines per store; rows past Sq
    // fall outside the buffer range and are dropped)
    const int ntok = min(TQ, a.Sq - tw0);
    const rsrc_t rd = make_rsrc(a.dq + ((long)b * a.Sq + tw0) * q_tok + (long)g * G * D,
                                (uint32_t)(((ntok - 1) * q_tok + (long)G * D) * 2));
    uint16_t* stg = stage_lds[wv];
#pragma unroll
    for (int hh = 0; hh < 2; ++hh) {
#pragma unroll
      for (int db2 = 0; db2 < Gm::ND / 2; ++db2) {
        const int db = hh * (Gm::ND / 2) + db2;
#pragma unroll
        for (int a4 = 0; a4 < 4; ++a4) {
          const f32x4 y = {dq[db][4 * a4] * a.scale, dq[db][4 * a4 + 1] * a.scale, dq[db][4 * a4 + 2] * a.scale,
                           dq[db][4 * a4 + 3] * a.scale};
          *(bf16x4*)&stg[Stg::off(col, 32 * db2 + 8 * a4 + 4 * half)] = __builtin_convertvector(y, bf16x4);
        }
      }
      wave_lds_sync();
#pragma unroll
      for (int it = 0; it < SIT; ++it) {
        const int u = it * 64 + lane;
        buf_store16(*(const u32x4*)&stg[Stg::off(u / HC, (u % HC) * 8)], rd,
                    wrow_voff + (uint32_t)((it * TPI * q_tok + hh * HD) * 2), 0);
      }
      wave_lds_sync();
    }
  };

  DqRows<D> ra, rb;
  float del_a = 0.0f, lse2_a = 0.0f, del_b = 0.0f, lse2_b = 0.0f;
  int loaded_hi = -1;
  if (blk0 < blk1) {
    loaded_hi = kt_hi(blk0);
    for (int kt = kt_lo(blk0); kt <= loaded_hi; ++kt) {
      load_tile(kt);
      store_tile(kt);
    }
    load_rows(ra, blk0);
    prep(ra, blk0, del_a, lse2_a);
  }
  __syncthreads();
  // one block with rows `cur` while `nxt` loads the next block's rows (their
  // per-row scalars are formed after the compute) and the next block's new
  // K/V tile, if any, is staged after the compute
  auto step = [&](const DqRows<D>& cur, float del_c, float lse2_c, DqRows<D>& nxt, float& del_n, float& lse2_n,
                  int blk) {
    const bool more = blk + 1 < blk1;
    const int new_kt = more ? kt_hi(blk + 1) : -1;
    const bool have_new = new_kt > loaded_hi;
    if (more) load_rows(nxt, blk + 1);
    if (have_new) load_tile(new_kt);
    block(cur, blk, del_c, lse2_c);
    if (have_new) {
      store_tile(new_kt);
      loaded_hi = new_kt;
    }
    if (more) prep(nxt, blk + 1, del_n, lse2_n);
    // Drain here, a block after the loads were issued: the next step then
    // starts with nothing in flight, so no wait the compiler derives for the
    // current rows can land on the prefetch issued at its top.
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
  };
  for (int blk = blk0; blk < blk1; blk += 2) {
    step(ra, del_a, lse2_a, rb, del_b, lse2_b, blk);
    if (blk + 1 < blk1) step(rb, del_b, lse2_b, ra, del_a, lse2_a, blk + 1);
  }

  // this strip's sink-gradient partial per head, fixed order
  if (a.sinks) {
    if (half == 0) sink_red[wv][col] = sterm;
    __syncthreads();
    if (tid < G) {
      float sum = 0.0f;
      for (int wq = 0; wq < NW; ++wq)
        for (int c = tid; c < 32; c += G) sum += sink_red[wq][c];
      a.sink_part[((long)b * spb + sidx) * a.Hq + g * G + tid] = -sum;
    }
  }
}

// Can the strip dQ kernel hold every block's window (plus the next block's
// new tile) in its ring?  Blocks start at positions q_offset + blk*TB.
static bool dq_strip_fits(const BwdArgs& a, int G) {
  if (a.window <= 0 || (G != 4 && G != 8)) return false;
  const int TB = (BKT / G) * 4;
  for (int blk = 0; blk < 2 * BKT / TB; ++blk) {
    const int p0 = a.q_offset + blk * TB;
    const int lo = max(0, p0 - a.window + 1) / BKT, hi = (p0 + TB - 1) / BKT;
    // the lowest tile a block can need is floor((p0 - W + 1) / 32) (or 0)
    const int lo_unclamped = (p0 - a.window + 1) >= 0 ? lo : -((-(p0 - a.window + 1) + BKT - 1) / BKT);
    if (hi - lo_unclamped + 1 + 1 > kDqRing) return false;
  }
  return true;
}

template <int D, int G>
hipError_t launch_bwd_dg(BwdArgs a, hipStream_t s) {
  // dQ first: it also leaves D = <dO, O> for dK/dV and the dsink partials
  int n_tb = 0;
  if constexpr (G == 4 || G == 8) {
    if (dq_strip_fits(a, G)) {
      const int TB = (BKT / G) * 4;
      n_tb = (a.Sq + TB - 1) / TB;
      int dev = 0, num_cu = 0;
      if (hipGetDevice(&dev) != hipSuccess ||
          hipDeviceGetAttribute(&num_cu, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || num_cu <= 0)
        num_cu = 256;
      const int bgs = a.B * a.Hkv;
      int spb = num_cu / bgs;
      if (spb < 1) spb = 1;
      if (spb > n_tb) spb = n_tb;
      a.strips_per_bg = spb;
      a.n_sink_parts = a.B * spb;
      if (n_tb > 0) {
        hipLaunchKernelGGL((bwd_dq_strip_kernel<D, G>), dim3(bgs * spb), dim3(256), 0, s, a);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
      }
    }
  }
  if (a.strips_per_bg == 0) {
    const int TB = (BKT / G) * kDqWaves;
    n_tb = (a.Sq + TB - 1) / TB;
    a.n_sink_parts = a.B * n_tb;
    if (n_tb > 0) {
      const int total = n_tb * a.B * a.Hkv;
      hipLaunchKernelGGL((bwd_dq_kernel<D, G, kDqWaves>), dim3(8 * ((total + 7) / 8)), dim3(kDqWaves * 64), 0, s, a);
      const hipError_t e = hipGetLastError();
      if (e != hipSuccess) return e;
    }
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
  const int n_kb = (a.Sk + kDkdvWaves * BKT - 1) / (kDkdvWaves * BKT);
  if (n_kb > 0) {
    const int total = n_kb * a.B * a.Hkv;
    hipLaunchKernelGGL((bwd_dkdv_kernel<D, G, kDkdvPrefetch, kDkdvWaves>), dim3(8 * ((total + 7) / 8)),
                       dim3(kDkdvWaves * 64), 0, s, a);
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
