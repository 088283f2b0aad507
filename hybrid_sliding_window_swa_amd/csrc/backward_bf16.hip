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
//   * bwd_fused_swa (sliding windows, D = 128, G in {4, 8}, q_offset a
//     multiple of 32 / G): dQ, dK, dV and the dsink partials in one pass per
//     query strip, see its section below; bwd_fuse_fixup adds the two
//     strips' partials of shared key tiles.  Other shapes use the split
//     kernels:
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
//   * bwd_dkdv: KV-parallel.  A wave owns 32 keys of one KV head and reads
//     their K and V rows as MFMA B operands from its LDS tile; the workgroup's
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

// ---------------------------------------------------------------- fused, sliding window
// dQ, dK, dV and the sink gradient of a sliding window in one pass over a
// strip of query blocks (the split kernels above read q and dO twice and
// compute S and dP twice).  One workgroup per (b, g, strip) of 8 waves:
//   * key waves 0..4: 32-key tile t belongs to wave t % 5 while it is live
//     (some query of the current block sees it); the wave keeps the tile's
//     dK^T and dV^T in its accumulators and, per block, computes S = Q K^T,
//     P, dP = dO V^T, dS, dV^T += dO^T P, dK^T += Q^T dS (the dK/dV kernel's
//     scheme) and leaves dS^T in LDS.  A window of W <= ~130 keys plus a
//     block of 32/G tokens meets at most five tiles, so every live tile has
//     its wave.  When a tile stops being live its dK, dV are written: in
//     bf16 when no other strip's queries see it, else as an fp32 partial
//     that bwd_fuse_fixup adds to the neighbouring strip's (fixed order).
//   * waves 5..7, one block behind: dQ^T = sum over the block's tiles of
//     K^T dS^T (D blocks 0 | 1 | 2, 3), with K^T and dS^T read transposed
//     from LDS; waves 5, 6 also stage the next block's q and dO rows into
//     LDS (direct-to-LDS loads) and form its D_i = <dO_i, O_i> and LSE from
//     global memory, wave 7 stages arriving K/V tiles.
// LDS: K tiles in six slots (the live tiles of the block computed, of the
// block whose dQ is formed, and the arriving one), V tiles likewise, q and
// dO double-buffered, dS^T per key wave double-buffered.  The 32 x 128 K,
// q and dO tiles are unpadded with XOR-swizzled 16-byte chunks (SwzTile),
// which keeps both their row reads and their transposed reads
// conflict-free within the 160 KiB.
constexpr int kFuseKeyWaves = 5;
constexpr int kFuseWaves = 8;
constexpr int kFuseSlots = 6;
constexpr int kFuseMinStrip = 512;         // tokens per strip at least
constexpr int kFuseMaxBoundaries = 256;    // strip boundaries per launch at most
constexpr int kFuseMaxBoundaryTiles = 5;   // tiles two strips share at most

// 32 rows x 128 bf16, rows of 256 bytes, 16-byte chunk c of row r stored at
// chunk c ^ swz(r), swz(r) = 4 (r % 4) + (r / 4) % 4.  A 16-byte operand read
// (16 consecutive rows, one chunk per clock group) meets 16 distinct chunks;
// a ds_read_b64_tr_b16 (4 consecutive rows x 64 bytes per 32 lanes) meets
// four distinct 64-byte bank groups.  Tile bases are 256-byte aligned, so a
// per-lane part can be XORed with compile-time chunk offsets.
struct SwzTile {
  static constexpr int BYTES = 32 * 256;
  static __device__ __forceinline__ int swz(int r) { return ((r & 3) << 2) | ((r >> 2) & 3); }
  // 16-byte operand read of chunk pair c (d in [16c + 8 half, +8)) by lane
  // (row lane % 32, half lane / 32): tile + (kop(lane) ^ 32 c)
  static __device__ __forceinline__ uint32_t kop(int lane) {
    const int r = lane & 31, h = lane >> 5;
    return (uint32_t)(r * 256 + 16 * (h ^ swz(r)));
  }
  // transposed read (PadTile::vt_operand's lane pattern) of rows
  // 16 kc + 8 hh + ..., output block db: tile + (tro(lane, hh) ^ 64 db) + 4096 kc
  static __device__ __forceinline__ uint32_t tro(int lane, int hh) {
    const int s = lane & 15, g4 = (lane >> 4) & 1, h = lane >> 5;
    const int row = 8 * hh + 4 * h + (s >> 2);
    const int unit = (2 * g4 + ((s & 3) >> 1)) ^ (2 * hh + h);
    return (uint32_t)(row * 256 + 64 * (s >> 2) + 16 * unit + 8 * (s & 1));
  }
  // global byte offset of the 16 bytes that DMA window i (rows 4i .. 4i+3)
  // delivers to lane `lane`, for rows row_off(r) bytes into the source
  static __device__ __forceinline__ int dma_chunk(int i, int lane) {
    return (lane & 15) ^ (((lane >> 4) << 2) | (i & 3));
  }
};

// dS^T tile per key wave: 32 keys x 32 queries bf16, rows of 64 bytes whose
// 8-byte units u sit at u ^ ((key / 4) % 8): the key waves' 8-byte row writes
// and the dQ waves' transposed reads are both conflict-free.
struct DsTile {
  static constexpr int BYTES = 32 * 64;
  // byte offset of the four queries 8 j + 4 half .. +3 of key row `key`
  static __device__ __forceinline__ uint32_t wr(int key, int half, int j) {
    return (uint32_t)(key * 64 + 8 * ((2 * j + half) ^ ((key >> 2) & 7)));
  }
  // transposed read of key rows 16 kc + 8 hh + ...: tile + ((tro(lane, hh) ^ 32 kc) + 1024 kc)
  static __device__ __forceinline__ uint32_t tro(int lane, int hh) {
    const int s = lane & 15, g4 = (lane >> 4) & 1, h = lane >> 5;
    const int row = 8 * hh + 4 * h + (s >> 2);
    return (uint32_t)(row * 64 + 8 * ((4 * g4 + (s & 3)) ^ (2 * hh + h)));
  }
};

__device__ __forceinline__ bf16x8 lds_rd16(uint32_t addr) { return *(const lds_bf16x8*)(uintptr_t)addr; }
__device__ __forceinline__ bf16x8 lds_tr16(uint32_t lo, uint32_t hi) {
  const i16x4 x = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(uintptr_t)lo);
  const i16x4 y = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(uintptr_t)hi);
  typedef short i16x8 __attribute__((ext_vector_type(8)));
  return __builtin_bit_cast(bf16x8, __builtin_shufflevector(x, y, 0, 1, 2, 3, 4, 5, 6, 7));
}

// Block n of the strip holds query tokens n*TQ .. n*TQ + TQ - 1 (q_offset is
// a multiple of TQ, so blocks are aligned in position).  Its live key tiles:
__device__ __forceinline__ int fuse_lo(const BwdArgs& a, int n, int TQ) {
  return max(0, a.q_offset + n * TQ - a.window + 1) / BKT;
}
__device__ __forceinline__ int fuse_hi(const BwdArgs& a, int n, int TQ) {
  return min(a.q_offset + n * TQ + TQ - 1, a.Sk - 1) / BKT;
}
// first key tile strip boundary j shares, and its position (the first query
// position of strip j + 1)
__device__ __forceinline__ int fuse_bpos(const BwdArgs& a, int j, int TQ) {
  const int nb = (a.Sq + TQ - 1) / TQ;
  return a.q_offset + (int)((long)(j + 1) * nb / a.fuse_spb) * TQ;
}

template <int G>
__global__ __launch_bounds__(kFuseWaves * 64) void bwd_fused_swa_kernel(BwdArgs a) {
  constexpr int D = 128;
  constexpr int TQ = BKT / G;
  constexpr int NKW = kFuseKeyWaves, NS = kFuseSlots;
  constexpr int VCH = D / 8 + 1;                   // V rows: pitch D + 8 (17 slots of 16 bytes)
  constexpr int NVI = (BKT * VCH + 63) / 64;       // direct-to-LDS loads per V tile
  constexpr uint32_t kOut = 0xFFFFFFF0u;           // an offset past any buffer range
  using VT = KTile<D>;
  __shared__ __attribute__((aligned(1024))) uint8_t k_lds[NS][SwzTile::BYTES];
  __shared__ __attribute__((aligned(1024))) uint8_t v_lds[NS][NVI * 1024];
  __shared__ __attribute__((aligned(1024))) uint8_t q_lds[2][SwzTile::BYTES];
  __shared__ __attribute__((aligned(1024))) uint8_t o_lds[2][SwzTile::BYTES];  // dO
  __shared__ __attribute__((aligned(1024))) uint8_t ds_lds[2][NKW][DsTile::BYTES];
  __shared__ float lse_lds[2][BKT];   // LSE * log2(e) per block row
  __shared__ float del_lds[2][BKT];   // D = <dO, O> per block row
  __shared__ float sink_red[BKT];

  const int tid = threadIdx.x, lane = tid & 63, wv = wave_index();
  const int half = lane >> 5, col = lane & 31;
  const int spb = a.fuse_spb;
  const int bg = blockIdx.x / spb, sidx = blockIdx.x - bg * spb;
  const int g = bg % a.Hkv, b = bg / a.Hkv;
  const int nb = (a.Sq + TQ - 1) / TQ;
  const int n0 = (int)((long)sidx * nb / spb), n1 = (int)((long)(sidx + 1) * nb / spb);
  const long q_tok = (long)a.Hq * D, kv_tok = (long)a.Hkv * D;
  const int W = a.window;
  const float c2 = a.scale_log2;

  // keys no query sees: zeros (the first strip below its first tile, the last
  // strip above its last one)
  {
    const int kz_lo = sidx == 0 ? 0 : a.Sk;
    const int kz_hi = sidx == 0 ? min(a.Sk, BKT * fuse_lo(a, 0, TQ)) : a.Sk;
    const int kz2 = sidx == spb - 1 ? min(a.Sk, BKT * (fuse_hi(a, nb - 1, TQ) + 1)) : a.Sk;
    const long kvb = (long)b * a.Sk * kv_tok + (long)g * D;
    for (int i = tid; i < (kz_hi - kz_lo) * (D / 8); i += kFuseWaves * 64) {
      const long off = kvb + (long)(kz_lo + i / (D / 8)) * kv_tok + (i % (D / 8)) * 8;
      *(u32x4*)(a.dk + off) = u32x4{};
      *(u32x4*)(a.dv + off) = u32x4{};
    }
    for (int i = tid; i < (a.Sk - kz2) * (D / 8); i += kFuseWaves * 64) {
      const long off = kvb + (long)(kz2 + i / (D / 8)) * kv_tok + (i % (D / 8)) * 8;
      *(u32x4*)(a.dk + off) = u32x4{};
      *(u32x4*)(a.dv + off) = u32x4{};
    }
  }
  if (n0 >= n1) return;

  // ---- staging (direct-to-LDS loads; the loop's s_waitcnt + barrier publish them)
  // q or dO rows of block n: row m is (token n*TQ + m / G, head g*G + m % G)
  auto dma_rows = [&](const uint16_t* src, uint32_t tile, int n) {
    const int t0 = n * TQ;
    const int ntok = min(TQ, a.Sq - t0);
    const uint16_t* first = src + ((long)b * a.Sq + t0) * q_tok + (long)g * G * D;
    const uint32_t bytes = (uint32_t)(((ntok - 1) * q_tok + (long)G * D) * 2);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int r = 4 * i + (lane >> 4);
      const uint32_t voff = (uint32_t)((((r / G) * q_tok + (long)(r % G) * D) * 2) + 16 * SwzTile::dma_chunk(i, lane));
      lds_dma16(first, bytes, tile + 1024u * i, voff);
    }
  };
  // K and V tile t (8 + NVI windows); this wave issues windows w0, w0 + step, ...
  auto dma_kv = [&](int t, int w0, int step) {
    const int kb = t * BKT;
    const int rows = min(BKT, a.Sk - kb);
    const long off = ((long)b * a.Sk + kb) * kv_tok + (long)g * D;
    const uint32_t bytes = (uint32_t)(((rows - 1) * kv_tok + D) * 2);
    for (int i = w0; i < 8 + NVI; i += step) {
      if (i < 8) {
        const int r = 4 * i + (lane >> 4);
        const uint32_t voff = (uint32_t)(r * kv_tok * 2) + 16u * SwzTile::dma_chunk(i, lane);
        lds_dma16(a.k + off, bytes, lds_addr(k_lds[t % NS]) + 1024u * i, voff);
      } else {
        const int P = 64 * (i - 8) + lane;
        const int r = P / VCH, ch = P - r * VCH;
        const uint32_t voff = (ch < D / 8 && r < BKT) ? (uint32_t)(r * kv_tok * 2) + 16u * ch : kOut;
        lds_dma16(a.v + off, bytes, lds_addr(v_lds[t % NS]) + 1024u * (i - 8), voff);
      }
    }
  };

  // ---- D = <dO, O> and LSE of block n (wave 7: two lanes per row, loaded
  // two blocks ahead of their use)
  const int drow = lane >> 1, dhr = lane & 1;
  const float sink_h = (a.sinks && wv == 7) ? a.sinks[g * G + drow % G] : 0.0f;
  float sterm = 0.0f;
  struct DRows {
    u32x4 o[8], d[8];
    float lse;
  };
  auto d_load = [&](DRows& r, int n) {
    const int t0 = n * TQ;
    const int ntok = min(TQ, a.Sq - t0);
    const long base = ((long)b * a.Sq + t0) * q_tok + (long)g * G * D;
    const uint32_t bytes = (uint32_t)(((ntok - 1) * q_tok + (long)G * D) * 2);
    const rsrc_t ro = make_rsrc(a.o + base, bytes), rd = make_rsrc(a.dout + base, bytes);
    const uint32_t off = (uint32_t)((((drow / G) * q_tok + (long)(drow % G) * D) + 64 * dhr) * 2);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      r.o[i] = buf_load16(ro, off + 16u * i, 0);
      r.d[i] = buf_load16(rd, off + 16u * i, 0);
    }
    const rsrc_t rl = make_rsrc(a.lse + ((long)b * a.Sq + t0) * a.Hq + g * G, (uint32_t)(((ntok - 1) * a.Hq + G) * 4));
    r.lse = __uint_as_float((uint32_t)__builtin_amdgcn_raw_buffer_load_b32(
        rl, (int)(((drow / G) * a.Hq + drow % G) * 4), 0, 0));
  };
  auto d_finish = [&](const DRows& r, int n) {
    float part = 0.0f;
#pragma unroll
    for (int i = 0; i < 8; ++i)
      part = dot_bf16x8(__builtin_bit_cast(bf16x8, r.d[i]), __builtin_bit_cast(bf16x8, r.o[i]), part);
    part += __shfl_xor(part, 1);
    if (dhr == 0) {
      lse_lds[n & 1][drow] = r.lse * kLog2e;
      del_lds[n & 1][drow] = part;
      if (a.sinks && n * TQ + drow / G < a.Sq) sterm += __expf(sink_h - r.lse) * part;
    }
  };
  // Block boundary: every wave's LDS writes (and the direct-to-LDS loads the
  // staging waves waited for) are visible after it; global loads and stores
  // may stay in flight across it.
  auto block_sync = [&]() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
  };

  // ---- key waves
  const uint32_t kop = SwzTile::kop(lane);
  const uint32_t tro0 = SwzTile::tro(lane, 0), tro1 = SwzTile::tro(lane, 1);
  const uint32_t vop = VT::k_lane_off(lane);
  f32x16 dk[4], dv[4];
#pragma unroll
  for (int db = 0; db < 4; ++db) {
    dk[db] = f32x16{};
    dv[db] = f32x16{};
  }
  auto key_block = [&](int n, int t) {
    const int buf = n & 1;
    const uint32_t qT = lds_addr(q_lds[buf]), oT = lds_addr(o_lds[buf]);
    const uint32_t qa = qT + kop, oa = oT + kop, ka = lds_addr(k_lds[t % NS]) + kop;
    const uint32_t va = lds_addr(v_lds[t % NS]) + vop;
    // S = Q K^T: lane (col = key), registers = query rows c_row(v, half);
    // operand reads run two chunks ahead of their MFMAs
    f32x16 s = {};
    {
      bf16x8 qr[3], kr[3];
#pragma unroll
      for (int c = 0; c < 2; ++c) {
        qr[c] = lds_rd16(qa ^ (32u * c));
        kr[c] = lds_rd16(ka ^ (32u * c));
      }
#pragma unroll
      for (int c = 0; c < 8; ++c) {
        if (c + 2 < 8) {
          qr[(c + 2) % 3] = lds_rd16(qa ^ (32u * (c + 2)));
          kr[(c + 2) % 3] = lds_rd16(ka ^ (32u * (c + 2)));
        }
        s = mfma32(qr[c % 3], kr[c % 3], s);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    // Masking: only the window (and keys past Sk, whose zero K rows would
    // otherwise get weight exp(-LSE)).  Query rows past Sq need none: their
    // q, dO rows, LSE and D read as zeros, so P = 1 there multiplies zero dO
    // rows and dS = P (0 - 0) = 0.
    const int pos0 = a.q_offset + n * TQ;
    const int kb = t * BKT, key = kb + col;
    const bool edge = !(kb + BKT - 1 <= pos0 && kb > pos0 + TQ - 1 - W) || kb + BKT > a.Sk;
    // the LSE and D of rows c_row(v, half): four runs of four rows, one
    // 16-byte read each
    typedef __attribute__((address_space(3))) f32x4 lds_f32x4;
    f32x4 l4[4], d4[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      l4[j] = ((const lds_f32x4*)lse_lds[buf])[2 * j + half];
      d4[j] = ((const lds_f32x4*)del_lds[buf])[2 * j + half];
    }
    float p[16];
#pragma unroll
    for (int v = 0; v < 16; ++v) p[v] = exp2_fast(fmaf(s[v], c2, -l4[v >> 2][v & 3]));
    if (edge) {
      // rows c_row(v, half) = 8 (v / 4) + 4 half + v % 4 belong to token
      // v / 4 (G = 8) or 2 (v / 4) + half (G = 4) of the block
      const bool kin = key < a.Sk;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int i = pos0 + (G == 8 ? j : 2 * j + half);
        const bool ok = kin && key <= i && key > i - W;
#pragma unroll
        for (int e = 0; e < 4; ++e) p[4 * j + e] = ok ? p[4 * j + e] : 0.0f;
      }
    }
    bf16x8 pb[2];
#pragma unroll
    for (int v = 0; v < 16; ++v) pb[v >> 3][v & 7] = (__bf16)p[v];
    // dP = dO V^T, and dV^T += dO^T P
    f32x16 dp = {};
#pragma unroll
    for (int c = 0; c < 8; ++c) dp = mfma32(lds_rd16(oa ^ (32u * c)), lds_rd16(va + 32u * c), dp);
    // (tile base + tro) ^ 64 db: the base is 256-byte aligned, so the XOR
    // only touches the per-lane part; 4096 kc becomes the read's immediate
    const uint32_t ot0 = oT + tro0, ot1 = oT + tro1;
#pragma unroll
    for (int kc = 0; kc < 2; ++kc)
#pragma unroll
      for (int db = 0; db < 4; ++db)
        dv[db] = mfma32(lds_tr16((ot0 ^ (64u * db)) + 4096u * kc, (ot1 ^ (64u * db)) + 4096u * kc), pb[kc], dv[db]);
    // dS = P (dP - D), and dS^T into this wave's LDS tile for dQ
    bf16x8 sb[2];
#pragma unroll
    for (int v = 0; v < 16; ++v) sb[v >> 3][v & 7] = (__bf16)(p[v] * (dp[v] - d4[v >> 2][v & 3]));
    const uint32_t dsT = lds_addr(ds_lds[buf][t % NKW]);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const u32x4 w4 = __builtin_bit_cast(u32x4, sb[j >> 1]);
      const u32x2 x2 = (j & 1) ? u32x2{w4[2], w4[3]} : u32x2{w4[0], w4[1]};
      *(__attribute__((address_space(3))) u32x2*)(uintptr_t)(dsT + DsTile::wr(col, half, j)) = x2;
    }
    // dK^T += Q^T dS
    const uint32_t qt0 = qT + tro0, qt1 = qT + tro1;
#pragma unroll
    for (int kc = 0; kc < 2; ++kc)
#pragma unroll
      for (int db = 0; db < 4; ++db)
        dk[db] = mfma32(lds_tr16((qt0 ^ (64u * db)) + 4096u * kc, (qt1 ^ (64u * db)) + 4096u * kc), sb[kc], dk[db]);
  };
  // tile t is done: bf16 dK, dV when only this strip sees it, else an fp32
  // partial for bwd_fuse_fixup (side 0: the earlier strip of the boundary)
  const int P0 = a.q_offset + n0 * TQ, P1 = a.q_offset + n1 * TQ;
  auto key_flush = [&](int t) {
    const int kb = t * BKT, key = kb + col;
    int side = -1, j = 0;
    if (sidx > 0 && kb <= P0 - 1) {
      side = 1;
      j = sidx - 1;
    } else if (sidx < spb - 1 && kb + BKT - 1 >= max(0, P1 - W + 1)) {
      side = 0;
      j = sidx;
    }
    if (side < 0) {
      if (key < a.Sk) {
        uint16_t* dkp = a.dk + ((long)b * a.Sk + key) * kv_tok + (long)g * D;
        uint16_t* dvp = a.dv + ((long)b * a.Sk + key) * kv_tok + (long)g * D;
#pragma unroll
        for (int db = 0; db < 4; ++db)
#pragma unroll
          for (int a4 = 0; a4 < 4; ++a4) {
            const f32x4 yk = {dk[db][4 * a4] * a.scale, dk[db][4 * a4 + 1] * a.scale, dk[db][4 * a4 + 2] * a.scale,
                              dk[db][4 * a4 + 3] * a.scale};
            const f32x4 yv = {dv[db][4 * a4], dv[db][4 * a4 + 1], dv[db][4 * a4 + 2], dv[db][4 * a4 + 3]};
            *(bf16x4*)(dkp + db * 32 + 8 * a4 + 4 * half) = __builtin_convertvector(yk, bf16x4);
            *(bf16x4*)(dvp + db * 32 + 8 * a4 + 4 * half) = __builtin_convertvector(yv, bf16x4);
          }
      }
    } else {
      const int tb0 = max(0, fuse_bpos(a, j, TQ) - W + 1) / BKT;
      float* pk = a.part + ((((long)bg * (spb - 1) + j) * a.fuse_nbt + (t - tb0)) * 2 + side) * (2 * BKT * D) +
                  col * D + 4 * half;
      float* pv = pk + BKT * D;
#pragma unroll
      for (int db = 0; db < 4; ++db)
#pragma unroll
        for (int a4 = 0; a4 < 4; ++a4) {
          *(f32x4*)(pk + db * 32 + 8 * a4) = f32x4{dk[db][4 * a4], dk[db][4 * a4 + 1], dk[db][4 * a4 + 2], dk[db][4 * a4 + 3]};
          *(f32x4*)(pv + db * 32 + 8 * a4) = f32x4{dv[db][4 * a4], dv[db][4 * a4 + 1], dv[db][4 * a4 + 2], dv[db][4 * a4 + 3]};
        }
    }
#pragma unroll
    for (int db = 0; db < 4; ++db) {
      dk[db] = f32x16{};
      dv[db] = f32x16{};
    }
  };

  // ---- dQ waves: dQ^T of block n (D blocks db0, db0 + 1 if two) from the
  // key waves' dS^T and the K tiles, then dq = scale * dQ
  const uint32_t dso0 = DsTile::tro(lane, 0), dso1 = DsTile::tro(lane, 1);
  // wave 5: D blocks 0, 1 (two = true); wave 6: 2; wave 7: 3.  `two` is
  // passed as a literal where it is known, so wave 7's code holds no second
  // accumulator next to its D rows.
  const int db0 = wv == 5 ? 0 : wv - 4;
  const uint32_t x0 = 64u * db0, x1 = 64u * (db0 + 1);
  f32x16 acc0 = {}, acc1 = {};
  // operands of one tile: dS^T (B) and K^T (A) for both 16-key chunks
  struct DqOps {
    bf16x8 bop[2], a0[2], a1[2];
  };
  auto dq_ops = [&](int t, int buf, bool two) {
    DqOps o;
    const uint32_t kT = lds_addr(k_lds[t % NS]);
    const uint32_t dT = lds_addr(ds_lds[buf][t % NKW]);
    const uint32_t k0 = kT + tro0, k1 = kT + tro1, d0 = dT + dso0, d1 = dT + dso1;
#pragma unroll
    for (int kc = 0; kc < 2; ++kc) {
      o.bop[kc] = lds_tr16((d0 ^ (32u * kc)) + 1024u * kc, (d1 ^ (32u * kc)) + 1024u * kc);
      o.a0[kc] = lds_tr16((k0 ^ x0) + 4096u * kc, (k1 ^ x0) + 4096u * kc);
      if (two) o.a1[kc] = lds_tr16((k0 ^ x1) + 4096u * kc, (k1 ^ x1) + 4096u * kc);
    }
    return o;
  };
  // dQ^T of block n into acc0 (acc1).  Straight-line over the at most five
  // live tiles, so every operand read can be issued ahead of the MFMAs: a
  // step past the block's last live tile reads that tile again with a zero
  // dS^T operand (its K and dS^T are finite, so it adds exact zeros).
  auto dq_compute = [&](int n, bool two) {
    const int buf = n & 1;
    const int tlo = fuse_lo(a, n, TQ), thi = fuse_hi(a, n, TQ);
    acc0 = f32x16{};
    acc1 = f32x16{};
    DqOps ops[NKW];
#pragma unroll
    for (int i = 0; i < NKW; ++i) {
      ops[i] = dq_ops(min(tlo + i, thi), buf, two);
      if (tlo + i > thi) {
        ops[i].bop[0] = bf16x8{};
        ops[i].bop[1] = bf16x8{};
      }
    }
#pragma unroll
    for (int i = 0; i < NKW; ++i)
#pragma unroll
      for (int kc = 0; kc < 2; ++kc) {
        acc0 = mfma32(ops[i].a0[kc], ops[i].bop[kc], acc0);
        if (two) acc1 = mfma32(ops[i].a1[kc], ops[i].bop[kc], acc1);
      }
  };
  // dq = scale * dQ^T of block n: lane (query col, half) holds d = 32 db +
  // 8 a4 + 4 half + 0..3; v_permlane32_swap gives lane half 0 the 8 values of
  // d = 32 db + 16 pr + 0..7 and lane half 1 those of 16 pr + 8..15, so every
  // lane stores 16 bytes per pair of a4
  auto dq_store = [&](int n, bool two) {
    const int tq = n * TQ + col / G;
    uint16_t* dqp = a.dq + ((long)b * a.Sq + tq) * q_tok + (long)(g * G + col % G) * D + 8 * half;
    auto store_db = [&](const f32x16& acc, int db) {
#pragma unroll
      for (int pr = 0; pr < 2; ++pr) {
        const f32x4 x = {acc[8 * pr] * a.scale, acc[8 * pr + 1] * a.scale, acc[8 * pr + 2] * a.scale,
                         acc[8 * pr + 3] * a.scale};
        const f32x4 y = {acc[8 * pr + 4] * a.scale, acc[8 * pr + 5] * a.scale, acc[8 * pr + 6] * a.scale,
                         acc[8 * pr + 7] * a.scale};
        const u32x2 xw = __builtin_bit_cast(u32x2, __builtin_convertvector(x, bf16x4));
        const u32x2 yw = __builtin_bit_cast(u32x2, __builtin_convertvector(y, bf16x4));
        const auto r0 = __builtin_amdgcn_permlane32_swap(xw[0], yw[0], false, false);
        const auto r1 = __builtin_amdgcn_permlane32_swap(xw[1], yw[1], false, false);
        if (tq < a.Sq) *(u32x4*)(dqp + 32 * db + 16 * pr) = u32x4{r0[0], r1[0], r0[1], r1[1]};
      }
    };
    store_db(acc0, db0);
    if (two) store_db(acc1, db0 + 1);
  };

  // ---- prologue: block n0's tiles, rows, D and LSE (and block n0 + 1's
  // rows for D in flight)
  for (int t = fuse_lo(a, n0, TQ); t <= fuse_hi(a, n0, TQ); ++t) dma_kv(t, wv, kFuseWaves);
  if (wv == 5) dma_rows(a.q, lds_addr(q_lds[n0 & 1]), n0);
  if (wv == 6) dma_rows(a.dout, lds_addr(o_lds[n0 & 1]), n0);
  __builtin_amdgcn_s_waitcnt(0);
  DRows dr0, dr1;
  if (wv == 7) {
    d_load(dr0, n0);
    d_finish(dr0, n0);
    if (n0 + 1 < n1) d_load(dr0, n0 + 1);
  }
  block_sync();

  // ---- main loops (the same number of barriers in every role): iteration n
  // computes block n's key tiles and block n - 1's dQ while block n + 1 is
  // staged; iteration n1 only finishes dQ
  if (wv < NKW) {
    for (int n = n0; n <= n1; ++n) {
      if (n < n1) {
        const int lo = fuse_lo(a, n, TQ), hi = fuse_hi(a, n, TQ);
        const int t = lo + (wv - lo % NKW + NKW) % NKW;
        if (t <= hi) {
          key_block(n, t);
          if (n + 1 == n1 || fuse_lo(a, n + 1, TQ) > t) key_flush(t);
        }
      }
      block_sync();
    }
  } else if (wv < 7) {
    // staging waves: q (wave 5) and dO (wave 6) rows of block n + 1, wave 6
    // also the arriving K/V tile, waited for before the barrier.  The dq of
    // block n - 2 is stored right after those loads are issued, so that the
    // wait does not also wait for stores issued just before it.
    for (int n = n0; n <= n1; ++n) {
      if (n + 1 < n1) {
        if (wv == 5) dma_rows(a.q, lds_addr(q_lds[(n + 1) & 1]), n + 1);
        if (wv == 6) {
          dma_rows(a.dout, lds_addr(o_lds[(n + 1) & 1]), n + 1);
          if (fuse_hi(a, n + 1, TQ) > fuse_hi(a, n, TQ)) dma_kv(fuse_hi(a, n + 1, TQ), 0, 1);
        }
      }
      if (n - 2 >= n0) dq_store(n - 2, wv == 5);
      if (n > n0) dq_compute(n - 1, wv == 5);
      __builtin_amdgcn_s_waitcnt(0);
      block_sync();
    }
    if (n1 - 1 >= n0) dq_store(n1 - 1, wv == 5);
  } else {
    // wave 7: D and LSE of block n + 1 from rows loaded an iteration earlier,
    // block n + 2's rows loaded meanwhile (two register sets, alternating)
    auto step = [&](int n, DRows& cur, DRows& nxt) {
      if (n + 2 < n1) d_load(nxt, n + 2);
      if (n > n0) {
        dq_compute(n - 1, false);
        dq_store(n - 1, false);
      }
      if (n + 1 < n1) d_finish(cur, n + 1);
      block_sync();
    };
    for (int n = n0; n <= n1; n += 2) {
      step(n, dr0, dr1);
      if (n + 1 <= n1) step(n + 1, dr1, dr0);
    }
  }

  // this strip's sink-gradient partial per head, fixed order
  if (a.sinks) {
    if (wv == 7 && dhr == 0) sink_red[drow] = sterm;
    __syncthreads();
    if (tid < G) {
      float sum = 0.0f;
      for (int m = tid; m < BKT; m += G) sum += sink_red[m];
      a.sink_part[((long)b * spb + sidx) * a.Hq + g * G + tid] = -sum;
    }
  }
}

// dK, dV of the key tiles two strips share: the two fp32 partials added in a
// fixed order (earlier strip first), scaled and rounded.  One workgroup per
// (b, g, boundary, tile).
__global__ __launch_bounds__(256) void bwd_fuse_fixup_kernel(BwdArgs a, int TQ) {
  constexpr int D = 128;
  const int nbt = a.fuse_nbt, nbd = a.fuse_spb - 1;
  int idx = blockIdx.x;
  const int i = idx % nbt;
  idx /= nbt;
  const int j = idx % nbd, bg = idx / nbd;
  const int g = bg % a.Hkv, b = bg / a.Hkv;
  const int Pj = fuse_bpos(a, j, TQ);
  const int tb0 = max(0, Pj - a.window + 1) / BKT, tb1 = (Pj - 1) / BKT;
  const int t = tb0 + i;
  if (t > tb1) return;
  const float* p0 = a.part + (((long)bg * nbd + j) * nbt + i) * 2 * (2 * BKT * D);
  const float* p1 = p0 + 2 * BKT * D;
  const long kv_tok = (long)a.Hkv * D;
  for (int e = threadIdx.x * 4; e < 2 * BKT * D; e += 256 * 4) {
    const int which = e / (BKT * D), r = (e / D) % BKT, d = e % D;
    const int key = t * BKT + r;
    if (key >= a.Sk) continue;
    const f32x4 x = *(const f32x4*)(p0 + e) + *(const f32x4*)(p1 + e);
    const f32x4 y = which == 0 ? x * a.scale : x;
    uint16_t* dst = (which == 0 ? a.dk : a.dv) + ((long)b * a.Sk + key) * kv_tok + (long)g * D + d;
    *(bf16x4*)dst = __builtin_convertvector(y, bf16x4);
  }
}

// Does the fused kernel apply, and with how many strips per (b, g)?
static bool fuse_plan(BwdArgs& a, int G, size_t part_bytes) {
  if (a.window <= 0 || a.D != 128 || (G != 4 && G != 8) || a.Sq <= 0) return false;
  const int TQ = BKT / G;
  if (a.q_offset % TQ != 0) return false;
  auto fl = [](int x) { return x >= 0 ? x / BKT : -((-x + BKT - 1) / BKT); };
  auto lo = [&](int p) { return fl(p - a.window + 1); };
  auto hi = [&](int p) { return fl(p + TQ - 1); };
  // block start positions repeat modulo 32: at most five live tiles per
  // block, six over three consecutive blocks (the K/V slots)
  for (int n = 1; n <= 2 * BKT / TQ + 1; ++n) {
    const int p = a.q_offset % BKT + n * TQ;
    if (hi(p) - lo(p) + 1 > kFuseKeyWaves) return false;
    if (hi(p + TQ) - lo(p - TQ) + 1 > kFuseSlots) return false;
  }
  const int nbt = max(1, (a.window - 2 + BKT - 1) / BKT + 1);
  if (nbt > kFuseMaxBoundaryTiles) return false;
  const int bgs = a.B * a.Hkv;
  const int min_len = max(kFuseMinStrip, a.window + 2 * BKT);
  int spb = min(kFuseMaxBoundaries / max(1, bgs), a.Sq / min_len);
  if (spb < 1) spb = 1;
  const size_t need = (size_t)bgs * (spb - 1) * nbt * 2 * 2 * BKT * 128 * 4;
  if (need > part_bytes) return false;
  a.fuse_spb = spb;
  a.fuse_nbt = nbt;
  return true;
}

template <int G>
hipError_t launch_bwd_fused(BwdArgs a, hipStream_t s) {
  const int TQ = BKT / G;
  const int spb = a.fuse_spb;
  a.n_sink_parts = a.B * spb;
  hipLaunchKernelGGL((bwd_fused_swa_kernel<G>), dim3(a.B * a.Hkv * spb), dim3(kFuseWaves * 64), 0, s, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (spb > 1) {
    hipLaunchKernelGGL(bwd_fuse_fixup_kernel, dim3(a.B * a.Hkv * (spb - 1) * a.fuse_nbt), dim3(256), 0, s, a, TQ);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (a.dsink) {
    if (a.sinks)
      hipLaunchKernelGGL(bwd_sink_reduce_kernel, dim3(a.Hq), dim3(256), 0, s, a);
    else
      hipLaunchKernelGGL(bwd_zero_kernel, dim3((a.Hq + 255) / 256), dim3(256), 0, s, a.dsink, a.Hq);
    e = hipGetLastError();
  }
  return e;
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
  if constexpr (G == 4 || G == 8) {
    if (a.part && fuse_plan(a, G, a.part_bytes)) return launch_bwd_fused<G>(a, s);
  }
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
  // sink partials: one per (request, dQ token block or strip) and head;
  // blocks hold at least 8 tokens (G <= 32)
  const long parts = (long)B * ((Sq + 7) / 8);
  const size_t delta_bytes = ((size_t)B * Sq * Hq * 4 + 255) / 256 * 256;
  p.delta_bytes = delta_bytes;
  p.part_offset = delta_bytes + ((size_t)parts * Hq * 4 + 255) / 256 * 256;
  // the fused kernel's shared-tile partials: at most kFuseMaxBoundaries strip
  // boundaries (only when a strip pair fits, Sq >= 2 * kFuseMinStrip), each
  // with kFuseMaxBoundaryTiles tiles x 2 sides x (dK, dV) x 32 keys x 128
  p.part_bytes = Sq >= 2 * kFuseMinStrip
                     ? (size_t)kFuseMaxBoundaries * kFuseMaxBoundaryTiles * 2 * 2 * BKT * 128 * 4
                     : 0;
  p.ws_bytes = p.part_offset + p.part_bytes;
  return p;
}

hipError_t launch_backward_bf16(BwdArgs a, const BwdPlan& p, hipStream_t s) {
  (void)p;
  return a.D == 128 ? launch_bwd_d<128>(a, s) : launch_bwd_d<64>(a, s);
}

}  // namespace swa
