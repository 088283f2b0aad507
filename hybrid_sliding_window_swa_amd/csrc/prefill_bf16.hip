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
//     GQA group.  Each wave owns 32 query rows: row m is (token m / G, head
//     m % G).
//   * Scores are computed transposed, S^T = K Q^T, with the 32x32x16 bf16
//     MFMA: lane l then holds 16 scores of ONE query (column l%32) and the
//     other 16 live in lane l^32, so the softmax row max needs one half swap
//     (v_permlane32_swap) and the row sum none until the end.  The
//     exponentiated scores P^T are already laid out as the B operand of
//     O^T += V^T P^T, so P never goes through LDS.
//   * V^T is the A operand of that product.  V tiles stay row-major in LDS;
//     ds_read_b64_tr_b16 transposes while reading.
//   * Key tiles are 32 keys.  Each wave visits only the tiles of its own
//     window and applies the causal / window mask on boundary tiles only.
//   * Online softmax in the log2 domain, fp32, started from the sink
//     (m = sink*log2e, l = 1), with a lazy rescale: the running max is only
//     raised when a score exceeds it by more than kRescaleTau.
//   * Software pipelining inside each wave: the score MFMAs of tile kt + 1
//     are issued between the exponentials of tile kt.
//
// prefill_swa_strip_kernel (sliding window, G in {4, 8}): persistent over a
//   strip of consecutive 32-token blocks of one (request, KV head).  The K/V
//   window lives in an LDS ring of 32-key tiles; each block adds one tile.
//   While a block is computed, the next block's queries and its new K/V tile
//   are already in flight, and the block's output is stored asynchronously,
//   so HBM streams continuously.
// prefill_bf16_kernel (global attention and any other shape): one workgroup
//   per token block, K/V tiles staged two at a time in a four-slot ring (K one
//   tile ahead of V, one barrier per two tiles), XCD-aware order with
//   the longest (latest) blocks first.
#include <type_traits>

#include "common.hpp"
#include "launch.hpp"

namespace swa {

namespace {

constexpr int KT = 32;  // keys per tile
// query rows and outputs of the one-workgroup-per-block kernel: streamed
// (every row touched once); its K/V tiles are re-read by later blocks
constexpr bool kGenericRowsNT = false;
constexpr int kMaskHi = 1, kMaskLo = 2, kMaskAll = 4;

template <int D>
struct TileGeom {
  static constexpr int NC = D / 16;             // 16-wide chunks of the QK^T contraction
  static constexpr int ND = D / 32;             // 32-wide blocks of d in the output
  static constexpr int K_ELEMS = KTile<D>::ELEMS;  // one K tile in LDS
  static constexpr int V_ELEMS = VTile<D>::ELEMS;  // one V tile in LDS (row-major)
  static constexpr int KCH = KT * D / 8;        // 16-byte chunks of a K (or V) tile
};

// Global -> register half of staging 32-key tiles of K and of V (possibly of
// different tiles), through raw buffer loads: the tile's first row is a
// scalar base, each thread's offset inside the tile is fixed, and rows at or
// past the given key end (the last key any query of the workgroup can see,
// plus one) read as zeros, whatever the caller's buffer holds there.
template <int D, int NT, int POL = kCacheDefault>
struct Stager {
  using Gm = TileGeom<D>;
  static constexpr int IT = (Gm::KCH + NT - 1) / NT;
  // every thread owns IT chunks (no lane predicate, no exec-mask branch)
  static constexpr bool kWhole = IT * NT == Gm::KCH;
  u32x4 kpre[IT];
  u32x4 vpre[IT];
  uint32_t voff[IT];  // byte offset of this thread's 16-byte chunks in a tile

  __device__ __forceinline__ void init(long kv_tok, int tid) {
#pragma unroll
    for (int i = 0; i < IT; ++i) {
      const int c = tid + i * NT;
      voff[i] = (uint32_t)(((c / (D / 8)) * kv_tok + (c % (D / 8)) * 8) * 2);
    }
  }
  static __device__ __forceinline__ rsrc_t tile(const uint16_t* g, long kv_tok, int kb, int Sk) {
    const int rows = min(KT, Sk - kb);
    return make_rsrc(g + (long)kb * kv_tok, (uint32_t)(((rows - 1) * kv_tok + D) * 2));
  }
  // The same range from a first-row pointer the caller advances itself:
  // rows * row_bytes - pad_bytes = ((rows - 1) * kv_tok + D) * 2 with
  // row_bytes = 2 kv_tok and pad_bytes = 2 (kv_tok - D), no 64-bit multiply.
  static __device__ __forceinline__ rsrc_t tile_at(const uint16_t* first_row, int kb, int Sk, uint32_t row_bytes,
                                                   uint32_t pad_bytes) {
    return make_rsrc(first_row, (uint32_t)min(KT, Sk - kb) * row_bytes - pad_bytes);
  }
  __device__ __forceinline__ void load_k(rsrc_t r, int tid) {
#pragma unroll
    for (int i = 0; i < IT; ++i)
      if (kWhole || tid + i * NT < Gm::KCH) kpre[i] = buf_load16<POL>(r, voff[i], 0);
  }
  __device__ __forceinline__ void load_v(rsrc_t r, int tid) {
#pragma unroll
    for (int i = 0; i < IT; ++i)
      if (kWhole || tid + i * NT < Gm::KCH) vpre[i] = buf_load16<POL>(r, voff[i], 0);
  }
  __device__ __forceinline__ void load_k(const uint16_t* kg, long kv_tok, int kb, int Sk, int tid) {
    load_k(tile(kg, kv_tok, kb, Sk), tid);
  }
  __device__ __forceinline__ void load_v(const uint16_t* vg, long kv_tok, int kb, int Sk, int tid) {
    load_v(tile(vg, kv_tok, kb, Sk), tid);
  }
  __device__ __forceinline__ void load(const uint16_t* kg, const uint16_t* vg, long kv_tok, int kb,
                                       int Sk, int tid) {
    load_k(kg, kv_tok, kb, Sk, tid);
    load_v(vg, kv_tok, kb, Sk, tid);
  }

  // Zero the loaded rows of the tile below tile-relative row r0: keys that no
  // query of the workgroup can see.  Such rows only get exact-zero weights,
  // but a zero weight times a non-finite value is still NaN inside P V, so
  // they must not carry whatever the caller's buffer holds there.
  __device__ __forceinline__ void zero_below(int r0, int tid) {
#pragma unroll
    for (int i = 0; i < IT; ++i) {
      if ((tid + i * NT) / (D / 8) < r0) {
        kpre[i] = u32x4{0u, 0u, 0u, 0u};
        vpre[i] = u32x4{0u, 0u, 0u, 0u};
      }
    }
  }

  // Register -> LDS half: row-major tiles with padded pitches.
  __device__ __forceinline__ void store_k(uint16_t* k_dst, int tid) const {
#pragma unroll
    for (int i = 0; i < IT; ++i) {
      const int c = tid + i * NT;
      if (kWhole || c < Gm::KCH) *(u32x4*)&k_dst[KTile<D>::off(c / (D / 8), (c % (D / 8)) * 8)] = kpre[i];
    }
  }
  __device__ __forceinline__ void store_v(uint16_t* v_dst, int tid) const {
#pragma unroll
    for (int i = 0; i < IT; ++i) {
      const int c = tid + i * NT;
      if (kWhole || c < Gm::KCH) *(u32x4*)&v_dst[VTile<D>::off(c / (D / 8), (c % (D / 8)) * 8)] = vpre[i];
    }
  }
  __device__ __forceinline__ void store(uint16_t* k_dst, uint16_t* v_dst, int tid) const {
    store_k(k_dst, tid);
    store_v(v_dst, tid);
  }
};

// Direct-to-LDS staging of a 32-key tile in the padded layouts of KTile and
// VTile (pitch D + 8 and D + 32): gfx950's buffer_load_dwordx4 ... lds writes
// the 16 bytes of lane l of a wave to LDS byte M0 + 16 l, so one load fills a
// 1 KiB window of 64 16-byte slots.  Window j of a tile covers slots 64 j ..
// 64 j + 63 (slot P = row * pitch16 + chunk); a slot in a row's padding, or
// past the tile's last row, gets an out-of-range offset and reads as zeros
// (no memory access).  NK / NV windows cover a K / V tile.
template <int D>
struct DmaTile {
  static constexpr int CPR = D / 8;                  // 16-byte chunks of a row
  static constexpr int KP = CPR + 1, VP = CPR + 4;   // pitches in 16-byte slots
  static constexpr int NK = (32 * KP + 63) / 64, NV = (32 * VP + 63) / 64;
  static constexpr int NPT = NK + NV;                // windows per K + V tile pair
  // an offset past any range, also with a few tiles' bytes added to it
  static constexpr uint32_t kOut = 0x80000000u;
  // byte offset in global memory of lane `lane`'s 16 bytes of window j of a
  // K (is_k) or V tile whose rows are row_bytes apart
  static __device__ __forceinline__ uint32_t voff(bool is_k, int j, int lane, uint32_t row_bytes) {
    const int pitch = is_k ? KP : VP;
    const int P = 64 * j + lane;
    const int row = P / pitch, ch = P - row * pitch;
    return (ch < CPR && row < 32) ? (uint32_t)row * row_bytes + (uint32_t)ch * 16u : kOut;
  }
  // One wave-wide load into the 1 KiB LDS window at byte address lds_byte
  // (lds_dma16).
  static __device__ __forceinline__ void load(const uint16_t* first_row, uint32_t num_records, uint32_t lds_byte,
                                              uint32_t voffset) {
    lds_dma16(first_row, num_records, lds_byte, voffset);
  }
};

struct NoExtra {
  __device__ __forceinline__ void operator()(int) const {}
};

// Per-lane state of one 32-query block; row m of the block is (token m / G,
// head m % G), and lane l holds query column l % 32.  RSUM: the row sums add
// the rounded weights (pack_sum<true>), else the weights before rounding.
template <int D, bool RSUM = false>
struct QState {
  using Gm = TileGeom<D>;
  bf16x8 q[Gm::NC];
  int qpos;
  float m_run, l_run;
  float mu;  // exponent shift of the tile being folded
  f32x16 acc[Gm::ND];

  __device__ __forceinline__ void load_q(const uint16_t* qbase, long q_tok, int tw0, int G, int g,
                                         int Sq, int q_offset, int col, int half) {
    const int tok = tw0 + col / G;
    const int h = g * G + col % G;
    qpos = q_offset + tok;
    if (tok < Sq) {
      const uint16_t* qp = qbase + (long)tok * q_tok + (long)h * D + half * 8;
#pragma unroll
      for (int c = 0; c < Gm::NC; ++c) q[c] = load_pol<kGenericRowsNT>((const bf16x8*)(qp + c * 16));
    } else {
#pragma unroll
      for (int c = 0; c < Gm::NC; ++c) q[c] = bf16x8{};
    }
  }

  // Start every row from its head's sink: m = sink*log2e, l = 1 (counted once,
  // in the lower half of the wave).  sink2 = sink * log2(e), or -inf for none.
  __device__ __forceinline__ void reset(float sink2, int half) {
    m_run = sink2;
    mu = sink2 == kNegInf ? 0.0f : sink2;
    l_run = (sink2 != kNegInf && half == 0) ? 1.0f : 0.0f;
#pragma unroll
    for (int db = 0; db < Gm::ND; ++db) acc[db] = f32x16{};
  }

  // Raw scores S^T = K Q^T of one 32-key tile in LDS.
  __device__ __forceinline__ f32x16 scores(const uint16_t* k_t, int lane) const {
    const lds_u16* kbase = lane_base(lds_addr(k_t), KTile<D>::k_lane_off(lane));
    bf16x8 ka[Gm::NC];
#pragma unroll
    for (int c = 0; c < Gm::NC; ++c) ka[c] = KTile<D>::k_operand(kbase, c);
    f32x16 s = {};
#pragma unroll
    for (int c = 0; c < Gm::NC; ++c) s = mfma32(ka[c], q[c], s);
    return s;
  }

  // Causal / window mask of the tile starting at key kb (masked scores ->
  // -inf).  mask: kMaskHi if some key of the tile lies after some query of
  // the wave, kMaskLo if some key lies below some query's window, kMaskAll to
  // drop the whole tile.
  __device__ __forceinline__ void apply_mask(f32x16& s, int kb, int mask, int window, int half) const {
    if (mask == kMaskAll) {
#pragma unroll
      for (int v = 0; v < 16; ++v) s[v] = kNegInf;
    } else if (mask) {
      // The key of register v sits at kb + 4*half + cv with cv = 8*(v/4) +
      // v%4, so with a = qpos - kb - 4*half it is valid iff a - W + 1 <= cv
      // <= a: one compare per score when only one bound can bite.
      const int a = qpos - kb - 4 * half;
      const int alo = a - window + 1;
      if (mask == kMaskHi) {
#pragma unroll
        for (int v = 0; v < 16; ++v) s[v] = (c_row(v, 0) <= a) ? s[v] : kNegInf;
      } else if (mask == kMaskLo) {
#pragma unroll
        for (int v = 0; v < 16; ++v) s[v] = (c_row(v, 0) >= alo) ? s[v] : kNegInf;
      } else {
#pragma unroll
        for (int v = 0; v < 16; ++v) s[v] = (c_row(v, 0) <= a && c_row(v, 0) >= alo) ? s[v] : kNegInf;
      }
    }
  }

  // Lazy rescale from the raw-score maximum mx of this lane's scores of a
  // tile (scale > 0 commutes with max), then the exponent shift mu.
  __device__ __forceinline__ void update_max(float mx, float c2) {
    mx = halves_max(mx) * c2;
    const float m_new = __builtin_elementwise_maximum(m_run, mx);
    const bool need = m_new > m_run + kRescaleTau;
    if (wave_any(need)) {
      const float alpha = need ? exp2_fast(m_run - m_new) : 1.0f;
      m_run = need ? m_new : m_run;
      l_run *= alpha;
#pragma unroll
      for (int db = 0; db < Gm::ND; ++db) acc[db] *= alpha;
    }
    mu = m_run == kNegInf ? 0.0f : m_run;
  }

  // Mask, row max and lazy rescale of a tile folded without a predecessor.
  __device__ __forceinline__ void prep(f32x16& s, int kb, int mask, int window, float c2, int half) {
    apply_mask(s, kb, mask, window, half);
    float mx = kNegInf;
#pragma unroll
    for (int v = 0; v < 16; ++v) mx = __builtin_elementwise_maximum(mx, s[v]);
    update_max(mx, c2);
  }

  // P = exp2(s*c2 - mu) rounded to bf16, l += the sum of the weights
  // (pack_sum), O^T += V^T P^T for the V tile v_t.  With NEXT the scores of
  // the K tile k_next (first key kb_next) are computed in the same
  // instruction stream, masked, reduced to their
  // row max and folded into the running max (so mu is ready for them) and
  // returned.  Each score MFMA is followed by a share of the exponentials
  // and their sums, each P V MFMA by a share of the next row max
  // (scheduling fences keep that order), so the matrix core and the vector
  // ALU of the SIMD work at the same time.
  // `extra(c)` runs right after score MFMA c (work that then issues while
  // the matrix core is busy, e.g. the next tiles' global loads).  With
  // PRE_IN the first KPRE K operands of k_next were read ahead into kpre;
  // with PRE_OUT this fold reads those of k_after (the tile the next fold
  // scores) into kpre during its P V MFMAs, so the next fold's first score
  // MFMAs do not wait for LDS.
  static constexpr int KPRE = Gm::NC < 4 ? Gm::NC : 4;
  template <bool NEXT, bool PRE_IN = false, bool PRE_OUT = false, typename X = NoExtra>
  __device__ __forceinline__ f32x16 fold(const f32x16& s, float c2, const uint16_t* v_t,
                                         const uint16_t* k_next, int kb_next, int mask_next,
                                         int window, int half, int lane, const X& extra = X(),
                                         bf16x8* kpre = nullptr, const uint16_t* k_after = nullptr) {
    constexpr int EPM = 16 / Gm::NC;  // exponentials per score MFMA
    const lds_u16* vbase = lane_base(lds_addr(v_t), VTile<D>::vt_lane_off(lane));
    f32x16 sn = {};
    bf16x8 pb[2];
    bf16x8 va[2][Gm::ND];
    if constexpr (NEXT) {
      const lds_u16* kbase = lane_base(lds_addr(k_next), KTile<D>::k_lane_off(lane));
      bf16x8 ka[Gm::NC];
#pragma unroll
      for (int c = 0; c < Gm::NC; ++c) ka[c] = (PRE_IN && c < KPRE) ? kpre[c] : KTile<D>::k_operand(kbase, c);
#pragma unroll
      for (int db = 0; db < Gm::ND; ++db) va[0][db] = VTile<D>::vt_operand(vbase, db, 0);
      __builtin_amdgcn_sched_barrier(0);
      // the packed weights pass through an empty asm so that the
      // exponentials stay next to their MFMA instead of sinking to the use
      uint32_t pw[8];
      // each group converts the previous group's exponentials after its
      // MFMA, so no conversion waits on the exponential just issued
      float ex[EPM];
#pragma unroll
      for (int c = 0; c < Gm::NC; ++c) {
        sn = mfma32(ka[c], q[c], sn);
        if (c > 0) {
#pragma unroll
          for (int e = 0; e < EPM; e += 2) pw[((c - 1) * EPM + e) >> 1] = pack_sum<RSUM>(ex[e], ex[e + 1], l_run);
        }
#pragma unroll
        for (int e = 0; e < EPM; ++e) {
          ex[e] = exp2_fast(fmaf(s[c * EPM + e], c2, -mu));
          __asm__ volatile("" : "+v"(ex[e]));
        }
        extra(c);
        __builtin_amdgcn_sched_barrier(0);
      }
#pragma unroll
      for (int e = 0; e < EPM; e += 2) pw[((Gm::NC - 1) * EPM + e) >> 1] = pack_sum<RSUM>(ex[e], ex[e + 1], l_run);
      pb[0] = __builtin_bit_cast(bf16x8, u32x4{pw[0], pw[1], pw[2], pw[3]});
      pb[1] = __builtin_bit_cast(bf16x8, u32x4{pw[4], pw[5], pw[6], pw[7]});
      apply_mask(sn, kb_next, mask_next, window, half);
      // O^T += V^T P^T (keys 16kc .. 16kc+15 per MFMA) with the row max of
      // the next scores in between; the second key half of V is read while
      // the first is multiplied
#pragma unroll
      for (int db = 0; db < Gm::ND; ++db) va[1][db] = VTile<D>::vt_operand(vbase, db, 1);
      float mx = kNegInf;
      constexpr int NPV = 2 * Gm::ND;
#pragma unroll
      for (int i = 0; i < NPV; ++i) {
        const int kc = i / Gm::ND, db = i % Gm::ND;
        acc[db] = mfma32(va[kc][db], pb[kc], acc[db]);
        if constexpr (PRE_OUT) {
          if (i == 1) {
            const lds_u16* abase = lane_base(lds_addr(k_after), KTile<D>::k_lane_off(lane));
#pragma unroll
            for (int c = 0; c < KPRE; ++c) kpre[c] = KTile<D>::k_operand(abase, c);
          }
        }
#pragma unroll
        for (int j = i * 8 / NPV; j < (i + 1) * 8 / NPV; ++j)
          mx = __builtin_elementwise_maximum(mx, __builtin_elementwise_maximum(sn[2 * j], sn[2 * j + 1]));
        __builtin_amdgcn_sched_barrier(0);
      }
      update_max(mx, c2);
    } else {
#pragma unroll
      for (int kc = 0; kc < 2; ++kc)
#pragma unroll
        for (int db = 0; db < Gm::ND; ++db) va[kc][db] = VTile<D>::vt_operand(vbase, db, kc);
      uint32_t pw[8];
#pragma unroll
      for (int j = 0; j < 8; ++j)
        pw[j] = pack_sum<RSUM>(exp2_fast(fmaf(s[2 * j], c2, -mu)), exp2_fast(fmaf(s[2 * j + 1], c2, -mu)), l_run);
      pb[0] = __builtin_bit_cast(bf16x8, u32x4{pw[0], pw[1], pw[2], pw[3]});
      pb[1] = __builtin_bit_cast(bf16x8, u32x4{pw[4], pw[5], pw[6], pw[7]});
#pragma unroll
      for (int kc = 0; kc < 2; ++kc)
#pragma unroll
        for (int db = 0; db < Gm::ND; ++db) acc[db] = mfma32(va[kc][db], pb[kc], acc[db]);
    }
    return sn;
  }

  // Fold of one tile whose rescale need is decided by its weights' sum (the
  // no-window loop): P = exp2(s*c2 - mu) with the current shift, rounded to
  // bf16, then this lane's sum of its 16 weights (pack_sum).  A weight above
  // 2^kRescaleTau forces that sum above it, so when no lane's sum exceeds it
  // every weight is bounded as under the max-based rule, and no row max is
  // needed: the check is one compare per lane before P V.  Otherwise (rare:
  // a score well above the running shift) the tile's true row max is taken,
  // the accumulator rescaled and the weights recomputed.  With NEXT the
  // score MFMAs of the K tile k_next run between the exponentials, the next
  // tile's mask is applied to them, and they are returned (raw).  `extra`,
  // kpre and k_after as in fold.
  template <bool NEXT, bool PRE_IN = false, bool PRE_OUT = false, typename X = NoExtra>
  __device__ __forceinline__ f32x16 fold_sum(f32x16 s, float c2, const uint16_t* v_t, const uint16_t* k_next,
                                             int kb_next, int mask_next, int window, int half, int lane,
                                             const X& extra = X(), bf16x8* kpre = nullptr,
                                             const uint16_t* k_after = nullptr) {
    constexpr int EPM = 16 / Gm::NC;  // exponentials per score MFMA
    constexpr int NPAIR = 8;          // packed weight pairs per tile
    const lds_u16* vbase = lane_base(lds_addr(v_t), VTile<D>::vt_lane_off(lane));
    f32x16 sn = {};
    uint32_t pw[NPAIR];
    float tsum = 0.0f;
    bf16x8 va[2][Gm::ND];
    if constexpr (NEXT) {
      const lds_u16* kbase = lane_base(lds_addr(k_next), KTile<D>::k_lane_off(lane));
      bf16x8 ka[Gm::NC];
#pragma unroll
      for (int c = 0; c < Gm::NC; ++c) ka[c] = (PRE_IN && c < KPRE) ? kpre[c] : KTile<D>::k_operand(kbase, c);
#pragma unroll
      for (int db = 0; db < Gm::ND; ++db) va[0][db] = VTile<D>::vt_operand(vbase, db, 0);
      __builtin_amdgcn_sched_barrier(0);
      // group c: score MFMA c; pack the previous group's weights and add
      // them to the sum; this group's exponentials
      float ex[EPM];
#pragma unroll
      for (int c = 0; c < Gm::NC; ++c) {
        sn = mfma32(ka[c], q[c], sn);
        if (c > 0) {
#pragma unroll
          for (int e = 0; e < EPM; e += 2) pw[((c - 1) * EPM + e) >> 1] = pack_sum<RSUM>(ex[e], ex[e + 1], tsum);
        }
#pragma unroll
        for (int e = 0; e < EPM; ++e) {
          ex[e] = exp2_fast(fmaf(s[c * EPM + e], c2, -mu));
          __asm__ volatile("" : "+v"(ex[e]));
        }
        extra(c);
        __builtin_amdgcn_sched_barrier(0);
      }
#pragma unroll
      for (int e = 0; e < EPM; e += 2) pw[((Gm::NC - 1) * EPM + e) >> 1] = pack_sum<RSUM>(ex[e], ex[e + 1], tsum);
    } else {
#pragma unroll
      for (int kc = 0; kc < 2; ++kc)
#pragma unroll
        for (int db = 0; db < Gm::ND; ++db) va[kc][db] = VTile<D>::vt_operand(vbase, db, kc);
#pragma unroll
      for (int j = 0; j < NPAIR; ++j)
        pw[j] = pack_sum<RSUM>(exp2_fast(fmaf(s[2 * j], c2, -mu)), exp2_fast(fmaf(s[2 * j + 1], c2, -mu)), tsum);
    }
    if (wave_any(!(tsum <= exp2_fast(kRescaleTau)))) {
      // a weight may exceed 2^tau (or be non-finite): shift by the tile's row max
      // (mu is the shift the accumulator and the sum are kept at: the
      // running max, or 0 while that is still -inf)
      float mx = kNegInf;
#pragma unroll
      for (int v = 0; v < 16; ++v) mx = __builtin_elementwise_maximum(mx, s[v]);
      // (alpha is exactly 1 where the shift does not move)
      const float m_new = __builtin_elementwise_maximum(mu, halves_max(mx) * c2);
      const float alpha = exp2_fast(mu - m_new);
      l_run *= alpha;
#pragma unroll
      for (int db = 0; db < Gm::ND; ++db) acc[db] *= alpha;
      mu = m_new;
      tsum = 0.0f;
#pragma unroll
      for (int j = 0; j < NPAIR; ++j)
        pw[j] = pack_sum<RSUM>(exp2_fast(fmaf(s[2 * j], c2, -mu)), exp2_fast(fmaf(s[2 * j + 1], c2, -mu)), tsum);
    }
    l_run += tsum;
    bf16x8 pb[2];
    pb[0] = __builtin_bit_cast(bf16x8, u32x4{pw[0], pw[1], pw[2], pw[3]});
    pb[1] = __builtin_bit_cast(bf16x8, u32x4{pw[4], pw[5], pw[6], pw[7]});
    if constexpr (NEXT) {
      apply_mask(sn, kb_next, mask_next, window, half);
#pragma unroll
      for (int db = 0; db < Gm::ND; ++db) va[1][db] = VTile<D>::vt_operand(vbase, db, 1);
    }
    constexpr int NPV = 2 * Gm::ND;
#pragma unroll
    for (int i = 0; i < NPV; ++i) {
      const int kc = i / Gm::ND, db = i % Gm::ND;
      acc[db] = mfma32(va[kc][db], pb[kc], acc[db]);
      if constexpr (NEXT && PRE_OUT) {
        if (i == 1) {
          const lds_u16* abase = lane_base(lds_addr(k_after), KTile<D>::k_lane_off(lane));
#pragma unroll
          for (int c = 0; c < KPRE; ++c) kpre[c] = KTile<D>::k_operand(abase, c);
        }
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    return sn;
  }

  // One step of the skewed pipeline of the no-window loop.  On entry pw
  // holds the packed bf16 weights P(t) of tile t (already summed into l) and
  // s the raw scores S(t+1) of tile t + 1.  The step issues O^T += V(t)^T
  // P(t)^T (V tile v_t) and the score MFMAs of tile t + 2 (K tile k_next2,
  // first key kb_next2) alternately, one of each per group, and between
  // them the exponentials of S(t+1) against the shift in use, their bf16
  // packing and their sum; then the rescale is decided from that sum as in
  // fold_sum.  On exit pw holds P(t+1) (summed into l) and the masked S(t+2)
  // is returned.  No MFMA of a step depends on the step's vector work, and
  // the score chain is interleaved with independent P V products, so the
  // matrix core has work while the exponentials issue.  Without PV (the
  // first step) only the scores and the weights are formed.  `extra(c)` as
  // in fold.
  // K and V^T operands of a step's first groups, read during the previous
  // step (skew_step's PRE_IN / PRE_OUT).
  static constexpr int SKEW_PRE = 2;
  struct SkewOps {
    bf16x8 k[SKEW_PRE];
    bf16x8 v[SKEW_PRE];
  };

  // The operands of group c are read SKEW_PRE groups ahead, during group c -
  // SKEW_PRE, so the reads of the eight waves spread over the step instead
  // of queueing at its start.  With PRE_IN the operands of groups 0 ..
  // SKEW_PRE - 1 come from ops (read by the previous step), else they are
  // read at the start; with PRE_OUT the last groups read those of the next
  // step (V tile v_after, K tile k_after) into ops.
  template <bool PV, int PRE_IN = 0, int PRE_OUT = 0, typename X = NoExtra>
  __device__ __forceinline__ f32x16 skew_step(const f32x16& s, uint32_t (&pw)[8], float c2, const uint16_t* v_t,
                                              const uint16_t* k_next2, int kb_next2, int mask_next2, int window,
                                              int half, int lane, const X& extra = X(), SkewOps* ops = nullptr,
                                              const uint16_t* v_after = nullptr, const uint16_t* k_after = nullptr) {
    constexpr int EPM = 16 / Gm::NC;  // exponentials per group
    constexpr int NPAIR = 8;          // packed weight pairs per tile
    constexpr int RA = SKEW_PRE;      // read-ahead distance in groups
    static_assert(Gm::NC == 2 * Gm::ND, "one P V MFMA per score MFMA");
    static_assert((PRE_IN == 0 || PRE_IN == RA) && (PRE_OUT == 0 || PRE_OUT == RA) && RA < Gm::NC,
                  "read-ahead depth");
    const lds_u16* kbase = lane_base(lds_addr(k_next2), KTile<D>::k_lane_off(lane));
    const lds_u16* vbase = PV ? lane_base(lds_addr(v_t), VTile<D>::vt_lane_off(lane)) : nullptr;
    bf16x8 ka[Gm::NC];
    bf16x8 va[2][Gm::ND];
    bf16x8 pb[2];
    auto read_group = [&](int c) {
      ka[c] = KTile<D>::k_operand(kbase, c);
      if constexpr (PV) va[c / Gm::ND][c % Gm::ND] = VTile<D>::vt_operand(vbase, c % Gm::ND, c / Gm::ND);
    };
#pragma unroll
    for (int c = 0; c < RA; ++c) {
      if (PRE_IN > 0) {
        ka[c] = ops->k[c];
        va[c / Gm::ND][c % Gm::ND] = ops->v[c];
      } else {
        read_group(c);
      }
    }
    if constexpr (PV) {
      pb[0] = __builtin_bit_cast(bf16x8, u32x4{pw[0], pw[1], pw[2], pw[3]});
      pb[1] = __builtin_bit_cast(bf16x8, u32x4{pw[4], pw[5], pw[6], pw[7]});
    }
    __builtin_amdgcn_sched_barrier(0);
    f32x16 sn = {};
    uint32_t pn[NPAIR];
    float tsum = 0.0f;
    float ex[EPM];
    // group c: score MFMA c; the operands of group c + RA; pack the previous
    // group's weights and add them to the sum; P V MFMA c; this group's
    // exponentials
#pragma unroll
    for (int c = 0; c < Gm::NC; ++c) {
      sn = mfma32(ka[c], q[c], sn);
      if (c + RA < Gm::NC) {
        read_group(c + RA);
      } else if constexpr (PRE_OUT > 0) {
        const int j = c + RA - Gm::NC;
        const lds_u16* kb2 = lane_base(lds_addr(k_after), KTile<D>::k_lane_off(lane));
        const lds_u16* vb2 = lane_base(lds_addr(v_after), VTile<D>::vt_lane_off(lane));
        ops->k[j] = KTile<D>::k_operand(kb2, j);
        ops->v[j] = VTile<D>::vt_operand(vb2, j % Gm::ND, j / Gm::ND);
      }
      if (c > 0) {
#pragma unroll
        for (int e = 0; e < EPM; e += 2) pn[((c - 1) * EPM + e) >> 1] = pack_sum<RSUM>(ex[e], ex[e + 1], tsum);
      }
      // the P V MFMA issues once the score MFMA is well under way, so the
      // wave does not stall on it with its vector work queued behind
      __builtin_amdgcn_sched_barrier(0);
      if constexpr (PV) acc[c % Gm::ND] = mfma32(va[c / Gm::ND][c % Gm::ND], pb[c / Gm::ND], acc[c % Gm::ND]);
#pragma unroll
      for (int e = 0; e < EPM; ++e) {
        ex[e] = exp2_fast(fmaf(s[c * EPM + e], c2, -mu));
        __asm__ volatile("" : "+v"(ex[e]));
      }
      extra(c);
      __builtin_amdgcn_sched_barrier(0);
    }
#pragma unroll
    for (int e = 0; e < EPM; e += 2) pn[((Gm::NC - 1) * EPM + e) >> 1] = pack_sum<RSUM>(ex[e], ex[e + 1], tsum);
    if (wave_any(!(tsum <= exp2_fast(kRescaleTau)))) {
      // as fold_sum: shift by the tile's row max, rescale what has been
      // accumulated (P V of tiles up to t, issued above), recompute
      float mx = kNegInf;
#pragma unroll
      for (int v = 0; v < 16; ++v) mx = __builtin_elementwise_maximum(mx, s[v]);
      const float m_new = __builtin_elementwise_maximum(mu, halves_max(mx) * c2);
      const float alpha = exp2_fast(mu - m_new);
      l_run *= alpha;
#pragma unroll
      for (int db = 0; db < Gm::ND; ++db) acc[db] *= alpha;
      mu = m_new;
      tsum = 0.0f;
#pragma unroll
      for (int j = 0; j < NPAIR; ++j)
        pn[j] = pack_sum<RSUM>(exp2_fast(fmaf(s[2 * j], c2, -mu)), exp2_fast(fmaf(s[2 * j + 1], c2, -mu)), tsum);
    }
    l_run += tsum;
#pragma unroll
    for (int j = 0; j < NPAIR; ++j) pw[j] = pn[j];
    apply_mask(sn, kb_next2, mask_next2, window, half);
    return sn;
  }

  // O^T += V^T P^T for the packed weights pw of the V tile v_t (the last
  // tile of the skewed pipeline).
  __device__ __forceinline__ void pv_only(const uint32_t (&pw)[8], const uint16_t* v_t, int lane) {
    const lds_u16* vbase = lane_base(lds_addr(v_t), VTile<D>::vt_lane_off(lane));
    bf16x8 va[2][Gm::ND];
#pragma unroll
    for (int kc = 0; kc < 2; ++kc)
#pragma unroll
      for (int db = 0; db < Gm::ND; ++db) va[kc][db] = VTile<D>::vt_operand(vbase, db, kc);
    const bf16x8 pb[2] = {__builtin_bit_cast(bf16x8, u32x4{pw[0], pw[1], pw[2], pw[3]}),
                          __builtin_bit_cast(bf16x8, u32x4{pw[4], pw[5], pw[6], pw[7]})};
#pragma unroll
    for (int kc = 0; kc < 2; ++kc)
#pragma unroll
      for (int db = 0; db < Gm::ND; ++db) acc[db] = mfma32(va[kc][db], pb[kc], acc[db]);
  }

  // Natural-log softmax denominator of each row, sink included, for the
  // backward: lse = (mu + log2 l) * ln 2, mu being the shift the accumulator
  // and l are kept at (the running max, or 0 while that is -inf), so the sum
  // is exact whatever the shift.  lse_b points at [b][0][0] of [B, Sq, Hq].
  __device__ __forceinline__ void store_lse(float* lse_b, int Hq, int tw0, int G, int g, int Sq, int col,
                                            int half) const {
    const float lt = halves_sum(l_run);
    const int tok = tw0 + col / G;
    if (half == 0 && tok < Sq) lse_b[(long)tok * Hq + g * G + col % G] = (mu + __builtin_amdgcn_logf(lt)) * kLn2;
  }

  // O = acc / l in bf16, one 8-byte store per 4 consecutive d.
  __device__ __forceinline__ void store_o(uint16_t* obase, long q_tok, int tw0, int G, int g, int Sq,
                                          int col, int half) {
    const int tok = tw0 + col / G;
    const int h = g * G + col % G;
    const float lt = halves_sum(l_run);
    if (tok >= Sq) return;
    const float inv = 1.0f / lt;
    uint16_t* op = obase + (long)tok * q_tok + (long)h * D;
#pragma unroll
    for (int db = 0; db < Gm::ND; ++db) {
#pragma unroll
      for (int a4 = 0; a4 < 4; ++a4) {
        const f32x4 y = {acc[db][4 * a4] * inv, acc[db][4 * a4 + 1] * inv, acc[db][4 * a4 + 2] * inv,
                         acc[db][4 * a4 + 3] * inv};
        store_pol<kGenericRowsNT>(__builtin_convertvector(y, bf16x4), (bf16x4*)(op + db * 32 + 8 * a4 + 4 * half));
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
// XCD-aware work order, longest (latest) blocks first.
//
// Without a window (NOWIN) the K/V tiles stream through a ring of eight
// "pair slots" in LDS, each holding one K tile and one V tile in the padded
// layouts of KTile / VTile, filled by direct-to-LDS loads in whole 1 KiB
// windows.  The waves run the skewed pipeline of QState::skew_step: step t
// multiplies P(t) into V(t), computes the scores of tile t + 2 and the
// weights of tile t + 1, so the pair slot that step t reads holds V(t) and
// K(t + 2), and step t fetches K(t + 6) and V(t + 4) into the slot step
// t + 4 reads (last read four steps earlier).  Slots are numbered from the
// first step of the four-step trips (single steps, a barrier each, come
// first), so a trip reads slots rb .. rb + 3 and fills (rb ^ 4) .. (rb ^ 4) +
// 3, rb alternating between 0 and 4: no slot index wraps inside a trip.
// With a window: a 4-slot K/V ring staged through registers, two tiles per
// barrier, each wave folding only the tiles of its own range (QState::fold).
// LSE: also save each row's log-sum-exp (p.lse).  The row sums add the
// rounded weights (QState's RSUM), so that a saved log-sum-exp matches the
// output, except in the plain no-window kernel, whose matrix core is the
// bottleneck: there they add the weights before rounding, off the
// matrix-core pipeline (pack_sum).
template <int D, int G, int NW, bool NOWIN, bool LSE>
__global__ __launch_bounds__(NW * 64) void prefill_bf16_kernel(PrefillArgs p) {
  using QS = QState<D, LSE || !NOWIN>;
  using Gm = TileGeom<D>;
  constexpr int NT = NW * 64;
  constexpr int TW = 32 / G;        // tokens per wave
  constexpr int TB = TW * NW;       // tokens per workgroup
  static_assert(32 % G == 0, "a 32-row block must hold whole tokens");
  using Dma = DmaTile<D>;

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
  const int W = NOWIN ? 0 : p.window;  // NOWIN is launched only for window 0
  const float c2 = p.scale_log2;

  QS st;
  st.load_q(p.q + qoff, q_tok, tw0, G, g, p.Sq, p.q_offset, col, half);

  const int tlast = min(t0 + TB, p.Sq) - 1;
  const int pos_lo = p.q_offset + t0, pos_hi = p.q_offset + tlast;
  // keys [key_lo, key_end) are the ones the workgroup's queries can see:
  // tile rows outside read as (or are set to) zeros
  const int key_lo = W > 0 ? max(0, pos_lo - W + 1) : 0, key_end = pos_hi + 1;
  const int kt_begin = key_lo / KT, kt_end = pos_hi / KT;
  // this wave's tiles: [wk0, wk1] (empty when its tokens are all past Sq)
  const int wpos_lo = p.q_offset + tw0;
  const int wpos_hi = p.q_offset + min(tw0 + TW, p.Sq) - 1;
  const int wk0 = max(kt_begin, (W > 0 ? max(0, wpos_lo - W + 1) : 0) / KT);
  const int wk1 = tw0 < p.Sq ? wpos_hi / KT : -1;
  const float sink = p.sinks ? p.sinks[g * G + col % G] : 0.0f;
  // (the mask of tile kt for this wave; kMaskAll before its first tile)
  auto tile_mask = [&](int kt) {
    int mask;
    tile_needed(kt * KT, wpos_lo, wpos_hi, W, mask);
    return !NOWIN && kt < wk0 ? kMaskAll : mask;
  };

  if constexpr (NOWIN) {
    constexpr int PAIR = (Dma::NK + Dma::NV) * 512;  // bf16 elements per pair slot: K tile, then V tile
    constexpr int VREG = Dma::NK * 512;              // the V tile's offset in a slot
    constexpr uint32_t PAIR_B = 2u * PAIR;
    // The NPT 1 KiB windows of a step's K + V tile pair, padded to WPW per
    // wave: wave wv fills windows wv, wv + NW, ..., WPW of them every step
    // (so its per-lane offsets are fixed); a window past NPT is a dummy whose
    // lanes all read out of range and write zeros into dma_sink (no memory
    // access), so every wave issues the same loads with no branch.
    constexpr int WPW = (Dma::NPT + NW - 1) / NW;
    static_assert(WPW + 1 <= Gm::NC, "one load per group of a step");
    __shared__ __attribute__((aligned(16))) uint16_t ring[8][PAIR];
    __shared__ __attribute__((aligned(16))) uint16_t dma_sink[512];

    const long tstride = (long)KT * kv_tok;
    const uint32_t row_b = (uint32_t)(2 * kv_tok), pad_b = (uint32_t)(2 * (kv_tok - D));
    const uint32_t tile_b = (uint32_t)KT * row_b;
    const uint32_t full_rec = tile_b - pad_b;
    // records of tile t: rows at or past key_end read as zeros
    auto tile_rec = [&](int t) {
      return t * KT + KT <= key_end ? full_rec : (uint32_t)(key_end - t * KT) * row_b - pad_b;
    };
    const int singles = (kt_end - kt_begin) & 3;
    const int kt0 = kt_begin + singles;  // first step of the four-step trips
    // pair slot read by step t (V(t), K(t + 2))
    auto pslot = [&](int t) { return (t - kt0) & 7; };
    const uint32_t ring0 = lds_addr(ring[0]);

    // this wave's windows: global byte offset per lane, LDS offset in a slot
    uint32_t dma_off[WPW], dma_lds[WPW];
    bool dma_k[WPW], dma_on[WPW];
#pragma unroll
    for (int k = 0; k < WPW; ++k) {
      const int rr = wv + NW * k;
      dma_on[k] = rr < Dma::NPT;
      dma_k[k] = rr < Dma::NK;
      const int win = dma_k[k] ? rr : rr - Dma::NK;
      dma_off[k] = dma_on[k] ? Dma::voff(dma_k[k], win, lane, row_b) : Dma::kOut;
      dma_lds[k] = dma_k[k] ? 1024u * (uint32_t)win : 2u * VREG + 1024u * (uint32_t)win;
    }
    const uint32_t sink_lds = lds_addr(dma_sink);

    // Prologue: K(kt_begin .. + 5) and V(kt_begin .. + 3), window i of them
    // by wave i mod NW; K(t) goes to the slot of step t - 2.
    {
      constexpr int PK = 6, PV = 4;
      for (int i = wv; i < PK * Dma::NK + PV * Dma::NV; i += NW) {
        const bool is_k = i < PK * Dma::NK;
        const int j = is_k ? i : i - PK * Dma::NK;
        const int nw = is_k ? Dma::NK : Dma::NV;
        const int t = kt_begin + j / nw, win = j % nw;
        if (t > kt_end) continue;
        const uint32_t lds = ring0 + (uint32_t)pslot(is_k ? t - 2 : t) * PAIR_B + (is_k ? 0u : 2u * VREG) +
                             1024u * (uint32_t)win;
        Dma::load((is_k ? kg : vg) + t * tstride, tile_rec(t), lds, Dma::voff(is_k, win, lane, row_b));
      }
    }
    st.reset(p.sinks ? sink * kLog2e : kNegInf, half);
    // drain the prologue loads (queries, first tiles): inside the loop the
    // only loads in flight are then the prefetches
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();

    // every wave's range starts at the workgroup's first tile, and a tile
    // past a wave's last query is masked whole by the causal bound, so every
    // wave folds every tile with no per-wave condition
    f32x16 s = st.scores(&ring[pslot(kt_begin - 2)][0], lane);
    st.prep(s, kt_begin * KT, tile_mask(kt_begin), W, c2, half);
    uint32_t pw[8];
    s = st.template skew_step<false>(s, pw, c2, nullptr, &ring[pslot(kt_begin - 1)][0], (kt_begin + 1) * KT,
                                     tile_mask(kt_begin + 1), W, half, lane);
    // the slots of K(kt_begin) and K(kt_begin + 1) are refilled two and three
    // steps on: every wave has read them before that
    __syncthreads();

    // General step t (single steps and the last trips): bounds-checked loads
    // of the tiles that exist, the mask of tile t + 2.
    auto general_step = [&](int t) {
      const int r = pslot(t);
      s = st.template skew_step<true>(s, pw, c2, &ring[r][VREG], &ring[r][0], (t + 2) * KT, tile_mask(t + 2), W,
                                      half, lane, [&](int c) {
                                        if (c >= 1 && c <= WPW) {
                                          const int k = c - 1;
                                          const int tt = t + (dma_k[k] ? 6 : 4);
                                          if (dma_on[k] && tt <= kt_end)
                                            Dma::load((dma_k[k] ? kg : vg) + tt * tstride, tile_rec(tt),
                                                      ring0 + (uint32_t)pslot(t + 4) * PAIR_B + dma_lds[k],
                                                      dma_off[k]);
                                        }
                                      });
    };
    int kt = kt_begin;
    for (; kt < kt0; ++kt) {
      general_step(kt);
      __builtin_amdgcn_s_waitcnt(0);
      __syncthreads();
    }
    if (wv >= NW / 2) __builtin_amdgcn_s_setprio(1);
    // Four-step trips.  Window k's loads of a trip share one buffer
    // descriptor based at the first row of the tile it fetches in the
    // trip's first step (K(kt + 6) or V(kt + 4)), with its range cut at
    // key_end: step i adds i tiles to the lane offsets, rows at or past
    // key_end (and tiles past kt_end) read as zeros without a memory access,
    // and lanes pointed at kOut (row padding, dummy windows) stay out of
    // range.  The score tiles of a trip need no mask unless its last one
    // (kt + 5) reaches a query position.
    const uint16_t* bp[WPW];
#pragma unroll
    for (int k = 0; k < WPW; ++k) bp[k] = dma_k[k] ? kg + (kt + 6) * tstride : vg + (kt + 4) * tstride;
    const uint32_t trip_rec = 3u * tile_b + full_rec;
    uint32_t m0_step[WPW];  // LDS stride of window k from one step to the next (0: the sink)
#pragma unroll
    for (int k = 0; k < WPW; ++k) m0_step[k] = dma_on[k] ? PAIR_B : 0u;
    for (uint32_t rb = 0; kt < kt_end; kt += 4, rb ^= 4u) {
      const bool masked = (kt + 5) * KT + KT - 1 > pos_lo;
      u32x4 desc[WPW];
      uint32_t m0k[WPW];
      // window k's descriptor for this trip, built in the first step right
      // before its first load (scalar work between that step's MFMAs rather
      // than at the trip start, where both waves of a SIMD sit after the barrier)
      auto make_desc = [&](int k) {
        // keys of window k's tiles this trip: from (kt + 6) or (kt + 4) tiles on
        const int key0 = (kt + (dma_k[k] ? 6 : 4)) * KT;
        const int rows = min(key_end - key0, 4 * KT);
        desc[k] = buffer_desc(bp[k], rows <= 0 ? 0u : min(trip_rec, (uint32_t)rows * row_b - pad_b));
        bp[k] += 4 * tstride;
        m0k[k] = dma_on[k] ? ring0 + (rb ^ 4u) * PAIR_B + dma_lds[k] : sink_lds;
      };
      // steps 1 .. 3 of the trip get their first operands read by the step
      // before (the slots of a trip are all resident since its barrier)
      typename QS::SkewOps ops;
      auto trip_step = [&](auto ic) {
        constexpr int i = decltype(ic)::value;
        uint16_t* slot = &ring[rb + i][0];
        uint16_t* after = &ring[rb + (i < 3 ? i + 1 : i)][0];
        constexpr int PRE = QS::SKEW_PRE;
        constexpr int PIN = i > 0 ? PRE : 0, POUT = i < 3 ? PRE : 0;
        s = st.template skew_step<true, PIN, POUT>(
            s, pw, c2, slot + VREG, slot, (kt + i + 2) * KT, masked ? tile_mask(kt + i + 2) : 0, W, half, lane,
            [&](int c) {
              if (c >= 1 && c <= WPW) {
                const int k = c - 1;
                if constexpr (i == 0) make_desc(k);
                lds_dma16_soff(desc[k], 0u, m0k[k] + (uint32_t)i * m0_step[k], dma_off[k] + (uint32_t)i * tile_b);
              }
            },
            &ops, after + VREG, after);
      };
      trip_step(std::integral_constant<int, 0>());
      trip_step(std::integral_constant<int, 1>());
      trip_step(std::integral_constant<int, 2>());
      trip_step(std::integral_constant<int, 3>());
      // every direct-to-LDS load of this wave has landed before the barrier
      // that hands the slots to the other waves
      __builtin_amdgcn_s_waitcnt(0);
      __syncthreads();
    }
    st.pv_only(pw, &ring[pslot(kt_end)][VREG], lane);
  } else {
    // K/V ring of four slots, staged through registers; tile t in slot
    // (t - kt_begin) % 4.  A step over two tiles kt, kt + 1 reads K(kt + 1),
    // K(kt + 2), V(kt), V(kt + 1) and stages K(kt + 3), K(kt + 4), V(kt + 2),
    // V(kt + 3); one barrier per two tiles.
    __shared__ __attribute__((aligned(16))) uint16_t k_lds[4][Gm::K_ELEMS];
    __shared__ __attribute__((aligned(16))) uint16_t v_lds[4][Gm::V_ELEMS];
    Stager<D, NT> s0, s1;
    s0.init(kv_tok, tid);
    s1.init(kv_tok, tid);
    {
      // the first PK K tiles and PV V tiles the loop expects resident: every
      // load is issued before the first LDS store, so the block start waits
      // for one memory round trip
      constexpr int PK = 3, PV = PK - 1;
      Stager<D, NT> pro[PK];
#pragma unroll
      for (int i = 0; i < PK; ++i) {
        pro[i].init(kv_tok, tid);
        if (kt_begin + i <= kt_end) {
          pro[i].load_k(kg, kv_tok, (kt_begin + i) * KT, key_end, tid);
          if (i < PV) pro[i].load_v(vg, kv_tok, (kt_begin + i) * KT, key_end, tid);
        }
      }
      pro[0].zero_below(key_lo - kt_begin * KT, tid);
#pragma unroll
      for (int i = 0; i < PK; ++i)
        if (kt_begin + i <= kt_end) {
          pro[i].store_k(k_lds[i], tid);
          if (i < PV) pro[i].store_v(v_lds[i], tid);
        }
    }
    st.reset(p.sinks ? sink * kLog2e : kNegInf, half);
    // drain the prologue loads (queries, first tiles): inside the loop the
    // only loads in flight are then the prefetches
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();

    // Each fold of tile kt also computes the scores of tile kt + 1 (discarded
    // after the last tile); the last tile of the workgroup is folded after
    // the loop.  A wave folds only the tiles of its own range, and in the
    // step before its first tile it folds a fully masked tile, which adds
    // nothing, to get those scores.
    f32x16 s = {};
    int kt = kt_begin;
    if (wk0 == kt_begin && wk1 >= 0) {
      s = st.scores(k_lds[0], lane);
      st.prep(s, kt_begin * KT, tile_mask(kt_begin), W, c2, half);
    }
    auto fold_step = [&](int kt) {
      if (kt + 1 >= wk0 && kt <= wk1) {
        const int r = kt - kt_begin;
        if (kt + 1 == wk0) st.prep(s, kt * KT, kMaskAll, W, c2, half);
        s = st.template fold<true>(s, c2, v_lds[r & 3], k_lds[(r + 1) & 3], (kt + 1) * KT, tile_mask(kt + 1), W,
                                   half, lane);
      }
    };
    if ((kt_end - kt_begin) & 1) {  // a single step first, so that pairs remain
      if (kt + 3 <= kt_end) s0.load_k(kg, kv_tok, (kt + 3) * KT, key_end, tid);
      if (kt + 2 <= kt_end) s0.load_v(vg, kv_tok, (kt + 2) * KT, key_end, tid);
      fold_step(kt);
      if (kt + 3 <= kt_end) s0.store_k(k_lds[3], tid);
      if (kt + 2 <= kt_end) s0.store_v(v_lds[2], tid);
      __syncthreads();
      ++kt;
    }
    // The second wave of each SIMD pair runs at a raised priority: otherwise
    // the older wave wins every issue tie, finishes its tiles first and idles
    // at the barrier while the younger one runs alone (measured: about 1%).
    if (wv >= NW / 2) __builtin_amdgcn_s_setprio(1);
    for (; kt < kt_end; kt += 2) {
      const int r = kt - kt_begin;
      if (kt + 3 <= kt_end) s0.load_k(kg, kv_tok, (kt + 3) * KT, key_end, tid);
      if (kt + 2 <= kt_end) s0.load_v(vg, kv_tok, (kt + 2) * KT, key_end, tid);
      if (kt + 4 <= kt_end) s1.load_k(kg, kv_tok, (kt + 4) * KT, key_end, tid);
      if (kt + 3 <= kt_end) s1.load_v(vg, kv_tok, (kt + 3) * KT, key_end, tid);
      fold_step(kt);
      fold_step(kt + 1);
      if (kt + 3 <= kt_end) s0.store_k(k_lds[(r + 3) & 3], tid);
      if (kt + 2 <= kt_end) s0.store_v(v_lds[(r + 2) & 3], tid);
      if (kt + 4 <= kt_end) s1.store_k(k_lds[r & 3], tid);
      if (kt + 3 <= kt_end) s1.store_v(v_lds[(r + 3) & 3], tid);
      __syncthreads();
    }
    if (kt_end >= wk0 && kt_end <= wk1)
      st.template fold<false>(s, c2, v_lds[(kt_end - kt_begin) & 3], nullptr, 0, 0, W, half, lane);
  }
  if (wk1 >= 0) {
    st.store_o(p.o + qoff, q_tok, tw0, G, g, p.Sq, col, half);
    if constexpr (LSE) st.store_lse(p.lse + (long)b * p.Sq * p.Hq, p.Hq, tw0, G, g, p.Sq, col, half);
  }
}

// ----------------------------------------------------------------------------
// Sliding window: persistent over a strip of 32-token blocks with an LDS ring.
// G waves per workgroup, each wave 32/G tokens x G heads (one 32-row block).
// A wave's 32 query rows are TW runs of G*D contiguous elements in q and o
// (the G heads of one token), so Q is loaded and O stored in whole rows,
// half a head_dim at a time, through a private 32 x D/2 LDS staging tile that
// converts between that layout and the MFMA register layout.
constexpr int kRingTiles = 6;
// Cache policies of the strip kernel's HBM traffic: every query row, K/V row
// and output row is touched once.
// Cache policies of the strip kernel's HBM traffic: query and output rows are
// touched once and streamed past the caches (measured 1-2% faster, 5% with
// RoPE); K/V tiles keep the default so that the window halo a strip shares
// with its neighbour stays cached.
constexpr int kStripQPolicy = kCacheNT;
constexpr int kStripKvPolicy = kCacheDefault;
constexpr int kStripOPolicy = kCacheNT;

constexpr int kStripPlain = 0, kStripRope = 1, kStripLse = 2;
constexpr double kRopeTwoPi = 6.283185307179586476925286766559;
constexpr double kRopeInvTwoPi = 0.15915494309189533576888376337251;

// MODE: kStripPlain, kStripRope (rotate the queries as they are staged) or
// kStripLse (also save each row's log-sum-exp); separate instantiations keep
// the plain kernel's registers to itself.
template <int D, int G, int MODE>
__global__ __launch_bounds__(G * 64) void prefill_swa_strip_kernel(PrefillArgs p) {
  constexpr bool ROPE = MODE == kStripRope;
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

  // ring slots rounded up to whole 1 KiB windows of direct-to-LDS loads
  // (each block's new tile arrives that way); the tile layout inside is
  // that of KTile / VTile
  using Dma = DmaTile<D>;
  __shared__ __attribute__((aligned(16))) uint16_t k_ring[NR][Dma::NK * 512];
  __shared__ __attribute__((aligned(16))) uint16_t v_ring[NR][Dma::NV * 512];
  __shared__ __attribute__((aligned(16))) uint16_t stage_lds[NW][Stg::ELEMS];
  // rotary embedding of the queries: cos / sin of (token, pair) for a wave's
  // TW tokens (entry tok * 32 + i), and of the turn by one block (TB tokens)
  __shared__ float2 rope_tab[ROPE ? NW : 1][ROPE ? TW * 32 : 1];
  __shared__ float2 rope_step[ROPE ? 32 : 1];

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

  // A wave's Q (or O) rows through a buffer resource over its TW tokens x G
  // heads: one 16-byte load instruction covers RPI rows (TPI tokens), lane l
  // taking row l / HC, chunk l % HC; tokens at or past Sq read zeros (their
  // outputs are never stored) and their stores are dropped.
  constexpr int RPI = 64 / HC;
  static_assert(RPI % G == 0, "a load instruction must cover whole tokens");
  constexpr int TPI = RPI / G;
  const uint32_t row_voff =
      (uint32_t)((((lane / HC) / G) * q_tok + ((lane / HC) % G) * D + (lane % HC) * 8) * 2);
  auto rows_rsrc = [&](const uint16_t* base, int tw0) {
    const int ntok = min(TW, p.Sq - tw0);
    const uint32_t bytes = ntok > 0 ? (uint32_t)(((ntok - 1) * q_tok + G * D) * 2) : 0u;
    return make_rsrc(base + qoff + (long)tw0 * q_tok, bytes);
  };
  // Every offset goes into the per-lane voffset: the buffer range check
  // ignores soffset, and a register soffset also makes the compiler drop the
  // wait state that protects a 16-byte store's data registers from the next
  // vector-ALU write.
  auto rows_voff = [&](int it, int hh) { return row_voff + (uint32_t)((it * TPI * q_tok + hh * HD) * 2); };

  // Q of a block in whole-row layout: chunk u = it*64 + lane of half hh is
  // row u / HC, 16-byte chunk u % HC of that half.
  u32x4 qpre[2][SIT];
  auto load_q_rows = [&](int tw0) {
    const rsrc_t r = rows_rsrc(p.q, tw0);
#pragma unroll
    for (int hh = 0; hh < 2; ++hh)
#pragma unroll
      for (int it = 0; it < SIT; ++it) qpre[hh][it] = buf_load16<kStripQPolicy>(r, rows_voff(it, hh), 0);
  };
  // (row sums of the rounded weights in every mode: the saved log-sum-exp
  // matches the output, and the plain and training forwards agree bit for
  // bit; the sum's matrix-pipeline instruction costs nothing here, where the
  // matrix core has slack)
  QState<D, true> st;
  // Partial rotary embedding of the staged first half-head (every rotated
  // dimension lies there: 2 * rope_hr <= D / 2) of rows at tokens tw0 ...
  // The wave's TW x rope_hr (cos, sin) live in LDS from block to block: the
  // first block of a strip and every 8th after it computes them exactly (the
  // angle reduced modulo 2*pi in fp64, then fp32 sincosf); the blocks between
  // turn the previous entries by the one-block step (TB more tokens), four
  // fp32 FMAs instead of a sine and a cosine.  Then all 64 lanes rotate the
  // 32 x rope_hr pairs in LDS, rounding back to bf16 (nearest even).
  auto rope_angle = [&](long pos, int i) {
    const double th = (double)pos * p.rope_inv_freq[i];
    const double r = th - rint(th * kRopeInvTwoPi) * kRopeTwoPi;
    float sn, cs;
    sincosf((float)r, &sn, &cs);
    return make_float2(cs, sn);
  };
  auto rotate_staged = [&](int tw0, bool exact) {
    const int hr = p.rope_hr;
    float2* tab = rope_tab[wv];
    // an opaque copy of the lane index: the per-lane addresses below are
    // recomputed here instead of being hoisted out of the block loop, where
    // they would hold registers through the attention itself
    int ln = lane;
    asm volatile("" : "+v"(ln));
    for (int e = ln; e < TW * 32; e += 64) {
      const int tok = e >> 5, i = e & 31;
      if (i < hr) {
        if (exact) {
          tab[e] = rope_angle(p.q_offset + tw0 + tok, i);
        } else {
          const float2 c = tab[e], d = rope_step[i];
          tab[e] = make_float2(c.x * d.x - c.y * d.y, c.y * d.x + c.x * d.y);
        }
      }
    }
    wave_lds_sync();
    // lane ln takes pairs it = ln + 64 j (row m = it / hr, pair i = it % hr);
    // every read is issued before the first write so the wave waits for LDS once
    constexpr int kMaxPairs = 32 * 32 / 64;
    const float inv_hr = 1.0f / (float)hr;
    uint32_t uw[kMaxPairs];
    float2 cs[kMaxPairs];
    int at[kMaxPairs];
#pragma unroll
    for (int j = 0; j < kMaxPairs; ++j) {
      const int it = ln + 64 * j;
      if (it < 32 * hr) {
        const int m = (int)(((float)it + 0.5f) * inv_hr), i = it - m * hr;
        at[j] = Stg::off(m, i);
        uw[j] = (uint32_t)stg[at[j]] | ((uint32_t)stg[at[j] + hr] << 16);
        cs[j] = tab[(m / G) * 32 + i];
      }
    }
#pragma unroll
    for (int j = 0; j < kMaxPairs; ++j) {
      const int it = ln + 64 * j;
      if (it < 32 * hr) {
        const float u = __uint_as_float(uw[j] << 16), w = __uint_as_float(uw[j] & 0xffff0000u);
        stg[at[j]] = __builtin_bit_cast(uint16_t, (__bf16)(u * cs[j].x - w * cs[j].y));
        stg[at[j] + hr] = __builtin_bit_cast(uint16_t, (__bf16)(w * cs[j].x + u * cs[j].y));
      }
    }
    wave_lds_sync();
  };
  // whole rows -> LDS -> MFMA B-operand layout (row col, d = 16c + 8*half)
  auto stage_q = [&](int tw0, bool exact) {
#pragma unroll
    for (int hh = 0; hh < 2; ++hh) {
#pragma unroll
      for (int it = 0; it < SIT; ++it) {
        const int u = it * 64 + lane;
        *(u32x4*)&stg[Stg::off(u / HC, (u % HC) * 8)] = qpre[hh][it];
      }
      wave_lds_sync();
      if constexpr (ROPE) {
        if (hh == 0) rotate_staged(tw0, exact);
      }
      const lds_u16* sbase = lane_base(lds_addr(stg), Stg::k_lane_off(lane));
#pragma unroll
      for (int c = 0; c < Gm::NC / 2; ++c)
        st.q[hh * (Gm::NC / 2) + c] = Stg::k_operand(sbase, c);
      wave_lds_sync();
    }
  };
  // O = acc / l: MFMA layout -> LDS -> whole rows, half a head at a time
  auto store_o_rows = [&](int tw0) {
    const rsrc_t orsrc = rows_rsrc(p.o, tw0);
    const float lt = halves_sum(st.l_run);
    const float inv = 1.0f / lt;
#pragma unroll
    for (int hh = 0; hh < 2; ++hh) {
#pragma unroll
      for (int db2 = 0; db2 < Gm::ND / 2; ++db2) {
        const int db = hh * (Gm::ND / 2) + db2;
#pragma unroll
        for (int a4 = 0; a4 < 4; ++a4) {
          const f32x4 y = {st.acc[db][4 * a4] * inv, st.acc[db][4 * a4 + 1] * inv,
                           st.acc[db][4 * a4 + 2] * inv, st.acc[db][4 * a4 + 3] * inv};
          *(bf16x4*)&stg[Stg::off(col, 32 * db2 + 8 * a4 + 4 * half)] = __builtin_convertvector(y, bf16x4);
        }
      }
      wave_lds_sync();
#pragma unroll
      for (int it = 0; it < SIT; ++it) {
        const int u = it * 64 + lane;
        buf_store16<kStripOPolicy>(*(const u32x4*)&stg[Stg::off(u / HC, (u % HC) * 8)], orsrc, rows_voff(it, hh), 0);
      }
      wave_lds_sync();
    }
  };

  Stager<D, NT, kStripKvPolicy> sg;
  sg.init(kv_tok, tid);
  const float sink2 = p.sinks ? p.sinks[g * G + col % G] * kLog2e : kNegInf;
  // keys [key_lo, key_end) are the ones the strip's queries can see: tile
  // rows outside read as (or are set to) zeros
  const int key_lo = max(0, p.q_offset + blk0 * TB - W + 1);
  const int key_end = p.q_offset + min(blk1 * TB, p.Sq);

  // prologue: the first block's queries and its whole window
  load_q_rows(blk0 * TB + wv * TW);
  int loaded_hi = kt_hi(blk0);
  for (int kt = kt_lo(blk0); kt <= loaded_hi; ++kt) {
    sg.load(kg, vg, kv_tok, kt * KT, key_end, tid);
    sg.zero_below(key_lo - kt * KT, tid);
    sg.store(k_ring[kt % NR], v_ring[kt % NR], tid);
  }
  if constexpr (ROPE) {
    if (tid < p.rope_hr) rope_step[tid] = rope_angle(TB, tid);
  }
  stage_q(blk0 * TB + wv * TW, true);
  // Drain every prologue load here, so that inside the loop the only loads in
  // flight are the prefetches and no wait inserted for the current queries
  // can stall on them.
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();

  // The next block's (at most one) new K/V tile goes straight from memory
  // into its ring slot: a K + V tile pair is NPT 1 KiB windows, wave wv
  // filling windows wv, wv + NW, ... (per-lane offsets fixed per wave).  The
  // slot held tile new_kt - NR, older than this block's window and the last
  // block's (read before the last barrier).
  constexpr int WPW = (Dma::NPT + NW - 1) / NW;
  const uint32_t row_b = (uint32_t)(2 * kv_tok), pad_b = (uint32_t)(2 * (kv_tok - D));
  uint32_t dma_off[WPW];
#pragma unroll
  for (int k = 0; k < WPW; ++k) {
    const int rr = wv + NW * k;
    dma_off[k] = rr < Dma::NPT ? Dma::voff(rr < Dma::NK, rr < Dma::NK ? rr : rr - Dma::NK, lane, row_b) : 0u;
  }
  auto dma_tile = [&](int t) {
    const uint16_t* kfirst = kg + (long)t * KT * kv_tok;
    const uint16_t* vfirst = vg + (long)t * KT * kv_tok;
    const uint32_t nrec = (uint32_t)min(KT, key_end - t * KT) * row_b - pad_b;
#pragma unroll
    for (int k = 0; k < WPW; ++k) {
      const int rr = wv + NW * k;
      if (rr < Dma::NK)
        Dma::load(kfirst, nrec, lds_addr(k_ring[t % NR]) + 1024u * rr, dma_off[k]);
      else if (rr < Dma::NPT)
        Dma::load(vfirst, nrec, lds_addr(v_ring[t % NR]) + 1024u * (rr - Dma::NK), dma_off[k]);
    }
  };

  for (int blk = blk0; blk < blk1; ++blk) {
    const int tw0 = blk * TB + wv * TW;
    const bool nxt = blk + 1 < blk1;
    // prefetch: (at most one) new K/V tile, then the next block's queries.
    // The tile's loads are older than the query loads, and vmcnt retires in
    // order, so the wait for the queries before they are staged (at the
    // block's end, before the barrier) also covers the tile.
    const int new_kt = nxt ? kt_hi(blk + 1) : -1;
    const bool have_new = new_kt > loaded_hi;
    if (have_new) dma_tile(new_kt);
    if (nxt) load_q_rows(tw0 + TB);

    // compute this block from the ring; the second wave of each SIMD pair
    // at a raised priority while the tiles are folded (see the
    // one-workgroup-per-block kernel)
    if (wv >= NW / 2) __builtin_amdgcn_s_setprio(1);
    st.qpos = p.q_offset + tw0 + col / G;
    st.reset(sink2, half);
    const bool wave_active = tw0 < p.Sq;
    if (wave_active) {
      const int wpos_lo = p.q_offset + tw0;
      const int wpos_hi = p.q_offset + min(tw0 + TW, p.Sq) - 1;
      // this wave's tiles, all resident in the ring; the scores of tile
      // kt + 1 are computed while tile kt is exponentiated
      const int wk0 = max(0, wpos_lo - W + 1) / KT, wk1 = wpos_hi / KT;
      auto tile_mask = [&](int kt) {
        int mask;
        tile_needed(kt * KT, wpos_lo, wpos_hi, W, mask);
        return mask;
      };
      f32x16 s = st.scores(k_ring[wk0 % NR], lane);
      st.prep(s, wk0 * KT, tile_mask(wk0), W, p.scale_log2, half);
      // two folds per trip: the scores alternate between two register
      // sets, so none is copied back to close the loop
      int kt = wk0;
      for (; kt + 1 < wk1; kt += 2) {
        const f32x16 s1 = st.template fold_sum<true>(s, p.scale_log2, v_ring[kt % NR], k_ring[(kt + 1) % NR],
                                                     (kt + 1) * KT, tile_mask(kt + 1), W, half, lane);
        s = st.template fold_sum<true>(s1, p.scale_log2, v_ring[(kt + 1) % NR], k_ring[(kt + 2) % NR],
                                       (kt + 2) * KT, tile_mask(kt + 2), W, half, lane);
      }
      if (kt < wk1)
        s = st.template fold_sum<true>(s, p.scale_log2, v_ring[kt % NR], k_ring[(kt + 1) % NR], (kt + 1) * KT,
                                       tile_mask(kt + 1), W, half, lane);
      st.template fold_sum<false>(s, p.scale_log2, v_ring[wk1 % NR], nullptr, 0, 0, W, half, lane);
    }
    __builtin_amdgcn_s_setprio(0);
    if (have_new) loaded_hi = new_kt;
    // the next block's queries into their operand registers first (their
    // wait then covers only loads: no output store has been issued yet),
    // then this block's output, through the same staging tile
    if (nxt) stage_q(tw0 + TB, ((blk + 1 - blk0) & 7) == 0);
    if (wave_active) {
      store_o_rows(tw0);
      if constexpr (MODE == kStripLse) st.store_lse(p.lse + (long)b * p.Sq * p.Hq, p.Hq, tw0, G, g, p.Sq, col, half);
    }
    // When a new tile was loaded, the query loads came after it and were
    // waited for before staging, so the tile has landed in every wave's
    // share by this barrier.
    __syncthreads();
  }
}

// ----------------------------------------------------------------------------
template <int D, int G, int NW>
static hipError_t launch_generic(const PrefillArgs& a0, hipStream_t stream) {
  PrefillArgs a = a0;
  constexpr int TB = (32 / G) * NW;
  a.n_tb = (a.Sq + TB - 1) / TB;
  a.total = a.B * a.Hkv * a.n_tb;
  a.per_xcd = (a.total + 7) / 8;
  dim3 grid(8 * a.per_xcd), block(NW * 64);
  if (a.window == 0 && a.lse)
    hipLaunchKernelGGL((prefill_bf16_kernel<D, G, NW, true, true>), grid, block, 0, stream, a);
  else if (a.window == 0)
    hipLaunchKernelGGL((prefill_bf16_kernel<D, G, NW, true, false>), grid, block, 0, stream, a);
  else if (a.lse)
    hipLaunchKernelGGL((prefill_bf16_kernel<D, G, NW, false, true>), grid, block, 0, stream, a);
  else
    hipLaunchKernelGGL((prefill_bf16_kernel<D, G, NW, false, false>), grid, block, 0, stream, a);
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
  if (a.rope_hr > 0)
    hipLaunchKernelGGL((prefill_swa_strip_kernel<D, G, kStripRope>), dim3(a.total), dim3(G * 64), 0, stream, a);
  else if (a.lse)
    hipLaunchKernelGGL((prefill_swa_strip_kernel<D, G, kStripLse>), dim3(a.total), dim3(G * 64), 0, stream, a);
  else
    hipLaunchKernelGGL((prefill_swa_strip_kernel<D, G, kStripPlain>), dim3(a.total), dim3(G * 64), 0, stream, a);
  return hipGetLastError();
}

static int floor_div(int x, int y) { return x >= 0 ? x / y : -((-x + y - 1) / y); }

bool prefill_uses_strip(const PrefillArgs& a) {
  // The strip kernel's ring must hold a block's window plus the next block's
  // new tile.  Blocks start at positions p = q_offset (mod 32), and the keys
  // p - W + 1 .. p + 31 of a block span floor((a + 31) / 32) -
  // floor((a - W + 1) / 32) + 1 tiles with a = q_offset mod 32.
  const int G = a.Hq / a.Hkv;
  const int al = a.q_offset % KT;
  const int span = a.window > 0 ? (al + KT - 1) / KT - floor_div(al - a.window + 1, KT) + 1 : 0;
  const bool ring_fits = a.window > 0 && span + 1 <= kRingTiles;
  return ring_fits && (G == 8 || G == 4) && (a.D == 64 || a.D == 128);
}

template <int D>
static hipError_t launch_d(const PrefillArgs& a, int G, hipStream_t s) {
  if (prefill_uses_strip(a)) {
    int dev = 0, num_cu = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&num_cu, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        num_cu <= 0)
      num_cu = 256;
    return G == 8 ? launch_strip<D, 8>(a, num_cu, s) : launch_strip<D, 4>(a, num_cu, s);
  }
  switch (G) {
    case 1: return launch_generic<D, 1, 8>(a, s);
    case 2: return launch_generic<D, 2, 8>(a, s);
    case 4: return launch_generic<D, 4, 8>(a, s);
    case 8: return launch_generic<D, 8, 8>(a, s);
    case 16: return launch_generic<D, 16, 8>(a, s);
    case 32: return launch_generic<D, 32, 8>(a, s);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_prefill_bf16(const PrefillArgs& a, hipStream_t s) {
  const int G = a.Hq / a.Hkv;
  return a.D == 128 ? launch_d<128>(a, G, s) : launch_d<64>(a, G, s);
}

}  // namespace swa
