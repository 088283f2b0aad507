// bf16 multi-token verify (q_len = 1 committed + drafts) over a ring-buffer
// sliding-window cache or a linear global cache, on gfx950 MFMA.
//
// What it computes: each of the q_len tokens under verification is a query
// at position L_b + t; it attends to the committed keys inside its window and
// to the new tokens 0..t, with the per-head sink in the denominator.  The
// release blog (section "Multi-Token Prediction") verifies 1 + 3 drafts in
// one pass "without increasing KV-cache I/O": here every K/V row read from
// HBM serves all G * q_len query rows of its KV head (8 heads x 4 tokens =
// one 32-column MFMA block), so the cache is streamed exactly once.
//
// Work decomposition
//   * Workgroup = (split of the cache rows, KV head g, request b), or, for
//     the split launches of long caches, (split, pair of KV heads, request):
//     NW waves per head, the two heads' waves reading the two heads' rows
//     of each cache position side by side.  Split 0 also takes the tile of
//     q_len new rows.  Within a head, wave w takes tiles w, w + NW, ... (32
//     rows each) and keeps its own online-softmax state for the 32*NB query
//     rows; a head's waves are merged through LDS at the end, in a fixed
//     order (bitwise deterministic).
//   * Split workgroups run longest first: all full splits, then each
//     request's partial split by decreasing length, so the tail is short.
//   * K and V tiles are staged row-major in a per-wave LDS tile (coalesced
//     16-byte loads of whole rows); K is read back as the MFMA A operand of
//     S^T = K Q^T, V with ds_read_b64_tr_b16 as the A operand of
//     O^T += V^T P^T.  The next tile's loads are issued before the current
//     tile is computed; on a wave's first tile the scores are computed from
//     its K half while its V half is still arriving, and the wave that owns
//     the tile of new rows computes that tile first.
//   * Rows past the end of the valid cache range are clamped to the last
//     valid row and masked out, so unused cache slots are never read and may
//     hold anything, NaN included.
//   * With one split per (request, KV head) the workgroup folds the sink and
//     writes O directly; otherwise it writes (max, sum, unnormalised O) to the
//     workspace and verify_combine merges the splits, folding the sink once.
#include <type_traits>

#include "common.hpp"
#include "launch.hpp"

namespace swa {

namespace {

// Cache-row range [c0, c1) (as cache slot indices) of split `s`, and the
// number of splits, for request length L.
struct SplitRange {
  int clo, ncache, ns;
};

__device__ __forceinline__ SplitRange split_range(const VerifyArgs& p, int L) {
  SplitRange r;
  if (p.ring) {
    r.clo = 0;
    r.ncache = min(L, p.slots);
  } else {
    r.clo = p.window > 0 ? max(0, L - p.window + 1) : 0;
    r.ncache = L - r.clo;
  }
  r.ns = max(1, (r.ncache + p.split_len - 1) / p.split_len);
  return r;
}

// Longest-first order of the split workgroups: every full split (split_len
// rows) first, then the one partial split of each request by decreasing size,
// KV head innermost.  Workgroups start in linear-id order, so the short work
// runs last and the tail stays short.  Every wave derives the order from
// cache_len (requests b = lane + 64c); returns false when linear id i has no
// work.  Used for up to kLptMaxB requests.  nh: the KV-head items per
// (request, split), g the item's index among them.
constexpr int kLptMaxB = 256;

__device__ bool lpt_item(const VerifyArgs& p, int nh, int i, int lane, int& b, int& g, int& s) {
  constexpr int CH = kLptMaxB / 64;
  int nfull[CH], rem[CH];
#pragma unroll
  for (int c = 0; c < CH; ++c) {
    const int bb = c * 64 + lane;
    nfull[c] = 0;
    rem[c] = -1;  // -1: no partial split
    if (bb < p.B) {
      const SplitRange sr = split_range(p, p.cache_len[bb]);
      nfull[c] = sr.ncache / p.split_len;
      const int rm = sr.ncache - nfull[c] * p.split_len;
      if (rm > 0 || sr.ncache == 0) rem[c] = rm;
    }
  }
  // full splits, in request order
  int acc = 0;
#pragma unroll
  for (int c = 0; c < CH; ++c) {
    if (c * 64 >= p.B) break;
    for (int l = 0; l < 64 && c * 64 + l < p.B; ++l) {
      const int n = __builtin_amdgcn_readlane(nfull[c], l) * nh;
      if (i < acc + n) {
        b = c * 64 + l;
        s = (i - acc) / nh;
        g = (i - acc) % nh;
        return true;
      }
      acc += n;
    }
  }
  // partial splits: this lane's requests ranked by (size desc, index asc)
  const int j = i - acc;
  const int target = j / nh;
  g = j % nh;
#pragma unroll
  for (int c = 0; c < CH; ++c) {
    if (c * 64 >= p.B) break;
    int rank = 0;
#pragma unroll
    for (int c2 = 0; c2 < CH; ++c2) {
      if (c2 * 64 >= p.B) break;
      for (int l = 0; l < 64 && c2 * 64 + l < p.B; ++l) {
        const int r2 = __builtin_amdgcn_readlane(rem[c2], l);
        const int b2 = c2 * 64 + l;
        rank += (r2 > rem[c] || (r2 == rem[c] && b2 < c * 64 + lane)) ? 1 : 0;
      }
    }
    const uint64_t hit = __ballot(rem[c] >= 0 && rank == target);
    if (hit) {
      const int l = __builtin_ctzll(hit);
      b = c * 64 + l;
      s = __builtin_amdgcn_readlane(nfull[c], l);
      return true;
    }
  }
  return false;
}

}  // namespace

// HP KV heads per workgroup (1 or 2), NW waves per head: the waves of the
// heads of a pair read adjacent 256-byte rows of the same cache positions at
// the same time, which HBM serves at the contiguous-read rate (measured:
// 7.04-7.17 TB/s for two heads' waves in one workgroup against 6.67-6.70 for
// one head per workgroup, on the same 8 GiB).  Each head's waves fold and
// merge exactly as with one head per workgroup.
template <int D, int NB, int NW, bool DIRECT, int HP = 1>
__global__ __launch_bounds__(NW * HP * 64) __attribute__((amdgpu_waves_per_eu(NB == 1 ? 2 : 1, NB == 1 ? 2 : 1))) void verify_bf16_kernel(VerifyArgs p) {
  constexpr int NC = D / 16;
  constexpr int ND = D / 32;
  constexpr int CPR = D / 8;                   // 16-byte chunks per row
  constexpr int LD_IT = 32 * CPR / 64;         // 16-byte loads per lane per tile (K or V)
  constexpr int ACC_N = NB * ND * 16;          // accumulator floats per lane
  constexpr int NQ_W = (NB * ND + NW - 1) / NW;  // output blocks each wave finishes
  static_assert((NW & (NW - 1)) == 0, "the merge tree pairs waves");

  static_assert(HP == 1 || NB == 1, "head pairs with one 32-row block per head");
  struct MergeLds {
    float acc[NW * HP][ACC_N][64];
  };
  struct TileLds {
    uint16_t k[NW * HP][KTile<D>::ELEMS];
    uint16_t v[NW * HP][VTile<D>::ELEMS];
  };
  // 4 KiB accumulator blocks that fit in a wave's own K and V tiles
  constexpr int KBLK = (int)(sizeof(uint16_t) * KTile<D>::ELEMS / 4096);
  constexpr int VBLK = (int)(sizeof(uint16_t) * VTile<D>::ELEMS / 4096);
  constexpr bool OWN_MERGE = NB * ND <= KBLK + VBLK;
  constexpr size_t LDS_MAIN =
      OWN_MERGE || sizeof(TileLds) > sizeof(MergeLds) ? sizeof(TileLds) : sizeof(MergeLds);
  __shared__ __attribute__((aligned(16))) unsigned char lds_main[LDS_MAIN];
  __shared__ float lds_m[NW * HP][NB * 32];
  __shared__ float lds_l[NW * HP][NB * 32];

  // grid (B * Hkv / HP, nsplit): workgroups are dealt to the 8 XCDs
  // round-robin by linear id, so with (request, KV head or head pair) as the
  // fastest dimension every XCD gets the same mix of long and short
  // requests; splits past a request's length exit at once.
  const int lane = threadIdx.x & 63;
  const int wv_all = wave_index();
  const int hs = wv_all / NW;  // this wave's head within the workgroup's pair
  const int nh = p.Hkv / HP;   // head items per (request, split)
  int g, b, s;
  if (DIRECT || p.B > kLptMaxB) {
    g = blockIdx.x % nh;
    b = blockIdx.x / nh;
    s = blockIdx.y;
  } else if (!lpt_item(p, nh, blockIdx.x + blockIdx.y * gridDim.x, lane, b, g, s)) {
    return;
  }
  g = g * HP + hs;
  const int L = p.cache_len[b];
  const SplitRange sr = split_range(p, L);
  if (s >= sr.ns) return;
  const int c0 = sr.clo + s * p.split_len;
  const int c1 = sr.clo + min((s + 1) * p.split_len, sr.ncache);
  const int ntc = (c1 - c0 + 31) / 32;          // cache tiles of this split
  const int ntiles = ntc + (s == 0 ? 1 : 0);    // + the tile of new rows

  const int G = p.Hq / p.Hkv;
  const int R = G * p.T;
  const int wv = wv_all - hs * NW;  // wave index among this head's NW
  const int half = lane >> 5, col = lane & 31;
  const long kv_tok = (long)p.Hkv * D;
  // ring: slot of the oldest committed position held, to map slot -> position
  const int ring_n = min(L, p.slots);
  const int ring_base_slot = p.ring ? (L - ring_n) % p.slots : 0;

  // ---- queries: row m = t * G + hh  ->  token t, head g*G + hh
  bf16x8 qreg[NB][NC];
  int qt[NB];
  float m_run[NB], l_run[NB];
  f32x16 acc[NB][ND];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
    const int m = nb * 32 + col;
    qt[nb] = -1;
#pragma unroll
    for (int c = 0; c < NC; ++c) qreg[nb][c] = bf16x8{};
    if (m < R) {
      const int t = m / G, h = g * G + m % G;
      qt[nb] = t;
      const uint16_t* qp = p.q + (((long)b * p.T + t) * p.Hq + h) * D + half * 8;
#pragma unroll
      for (int c = 0; c < NC; ++c) qreg[nb][c] = *(const bf16x8*)(qp + c * 16);
    }
    m_run[nb] = kNegInf;
    l_run[nb] = 0.0f;
#pragma unroll
    for (int db = 0; db < ND; ++db) acc[nb][db] = f32x16{};
  }

  uint16_t* k_t = ((TileLds*)lds_main)->k[wv_all];
  uint16_t* v_t = ((TileLds*)lds_main)->v[wv_all];
  const long bg_off = ((long)b * p.slots * p.Hkv + g) * D;
  const long bg_new = ((long)b * p.T * p.Hkv + g) * D;

  // Element offset (from the cache or new-row base) of row r (0..31) of tile
  // j.  Rows past the valid range are clamped to the last valid row: they are
  // masked out of the softmax and their (finite, committed) values get weight
  // exactly 0, so unused cache slots are never read and no zero-fill is needed.
  auto row_off = [&](int j, int r) -> long {
    if (s == 0 && j == ntc) return bg_new + (long)min(r, p.T - 1) * kv_tok;
    return bg_off + (long)min(c0 + j * 32 + r, c1 - 1) * kv_tok;
  };

  // Tile staging: load i of a lane covers row 4i + lane/16 (D = 128), chunk
  // lane%16: every load instruction reads whole 256-byte rows.
  u32x4 kpre[LD_IT], vpre[LD_IT];
  auto load_tile = [&](int j) {
    const bool nw = (s == 0 && j == ntc);
    const uint16_t* kb = nw ? p.k_new : p.k_cache;
    const uint16_t* vb = nw ? p.v_new : p.v_cache;
    // every cache row is read once: non-temporal, so the stream does not
    // displace reused data in the L2 and the Infinity Cache (measured:
    // 5.6 -> 6.1 TB/s on the 64-request global cache).  All K loads are
    // issued before the V loads, so that the K half can be stored (and its
    // scores computed) while V is still arriving.
#pragma unroll
    for (int i = 0; i < LD_IT; ++i) {
      const int c = lane + 64 * i;
      kpre[i] = __builtin_nontemporal_load((const u32x4*)(kb + row_off(j, c / CPR) + (c % CPR) * 8));
    }
#pragma unroll
    for (int i = 0; i < LD_IT; ++i) {
      const int c = lane + 64 * i;
      vpre[i] = __builtin_nontemporal_load((const u32x4*)(vb + row_off(j, c / CPR) + (c % CPR) * 8));
    }
  };
  auto store_k = [&]() {
#pragma unroll
    for (int i = 0; i < LD_IT; ++i) {
      const int c = lane + 64 * i;
      *(u32x4*)&k_t[KTile<D>::off(c / CPR, (c % CPR) * 8)] = kpre[i];
    }
  };
  auto store_v = [&]() {
#pragma unroll
    for (int i = 0; i < LD_IT; ++i) {
      const int c = lane + 64 * i;
      *(u32x4*)&v_t[VTile<D>::off(c / CPR, (c % CPR) * 8)] = vpre[i];
    }
  };

  // The tile of new rows (split 0's last) holds only T distinct rows.  The
  // wave that owns it computes it first: its T rows (LDN loads per lane) are
  // issued in the prologue ahead of the wave's first cache tile, and the
  // wave waits only for them, so the new tile is computed while the cache
  // tile is still arriving instead of after it.  Rows T..31 of that LDS tile
  // are zeros (masked; zero V rows keep P V finite).  With more than
  // 64 * LDN / CPR new rows the tile is an ordinary last tile instead.
  constexpr int LDN = 2;                       // 16-byte loads per lane for T rows
  const bool new_first = s == 0 && ntc % NW == wv && p.T * CPR <= 64 * LDN;
  // this wave's tiles: wv, wv + NW, ... (the new tile, when it has it, first)
  const int nt_w = wv < ntiles ? (ntiles - 1 - wv) / NW + 1 : 0;
  auto tile_of = [&](int i) { return new_first ? (i == 0 ? ntc : wv + (i - 1) * NW) : wv + i * NW; };
  u32x4 nk[LDN], nv[LDN];
  auto load_new = [&]() {
#pragma unroll
    for (int i = 0; i < LDN; ++i) {
      const int c = lane + 64 * i;
      const long o = bg_new + (long)min(c / CPR, p.T - 1) * kv_tok + (c % CPR) * 8;
      nk[i] = __builtin_nontemporal_load((const u32x4*)(p.k_new + o));
      nv[i] = __builtin_nontemporal_load((const u32x4*)(p.v_new + o));
    }
  };
  auto store_new = [&](bool is_v) {
    const u32x4 zero = {0u, 0u, 0u, 0u};
#pragma unroll
    for (int i = 0; i < LD_IT; ++i) {
      const int c = lane + 64 * i;
      const bool have = i < LDN && c < p.T * CPR;
      if (is_v)
        *(u32x4*)&v_t[VTile<D>::off(c / CPR, (c % CPR) * 8)] = have ? nv[i < LDN ? i : 0] : zero;
      else
        *(u32x4*)&k_t[KTile<D>::off(c / CPR, (c % CPR) * 8)] = have ? nk[i < LDN ? i : 0] : zero;
    }
  };

  // Prologue: the first tile's K into LDS, its V stored after its scores
  // (the V half of its loads has the scores' time to arrive) and only then
  // the next tile's loads issued, since they reuse the registers; with the
  // new tile first, its K and V, the next (cache) tile's loads staying in
  // flight behind it.  From the second tile on, the next tile's loads are
  // issued at the top of each step and its K and V stored at the end.
  if (new_first) {
    load_new();
    // The next tile's loads, or, when the wave has no cache tile, the new
    // tile's own rows again (never used): one path, so the compiler's waits
    // for the T new rows leave these loads in flight.
    load_tile(nt_w > 1 ? tile_of(1) : ntc);
    store_new(false);
    store_new(true);
  } else if (nt_w > 0) {
    load_tile(tile_of(0));
    store_k();
  }
  // One step per tile; the first is a copy of its own (FIRST), so that the
  // two schedules do not share one loop body's registers.
  auto step = [&](auto first_c, int i) {
    constexpr bool FIRST = decltype(first_c)::value;
    const int j = tile_of(i);
    const bool more = i + 1 < nt_w;
    if (!FIRST && more) load_tile(tile_of(i + 1));
    wave_lds_sync();

    f32x16 sc[NB];
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) sc[nb] = f32x16{};
    const lds_u16* kbase = lane_base(lds_addr(k_t), KTile<D>::k_lane_off(lane));
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      const bf16x8 a = KTile<D>::k_operand(kbase, c);
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) sc[nb] = mfma32(a, qreg[nb][c], sc[nb]);
    }
    if (FIRST && !new_first) {
      store_v();
      if (more) load_tile(tile_of(1));
    }
    // Which rows of the tile a query sees, as two range tests per element
    // with per-tile and per-lane bounds (no per-element branches): row r is
    // visible iff a = a0 + r < a_hi and b = b0 + r (taken into [0, slots) by
    // adding slots when negative) > b_lo.
    //   new tile:  r < min(T, t + 1) (token r at position L + r, tokens 0..t
    //              visible) and r > t - window;
    //   cache:     slot ci = c0 + 32 j + r < c1, and its position above
    //              L + t - window: position ci in a linear cache, L - ring_n
    //              + e with e = (ci - ring_base_slot) mod slots in a ring.
    const bool is_new_tile = (s == 0 && j == ntc);
    const int cb = c0 + j * 32;
    const int a0 = is_new_tile ? 0 : cb;
    const int b0 = is_new_tile ? 0 : (p.ring ? cb - ring_base_slot : cb);
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      const int t = qt[nb];
      int a_hi = is_new_tile ? min(p.T, t + 1) : c1;
      a_hi = t < 0 ? INT32_MIN : a_hi;  // padding rows see nothing
      const int b_lo = p.window <= 0 ? -1 : (is_new_tile ? 0 : (p.ring ? ring_n : L)) + t - p.window;
      float mx = kNegInf;
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int r = c_row(v, half);
        int b = b0 + r;
        b += b < 0 ? p.slots : 0;
        const bool ok = (a0 + r < a_hi) & (b > b_lo);
        const float x = ok ? sc[nb][v] * p.scale_log2 : kNegInf;
        sc[nb][v] = x;
        mx = fmaxf(mx, x);
      }
      mx = halves_max(mx);
      const float m_new = fmaxf(m_run[nb], mx);
      const bool need = m_new > m_run[nb] + kRescaleTau;
      // A wave's first tile finds its accumulators and sum still zero: only
      // the max moves.  Later, the rescale is a real branch (the empty asm
      // keeps the compiler from turning it into unconditional multiplies),
      // taken only when some row's max has grown past the threshold.
      if (!FIRST && wave_any(need)) {
        __asm__ volatile("");
        const float alpha = need ? exp2_fast(m_run[nb] - m_new) : 1.0f;
        l_run[nb] *= alpha;
#pragma unroll
        for (int db = 0; db < ND; ++db) acc[nb][db] *= alpha;
      }
      m_run[nb] = need ? m_new : m_run[nb];
      const float mu = m_run[nb] == kNegInf ? 0.0f : m_run[nb];
      uint32_t pw[8];
#pragma unroll
      for (int j = 0; j < 8; ++j)
        pw[j] = pack_sum<true>(exp2_fast(sc[nb][2 * j] - mu), exp2_fast(sc[nb][2 * j + 1] - mu), l_run[nb]);
      const bf16x8 pb[2] = {__builtin_bit_cast(bf16x8, u32x4{pw[0], pw[1], pw[2], pw[3]}),
                            __builtin_bit_cast(bf16x8, u32x4{pw[4], pw[5], pw[6], pw[7]})};
      if (FIRST) wave_lds_sync();  // this step stored the V half
      const lds_u16* vbase = lane_base(lds_addr(v_t), VTile<D>::vt_lane_off(lane));
#pragma unroll
      for (int kc = 0; kc < 2; ++kc) {
#pragma unroll
        for (int db = 0; db < ND; ++db)
          acc[nb][db] = mfma32(VTile<D>::vt_operand(vbase, db, kc), pb[kc], acc[nb][db]);
      }
    }
    wave_lds_sync();
    if (more) {
      store_k();
      store_v();
    }
  };
  if (nt_w > 0) step(std::true_type{}, 0);
  for (int i = 1; i < nt_w; ++i) step(std::false_type{}, i);

  // ---- merge the waves.  Each wave leaves its running max and sum per query
  // row in lds_m / lds_l and its unscaled accumulators in LDS; after one
  // barrier, wave w finishes output blocks q = w, w + NW, ... (q = nb * ND +
  // db): the common max M of the row over the waves, l = sum_w l_w 2^(m_w -
  // M), and the sum over the waves of acc_w 2^(m_w - M) in a fixed pairwise
  // order ((w0 + w2) + (w1 + w3) for four waves: bitwise deterministic).
  // When a wave's accumulators fit in its own K/V tile (NB = 1) they go
  // there as soon as the wave is done with its tiles; otherwise into a merge
  // area over all the tiles, behind a barrier.  A block is 16 floats per
  // lane, stored as 4 x 64 lane-contiguous 16-byte entries.
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
    const float lt = halves_sum(l_run[nb]);
    if (half == 0) {
      lds_m[wv_all][nb * 32 + col] = m_run[nb];
      lds_l[wv_all][nb * 32 + col] = lt;
    }
  }
  TileLds* tl = (TileLds*)lds_main;
  MergeLds* ml = (MergeLds*)lds_main;
  // (w: a wave of this head)
  auto blk_ptr = [&](int w, int q) -> f32x4* {
    const int wa = hs * NW + w;
    if constexpr (OWN_MERGE) {
      return q < KBLK ? (f32x4*)tl->k[wa] + q * 256 : (f32x4*)tl->v[wa] + (q - KBLK) * 256;
    } else {
      return (f32x4*)&ml->acc[wa][q * 16][0];
    }
  };
  if constexpr (!OWN_MERGE) __syncthreads();  // every wave is done with its tiles
#pragma unroll
  for (int nb = 0; nb < NB; ++nb)
#pragma unroll
    for (int db = 0; db < ND; ++db) {
      f32x4* bp = blk_ptr(wv, nb * ND + db);
#pragma unroll
      for (int v4 = 0; v4 < 4; ++v4)
        bp[v4 * 64 + lane] = f32x4{acc[nb][db][4 * v4], acc[nb][db][4 * v4 + 1], acc[nb][db][4 * v4 + 2],
                                   acc[nb][db][4 * v4 + 3]};
    }
  __syncthreads();
#pragma unroll
  for (int qi = 0; qi < NQ_W; ++qi) {
    const int q = wv + qi * NW;
    if (q >= NB * ND) break;
    const int nb = q / ND, db = q % ND;
    float mw[NW], fw[NW];
    float mA = kNegInf;
#pragma unroll
    for (int w = 0; w < NW; ++w) {
      mw[w] = lds_m[hs * NW + w][nb * 32 + col];
      mA = fmaxf(mA, mw[w]);
    }
    float lA = 0.0f;
#pragma unroll
    for (int w = 0; w < NW; ++w) {
      fw[w] = mw[w] == kNegInf ? 0.0f : exp2_fast(mw[w] - mA);
      lA += mw[w] == kNegInf ? 0.0f : lds_l[hs * NW + w][nb * 32 + col] * fw[w];
    }
    f32x16 y;
#pragma unroll
    for (int v4 = 0; v4 < 4; ++v4) {
      f32x4 x[NW];
#pragma unroll
      for (int w = 0; w < NW; ++w) x[w] = blk_ptr(w, q)[v4 * 64 + lane] * fw[w];
#pragma unroll
      for (int r = NW / 2; r >= 1; r /= 2)
#pragma unroll
        for (int w = 0; w < r; ++w) x[w] += x[w + r];
#pragma unroll
      for (int e = 0; e < 4; ++e) y[4 * v4 + e] = x[0][e];
    }
    const int m = nb * 32 + col;
    if (DIRECT) {
      if (m >= R) continue;
      const int t = m / G, h = g * G + m % G;
      const float sink2 = p.sinks ? p.sinks[h] * kLog2e : kNegInf;
      const float M = fmaxf(mA, sink2);
      const float f = mA == kNegInf ? 0.0f : exp2_fast(mA - M);
      const float denom = lA * f + (sink2 == kNegInf ? 0.0f : exp2_fast(sink2 - M));
      const float scale = f / denom;
      uint16_t* op = p.o + (((long)b * p.T + t) * p.Hq + h) * D + db * 32 + 4 * half;
#pragma unroll
      for (int a4 = 0; a4 < 4; ++a4) {
        const f32x4 z = {y[4 * a4] * scale, y[4 * a4 + 1] * scale, y[4 * a4 + 2] * scale, y[4 * a4 + 3] * scale};
        *(bf16x4*)(op + 8 * a4) = __builtin_convertvector(z, bf16x4);
      }
    } else {
      const long prow = (((long)b * p.Hkv + g) * p.nsplit + s) * p.r_pad + m;
      float* op = p.ws_o + prow * D + db * 32 + 4 * half;
#pragma unroll
      for (int a4 = 0; a4 < 4; ++a4)
        *(f32x4*)(op + 8 * a4) = f32x4{y[4 * a4], y[4 * a4 + 1], y[4 * a4 + 2], y[4 * a4 + 3]};
      if (db == 0 && half == 0) {
        p.ws_ml[prow * 2] = mA;
        p.ws_ml[prow * 2 + 1] = lA;
      }
    }
  }
}

// Merge the splits of one (request, KV head): M = max(max_s m_s, sink),
// l = sum_s l_s 2^(m_s - M) + 2^(sink - M), O = sum_s O_s 2^(m_s - M) / l.
// Grid (B * Hkv, row groups): one thread per (row, 4 columns).  The splits
// are taken kCombineBatch at a time with every load of a batch issued before
// its first use (splits past the request's count alias its last split and get
// weight zero), the running state rescaled between batches, so the kernel
// waits on memory once per batch.
constexpr int kCombineBatch = 8;

template <int D>
__global__ __launch_bounds__(256) void verify_combine_kernel(VerifyArgs p) {
  const int g = blockIdx.x % p.Hkv, b = blockIdx.x / p.Hkv;
  const int G = p.Hq / p.Hkv;
  const int R = G * p.T;
  constexpr int TPR = D / 4;            // threads per row (4 floats each)
  constexpr int RPP = 256 / TPR;        // rows per workgroup
  const int tid = threadIdx.x;
  const int m = blockIdx.y * RPP + tid / TPR;
  if (m >= R) return;
  const int d = (tid % TPR) * 4;
  const int L = p.cache_len[b];
  const int ns = split_range(p, L).ns;
  const int t = m / G, h = g * G + m % G;
  const long base = ((long)b * p.Hkv + g) * p.nsplit * p.r_pad + m;
  const float sink2 = p.sinks ? p.sinks[h] * kLog2e : kNegInf;
  float M = kNegInf, l = 0.0f;
  f32x4 o = {0.0f, 0.0f, 0.0f, 0.0f};
  for (int s0 = 0; s0 < ns; s0 += kCombineBatch) {
    float ms[kCombineBatch], ls[kCombineBatch];
    f32x4 xs[kCombineBatch];
#pragma unroll
    for (int i = 0; i < kCombineBatch; ++i) {
      const long row = base + (long)min(s0 + i, ns - 1) * p.r_pad;
      const float2 ml = *(const float2*)(p.ws_ml + row * 2);
      ms[i] = s0 + i < ns ? ml.x : kNegInf;
      ls[i] = ml.y;
      xs[i] = *(const f32x4*)(p.ws_o + row * D + d);
    }
    float Mb = M;
#pragma unroll
    for (int i = 0; i < kCombineBatch; ++i) Mb = fmaxf(Mb, ms[i]);
    if (Mb == kNegInf) continue;
    const float fo = M == kNegInf ? 0.0f : exp2_fast(M - Mb);
    l *= fo;
    o *= fo;
#pragma unroll
    for (int i = 0; i < kCombineBatch; ++i) {
      const float f = ms[i] == kNegInf ? 0.0f : exp2_fast(ms[i] - Mb);
      l += ls[i] * f;
      o += xs[i] * f;
    }
    M = Mb;
  }
  if (sink2 != kNegInf) {
    const float Mt = fmaxf(M, sink2);
    const float fo = M == kNegInf ? 0.0f : exp2_fast(M - Mt);
    l = l * fo + exp2_fast(sink2 - Mt);
    o *= fo;
  }
  o *= 1.0f / l;
  uint16_t* op = p.o + (((long)b * p.T + t) * p.Hq + h) * D + d;
  *(bf16x4*)op = __builtin_convertvector(o, bf16x4);
}

VerifyPlan plan_verify_bf16(int B, int T, int Hq, int Hkv, int D, int slots, int ring, int window) {
  VerifyPlan pl;
  const int G = Hq / Hkv;
  const int R = G * T;
  pl.nb = R <= 32 ? 1 : 2;
  pl.waves = pl.nb == 1 ? 4 : 2;
  // split launches pair the KV heads (two per workgroup) when they can
  const int head_items = pl.nb == 1 && Hkv % 2 == 0 ? Hkv / 2 : Hkv;
  const int unit = 32 * pl.waves;
  // most cache rows one request can need
  long max_rows = slots;
  if (!ring && window > 0 && window - 1 < max_rows) max_rows = window - 1;
  if (max_rows < 1) max_rows = 1;
  // aim for about 256 workgroups (one per CU) or more, splits of at most
  // 16384 rows.  Measured with longest-first order: the 64-request
  // global-cache verify is best at 16384 rows (fewer workgroups and
  // partials, the short partial splits close the tail); one request at
  // 262144 rows takes 0.18 ms with 8192-row splits (264 workgroups) against
  // 0.21 ms with 2048 (1032) and 0.24 ms with 1024.
  long want = max_rows * (long)B * head_items / 256;
  long sl = unit;
  while (sl < want && sl < 16384) sl *= 2;
  if (sl < unit) sl = unit;
  sl = (sl + unit - 1) / unit * unit;
  pl.split_len = (int)sl;
  pl.nsplit = (int)((max_rows + sl - 1) / sl);
  if (pl.nsplit < 1) pl.nsplit = 1;
  const long r_pad = 32L * pl.nb;
  pl.ws_bytes = pl.nsplit == 1 ? 0
                               : (size_t)B * Hkv * pl.nsplit * r_pad * (size_t)(D + 2) * sizeof(float);
  return pl;
}

template <int D, int NB, int NW, int HP>
static hipError_t launch_verify_t(VerifyArgs a, const VerifyPlan& pl, hipStream_t s) {
  dim3 grid(a.B * a.Hkv / HP, pl.nsplit), block(NW * HP * 64);
  if (pl.nsplit == 1) {
    hipLaunchKernelGGL((verify_bf16_kernel<D, NB, NW, true, HP>), grid, block, 0, s, a);
    return hipGetLastError();
  }
  hipLaunchKernelGGL((verify_bf16_kernel<D, NB, NW, false, HP>), grid, block, 0, s, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  constexpr int RPP = 256 / (D / 4);
  const int R = (a.Hq / a.Hkv) * a.T;
  hipLaunchKernelGGL((verify_combine_kernel<D>), dim3(a.B * a.Hkv, (R + RPP - 1) / RPP), dim3(256), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_verify_bf16(const VerifyArgs& a0, const VerifyPlan& pl, hipStream_t s) {
  VerifyArgs a = a0;
  a.split_len = pl.split_len;
  a.nsplit = pl.nsplit;
  a.r_pad = 32 * pl.nb;
  // head pairs for the split (long-cache) launches, which stream from HBM,
  // when one 32-row block serves a head and the heads pair up; a one-split
  // launch (the SWA ring, short contexts) is bound by its latency, and after
  // an Infinity-Cache flush the 64-request ring verify measured 16.5 us with
  // one head per workgroup against 19.7 us with pairs
  const bool pairs = pl.nb == 1 && a.Hkv % 2 == 0 && pl.nsplit > 1;
  if (a.D == 128) {
    if (pl.nb == 1) return pairs ? launch_verify_t<128, 1, 4, 2>(a, pl, s) : launch_verify_t<128, 1, 4, 1>(a, pl, s);
    return launch_verify_t<128, 2, 2, 1>(a, pl, s);
  }
  if (pl.nb == 1) return pairs ? launch_verify_t<64, 1, 4, 2>(a, pl, s) : launch_verify_t<64, 1, 4, 1>(a, pl, s);
  return launch_verify_t<64, 2, 2, 1>(a, pl, s);
}

}  // namespace swa
