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
//   * Workgroup = (split of the cache rows, KV head g, request b).  Split 0
//     also takes the tile of q_len new rows.  Within a workgroup, wave w takes
//     tiles w, w + NW, ... (32 rows each) and keeps its own online-softmax
//     state for the 32*NB query rows; the waves are merged through LDS at
//     the end, in a fixed order (bitwise deterministic).
//   * Split workgroups run longest first: all full splits, then each
//     request's partial split by decreasing length, so the tail is short.
//   * K and V tiles are staged row-major in a per-wave LDS tile (coalesced
//     16-byte loads of whole rows); K is read back as the MFMA A operand of
//     S^T = K Q^T, V with ds_read_b64_tr_b16 as the A operand of
//     O^T += V^T P^T.  The next tile's loads are issued before the current
//     tile is computed.
//   * Rows past the end of the valid cache range are clamped to the last
//     valid row and masked out, so unused cache slots are never read and may
//     hold anything, NaN included.
//   * With one split per (request, KV head) the workgroup folds the sink and
//     writes O directly; otherwise it writes (max, sum, unnormalised O) to the
//     workspace and verify_combine merges the splits, folding the sink once.
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
// work.  Used for up to kLptMaxB requests.
constexpr int kLptMaxB = 256;

__device__ bool lpt_item(const VerifyArgs& p, int i, int lane, int& b, int& g, int& s) {
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
      const int n = __builtin_amdgcn_readlane(nfull[c], l) * p.Hkv;
      if (i < acc + n) {
        b = c * 64 + l;
        s = (i - acc) / p.Hkv;
        g = (i - acc) % p.Hkv;
        return true;
      }
      acc += n;
    }
  }
  // partial splits: this lane's requests ranked by (size desc, index asc)
  const int j = i - acc;
  const int target = j / p.Hkv;
  g = j % p.Hkv;
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

template <int D, int NB, int NW, bool DIRECT>
__global__ __launch_bounds__(NW * 64) __attribute__((amdgpu_waves_per_eu(NB == 1 ? 2 : 1, NB == 1 ? 2 : 1))) void verify_bf16_kernel(VerifyArgs p) {
  constexpr int NC = D / 16;
  constexpr int ND = D / 32;
  constexpr int CPR = D / 8;                   // 16-byte chunks per row
  constexpr int LD_IT = 32 * CPR / 64;         // 16-byte loads per lane per tile (K or V)
  constexpr int ACC_N = NB * ND * 16;          // accumulator floats per lane
  constexpr int MERGE_SLOTS = NW / 2 > 0 ? NW / 2 : 1;

  struct MergeLds {
    float acc[MERGE_SLOTS][ACC_N][64];
  };
  struct TileLds {
    uint16_t k[NW][KTile<D>::ELEMS];
    uint16_t v[NW][VTile<D>::ELEMS];
  };
  constexpr size_t LDS_MAIN = sizeof(MergeLds) > sizeof(TileLds) ? sizeof(MergeLds) : sizeof(TileLds);
  __shared__ __attribute__((aligned(16))) unsigned char lds_main[LDS_MAIN];
  __shared__ float lds_m[NW][NB * 32];
  __shared__ float lds_l[NW][NB * 32];

  // grid (B * Hkv, nsplit): workgroups are dealt to the 8 XCDs round-robin by
  // linear id, so with (request, KV head) as the fastest dimension every XCD
  // gets the same mix of long and short requests (with 8 KV heads, XCD = KV
  // head); splits past a request's length exit at once.
  const int lane = threadIdx.x & 63;
  int g, b, s;
  if (DIRECT || p.B > kLptMaxB) {
    g = blockIdx.x % p.Hkv;
    b = blockIdx.x / p.Hkv;
    s = blockIdx.y;
  } else if (!lpt_item(p, blockIdx.x + blockIdx.y * gridDim.x, lane, b, g, s)) {
    return;
  }
  const int L = p.cache_len[b];
  const SplitRange sr = split_range(p, L);
  if (s >= sr.ns) return;
  const int c0 = sr.clo + s * p.split_len;
  const int c1 = sr.clo + min((s + 1) * p.split_len, sr.ncache);
  const int ntc = (c1 - c0 + 31) / 32;          // cache tiles of this split
  const int ntiles = ntc + (s == 0 ? 1 : 0);    // + the tile of new rows

  const int G = p.Hq / p.Hkv;
  const int R = G * p.T;
  const int tid = threadIdx.x, wv = wave_index();
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

  uint16_t* k_t = ((TileLds*)lds_main)->k[wv];
  uint16_t* v_t = ((TileLds*)lds_main)->v[wv];
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
#pragma unroll
    for (int i = 0; i < LD_IT; ++i) {
      const int c = lane + 64 * i;
      const long o = row_off(j, c / CPR) + (c % CPR) * 8;
      // every cache row is read once: non-temporal, so the stream does not
      // displace reused data in the L2 and the Infinity Cache (measured:
      // 5.6 -> 6.1 TB/s on the 64-request global cache)
      kpre[i] = __builtin_nontemporal_load((const u32x4*)(kb + o));
      vpre[i] = __builtin_nontemporal_load((const u32x4*)(vb + o));
    }
  };
  auto store_tile = [&]() {
#pragma unroll
    for (int i = 0; i < LD_IT; ++i) {
      const int c = lane + 64 * i;
      *(u32x4*)&k_t[KTile<D>::off(c / CPR, (c % CPR) * 8)] = kpre[i];
      *(u32x4*)&v_t[VTile<D>::off(c / CPR, (c % CPR) * 8)] = vpre[i];
    }
  };

  if (wv < ntiles) {
    load_tile(wv);
    store_tile();
  }
  // Drain the prologue loads (queries, first tile) so that inside the loop
  // the only loads in flight are the prefetch of the next tile and nothing
  // waits on it before the current tile is computed.
  __builtin_amdgcn_s_waitcnt(0);
  for (int j = wv; j < ntiles; j += NW) {
    const bool more = j + NW < ntiles;
    if (more) load_tile(j + NW);
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
    const bool is_new_tile = (s == 0 && j == ntc);
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      const int t = qt[nb];
      float mx = kNegInf;
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int r = c_row(v, half);
        bool ok;
        if (is_new_tile) {
          // new token u at position L + u, visible to query t iff u <= t and in window
          ok = t >= 0 && r < p.T && r <= t && (p.window <= 0 || r > t - p.window);
        } else {
          const int ci = c0 + j * 32 + r;
          int pos = ci;
          if (p.ring) {
            const int d = ci - ring_base_slot;
            pos = L - ring_n + (d >= 0 ? d : d + p.slots);
          }
          ok = t >= 0 && ci < c1 && (p.window <= 0 || pos > L + t - p.window);
        }
        const float x = ok ? sc[nb][v] * p.scale_log2 : kNegInf;
        sc[nb][v] = x;
        mx = fmaxf(mx, x);
      }
      mx = halves_max(mx);
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
#pragma unroll
      for (int v = 0; v < 16; ++v) pb[v >> 3][v & 7] = (__bf16)exp2_fast(sc[nb][v] - mu);
      l_run[nb] = sum_bf16x16(pb[0], pb[1], l_run[nb]);
      const lds_u16* vbase = lane_base(lds_addr(v_t), VTile<D>::vt_lane_off(lane));
#pragma unroll
      for (int kc = 0; kc < 2; ++kc) {
#pragma unroll
        for (int db = 0; db < ND; ++db)
          acc[nb][db] = mfma32(VTile<D>::vt_operand(vbase, db, kc), pb[kc], acc[nb][db]);
      }
    }
    wave_lds_sync();
    if (more) store_tile();
  }

  // ---- merge the waves: common max, then a fixed-order pairwise sum in LDS
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
    const float lt = halves_sum(l_run[nb]);
    if (half == 0) {
      lds_m[wv][nb * 32 + col] = m_run[nb];
      lds_l[wv][nb * 32 + col] = lt;
    }
  }
  __syncthreads();
  float m_all[NB], l_all[NB];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
    float mm = kNegInf;
#pragma unroll
    for (int w = 0; w < NW; ++w) mm = fmaxf(mm, lds_m[w][nb * 32 + col]);
    float ll = 0.0f;
#pragma unroll
    for (int w = 0; w < NW; ++w) {
      const float mw = lds_m[w][nb * 32 + col];
      ll += mw == kNegInf ? 0.0f : lds_l[w][nb * 32 + col] * exp2_fast(mw - mm);
    }
    m_all[nb] = mm;
    l_all[nb] = ll;
    const float f = m_run[nb] == kNegInf ? 0.0f : exp2_fast(m_run[nb] - mm);
#pragma unroll
    for (int db = 0; db < ND; ++db) acc[nb][db] *= f;
  }
  MergeLds* ml = (MergeLds*)lds_main;
#pragma unroll
  for (int r = NW / 2; r >= 1; r /= 2) {
    if (wv >= r && wv < 2 * r) {
#pragma unroll
      for (int nb = 0; nb < NB; ++nb)
#pragma unroll
        for (int db = 0; db < ND; ++db)
#pragma unroll
          for (int v = 0; v < 16; ++v) ml->acc[wv - r][(nb * ND + db) * 16 + v][lane] = acc[nb][db][v];
    }
    __syncthreads();
    if (wv < r) {
#pragma unroll
      for (int nb = 0; nb < NB; ++nb)
#pragma unroll
        for (int db = 0; db < ND; ++db)
#pragma unroll
          for (int v = 0; v < 16; ++v) acc[nb][db][v] += ml->acc[wv][(nb * ND + db) * 16 + v][lane];
    }
    __syncthreads();
  }
  if (wv != 0) return;

  // ---- wave 0 writes the result of this split
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
    const int m = nb * 32 + col;
    if (DIRECT) {
      if (m >= R) continue;
      const int t = m / G, h = g * G + m % G;
      const float sink2 = p.sinks ? p.sinks[h] * kLog2e : kNegInf;
      const float M = fmaxf(m_all[nb], sink2);
      const float f = m_all[nb] == kNegInf ? 0.0f : exp2_fast(m_all[nb] - M);
      const float denom = l_all[nb] * f + (sink2 == kNegInf ? 0.0f : exp2_fast(sink2 - M));
      const float scale = f / denom;
      uint16_t* op = p.o + (((long)b * p.T + t) * p.Hq + h) * D;
#pragma unroll
      for (int db = 0; db < ND; ++db) {
#pragma unroll
        for (int a4 = 0; a4 < 4; ++a4) {
          const f32x4 y = {acc[nb][db][4 * a4] * scale, acc[nb][db][4 * a4 + 1] * scale,
                           acc[nb][db][4 * a4 + 2] * scale, acc[nb][db][4 * a4 + 3] * scale};
          *(bf16x4*)(op + db * 32 + 8 * a4 + 4 * half) = __builtin_convertvector(y, bf16x4);
        }
      }
    } else {
      const long prow = (((long)b * p.Hkv + g) * p.nsplit + s) * p.r_pad + m;
      float* op = p.ws_o + prow * D;
#pragma unroll
      for (int db = 0; db < ND; ++db) {
#pragma unroll
        for (int a4 = 0; a4 < 4; ++a4) {
          const f32x4 y = {acc[nb][db][4 * a4], acc[nb][db][4 * a4 + 1], acc[nb][db][4 * a4 + 2],
                           acc[nb][db][4 * a4 + 3]};
          *(f32x4*)(op + db * 32 + 8 * a4 + 4 * half) = y;
        }
      }
      if (half == 0) {
        p.ws_ml[prow * 2] = m_all[nb];
        p.ws_ml[prow * 2 + 1] = l_all[nb];
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
  long want = max_rows * (long)B * Hkv / 256;
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

template <int D, int NB, int NW>
static hipError_t launch_verify_t(VerifyArgs a, const VerifyPlan& pl, hipStream_t s) {
  dim3 grid(a.B * a.Hkv, pl.nsplit), block(NW * 64);
  if (pl.nsplit == 1) {
    hipLaunchKernelGGL((verify_bf16_kernel<D, NB, NW, true>), grid, block, 0, s, a);
    return hipGetLastError();
  }
  hipLaunchKernelGGL((verify_bf16_kernel<D, NB, NW, false>), grid, block, 0, s, a);
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
  if (a.D == 128) {
    return pl.nb == 1 ? launch_verify_t<128, 1, 4>(a, pl, s) : launch_verify_t<128, 2, 2>(a, pl, s);
  }
  return pl.nb == 1 ? launch_verify_t<64, 1, 4>(a, pl, s) : launch_verify_t<64, 2, 2>(a, pl, s);
}

}  // namespace swa
