// Internal kernel-launch interface between the C-ABI entry points and the
// kernels.  All pointers are device pointers; arguments are already validated.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace swa {

struct PrefillArgs {
  const uint16_t* q;  // bf16 bits, or fp32 reinterpreted by the fp32 kernel
  const uint16_t* k;
  const uint16_t* v;
  const float* sinks;
  uint16_t* o;
  float* lse;         // [B, Sq, Hq] natural-log softmax denominators, or null
  int B, Sq, Sk, Hq, Hkv, D;
  int window, q_offset;
  float scale;        // sm_scale
  float scale_log2;   // sm_scale * log2(e)
  // partial rotary embedding of the queries, applied as they are staged
  // (sliding-window strip kernel only): rope_hr pairs (i, i + rope_hr), pair
  // i turned by position * rope_inv_freq[i]; rope_hr == 0 leaves q as is
  int rope_hr;
  double rope_inv_freq[32];
  // filled by the launcher
  int n_tb, total, per_xcd;
};

struct VerifyArgs {
  const uint16_t* q;
  const uint16_t* k_new;
  const uint16_t* v_new;
  const uint16_t* k_cache;
  const uint16_t* v_cache;
  const int32_t* cache_len;
  const float* sinks;
  uint16_t* o;
  float* ws_o;   // [B][Hkv][nsplit][R_pad][D] split partial outputs
  float* ws_ml;  // [B][Hkv][nsplit][R_pad][2] split running max (log2) and sum
  int B, T, Hq, Hkv, D;
  int slots, ring, window;
  float scale;
  float scale_log2;
  int split_len;   // cache rows per split (multiple of 32 * waves)
  int nsplit;      // splits per (request, KV head) the workspace holds
  int r_pad;       // query rows per (request, KV head), padded to 32 * NB
};

struct AppendArgs {
  uint8_t* k_cache;
  uint8_t* v_cache;
  const uint8_t* k_new;
  const uint8_t* v_new;
  const int32_t* cache_len;
  const int32_t* n_append;
  int B, T, row_bytes, slots, ring;
};

hipError_t launch_prefill_bf16(const PrefillArgs& a, hipStream_t s);

struct BwdArgs {
  const uint16_t* q;      // [B, Sq, Hq, D] bf16
  const uint16_t* k;      // [B, Sk, Hkv, D]
  const uint16_t* v;
  const float* sinks;     // [Hq] or null
  const uint16_t* o;      // forward output [B, Sq, Hq, D]
  const uint16_t* dout;   // dL/dO [B, Sq, Hq, D]
  const float* lse;       // forward log-sum-exp [B, Sq, Hq] (natural log, sink included)
  uint16_t* dq;
  uint16_t* dk;
  uint16_t* dv;
  float* dsink;           // [Hq] or null
  float* delta;           // workspace: <dO, O> per row [B, Sq, Hq]
  float* sink_part;       // workspace: [n_sink_parts][Hq] partial sink gradients
  int B, Sq, Sk, Hq, Hkv, D;
  int window, q_offset;
  float scale, scale_log2;
  int n_sink_parts;       // set by the launcher
  int strips_per_bg;      // set by the launcher (0: the non-persistent dQ kernel)
  float* part;            // workspace: fp32 dK/dV partials of key tiles two strips share
  size_t part_bytes;
  int fuse_spb, fuse_nbt; // set by the launcher for the fused sliding-window kernel
};

struct BwdPlan {
  size_t delta_bytes; // bytes of the delta array (256-byte rounded)
  size_t part_offset; // byte offset of the fused kernel's partials
  size_t part_bytes;
  size_t ws_bytes;
};
BwdPlan plan_backward(int B, int Sq, int Hq);
hipError_t launch_backward_bf16(BwdArgs a, const BwdPlan& p, hipStream_t s);
// Whether launch_prefill_bf16 runs these arguments on the sliding-window strip
// kernel (the only prefill kernel that rotates queries as it stages them).
bool prefill_uses_strip(const PrefillArgs& a);
hipError_t launch_prefill_f32(const PrefillArgs& a, hipStream_t s);

// Verify plan shared by the workspace query and the launch.
struct VerifyPlan {
  int nb;         // 32-row query blocks per (request, KV head)
  int waves;      // waves per workgroup
  int split_len;  // cache rows per split
  int nsplit;     // splits per (request, KV head)
  size_t ws_bytes;
};
VerifyPlan plan_verify_bf16(int B, int T, int Hq, int Hkv, int D, int slots, int ring, int window);
hipError_t launch_verify_bf16(const VerifyArgs& a, const VerifyPlan& plan, hipStream_t s);
hipError_t launch_verify_f32(const VerifyArgs& a, hipStream_t s);

hipError_t launch_append(const AppendArgs& a, hipStream_t s);

struct AcceptArgs {
  const void* logits;     // [B][T][V] fp32 or bf16 bits
  const int32_t* draft;   // [B][T-1]
  int32_t* target;        // [B][T]
  int32_t* n_append;      // [B]
  float* ws_v;            // [B*T][nchunk] chunk maxima
  int32_t* ws_i;          // [B*T][nchunk] lowest index of each chunk maximum (set by the launcher)
  long V;
  int B, T, elem_bytes;
  long chunk_len;         // set by the launcher
  int nchunk;             // set by the launcher
};

struct AcceptPlan {
  long chunk_len;  // logits per chunk (a multiple of 1024)
  int nchunk;      // chunks per row
  size_t ws_bytes;
};
AcceptPlan plan_accept(int B, int T, long V);
hipError_t launch_accept(AcceptArgs a, const AcceptPlan& p, hipStream_t s);
hipError_t launch_advance(int32_t* cache_len, const int32_t* n_append, int B, hipStream_t s);

struct RopeArgs {
  void* x;               // [B][S][H][D], rotated in place
  const int32_t* pos0;   // [B] or null
  long rows;             // B * S * H
  int pos_offset;
  int B, S, H, D, rot, esize;
  double log2_base;
  int nv, pitch_dw, rows_blk;  // set by the launcher
};

struct RopePlan {
  int nv;          // 16-byte vectors per row that hold the rotated dimensions
  int pitch_dw;    // LDS row pitch in dwords (odd)
  int rows_blk;    // rows per workgroup
  size_t lds_bytes;
};
RopePlan plan_rope(int H, int D, int rot, int esize);
hipError_t launch_rope(RopeArgs a, hipStream_t s);

}  // namespace swa
