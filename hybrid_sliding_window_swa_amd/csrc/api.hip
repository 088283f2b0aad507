// C-ABI entry points: validate on the host, then enqueue the kernels on the
// caller's stream.  No allocation, no synchronisation, no state.
#include <math.h>

#include "launch.hpp"
#include "swa_attn.h"
#include "validate.h"

using namespace swa;

namespace {

constexpr float kLog2eHost = 1.4426950408889634f;

swa_status_t from_hip(hipError_t e) { return e == hipSuccess ? SWA_OK : SWA_ERR_LAUNCH; }

}  // namespace

extern "C" {

const char* swa_status_string(swa_status_t status) {
  switch (status) {
    case SWA_OK: return "ok";
    case SWA_ERR_NULL: return "a required pointer is NULL";
    case SWA_ERR_SHAPE: return "sizes violate a shape rule";
    case SWA_ERR_UNSUPPORTED: return "unsupported dtype, head_dim or head grouping, or sm_scale not finite > 0";
    case SWA_ERR_WORKSPACE: return "workspace missing or too small";
    case SWA_ERR_LAUNCH: return "kernel launch failed";
  }
  return "unknown status";
}

namespace {

PrefillArgs prefill_args(const void* q, const void* k, const void* v, const float* sinks, void* o, int B,
                         int Sq, int Sk, int Hq, int Hkv, int D, int window, int q_offset, float sm_scale) {
  PrefillArgs a = {};
  a.q = (const uint16_t*)q;
  a.k = (const uint16_t*)k;
  a.v = (const uint16_t*)v;
  a.sinks = sinks;
  a.o = (uint16_t*)o;
  a.B = B;
  a.Sq = Sq;
  a.Sk = Sk;
  a.Hq = Hq;
  a.Hkv = Hkv;
  a.D = D;
  a.window = window > 0 ? window : 0;
  a.q_offset = q_offset;
  a.scale = sm_scale;
  a.scale_log2 = sm_scale * kLog2eHost;
  return a;
}

}  // namespace

swa_status_t swa_attn_prefill(const void* q, const void* k, const void* v, const float* sinks,
                              void* o, int B, int Sq, int Sk, int Hq, int Hkv, int D, int window,
                              int q_offset, float sm_scale, swa_dtype_t dtype, void* stream) {
  swa_status_t st = swa_validate_prefill(q, k, v, o, B, Sq, Sk, Hq, Hkv, D, window, q_offset,
                                         sm_scale, dtype);
  if (st != SWA_OK || B == 0 || Sq == 0) return st;
  const PrefillArgs a = prefill_args(q, k, v, sinks, o, B, Sq, Sk, Hq, Hkv, D, window, q_offset, sm_scale);
  hipStream_t s = (hipStream_t)stream;
  return from_hip(dtype == SWA_BF16 ? launch_prefill_bf16(a, s) : launch_prefill_f32(a, s));
}

swa_status_t swa_attn_prefill_rope(const void* q, const void* k, const void* v, const float* sinks,
                                   void* o, int B, int Sq, int Sk, int Hq, int Hkv, int D, int window,
                                   int q_offset, float sm_scale, int rot_dim, float rope_base,
                                   swa_dtype_t dtype, void* stream) {
  swa_status_t st = swa_validate_prefill(q, k, v, o, B, Sq, Sk, Hq, Hkv, D, window, q_offset,
                                         sm_scale, dtype);
  if (st != SWA_OK) return st;
  if (rot_dim < 0 || (rot_dim & 1) || rot_dim > D) return SWA_ERR_SHAPE;
  if (!(rope_base > 0.0f) || rope_base > 3.0e38f) return SWA_ERR_UNSUPPORTED;
  if (B == 0 || Sq == 0) return SWA_OK;
  PrefillArgs a = prefill_args(q, k, v, sinks, o, B, Sq, Sk, Hq, Hkv, D, window, q_offset, sm_scale);
  if (rot_dim > 0 && (dtype != SWA_BF16 || rot_dim > D / 2 || !prefill_uses_strip(a)))
    return SWA_ERR_UNSUPPORTED;
  a.rope_hr = rot_dim / 2;
  for (int i = 0; i < a.rope_hr; ++i) a.rope_inv_freq[i] = pow((double)rope_base, -2.0 * i / rot_dim);
  hipStream_t s = (hipStream_t)stream;
  return from_hip(dtype == SWA_BF16 ? launch_prefill_bf16(a, s) : launch_prefill_f32(a, s));
}

swa_status_t swa_attn_prefill_lse(const void* q, const void* k, const void* v, const float* sinks,
                                  void* o, float* lse, int B, int Sq, int Sk, int Hq, int Hkv, int D,
                                  int window, int q_offset, float sm_scale, swa_dtype_t dtype, void* stream) {
  swa_status_t st = swa_validate_prefill(q, k, v, o, B, Sq, Sk, Hq, Hkv, D, window, q_offset,
                                         sm_scale, dtype);
  if (st != SWA_OK) return st;
  if (dtype != SWA_BF16) return SWA_ERR_UNSUPPORTED;
  if (B == 0 || Sq == 0) return SWA_OK;
  if (!lse) return SWA_ERR_NULL;
  PrefillArgs a = prefill_args(q, k, v, sinks, o, B, Sq, Sk, Hq, Hkv, D, window, q_offset, sm_scale);
  a.lse = lse;
  return from_hip(launch_prefill_bf16(a, (hipStream_t)stream));
}

size_t swa_attn_backward_workspace_bytes(int B, int Sq, int Hq) {
  if (B < 0 || Sq < 0 || Hq <= 0) return 0;
  return plan_backward(B, Sq, Hq).ws_bytes;
}

swa_status_t swa_attn_backward(const void* q, const void* k, const void* v, const float* sinks,
                               const void* o, const float* lse, const void* dout, void* dq, void* dk,
                               void* dv, float* dsink, int B, int Sq, int Sk, int Hq, int Hkv, int D,
                               int window, int q_offset, float sm_scale, swa_dtype_t dtype,
                               void* workspace, size_t workspace_bytes, void* stream) {
  swa_status_t st = swa_validate_prefill(q, k, v, o, B, Sq, Sk, Hq, Hkv, D, window, q_offset,
                                         sm_scale, dtype);
  if (st != SWA_OK) return st;
  if (dtype != SWA_BF16) return SWA_ERR_UNSUPPORTED;
  if (B == 0) return SWA_OK;
  if (!dk || !dv || (Sq > 0 && (!lse || !dout || !dq))) return SWA_ERR_NULL;
  const BwdPlan plan = plan_backward(B, Sq, Hq);
  if (!workspace || workspace_bytes < plan.ws_bytes || ((uintptr_t)workspace & 255u) != 0)
    return SWA_ERR_WORKSPACE;
  BwdArgs a = {};
  a.q = (const uint16_t*)q;
  a.k = (const uint16_t*)k;
  a.v = (const uint16_t*)v;
  a.sinks = sinks;
  a.o = (const uint16_t*)o;
  a.dout = (const uint16_t*)dout;
  a.lse = lse;
  a.dq = (uint16_t*)dq;
  a.dk = (uint16_t*)dk;
  a.dv = (uint16_t*)dv;
  a.dsink = dsink;
  a.delta = (float*)workspace;
  a.sink_part = (float*)((char*)workspace + plan.delta_bytes);
  a.part = plan.part_bytes ? (float*)((char*)workspace + plan.part_offset) : nullptr;
  a.part_bytes = plan.part_bytes;
  a.B = B;
  a.Sq = Sq;
  a.Sk = Sk;
  a.Hq = Hq;
  a.Hkv = Hkv;
  a.D = D;
  a.window = window > 0 ? window : 0;
  a.q_offset = q_offset;
  a.scale = sm_scale;
  a.scale_log2 = sm_scale * kLog2eHost;
  return from_hip(launch_backward_bf16(a, plan, (hipStream_t)stream));
}

size_t swa_attn_verify_workspace_bytes(int B, int q_len, int Hq, int Hkv, int D, int cache_slots,
                                       int ring, int window, swa_dtype_t dtype) {
  if (swa_validate_verify_shape(B, q_len, Hq, Hkv, D, cache_slots, ring, window, dtype) != SWA_OK)
    return 0;
  if (dtype != SWA_BF16 || B == 0) return 0;
  return plan_verify_bf16(B, q_len, Hq, Hkv, D, cache_slots, ring, window).ws_bytes;
}

swa_status_t swa_attn_verify(const void* q, const void* k_new, const void* v_new,
                             const void* k_cache, const void* v_cache, const int32_t* cache_len,
                             const float* sinks, void* o, int B, int q_len, int Hq, int Hkv, int D,
                             int cache_slots, int ring, int window, float sm_scale,
                             swa_dtype_t dtype, void* workspace, size_t workspace_bytes,
                             void* stream) {
  swa_status_t st =
      swa_validate_verify_shape(B, q_len, Hq, Hkv, D, cache_slots, ring, window, dtype);
  if (st == SWA_OK) st = swa_validate_scale(sm_scale);
  if (st != SWA_OK || B == 0) return st;
  st = swa_validate_verify_ptrs(q, k_new, v_new, k_cache, v_cache, cache_len, o);
  if (st != SWA_OK) return st;
  VerifyArgs a = {};
  a.q = (const uint16_t*)q;
  a.k_new = (const uint16_t*)k_new;
  a.v_new = (const uint16_t*)v_new;
  a.k_cache = (const uint16_t*)k_cache;
  a.v_cache = (const uint16_t*)v_cache;
  a.cache_len = cache_len;
  a.sinks = sinks;
  a.o = (uint16_t*)o;
  a.B = B;
  a.T = q_len;
  a.Hq = Hq;
  a.Hkv = Hkv;
  a.D = D;
  a.slots = cache_slots;
  a.ring = ring;
  a.window = window > 0 ? window : 0;
  a.scale = sm_scale;
  a.scale_log2 = sm_scale * kLog2eHost;
  hipStream_t s = (hipStream_t)stream;
  if (dtype == SWA_F32) return from_hip(launch_verify_f32(a, s));
  const VerifyPlan plan = plan_verify_bf16(B, q_len, Hq, Hkv, D, cache_slots, ring, window);
  if (plan.ws_bytes > 0) {
    if (!workspace || workspace_bytes < plan.ws_bytes || ((uintptr_t)workspace & 255u) != 0)
      return SWA_ERR_WORKSPACE;
    a.ws_o = (float*)workspace;
    a.ws_ml = a.ws_o + (size_t)B * Hkv * plan.nsplit * (32 * plan.nb) * D;
  }
  return from_hip(launch_verify_bf16(a, plan, s));
}

swa_status_t kv_ring_append(void* k_cache, void* v_cache, const void* k_new, const void* v_new,
                            const int32_t* cache_len, const int32_t* n_append, int B, int q_len,
                            int Hkv, int D, int cache_slots, int ring, swa_dtype_t dtype,
                            void* stream) {
  swa_status_t st = swa_validate_append(k_cache, v_cache, k_new, v_new, cache_len, n_append, B,
                                        q_len, Hkv, D, cache_slots, ring, dtype);
  if (st != SWA_OK || B == 0) return st;
  AppendArgs a = {};
  a.k_cache = (uint8_t*)k_cache;
  a.v_cache = (uint8_t*)v_cache;
  a.k_new = (const uint8_t*)k_new;
  a.v_new = (const uint8_t*)v_new;
  a.cache_len = cache_len;
  a.n_append = n_append;
  a.B = B;
  a.T = q_len;
  a.row_bytes = Hkv * D * (dtype == SWA_BF16 ? 2 : 4);
  a.slots = cache_slots;
  a.ring = ring;
  return from_hip(launch_append(a, (hipStream_t)stream));
}

size_t swa_mtp_accept_workspace_bytes(int B, int q_len, int64_t vocab) {
  if (swa_validate_accept((const void*)1, (const void*)1, (const void*)1, (const void*)1, B, q_len,
                          vocab, SWA_F32) != SWA_OK || B == 0)
    return 0;
  return plan_accept(B, q_len, (long)vocab).ws_bytes;
}

swa_status_t swa_mtp_greedy_accept(const void* logits, const int32_t* draft, int32_t* target,
                                   int32_t* n_append, int B, int q_len, int64_t vocab,
                                   swa_dtype_t dtype, void* workspace, size_t workspace_bytes,
                                   void* stream) {
  swa_status_t st = swa_validate_accept(logits, draft, target, n_append, B, q_len, vocab, dtype);
  if (st != SWA_OK || B == 0) return st;
  const AcceptPlan plan = plan_accept(B, q_len, (long)vocab);
  if (!workspace || workspace_bytes < plan.ws_bytes || ((uintptr_t)workspace & 3u) != 0)
    return SWA_ERR_WORKSPACE;
  AcceptArgs a = {};
  a.logits = logits;
  a.draft = draft;
  a.target = target;
  a.n_append = n_append;
  a.ws_v = (float*)workspace;
  a.V = (long)vocab;
  a.B = B;
  a.T = q_len;
  a.elem_bytes = dtype == SWA_BF16 ? 2 : 4;
  return from_hip(launch_accept(a, plan, (hipStream_t)stream));
}

swa_status_t swa_cache_advance(int32_t* cache_len, const int32_t* n_append, int B, void* stream) {
  swa_status_t st = swa_validate_advance(cache_len, n_append, B);
  if (st != SWA_OK || B == 0) return st;
  return from_hip(launch_advance(cache_len, n_append, B, (hipStream_t)stream));
}

swa_status_t swa_rope_apply(void* x, const int32_t* pos0, int pos_offset, int B, int S, int H, int D,
                            int rot_dim, float base, swa_dtype_t dtype, void* stream) {
  swa_status_t st = swa_validate_rope(x, B, S, H, D, rot_dim, pos_offset, base, dtype);
  if (st != SWA_OK || B == 0 || S == 0 || rot_dim == 0) return st;
  RopeArgs a = {};
  a.x = x;
  a.pos0 = pos0;
  a.pos_offset = pos_offset;
  a.rows = (long)B * S * H;
  a.B = B;
  a.S = S;
  a.H = H;
  a.D = D;
  a.rot = rot_dim;
  a.esize = dtype == SWA_BF16 ? 2 : 4;
  a.log2_base = log2((double)base);
  return from_hip(launch_rope(a, (hipStream_t)stream));
}

}  // extern "C"
