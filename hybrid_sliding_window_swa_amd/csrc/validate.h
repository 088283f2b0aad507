/* Host-side argument validation of the C ABI.  Plain C with no HIP
 * dependency, so the rules can be exercised without a GPU. */
#ifndef SWA_VALIDATE_H
#define SWA_VALIDATE_H

#include "swa_attn.h"

#ifdef __cplusplus
extern "C" {
#endif

swa_status_t swa_validate_prefill(const void *q, const void *k, const void *v, const void *o,
                                  int B, int Sq, int Sk, int Hq, int Hkv, int D,
                                  int window, int q_offset, float sm_scale, swa_dtype_t dtype);

swa_status_t swa_validate_verify_shape(int B, int q_len, int Hq, int Hkv, int D,
                                       int cache_slots, int ring, int window, swa_dtype_t dtype);

/* sm_scale must be finite and positive. */
swa_status_t swa_validate_scale(float sm_scale);

swa_status_t swa_validate_verify_ptrs(const void *q, const void *k_new, const void *v_new,
                                      const void *k_cache, const void *v_cache,
                                      const void *cache_len, const void *o);

swa_status_t swa_validate_append(const void *k_cache, const void *v_cache, const void *k_new,
                                 const void *v_new, const void *cache_len, const void *n_append,
                                 int B, int q_len, int Hkv, int D, int cache_slots, int ring,
                                 swa_dtype_t dtype);

/* B * q_len <= 65535 (one workgroup row per logits row), 1 <= vocab < 2^31. */
swa_status_t swa_validate_accept(const void *logits, const void *draft, const void *target,
                                 const void *n_append, int B, int q_len, long long vocab,
                                 swa_dtype_t dtype);

swa_status_t swa_validate_advance(const void *cache_len, const void *n_append, int B);

/* D % 8 == 0, D <= 256, rot_dim even in [0, D], x 16-byte aligned. */
swa_status_t swa_validate_rope(const void *x, int B, int S, int H, int D, int rot_dim,
                               int pos_offset, float base, swa_dtype_t dtype);

#ifdef __cplusplus
}
#endif

#endif
