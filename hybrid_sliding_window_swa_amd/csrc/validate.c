/* Host-side argument validation of the C ABI (no HIP dependency). */
#include "validate.h"

static int dtype_ok(swa_dtype_t dt) { return dt == SWA_F32 || dt == SWA_BF16; }
static int head_dim_ok(int D) { return D == 64 || D == 128; }

swa_status_t swa_validate_scale(float sm_scale)
{
    /* finite and > 0 (NaN fails the comparison) */
    if (!(sm_scale > 0.0f) || sm_scale > 3.0e38f)
        return SWA_ERR_UNSUPPORTED;
    return SWA_OK;
}

swa_status_t swa_validate_prefill(const void *q, const void *k, const void *v, const void *o,
                                  int B, int Sq, int Sk, int Hq, int Hkv, int D,
                                  int window, int q_offset, float sm_scale, swa_dtype_t dtype)
{
    (void)window;
    if (!dtype_ok(dtype))
        return SWA_ERR_UNSUPPORTED;
    if (swa_validate_scale(sm_scale) != SWA_OK)
        return SWA_ERR_UNSUPPORTED;
    if (B < 0 || Sq < 0 || Sk < 0 || Hq <= 0 || Hkv <= 0 || Hq % Hkv != 0)
        return SWA_ERR_SHAPE;
    if (q_offset < 0 || (long long)q_offset + Sq > Sk)
        return SWA_ERR_SHAPE;
    if (!head_dim_ok(D))
        return SWA_ERR_UNSUPPORTED;
    {
        const int G = Hq / Hkv;
        if (dtype == SWA_BF16 && (G > 32 || 32 % G != 0))
            return SWA_ERR_UNSUPPORTED;
        if (dtype == SWA_F32 && G > 128)
            return SWA_ERR_UNSUPPORTED;
    }
    /* element offsets must fit in 64-bit and per-tensor token counts in int */
    if ((long long)B * Sq * Hq * D > (1LL << 46) || (long long)B * Sk * Hkv * D > (1LL << 46))
        return SWA_ERR_SHAPE;
    if (B == 0 || Sq == 0)
        return SWA_OK;
    if (!q || !k || !v || !o)
        return SWA_ERR_NULL;
    return SWA_OK;
}

swa_status_t swa_validate_verify_shape(int B, int q_len, int Hq, int Hkv, int D,
                                       int cache_slots, int ring, int window, swa_dtype_t dtype)
{
    if (!dtype_ok(dtype))
        return SWA_ERR_UNSUPPORTED;
    if (B < 0 || q_len < 1 || q_len > 16 || Hq <= 0 || Hkv <= 0 || Hq % Hkv != 0 ||
        cache_slots < 1 || (ring != 0 && ring != 1))
        return SWA_ERR_SHAPE;
    if (ring && (window < 1 || cache_slots < window))
        return SWA_ERR_SHAPE;
    if (!head_dim_ok(D))
        return SWA_ERR_UNSUPPORTED;
    {
        const int rows = (Hq / Hkv) * q_len;
        if (dtype == SWA_BF16 && rows > 64)
            return SWA_ERR_UNSUPPORTED;
        if (dtype == SWA_F32 && rows > 256)
            return SWA_ERR_UNSUPPORTED;
    }
    if ((long long)B * cache_slots * Hkv * D > (1LL << 46))
        return SWA_ERR_SHAPE;
    return SWA_OK;
}

swa_status_t swa_validate_verify_ptrs(const void *q, const void *k_new, const void *v_new,
                                      const void *k_cache, const void *v_cache,
                                      const void *cache_len, const void *o)
{
    if (!q || !k_new || !v_new || !k_cache || !v_cache || !cache_len || !o)
        return SWA_ERR_NULL;
    return SWA_OK;
}

swa_status_t swa_validate_append(const void *k_cache, const void *v_cache, const void *k_new,
                                 const void *v_new, const void *cache_len, const void *n_append,
                                 int B, int q_len, int Hkv, int D, int cache_slots, int ring,
                                 swa_dtype_t dtype)
{
    if (!dtype_ok(dtype))
        return SWA_ERR_UNSUPPORTED;
    if (B < 0 || q_len < 1 || q_len > 16 || Hkv <= 0 || D <= 0 || cache_slots < 1 ||
        (ring != 0 && ring != 1))
        return SWA_ERR_SHAPE;
    {
        const long long row = (long long)Hkv * D * (dtype == SWA_BF16 ? 2 : 4);
        if (row % 16 != 0)
            return SWA_ERR_UNSUPPORTED;
    }
    if (B == 0)
        return SWA_OK;
    if (!k_cache || !v_cache || !k_new || !v_new || !cache_len || !n_append)
        return SWA_ERR_NULL;
    return SWA_OK;
}

swa_status_t swa_validate_accept(const void *logits, const void *draft, const void *target,
                                 const void *n_append, int B, int q_len, long long vocab,
                                 swa_dtype_t dtype)
{
    if (!dtype_ok(dtype))
        return SWA_ERR_UNSUPPORTED;
    if (B < 0 || q_len < 1 || q_len > 16 || vocab < 1 || vocab > 2147483647LL ||
        (long long)B * q_len > 65535)
        return SWA_ERR_SHAPE;
    if (B == 0)
        return SWA_OK;
    if (!logits || !target || !n_append || (q_len > 1 && !draft))
        return SWA_ERR_NULL;
    return SWA_OK;
}

swa_status_t swa_validate_advance(const void *cache_len, const void *n_append, int B)
{
    if (B < 0)
        return SWA_ERR_SHAPE;
    if (B == 0)
        return SWA_OK;
    if (!cache_len || !n_append)
        return SWA_ERR_NULL;
    return SWA_OK;
}

swa_status_t swa_validate_rope(const void *x, int B, int S, int H, int D, int rot_dim,
                               int pos_offset, float base, swa_dtype_t dtype)
{
    if (!dtype_ok(dtype))
        return SWA_ERR_UNSUPPORTED;
    if (B < 0 || S < 0 || H <= 0 || pos_offset < 0)
        return SWA_ERR_SHAPE;
    if (D <= 0 || D > 256 || D % 8 != 0 || rot_dim < 0 || rot_dim > D || (rot_dim & 1))
        return SWA_ERR_SHAPE;
    if (!(base > 0.0f) || base > 3.0e38f)
        return SWA_ERR_UNSUPPORTED;
    if (B == 0 || S == 0 || rot_dim == 0)
        return SWA_OK;
    if (!x)
        return SWA_ERR_NULL;
    if (((unsigned long long)(size_t)x) % 16 != 0)
        return SWA_ERR_UNSUPPORTED;
    return SWA_OK;
}
