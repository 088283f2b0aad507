/*
 * swa_attn.h -- C ABI of the MI355X (gfx950) sliding-window / global
 * attention library with per-head attention sinks.
 *
 * The operation (from the pages on MiMo-V2-Flash):
 *   - Sliding-window attention with a window of W = 128 tokens, interleaved
 *     5:1 with global attention (W = infinity) in the same model; the MTP
 *     draft layers use the sliding window too.  MiMo-V2-Flash technical-report
 *     digest (fanfer.top), section "MiMo-V2-Flash Model Architecture"; release
 *     blog (aihot.news), section on pushing efficiency to the limit.
 *   - A learnable attention-sink bias per head in the gpt-oss style: the sink
 *     logit adds exp(sink) to the softmax denominator and carries no value.
 *     Technical-report digest, paragraph "Hybrid Sliding Window Attention
 *     Architecture".
 *   - MTP self-speculative decoding: the main model verifies 1 committed + 3
 *     draft tokens in one pass without extra KV-cache I/O, accepts a prefix
 *     and discards the rest.  Release blog, section "Multi-Token Prediction"
 *     (verify diagram and the paragraph after it).
 *   - The SWA layers keep a fixed-size KV cache.  Release blog, section on
 *     pushing efficiency to the limit.
 *
 * Definition computed by every entry point, for request b, query head h,
 * query at absolute position i (G = Hq / Hkv, KV head g = h / G):
 *   J(i) = { j : max(0, i - W + 1) <= j <= i }   (W keys including self;
 *          all j <= i when window <= 0)
 *   s_j  = sm_scale * <q, K[j, g]>
 *   O    = sum_{j in J(i)} exp(s_j) V[j, g] / (exp(sink_h) + sum_{j in J(i)} exp(s_j))
 * With sinks == NULL (or a sink of -inf) the exp(sink_h) term is absent.
 *
 * Conventions common to all entry points
 *   - Tensors are dense, row-major, token-major: [B, S, H, D] (the last index
 *     is contiguous).  Every data pointer is a DEVICE pointer (hipMalloc'd or
 *     from a framework allocator) owned by the caller.  The library allocates
 *     no memory and keeps no state between calls (the one exception is the
 *     fixed per-GPU array of swa_attn_verify_noalloc, part of the library's
 *     device code; see there).
 *   - `stream` is a hipStream_t passed as void* (NULL = the null stream).
 *     Calls only enqueue work on it and return without synchronising.
 *   - Host-visible arguments are validated before anything is launched; on a
 *     failure a nonzero status is returned and nothing is enqueued.
 *     Values that live in device memory (cache_len, n_append) cannot be
 *     checked without a synchronisation and are PRECONDITIONS (listed per
 *     entry point); violating them is undefined behaviour.
 *   - dtype SWA_BF16: q, k, v, o and caches are bfloat16; scores, softmax and
 *     accumulation are fp32, the attention weights are rounded to bf16 before
 *     the value product (the row sum that divides O adds the rounded
 *     weights, or, in the global-attention prefill, the weights before that
 *     rounding), and O is rounded to bf16 (round to nearest even).
 *     dtype SWA_F32: everything is fp32 and nothing is rounded to bf16.
 *   - sinks, when given, are fp32 [Hq] device values: finite or -inf.
 *   - Supported: D in {64, 128}; Hq % Hkv == 0.  The bf16 paths also need
 *     32 % (Hq / Hkv) == 0 (prefill) and (Hq / Hkv) * q_len <= 64 (verify).
 */
#ifndef SWA_ATTN_H
#define SWA_ATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Entry points are the only symbols the shared library exports. */
#if defined(__GNUC__) || defined(__clang__)
#define SWA_API __attribute__((visibility("default")))
#else
#define SWA_API
#endif

typedef enum {
    SWA_OK = 0,
    SWA_ERR_NULL = 1,        /* a required pointer is NULL */
    SWA_ERR_SHAPE = 2,       /* sizes violate a shape rule */
    SWA_ERR_UNSUPPORTED = 3, /* not implemented (dtype, D, grouping) or sm_scale not finite > 0 */
    SWA_ERR_WORKSPACE = 4,   /* workspace missing or smaller than required */
    SWA_ERR_LAUNCH = 5       /* the HIP runtime reported a launch error */
} swa_status_t;

typedef enum { SWA_F32 = 0, SWA_BF16 = 1 } swa_dtype_t;

/* Static, NUL-terminated description of a status code. */
SWA_API const char *swa_status_string(swa_status_t status);

/*
 * Causal prefill (also chunked prefill and prefill after a cached prefix).
 *   q      [B, Sq, Hq, D]   queries; query row r sits at absolute position
 *                           q_offset + r
 *   k, v   [B, Sk, Hkv, D]  keys / values of positions 0 .. Sk-1
 *   sinks  [Hq] fp32 or NULL
 *   o      [B, Sq, Hq, D]   output (same dtype as q); must not alias inputs
 *   window >= 1: sliding window of `window` keys including the query's own
 *          position; <= 0: global causal attention
 *   q_offset  0 <= q_offset and q_offset + Sq <= Sk.  Fresh prefill uses 0; a
 *          chunk [c0, c0 + C) of a long sequence passes its queries, the full
 *          k / v and q_offset = c0 (only keys >= c0 - window + 1 are read).
 *   sm_scale  multiplier of q.k (normally 1/sqrt(D)), finite and > 0; the
 *          sink is not scaled.
 * Rows of k / v that no query of the call can see -- positions below
 * max(0, q_offset - window + 1) (none for global attention) and at or above
 * q_offset + Sq -- are never used and may hold anything, NaN included (e.g.
 * the unfilled tail of a cache behind a chunk, or stale rows below the
 * window).  Inside that range a non-finite value can also reach outputs of
 * nearby queries whose windows exclude it (masked weights are exact zeros,
 * but they still multiply the loaded value rows of a 32-key tile).
 * B == 0 or Sq == 0 is a valid no-op.
 */
SWA_API swa_status_t swa_attn_prefill(const void *q, const void *k, const void *v,
                              const float *sinks, void *o,
                              int B, int Sq, int Sk, int Hq, int Hkv, int D,
                              int window, int q_offset, float sm_scale,
                              swa_dtype_t dtype, void *stream);

/*
 * Causal prefill with the queries' partial rotary embedding applied as they
 * are loaded: O = attention(R(q), k, v), where R rotates the first rot_dim
 * dimensions of every query head by its position (q_offset + r) exactly as
 * swa_rope_apply does (pairs (i, i + rot_dim/2), angle pos *
 * rope_base^(-2i/rot_dim); technical-report digest, "Pre-training", and the
 * model card config extract for the factor 0.334).  q is only read.  The keys
 * must already be rotated (swa_rope_apply once, or a cache of rotated keys).
 * Other arguments as swa_attn_prefill; rot_dim == 0 is swa_attn_prefill.
 * Supported with rot_dim > 0: SWA_BF16, rot_dim even and <= D / 2, and the
 * sliding-window configurations of the strip kernel (window >= 1 with at most
 * about 128 + 31 keys per 32-query block, Hq / Hkv of 4 or 8); otherwise
 * SWA_ERR_UNSUPPORTED, and the caller applies swa_rope_apply to a copy of q
 * and calls swa_attn_prefill (for global attention that extra pass costs
 * under one percent of the prefill).
 */
SWA_API swa_status_t swa_attn_prefill_rope(const void *q, const void *k, const void *v,
                                   const float *sinks, void *o,
                                   int B, int Sq, int Sk, int Hq, int Hkv, int D,
                                   int window, int q_offset, float sm_scale,
                                   int rot_dim, float rope_base,
                                   swa_dtype_t dtype, void *stream);

/*
 * Training forward: swa_attn_prefill that also saves, per query row, the
 * natural-log softmax denominator with the sink,
 *   lse[b, r, h] = log(exp(sink_h) + sum_{j in J(i)} exp(s_j)),
 * which swa_attn_backward needs.  lse [B, Sq, Hq] fp32 DEVICE.  SWA_BF16 only;
 * other arguments and rules as swa_attn_prefill.  The row sums (o's divisor
 * and lse) add the attention weights after their rounding to bf16, the
 * weights that enter P V, so that lse matches o for the backward; where
 * swa_attn_prefill adds them before the rounding (global attention; at
 * most 2^-9 apart relatively) the two outputs can differ at bf16 rounding
 * level, elsewhere they are equal.
 */
SWA_API swa_status_t swa_attn_prefill_lse(const void *q, const void *k, const void *v,
                                  const float *sinks, void *o, float *lse,
                                  int B, int Sq, int Sk, int Hq, int Hkv, int D,
                                  int window, int q_offset, float sm_scale,
                                  swa_dtype_t dtype, void *stream);

/* Bytes of device workspace swa_attn_backward needs: per-row <dO, O>, the
 * per-workgroup partial sink gradients, and, for Sq >= 1024, a fixed 80 MiB
 * for the fp32 dK/dV partials of key tiles that two query strips of the
 * sliding-window kernel share (at most 256 strip boundaries x 5 tiles).
 * 0 for invalid sizes. */
SWA_API size_t swa_attn_backward_workspace_bytes(int B, int Sq, int Hq);

/*
 * Backward of the prefill: the gradients of L = sum(dout * O) for
 * O = swa_attn_prefill(q, k, v, sinks) (the definition at the top of this
 * file differentiated; the pages give no training kernel, and MTP-accelerated
 * RL training, report digest "Model Architecture", needs one):
 *   P = exp(s - lse), D_i = <dout_i, O_i>, dS = P (dout V^T - D),
 *   dq = sm_scale dS K, dk = sm_scale dS^T q, dv = P^T dout,
 *   dsink_h = -sum_i exp(sink_h - lse_i) D_i   (the sink is not scaled and
 *   carries no value).
 *   q, o, dout, dq   [B, Sq, Hq, D] bf16 DEVICE;  k, v, dk, dv [B, Sk, Hkv, D];
 *   o, lse           from swa_attn_prefill_lse on the same inputs;
 *   sinks [Hq] fp32 or NULL;  dsink [Hq] fp32 DEVICE output, or NULL to skip
 *   (zeros when sinks is NULL);
 *   workspace        device buffer, 256-byte aligned, of at least
 *                    swa_attn_backward_workspace_bytes(B, Sq, Hq) bytes.
 * Every element of dq, dk and dv is written (keys no query sees get zeros).
 * Accumulation is fp32; P and dS are rounded to bf16 for the matrix cores;
 * dq, dk, dv are rounded to bf16 (nearest even); dsink and the dK/dV of key
 * tiles shared by two query strips are summed in a fixed order
 * (deterministic).  SWA_BF16 only; shape rules as swa_attn_prefill.
 * Unlike the forward, the backward reads whole 32-key tiles around each
 * window and multiplies rows outside it by zero weights, so k and v must be
 * finite for all Sk rows.  Calls sharing a workspace must not overlap.
 */
SWA_API swa_status_t swa_attn_backward(const void *q, const void *k, const void *v,
                               const float *sinks, const void *o, const float *lse,
                               const void *dout, void *dq, void *dk, void *dv, float *dsink,
                               int B, int Sq, int Sk, int Hq, int Hkv, int D,
                               int window, int q_offset, float sm_scale, swa_dtype_t dtype,
                               void *workspace, size_t workspace_bytes, void *stream);

/*
 * Bytes of device workspace swa_attn_verify needs for these sizes (split-KV
 * partial results: running max, running sum and unnormalised output per
 * query row and split).  0 when the arguments are invalid.
 */
SWA_API size_t swa_attn_verify_workspace_bytes(int B, int q_len, int Hq, int Hkv, int D,
                                       int cache_slots, int ring, int window,
                                       swa_dtype_t dtype);

/*
 * Multi-token verify step (q_len = 1 + number of drafts; q_len = 1 is plain
 * decode) over a KV cache.
 *   q             [B, q_len, Hq, D]   token t of request b sits at position
 *                                     cache_len[b] + t
 *   k_new, v_new  [B, q_len, Hkv, D]  keys / values of the tokens under
 *                                     verification (not yet in the cache);
 *                                     token t sees new tokens 0..t
 *   k_cache, v_cache [B, cache_slots, Hkv, D]
 *       ring == 1: ring buffer, position p lives in slot p % cache_slots;
 *                  requires window >= 1 and cache_slots >= window.  Holds the
 *                  last min(L_b, cache_slots) committed positions.
 *       ring == 0: linear cache, position p lives in slot p.
 *   cache_len     [B] int32 DEVICE array: L_b committed tokens per request.
 *   sinks [Hq] fp32 or NULL;  o [B, q_len, Hq, D] output;
 *   sm_scale finite and > 0 (the sink is not scaled).
 *   workspace     device buffer of at least
 *                 swa_attn_verify_workspace_bytes(...) bytes (any alignment
 *                 of 256 bytes or more); its contents are scratch.
 * Device-side preconditions (not checked): 0 <= L_b; for ring == 0,
 * L_b <= cache_slots.  Cache slots that hold no committed position are never
 * read (they may hold NaN).  Calls that share a workspace must not overlap.
 */
SWA_API swa_status_t swa_attn_verify(const void *q, const void *k_new, const void *v_new,
                             const void *k_cache, const void *v_cache,
                             const int32_t *cache_len, const float *sinks, void *o,
                             int B, int q_len, int Hq, int Hkv, int D,
                             int cache_slots, int ring, int window, float sm_scale,
                             swa_dtype_t dtype, void *workspace, size_t workspace_bytes,
                             void *stream);

/*
 * swa_attn_verify without a workspace argument, for callers that cannot
 * allocate device memory: code under HIP graph capture, tight serving loops
 * and harnesses that forbid allocation.  Same arguments (minus workspace and
 * workspace_bytes), validation, kernels and results as swa_attn_verify.  The
 * split partials live in a fixed device array inside the library, one copy
 * per GPU, allocated when the library's code is loaded on that GPU and held
 * until the process ends; the call itself allocates nothing.
 *   Maximum: swa_attn_verify_workspace_bytes(...) of the same arguments must
 *   not exceed SWA_VERIFY_NOALLOC_SCRATCH_BYTES (64 MiB, e.g. 64 requests x 8
 *   KV heads over 65536-slot global caches need 34 MB, one request over
 *   262144 slots 8.5 MB); larger sizes return SWA_ERR_WORKSPACE with nothing
 *   enqueued.
 *   All calls on one GPU share that GPU's array, so calls that overlap on
 *   one GPU (other streams, other host threads) race and must be ordered by
 *   the caller.  Nothing in the array has to start at zero.
 *   The first call on each GPU looks up the array's device address (no
 *   allocation); make it once outside capture if the runtime forbids that
 *   lookup during capture.
 */
#define SWA_VERIFY_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)
SWA_API swa_status_t swa_attn_verify_noalloc(const void *q, const void *k_new, const void *v_new,
                                     const void *k_cache, const void *v_cache,
                                     const int32_t *cache_len, const float *sinks, void *o,
                                     int B, int q_len, int Hq, int Hkv, int D,
                                     int cache_slots, int ring, int window, float sm_scale,
                                     swa_dtype_t dtype, void *stream);

/*
 * Commit accepted tokens after a verify step.  For every request b and every
 * t < n_append[b], row t of k_new / v_new [B, q_len, Hkv, D] is copied to the
 * slot of position cache_len[b] + t: slot (cache_len[b] + t) % cache_slots
 * when ring == 1, slot cache_len[b] + t when ring == 0.  No other slot
 * changes, cache_len is only read (the caller advances it by n_append), and
 * rejected drafts never touch the cache (release blog, section
 * "Multi-Token Prediction": accept a prefix, reject one token, discard the
 * rest).
 *   cache_len, n_append: [B] int32 DEVICE arrays.
 * Device-side preconditions (not checked): 0 <= n_append[b] <= q_len,
 * 0 <= cache_len[b], and for ring == 0 cache_len[b] + n_append[b] <= cache_slots.
 * Works for either dtype (a copy of 2- or 4-byte elements).
 */
SWA_API swa_status_t kv_ring_append(void *k_cache, void *v_cache,
                            const void *k_new, const void *v_new,
                            const int32_t *cache_len, const int32_t *n_append,
                            int B, int q_len, int Hkv, int D, int cache_slots, int ring,
                            swa_dtype_t dtype, void *stream);

/*
 * Bytes of device workspace swa_mtp_greedy_accept needs (per-chunk maxima
 * and their indices).  0 when the sizes are invalid or B == 0.
 */
SWA_API size_t swa_mtp_accept_workspace_bytes(int B, int q_len, int64_t vocab);

/*
 * Greedy acceptance of draft tokens after a verify pass (self-speculative
 * decoding with the MTP heads as the draft model; release blog, section
 * "Multi-Token Prediction", verify diagram: accept a prefix, reject the first
 * mismatch, discard the rest).
 *   logits   [B, q_len, vocab] DEVICE, fp32 (SWA_F32) or bf16 (SWA_BF16):
 *            the main model's scores at the q_len verified positions; bf16 is
 *            widened to fp32 exactly before comparing.
 *   draft    [B, q_len - 1] int32 DEVICE: the token drafted for position t+1,
 *            compared with the prediction at position t; may be NULL when
 *            q_len == 1.
 *   target   [B, q_len] int32 DEVICE output: argmax over the vocabulary of
 *            each row, the lowest index among equal maxima.  target[b, t] is
 *            the main model's token for position t + 1; the entry at the
 *            first rejected draft is the corrected token.
 *   n_append [B] int32 DEVICE output: 1 + the number of leading drafts with
 *            draft[b, t] == target[b, t] (1 <= n_append <= q_len): the rows of
 *            the verified tokens whose K/V enter the caches (kv_ring_append).
 *   workspace  device buffer, 4-byte aligned, of at least
 *            swa_mtp_accept_workspace_bytes(B, q_len, vocab) bytes; scratch.
 * Sizes: 1 <= q_len <= 16, 1 <= vocab < 2^31, B * q_len <= 65535.
 * NaN logits are never selected (a row of only NaN gives index 0).
 * B == 0 is a no-op.  Calls sharing a workspace must not overlap.
 */
SWA_API swa_status_t swa_mtp_greedy_accept(const void *logits, const int32_t *draft,
                                   int32_t *target, int32_t *n_append,
                                   int B, int q_len, int64_t vocab, swa_dtype_t dtype,
                                   void *workspace, size_t workspace_bytes, void *stream);

/*
 * cache_len[b] += n_append[b] for b < B (both [B] int32 DEVICE arrays): the
 * committed length after every layer's kv_ring_append of the same step (the
 * appends read the old length).  B == 0 is a no-op.
 */
SWA_API swa_status_t swa_cache_advance(int32_t *cache_len, const int32_t *n_append, int B,
                               void *stream);

/*
 * Partial rotary position embedding, in place, on query or key rows before
 * attention (technical-report digest, "Pre-training": RoPE base 10000 for the
 * sliding-window layers, 640000 for the global layers, 5000000 after the
 * 256K extension; model card config extract: partial_rotary_factor 0.334).
 *   x  [B, S, H, D] DEVICE (bf16 or fp32), 16-byte aligned, rotated in place.
 *      Row s of request b sits at position (pos0 ? pos0[b] : 0) + pos_offset + s.
 *   pos0  [B] int32 DEVICE or NULL (e.g. cache_len for the rows under
 *      verification); pos_offset >= 0 (e.g. q_offset for a prefill chunk).
 *   rot_dim  even, 0 <= rot_dim <= D: the first rot_dim dimensions of each
 *      head rotate in rot_dim/2 pairs (i, i + rot_dim/2) by the angle
 *      pos * base^(-2i / rot_dim); the rest are untouched.  With the model's
 *      factor 0.334, rot_dim = 2 * floor(0.334 * D / 2) (42 for D = 128).
 *   base  finite and > 0.
 * The angle is reduced modulo 2*pi in fp64 before an fp32 sine / cosine, so
 * rotations stay accurate at positions of 2^18 and beyond.  Keys go through
 * it once (before prefill, or k_new before verify and kv_ring_append, so the
 * caches hold rotated keys); queries before every attention call.
 * Requires D % 8 == 0 and D <= 256.  Device-side precondition: positions are
 * >= 0 and below 2^31.  B == 0, S == 0 or rot_dim == 0 is a no-op.
 */
SWA_API swa_status_t swa_rope_apply(void *x, const int32_t *pos0, int pos_offset,
                            int B, int S, int H, int D, int rot_dim, float base,
                            swa_dtype_t dtype, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* SWA_ATTN_H */
