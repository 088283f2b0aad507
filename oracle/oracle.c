/*
 * CPU oracle for sliding-window / global causal attention with a per-head
 * attention sink.  TEST INFRASTRUCTURE ONLY: the tests, the smoke check and
 * the benchmark's CPU-baseline leg call it; the GPU library never does.  It
 * shares no code, header, table or helper with the GPU path.
 *
 * Plain C99 + OpenMP.  Inputs arrive as fp32 (the exact upcast of bf16 or
 * fp32 data); every step is computed in fp64 with libm's exp/log, two-pass
 * (all scores, then their maximum, then the normaliser, then the output).
 *
 * What is computed (the plain definition the GPU kernels must reproduce):
 *   For request b, query head h and a query at absolute position i:
 *     g     = h / (Hq / Hkv)                    contiguous GQA groups
 *     J(i)  = { j : max(0, i - W + 1) <= j <= i }   W keys including self;
 *             { j : 0 <= j <= i } when W <= 0 (global attention)
 *     s_j   = sm_scale * sum_d q[d] * K[j, g, d]
 *     m     = max(sink_h, max_{j in J} s_j)
 *     Z     = exp(sink_h - m) + sum_{j in J} exp(s_j - m)
 *     O[d]  = sum_{j in J} exp(s_j - m) / Z * V[j, g, d]
 *   The sink adds exp(sink_h) to the softmax denominator and carries no
 *   value; no sink (NULL) removes that term.
 *
 * Sources (the web pages on MiMo-V2-Flash):
 *   - sliding window of W = 128 tokens interleaved with global attention
 *     5:1: MiMo-V2-Flash technical-report digest (fanfer.top), section
 *     "MiMo-V2-Flash Model Architecture"; release blog (aihot.news), section
 *     on pushing efficiency to the limit.
 *   - learnable attention-sink bias in the gpt-oss style: technical-report
 *     digest, paragraph "Hybrid Sliding Window Attention Architecture" (its
 *     formula image is missing; the reading above is the gpt-oss one).
 *   - verify of 1 committed + 3 draft tokens in one pass, and the
 *     accept/accept/reject/discard example: release blog, section
 *     "Multi-Token Prediction" (verify diagram).
 *   - fixed-size SWA KV cache: release blog, section on pushing efficiency.
 * Readings where the pages are silent (window edge, GQA grouping, causal
 * offsets, cache layout) are listed with the design notes of the repository.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* Error codes of the oracle entry points. */
#define ORC_OK 0
#define ORC_BAD_ARGS 1
#define ORC_HISTORY_SHORT 2
#define ORC_NO_MEMORY 3

int oracle_num_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/*
 * One query vector against a key set made of up to two segments (segment A,
 * then segment B), each a run of consecutive rows with a row stride in
 * floats.  Writes O[D]; optionally the log of the full denominator
 * (log(exp(sink) + sum exp(s_j))), the sink's probability mass and the
 * per-key weights (in key order: segment A then segment B).
 * `sbuf` must hold nA + nB doubles.
 */
static void attend(const float *qv, int D, double scale, const double *sink,
                   const float *kA, const float *vA, long nA, long strideA,
                   const float *kB, const float *vB, long nB, long strideB,
                   double *out, double *lse_out, double *psink_out, double *w_out,
                   double *sbuf)
{
    long n = nA + nB;
    long j;
    int d;

    /* 1. scores s_j = scale * <q, k_j> */
    for (j = 0; j < n; ++j) {
        const float *kr = (j < nA) ? kA + j * strideA : kB + (j - nA) * strideB;
        double acc = 0.0;
        for (d = 0; d < D; ++d)
            acc += (double)qv[d] * (double)kr[d];
        sbuf[j] = scale * acc;
    }

    /* 2. maximum over the sink logit and the scores */
    double m = sink ? *sink : -INFINITY;
    for (j = 0; j < n; ++j)
        if (sbuf[j] > m)
            m = sbuf[j];

    /* 3. normaliser: the sink's exp term plus every key's */
    double z = sink ? exp(*sink - m) : 0.0;
    for (j = 0; j < n; ++j)
        z += exp(sbuf[j] - m);

    /* 4. output: weighted sum of value rows (the sink contributes no value) */
    for (d = 0; d < D; ++d)
        out[d] = 0.0;
    for (j = 0; j < n; ++j) {
        const float *vr = (j < nA) ? vA + j * strideA : vB + (j - nA) * strideB;
        double w = exp(sbuf[j] - m) / z;
        if (w_out)
            w_out[j] = w;
        for (d = 0; d < D; ++d)
            out[d] += w * (double)vr[d];
    }
    if (lse_out)
        *lse_out = m + log(z);
    if (psink_out)
        *psink_out = sink ? exp(*sink - m) / z : 0.0;
}

/* Lowest key position of the window of a query at position i. */
static long window_lo(long i, int window)
{
    if (window <= 0)
        return 0;
    long lo = i - (long)window + 1;
    return lo < 0 ? 0 : lo;
}

/*
 * Prefill over whole tensors.
 *   q [B, Sq, Hq, D], k/v [B, Sk, Hkv, D] (fp32), sinks [Hq] or NULL,
 *   o [B, Sq, Hq, D] (fp64).  Query row r sits at position q_offset + r.
 *   lse, psink: optional [B, Sq, Hq].  weights: optional [B, Sq, Hq, Sk],
 *   zero outside the window.
 */
int oracle_prefill(const float *q, const float *k, const float *v, const double *sinks,
                   double *o, double *lse, double *psink, double *weights,
                   int B, int Sq, int Sk, int Hq, int Hkv, int D,
                   int window, int q_offset, double sm_scale)
{
    if (B < 0 || Sq < 0 || Sk < 0 || Hq <= 0 || Hkv <= 0 || D <= 0 || Hq % Hkv != 0 ||
        q_offset < 0 || (long)q_offset + Sq > Sk)
        return ORC_BAD_ARGS;
    const int G = Hq / Hkv;
    const long total = (long)B * Sq * Hq;
    int err = ORC_OK;

#pragma omp parallel
    {
        double *sbuf = (double *)malloc(sizeof(double) * (size_t)(Sk > 0 ? Sk : 1));
        double *wbuf = weights ? (double *)malloc(sizeof(double) * (size_t)(Sk > 0 ? Sk : 1)) : NULL;
        if (!sbuf || (weights && !wbuf)) {
#pragma omp atomic write
            err = ORC_NO_MEMORY;
        } else {
            long idx;
#pragma omp for schedule(dynamic, 16)
            for (idx = 0; idx < total; ++idx) {
                long b = idx / ((long)Sq * Hq);
                long r = (idx / Hq) % Sq;
                int h = (int)(idx % Hq);
                int g = h / G;
                long i = (long)q_offset + r;
                long lo = window_lo(i, window);
                long n = i - lo + 1;
                const float *qv = q + ((b * Sq + r) * Hq + h) * (long)D;
                const float *kb = k + ((b * Sk + lo) * Hkv + g) * (long)D;
                const float *vb = v + ((b * Sk + lo) * Hkv + g) * (long)D;
                double *ov = o + ((b * Sq + r) * Hq + h) * (long)D;
                long row = (b * Sq + r) * Hq + h;
                attend(qv, D, sm_scale, sinks ? &sinks[h] : NULL,
                       kb, vb, n, (long)Hkv * D, NULL, NULL, 0, 0,
                       ov, lse ? &lse[row] : NULL, psink ? &psink[row] : NULL,
                       wbuf, sbuf);
                if (weights) {
                    double *wr = weights + row * (long)Sk;
                    memset(wr, 0, sizeof(double) * (size_t)Sk);
                    memcpy(wr + lo, wbuf, sizeof(double) * (size_t)n);
                }
            }
        }
        free(sbuf);
        free(wbuf);
    }
    return err;
}

/*
 * Prefill for selected query rows of one request.
 *   q_rows [n, Hq, D]: the query vectors of rows rows[0..n-1] (row r sits at
 *   position q_offset + r).  k/v [nk, Hkv, D] hold key positions
 *   k_base .. k_base + nk - 1.  o [n, Hq, D] (fp64).
 * Returns ORC_HISTORY_SHORT if a needed key lies outside the given slice.
 */
int oracle_prefill_rows(const float *q_rows, const int64_t *rows, long n,
                        const float *k, const float *v, long k_base, long nk,
                        const double *sinks, double *o,
                        int Hq, int Hkv, int D, int window, long q_offset, double sm_scale)
{
    if (n < 0 || Hq <= 0 || Hkv <= 0 || D <= 0 || Hq % Hkv != 0 || nk < 0 || k_base < 0)
        return ORC_BAD_ARGS;
    const int G = Hq / Hkv;
    long idx;
    for (idx = 0; idx < n; ++idx) {
        long i = q_offset + rows[idx];
        if (window_lo(i, window) < k_base || i >= k_base + nk)
            return ORC_HISTORY_SHORT;
    }
    const long total = n * Hq;
    int err = ORC_OK;
#pragma omp parallel
    {
        double *sbuf = (double *)malloc(sizeof(double) * (size_t)(nk > 0 ? nk : 1));
        if (!sbuf) {
#pragma omp atomic write
            err = ORC_NO_MEMORY;
        } else {
            long t;
#pragma omp for schedule(dynamic, 4)
            for (t = 0; t < total; ++t) {
                long a = t / Hq;
                int h = (int)(t % Hq);
                int g = h / G;
                long i = q_offset + rows[a];
                long lo = window_lo(i, window);
                const float *kb = k + ((lo - k_base) * Hkv + g) * (long)D;
                const float *vb = v + ((lo - k_base) * Hkv + g) * (long)D;
                attend(q_rows + (a * Hq + h) * (long)D, D, sm_scale, sinks ? &sinks[h] : NULL,
                       kb, vb, i - lo + 1, (long)Hkv * D, NULL, NULL, 0, 0,
                       o + (a * Hq + h) * (long)D, NULL, NULL, NULL, sbuf);
            }
        }
        free(sbuf);
    }
    return err;
}

/*
 * Verify: q_len = T new tokens per request, scored in one pass.
 *   Request b has L_b = cache_len[b] committed tokens.  Its logical history
 *   k_hist/v_hist [B, Hlen, Hkv, D] holds position hist_base[b] + r in row r
 *   (only rows for positions < L_b are read).  The T tokens under
 *   verification sit at positions L_b .. L_b + T - 1 with keys/values
 *   k_new/v_new [B, T, Hkv, D].  Query t (q [B, T, Hq, D]) sees history
 *   positions and new tokens u <= t inside its window.  o [B, T, Hq, D].
 * The oracle reads the logical history only, never a ring layout.
 */
int oracle_verify(const float *q, const float *k_new, const float *v_new,
                  const float *k_hist, const float *v_hist, const int64_t *hist_base,
                  const int64_t *cache_len, const double *sinks, double *o,
                  int B, int T, int Hq, int Hkv, int D, long Hlen, int window, double sm_scale)
{
    if (B < 0 || T <= 0 || Hq <= 0 || Hkv <= 0 || D <= 0 || Hq % Hkv != 0 || Hlen < 0)
        return ORC_BAD_ARGS;
    const int G = Hq / Hkv;
    int b;
    for (b = 0; b < B; ++b) {
        long L = cache_len[b];
        if (L < 0 || hist_base[b] < 0 || hist_base[b] > L)
            return ORC_BAD_ARGS;
        /* the lowest window position over the T queries is that of t = 0 */
        long lo = window_lo(L, window);
        if (lo < L && (lo < hist_base[b] || L - hist_base[b] > Hlen))
            return ORC_HISTORY_SHORT;
    }
    const long total = (long)B * T * Hq;
    int err = ORC_OK;
#pragma omp parallel
    {
        double *sbuf = (double *)malloc(sizeof(double) * (size_t)(Hlen + T + 1));
        if (!sbuf) {
#pragma omp atomic write
            err = ORC_NO_MEMORY;
        } else {
            long idx;
#pragma omp for schedule(dynamic, 4)
            for (idx = 0; idx < total; ++idx) {
                long bb = idx / ((long)T * Hq);
                long t = (idx / Hq) % T;
                int h = (int)(idx % Hq);
                int g = h / G;
                long L = cache_len[bb];
                long i = L + t;
                long lo = window_lo(i, window);
                /* segment A: committed positions lo .. L-1 from the history */
                long nA = lo < L ? L - lo : 0;
                long rowA = lo - hist_base[bb];
                const float *kA = k_hist + ((bb * Hlen + (nA ? rowA : 0)) * Hkv + g) * (long)D;
                const float *vA = v_hist + ((bb * Hlen + (nA ? rowA : 0)) * Hkv + g) * (long)D;
                /* segment B: new tokens u0 .. t (u0 > 0 only if the window is shorter than t+1) */
                long u0 = lo > L ? lo - L : 0;
                long nB = t - u0 + 1;
                const float *kB = k_new + ((bb * T + u0) * Hkv + g) * (long)D;
                const float *vB = v_new + ((bb * T + u0) * Hkv + g) * (long)D;
                attend(q + ((bb * T + t) * Hq + h) * (long)D, D, sm_scale,
                       sinks ? &sinks[h] : NULL,
                       kA, vA, nA, (long)Hkv * D, kB, vB, nB, (long)Hkv * D,
                       o + ((bb * T + t) * Hq + h) * (long)D, NULL, NULL, NULL, sbuf);
            }
        }
        free(sbuf);
    }
    return err;
}

/*
 * Commit accepted tokens to a KV cache (bytewise copy, any element size).
 *   caches [B, slots, Hkv, D], new rows [B, T, Hkv, D].  For every request b
 *   and every t < n_append[b], the row of position p = cache_len[b] + t goes
 *   to slot p % slots (ring) or slot p (linear); nothing else changes.
 *   Accepting a prefix of the drafts and discarding the rest follows the
 *   verify diagram of the release blog, section "Multi-Token Prediction".
 */
int oracle_ring_append(unsigned char *k_cache, unsigned char *v_cache,
                       const unsigned char *k_new, const unsigned char *v_new,
                       const int64_t *cache_len, const int64_t *n_append,
                       int B, int T, int Hkv, int D, long slots, int ring, int elem_bytes)
{
    if (B < 0 || T < 0 || Hkv <= 0 || D <= 0 || slots <= 0 || elem_bytes <= 0)
        return ORC_BAD_ARGS;
    const size_t rowb = (size_t)Hkv * D * elem_bytes;
    int b;
    for (b = 0; b < B; ++b) {
        long t;
        if (n_append[b] < 0 || n_append[b] > T || cache_len[b] < 0)
            return ORC_BAD_ARGS;
        for (t = 0; t < n_append[b]; ++t) {
            long p = cache_len[b] + t;
            long slot = ring ? p % slots : p;
            if (slot >= slots)
                return ORC_BAD_ARGS;
            memcpy(k_cache + ((size_t)b * slots + slot) * rowb, k_new + ((size_t)b * T + t) * rowb, rowb);
            memcpy(v_cache + ((size_t)b * slots + slot) * rowb, v_new + ((size_t)b * T + t) * rowb, rowb);
        }
    }
    return ORC_OK;
}

/*
 * Greedy acceptance of draft tokens after a verify pass (self-speculative
 * decoding with the MTP heads as the draft model: release blog, section
 * "Multi-Token Prediction", and its verify diagram).
 *   logits [B, T, V]: the target model's scores at the T positions under
 *   verification; draft [B, T - 1]: the token proposed for position t + 1.
 *   target[b, t] = argmax_v logits[b, t, v]  (the lowest index among equal
 *   maxima).  Draft t is accepted when target[b, t] == draft[b, t] and every
 *   earlier draft was accepted.  n_append[b] = 1 + accepted: the first
 *   verified token (already committed by the model) plus the accepted drafts
 *   are the rows whose K/V join the cache.
 */
int oracle_greedy_accept(const float *logits, const int32_t *draft, int B, int T, long V,
                         int32_t *target, int32_t *n_append)
{
    if (B < 0 || T < 1 || V < 1)
        return ORC_BAD_ARGS;
    int b;
    for (b = 0; b < B; ++b) {
        int t, accepted = 0, open = 1;
        for (t = 0; t < T; ++t) {
            const float *row = logits + ((size_t)b * T + t) * (size_t)V;
            long best = 0, v;
            for (v = 1; v < V; ++v)
                if (row[v] > row[best])
                    best = v;
            target[(size_t)b * T + t] = (int32_t)best;
        }
        for (t = 0; t + 1 < T && open; ++t) {
            if (target[(size_t)b * T + t] == draft[(size_t)b * (T - 1) + t])
                ++accepted;
            else
                open = 0;
        }
        n_append[b] = 1 + accepted;
    }
    return ORC_OK;
}

/*
 * Partial rotary position embedding on the query / key rows.
 *   Technical-report digest, "Pre-training" (long-context extension): RoPE
 *   base 10000 for the sliding-window layers, 640000 for the global layers,
 *   raised to 5000000 for the 256K stage; the model card's config extract
 *   ("lightweight multi-token prediction" section of the model download
 *   page) gives partial_rotary_factor 0.334.
 * Readings (the pages fix neither): only the first `rot` dimensions of each
 * head rotate, in rot/2 pairs (i, i + rot/2) (the half-split pairing), with
 * pair i turned by the angle pos * base^(-2i / rot); the other dimensions pass
 * through.  x, out: [rows, H, D]; pos[r] is the position of row r.
 *   out[i]         = x[i] cos(a_i) - x[i + rot/2] sin(a_i)
 *   out[i + rot/2] = x[i + rot/2] cos(a_i) + x[i] sin(a_i)
 */
int oracle_rope(const double *x, double *out, const int64_t *pos, long rows, int H, int D,
                int rot, double base)
{
    if (rows < 0 || H <= 0 || D <= 0 || rot < 0 || rot > D || (rot & 1) || !(base > 0.0))
        return ORC_BAD_ARGS;
    const int half = rot / 2;
    long r;
#pragma omp parallel for schedule(static)
    for (r = 0; r < rows; ++r) {
        int h, i;
        for (h = 0; h < H; ++h) {
            const double *xr = x + ((size_t)r * H + h) * D;
            double *orow = out + ((size_t)r * H + h) * D;
            for (i = 0; i < D; ++i)
                orow[i] = xr[i];
            for (i = 0; i < half; ++i) {
                const double angle = (double)pos[r] * pow(base, -2.0 * i / rot);
                const double c = cos(angle), s = sin(angle);
                const double a = xr[i], b = xr[i + half];
                orow[i] = a * c - b * s;
                orow[i + half] = b * c + a * s;
            }
        }
    }
    return ORC_OK;
}

/*
 * Backward of the prefill: gradients of L = sum(dout * O) with respect to q,
 * k, v and the sinks (the definition above differentiated; the pages give
 * no training kernel, and the MTP-accelerated RL training the report digest
 * describes in "Model Architecture" needs these gradients).
 *   For a query row with weights w_j (the softmax over its window with the
 *   sink in the denominator), sink mass p_s and output O:
 *     delta  = <dout, O>
 *     dP_j   = <dout, V_j>
 *     dS_j   = w_j * (dP_j - delta)
 *     dq     = sm_scale * sum_j dS_j K_j
 *     dK_j  += sm_scale * dS_j q         dV_j += w_j * dout
 *     dsink_h += -p_s * delta            (the sink logit is not scaled and
 *                                         carries no value)
 *   q, dout [B, Sq, Hq, D]; k, v [B, Sk, Hkv, D] (fp32 in); dq, dk, dv fp64 of
 *   the same shapes; dsink [Hq] fp64 (ignored when sinks == NULL).
 * One thread owns every query row of a (request, KV head), so the key
 * gradients need no atomics; per-request sink gradients are summed last.
 */
int oracle_prefill_backward(const float *q, const float *k, const float *v, const double *sinks,
                            const float *dout, double *dq, double *dk, double *dv, double *dsink,
                            int B, int Sq, int Sk, int Hq, int Hkv, int D,
                            int window, int q_offset, double sm_scale)
{
    if (B < 0 || Sq < 0 || Sk < 0 || Hq <= 0 || Hkv <= 0 || D <= 0 || Hq % Hkv != 0 ||
        q_offset < 0 || (long)q_offset + Sq > Sk)
        return ORC_BAD_ARGS;
    const int G = Hq / Hkv;
    const long groups = (long)B * Hkv;
    double *dsink_b = (double *)calloc((size_t)B * Hq + 1, sizeof(double));
    if (!dsink_b)
        return ORC_NO_MEMORY;
    memset(dk, 0, sizeof(double) * (size_t)B * Sk * Hkv * D);
    memset(dv, 0, sizeof(double) * (size_t)B * Sk * Hkv * D);
    int err = ORC_OK;

#pragma omp parallel
    {
        double *sbuf = (double *)malloc(sizeof(double) * (size_t)(Sk > 0 ? Sk : 1));
        double *wbuf = (double *)malloc(sizeof(double) * (size_t)(Sk > 0 ? Sk : 1));
        double *obuf = (double *)malloc(sizeof(double) * (size_t)D);
        if (!sbuf || !wbuf || !obuf) {
#pragma omp atomic write
            err = ORC_NO_MEMORY;
        } else {
            long bg;
#pragma omp for schedule(dynamic, 1)
            for (bg = 0; bg < groups; ++bg) {
                const long b = bg / Hkv;
                const int g = (int)(bg % Hkv);
                long r;
                int hh, d;
                for (r = 0; r < Sq; ++r) {
                    for (hh = 0; hh < G; ++hh) {
                        const int h = g * G + hh;
                        const long i = (long)q_offset + r;
                        const long lo = window_lo(i, window);
                        const long n = i - lo + 1;
                        const long row = (b * Sq + r) * Hq + h;
                        const float *qv = q + row * (long)D;
                        const float *go = dout + row * (long)D;
                        const float *kb = k + ((b * Sk + lo) * Hkv + g) * (long)D;
                        const float *vb = v + ((b * Sk + lo) * Hkv + g) * (long)D;
                        double psink = 0.0;
                        attend(qv, D, sm_scale, sinks ? &sinks[h] : NULL, kb, vb, n, (long)Hkv * D,
                               NULL, NULL, 0, 0, obuf, NULL, &psink, wbuf, sbuf);
                        double delta = 0.0;
                        for (d = 0; d < D; ++d)
                            delta += (double)go[d] * obuf[d];
                        double *dqv = dq + row * (long)D;
                        for (d = 0; d < D; ++d)
                            dqv[d] = 0.0;
                        long j;
                        for (j = 0; j < n; ++j) {
                            const float *kr = kb + j * (long)Hkv * D;
                            const float *vr = vb + j * (long)Hkv * D;
                            double dp = 0.0;
                            for (d = 0; d < D; ++d)
                                dp += (double)go[d] * (double)vr[d];
                            const double ds = wbuf[j] * (dp - delta);
                            double *dkr = dk + ((b * Sk + lo + j) * Hkv + g) * (long)D;
                            double *dvr = dv + ((b * Sk + lo + j) * Hkv + g) * (long)D;
                            for (d = 0; d < D; ++d) {
                                dqv[d] += sm_scale * ds * (double)kr[d];
                                dkr[d] += sm_scale * ds * (double)qv[d];
                                dvr[d] += wbuf[j] * (double)go[d];
                            }
                        }
                        dsink_b[b * Hq + h] += -psink * delta;
                    }
                }
            }
        }
        free(sbuf);
        free(wbuf);
        free(obuf);
    }
    if (dsink) {
        int h;
        long b;
        for (h = 0; h < Hq; ++h) {
            double acc = 0.0;
            for (b = 0; b < B; ++b)
                acc += dsink_b[b * Hq + h];
            dsink[h] = sinks ? acc : 0.0;
        }
    }
    free(dsink_b);
    return err;
}
