/*
 * q8kv_oracle.c -- plain, slow CPU oracle for q8 single-query decode attention.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path may include, link,
 * load or call this file.  It shares no code, header, constant table or helper
 * with the HIP library; the only thing both sides see are the seeded inputs.
 *
 * Sources (web pages, cited by title and section):
 *   [9-2]  "0.8MB 跑通 Qwen | 第 9-2 篇: flash_attn_single_q_q8_neon -- 单 q 单遍扫全 KV"
 *          (developer.aliyun.com article 1767760): §1 (why one pass suffices),
 *          §2 segment 1 (Q quantized once in 32-element blocks),
 *          §2 segment 2 (per-token score and online softmax over blocked q8 KV),
 *          §2 segment 3 (single division at the end), §3 (two-pass equivalence),
 *          §4 (debug observables: loop count, M non-decreasing).
 *   [9-3]  "q8 KV 精度对照实验" (www.0539edu.com news 4660027): §1 (reference
 *          attention: scores, max-subtracted softmax, weighted V), §2 (the
 *          kv_quantize_per_head write rule), §3 (printed fp32-vs-q8 gap).
 *
 * Readings of points the pages leave open (each one is listed with its reason
 * in the design notes of this repository):
 *   - K/V row quantizer: d = a * fl(1/127), r = 127/a (IEEE fp32 division),
 *     code = clamp(roundf(x * r), -127, 127), roundf = half away from zero.
 *     The stored per-(token, head) value is d (the max-abs/127 step).
 *   - Rows with max-abs a < 1e-6 use a = 1 (same guard the Q quantizer prints).
 *   - Q quantizer: code = truncation toward zero of clamp(q * r, -128, 127)
 *     (the printed conversion has no rounding call).
 *   - Query head h reads KV head h / (nq / nkv).
 *   - A sequence of length 0 gives an all-zero output row.
 *
 * Arithmetic: every fp32 step of the quantizers is a single IEEE operation
 * (built with -ffp-contract=off, no fast-math) so that codes and scales are a
 * bit-exact definition.  Attention runs in double over values dequantized
 * exactly in double (an int8 code times an fp32 scale needs at most 32
 * significant bits), so the only roundings are the double ones and the final
 * conversion of the output to fp32.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* fl(1/127): the step multiplier both quantizers use ([9-2] §2 segment 1). */
static const float ORC_INV127 = 1.0f / 127.0f;
/* Guard: a block or row whose max-abs is below this is treated as max-abs 1. */
static const float ORC_GUARD = 1e-6f;

/* ---------------------------------------------------------------- O1 ----- */
/* Per-(token, KV head) quantizer of one row of hd values ([9-3] §2: one scale
 * shared by the head's hd dimensions; scale = max-abs/127, code = round(x /
 * scale) clamped to [-127, 127], dequantized value = code * scale). */
void orc_quantize_kv_row(const float *x, int hd, int8_t *codes, float *step)
{
    float a = 0.0f;
    for (int i = 0; i < hd; ++i) {
        float m = fabsf(x[i]);
        if (m > a) a = m;
    }
    if (a < ORC_GUARD) a = 1.0f;
    float d = a * ORC_INV127;     /* stored step */
    float r = 127.0f / a;         /* reciprocal step, one correctly rounded division */
    for (int i = 0; i < hd; ++i) {
        float y = x[i] * r;       /* one fp32 product, not fused with anything */
        float c = roundf(y);
        if (c > 127.0f) c = 127.0f;
        if (c < -127.0f) c = -127.0f;
        codes[i] = (int8_t)c;
    }
    *step = d;
}

void orc_quantize_kv_rows(const float *x, int64_t rows, int hd, int8_t *codes, float *steps)
{
    for (int64_t r = 0; r < rows; ++r)
        orc_quantize_kv_row(x + r * hd, hd, codes + r * hd, steps + r);
}

/* ---------------------------------------------------------------- O2 ----- */
/* Q quantizer ([9-2] §2 segment 1): the query row is cut into blocks of 32;
 * each block gets its own max-abs m (guarded to 1 below 1e-6), block scale
 * qsc = m * fl(1/127), and codes = trunc(clamp(q * (127/m), -128, 127)). */
void orc_quantize_q(const float *q, int hd, int8_t *codes, float *qsc)
{
    for (int blk = 0; blk < hd / 32; ++blk) {
        const float *qb = q + 32 * blk;
        float m = 0.0f;
        for (int i = 0; i < 32; ++i) {
            float v = fabsf(qb[i]);
            if (v > m) m = v;
        }
        if (m < ORC_GUARD) m = 1.0f;
        qsc[blk] = m * ORC_INV127;
        float r = 127.0f / m;
        for (int i = 0; i < 32; ++i) {
            float y = qb[i] * r;
            if (y > 127.0f) y = 127.0f;
            if (y < -128.0f) y = -128.0f;
            codes[32 * blk + i] = (int8_t)y;   /* C conversion truncates toward zero */
        }
    }
}

void orc_quantize_q_rows(const float *q, int64_t rows, int hd, int8_t *codes, float *qsc)
{
    for (int64_t r = 0; r < rows; ++r)
        orc_quantize_q(q + r * hd, hd, codes + r * hd, qsc + r * (hd / 32));
}

/* ---------------------------------------------------------------- O3 ----- */
/* Exact integer dot product of each 32-element block of Q codes with the same
 * block of K codes ([9-2] §2 segment 2: one int32 sum per 32-block, rescaled
 * by that block's Q scale afterwards).  Summed in int64; returns 1 if any
 * block sum would not fit int32, else 0. */
int orc_block_partials(const int8_t *cq, const int8_t *ck, int hd, int32_t *out)
{
    int overflow = 0;
    for (int blk = 0; blk < hd / 32; ++blk) {
        int64_t s = 0;
        for (int i = 32 * blk; i < 32 * blk + 32; ++i)
            s += (int64_t)cq[i] * (int64_t)ck[i];
        if (s > INT32_MAX || s < INT32_MIN) overflow = 1;
        out[blk] = (int32_t)s;
    }
    return overflow;
}

/* ----------------------------------------------------------- O5 - O7 ----- */
/* Textbook attention for one query over n keys, three passes ([9-3] §1 and
 * [9-2] §1): all scores s_t = scale * <q, k_t>; then m = max s, w_t =
 * exp(s_t - m), S = sum w_t; then out = sum w_t v_t / S.  Everything double.
 * n == 0 gives a zero vector. */
void orc_attend_dense(const double *q, const double *k, const double *v,
                      int64_t n, int hd, double scale, double *out)
{
    for (int i = 0; i < hd; ++i) out[i] = 0.0;
    if (n <= 0) return;
    double *s = (double *)malloc(sizeof(double) * (size_t)n);
    /* pass 1: scores */
    for (int64_t t = 0; t < n; ++t) {
        double dot = 0.0;
        for (int i = 0; i < hd; ++i) dot += q[i] * k[t * hd + i];
        s[t] = scale * dot;
    }
    /* pass 2: max, weights, sum */
    double m = s[0];
    for (int64_t t = 1; t < n; ++t)
        if (s[t] > m) m = s[t];
    double S = 0.0;
    for (int64_t t = 0; t < n; ++t) {
        s[t] = exp(s[t] - m);
        S += s[t];
    }
    /* pass 3: weighted V, one division */
    for (int64_t t = 0; t < n; ++t)
        for (int i = 0; i < hd; ++i) out[i] += s[t] * v[t * hd + i];
    for (int i = 0; i < hd; ++i) out[i] /= S;
    free(s);
}

/* ---------------------------------------------------------------- O8 ----- */
/* Blocked KV layout ([9-2] §2 segment 2: token t lives in block t / kv_bs at
 * row t % kv_bs; a row holds all KV heads, head kh at offset kh * hd).
 * Physical block ids come from a per-sequence block table.
 *   k_codes, v_codes : [num_blocks][kv_bs][nkv * hd] int8
 *   k_step,  v_step  : [num_blocks][kv_bs][nkv]      fp32 (the stored d)
 * Returns the flat row index (block * kv_bs + row), or -1 if the block id is
 * outside [0, num_blocks). */
static int64_t orc_row_of(const int32_t *block_table, int max_blocks_per_seq, int b,
                          int64_t t, int kv_bs, int num_blocks)
{
    int32_t blk = block_table[(int64_t)b * max_blocks_per_seq + t / kv_bs];
    if (blk < 0 || blk >= num_blocks) return -1;
    return (int64_t)blk * kv_bs + t % kv_bs;
}

/* ------------------------------------------------------------ O4 + O8 ---- */
/* One (sequence b, query head h) of decode attention over the blocked q8
 * cache: quantize q (O2), dequantize the query and every visible key/value
 * row of KV head h / (nq/nkv) exactly (code times its scale, in double), then
 * run the three-pass attention.  Writes hd fp32 values to o (zeros when the
 * length is 0).  Returns 0, or -1 on a bad length or block id (o = zeros). */
static int orc_one_row_n(int b, int h, int nq, int nkv, int hd, int kv_bs,
                         const int32_t *block_table, int max_blocks_per_seq, int64_t n, int num_blocks,
                         const int8_t *k_codes, const int8_t *v_codes,
                         const float *k_step, const float *v_step,
                         const float *q_row, float scale, float *o)
{
    int kh = h / (nq / nkv);
    for (int i = 0; i < hd; ++i) o[i] = 0.0f;
    if (n < 0 || n > (int64_t)max_blocks_per_seq * kv_bs) return -1;
    if (n == 0) return 0;
    int8_t *cq = (int8_t *)malloc((size_t)hd);
    float *qsc = (float *)malloc(sizeof(float) * (size_t)(hd / 32));
    double *qh = (double *)malloc(sizeof(double) * (size_t)hd);
    double *kk = (double *)malloc(sizeof(double) * (size_t)(n * hd));
    double *vv = (double *)malloc(sizeof(double) * (size_t)(n * hd));
    double *oh = (double *)malloc(sizeof(double) * (size_t)hd);
    orc_quantize_q(q_row, hd, cq, qsc);
    for (int i = 0; i < hd; ++i) qh[i] = (double)cq[i] * (double)qsc[i / 32];
    int rc = 0;
    for (int64_t t = 0; t < n; ++t) {
        int64_t r = orc_row_of(block_table, max_blocks_per_seq, b, t, kv_bs, num_blocks);
        if (r < 0) { rc = -1; break; }
        const int8_t *ck = k_codes + (r * nkv + kh) * hd;
        const int8_t *cv = v_codes + (r * nkv + kh) * hd;
        double dk = (double)k_step[r * nkv + kh];
        double dv = (double)v_step[r * nkv + kh];
        for (int i = 0; i < hd; ++i) {
            kk[t * hd + i] = (double)ck[i] * dk;
            vv[t * hd + i] = (double)cv[i] * dv;
        }
    }
    if (rc == 0) {
        orc_attend_dense(qh, kk, vv, n, hd, (double)scale, oh);
        for (int i = 0; i < hd; ++i) o[i] = (float)oh[i];
    }
    free(cq); free(qsc); free(qh); free(kk); free(vv); free(oh);
    return rc;
}

/* The same over the sequence's whole visible history (n = seq_lens[b]). */
static int orc_one_row(int b, int h, int nq, int nkv, int hd, int kv_bs,
                       const int32_t *block_table, int max_blocks_per_seq,
                       const int32_t *seq_lens, int num_blocks,
                       const int8_t *k_codes, const int8_t *v_codes,
                       const float *k_step, const float *v_step,
                       const float *q_row, float scale, float *o)
{
    return orc_one_row_n(b, h, nq, nkv, hd, kv_bs, block_table, max_blocks_per_seq, seq_lens[b], num_blocks,
                         k_codes, v_codes, k_step, v_step, q_row, scale, o);
}

/* Every (b, h) of a batch.  q, out: [batch][nq][hd] fp32.  Returns 0, or -1
 * if any row had a bad length or block id (those rows are zeros). */
int orc_decode_attn(int batch, int nq, int nkv, int hd, int kv_bs,
                    const int32_t *block_table, int max_blocks_per_seq,
                    const int32_t *seq_lens, int num_blocks,
                    const int8_t *k_codes, const int8_t *v_codes,
                    const float *k_step, const float *v_step,
                    const float *q, float scale, float *out, int nthreads)
{
    int status = 0;
    int64_t rows = (int64_t)batch * nq;
    if (nthreads < 1) nthreads = 1;
#pragma omp parallel for schedule(dynamic, 1) num_threads(nthreads)
    for (int64_t bh = 0; bh < rows; ++bh) {
        int rc = orc_one_row((int)(bh / nq), (int)(bh % nq), nq, nkv, hd, kv_bs,
                             block_table, max_blocks_per_seq, seq_lens, num_blocks,
                             k_codes, v_codes, k_step, v_step,
                             q + bh * hd, scale, out + bh * hd);
        if (rc) {
#pragma omp atomic write
            status = -1;
        }
    }
    return status;
}

/* The same, for a chosen list of rows only (rows_bh[r] = b * nq + h), so that
 * a full-size batch can be checked on samples.  out: [n_rows][hd]. */
int orc_decode_attn_rows(int nq, int nkv, int hd, int kv_bs,
                         const int32_t *block_table, int max_blocks_per_seq,
                         const int32_t *seq_lens, int num_blocks,
                         const int8_t *k_codes, const int8_t *v_codes,
                         const float *k_step, const float *v_step,
                         const float *q, float scale,
                         const int64_t *rows_bh, int n_rows, float *out, int nthreads)
{
    int status = 0;
    if (nthreads < 1) nthreads = 1;
#pragma omp parallel for schedule(dynamic, 1) num_threads(nthreads)
    for (int r = 0; r < n_rows; ++r) {
        int64_t bh = rows_bh[r];
        int rc = orc_one_row((int)(bh / nq), (int)(bh % nq), nq, nkv, hd, kv_bs,
                             block_table, max_blocks_per_seq, seq_lens, num_blocks,
                             k_codes, v_codes, k_step, v_step,
                             q + bh * hd, scale, out + (int64_t)r * hd);
        if (rc) {
#pragma omp atomic write
            status = -1;
        }
    }
    return status;
}

/* ------------------------------------------------------------ O10 ------- */
/* The fp32 mirror cache and its exact attention ([9-3] §3 closing note: the
 * engine also stores every new K/V row in a float cache, so quantized and
 * exact attention coexist; [9-3] §1: the exact baseline is the standard
 * attention over the raw fp32 K/V).  Mirror layout = the code layout with
 * fp32 elements: [num_blocks][kv_bs][nkv * hd].  The query is used as given
 * (no quantization); everything else as O5-O8: one (b, h) row, three passes
 * in double, zeros for length 0, -1 on a bad length or block id. */
static int orc_one_row_f32(int b, int h, int nq, int nkv, int hd, int kv_bs,
                           const int32_t *block_table, int max_blocks_per_seq,
                           const int32_t *seq_lens, int num_blocks,
                           const float *k_f32, const float *v_f32,
                           const float *q_row, float scale, float *o)
{
    int kh = h / (nq / nkv);
    int64_t n = seq_lens[b];
    for (int i = 0; i < hd; ++i) o[i] = 0.0f;
    if (n < 0 || n > (int64_t)max_blocks_per_seq * kv_bs) return -1;
    if (n == 0) return 0;
    double *qh = (double *)malloc(sizeof(double) * (size_t)hd);
    double *kk = (double *)malloc(sizeof(double) * (size_t)(n * hd));
    double *vv = (double *)malloc(sizeof(double) * (size_t)(n * hd));
    double *oh = (double *)malloc(sizeof(double) * (size_t)hd);
    for (int i = 0; i < hd; ++i) qh[i] = (double)q_row[i];
    int rc = 0;
    for (int64_t t = 0; t < n; ++t) {
        int64_t r = orc_row_of(block_table, max_blocks_per_seq, b, t, kv_bs, num_blocks);
        if (r < 0) { rc = -1; break; }
        const float *kr = k_f32 + (r * nkv + kh) * hd;
        const float *vr = v_f32 + (r * nkv + kh) * hd;
        for (int i = 0; i < hd; ++i) {
            kk[t * hd + i] = (double)kr[i];
            vv[t * hd + i] = (double)vr[i];
        }
    }
    if (rc == 0) {
        orc_attend_dense(qh, kk, vv, n, hd, (double)scale, oh);
        for (int i = 0; i < hd; ++i) o[i] = (float)oh[i];
    }
    free(qh); free(kk); free(vv); free(oh);
    return rc;
}

/* Rows rows_bh[r] = b * nq + h of exact decode attention over the fp32
 * mirror (rows_bh == NULL: every (b, h), r = b * nq + h).  out: [n_rows][hd]. */
int orc_decode_attn_f32(int batch, int nq, int nkv, int hd, int kv_bs,
                        const int32_t *block_table, int max_blocks_per_seq,
                        const int32_t *seq_lens, int num_blocks,
                        const float *k_f32, const float *v_f32,
                        const float *q, float scale,
                        const int64_t *rows_bh, int n_rows, float *out, int nthreads)
{
    int status = 0;
    if (rows_bh == NULL) n_rows = batch * nq;
    if (nthreads < 1) nthreads = 1;
#pragma omp parallel for schedule(dynamic, 1) num_threads(nthreads)
    for (int r = 0; r < n_rows; ++r) {
        int64_t bh = rows_bh ? rows_bh[r] : r;
        int rc = orc_one_row_f32((int)(bh / nq), (int)(bh % nq), nq, nkv, hd, kv_bs,
                                 block_table, max_blocks_per_seq, seq_lens, num_blocks,
                                 k_f32, v_f32, q + bh * hd, scale, out + (int64_t)r * hd);
        if (rc) {
#pragma omp atomic write
            status = -1;
        }
    }
    return status;
}

/* Block partials of every visible token against every query head, over the
 * blocked cache: partials[b][h][t][blk] for t < seq_lens[b]; entries with
 * t >= seq_lens[b] (up to max_seq_len) are 0.  Returns 0, 1 if an int32
 * overflow would occur, -1 on a bad length or block id. */
int orc_qk_partials(int batch, int nq, int nkv, int hd, int kv_bs,
                    const int32_t *block_table, int max_blocks_per_seq,
                    const int32_t *seq_lens, int num_blocks, int max_seq_len,
                    const int8_t *k_codes, const float *q, int32_t *partials)
{
    int status = 0;
    int group = nq / nkv, nblk = hd / 32;
    int8_t *cq = (int8_t *)malloc((size_t)hd);
    float *qsc = (float *)malloc(sizeof(float) * (size_t)nblk);
    for (int b = 0; b < batch; ++b) {
        for (int h = 0; h < nq; ++h) {
            int kh = h / group;
            int32_t *p = partials + ((int64_t)b * nq + h) * (int64_t)max_seq_len * nblk;
            memset(p, 0, sizeof(int32_t) * (size_t)max_seq_len * (size_t)nblk);
            int64_t n = seq_lens[b];
            if (n < 0 || n > max_seq_len) { status = -1; continue; }
            orc_quantize_q(q + ((int64_t)b * nq + h) * hd, hd, cq, qsc);
            for (int64_t t = 0; t < n; ++t) {
                int64_t r = orc_row_of(block_table, max_blocks_per_seq, b, t, kv_bs, num_blocks);
                if (r < 0) { status = -1; break; }
                if (orc_block_partials(cq, k_codes + (r * nkv + kh) * hd, hd, p + t * nblk))
                    status = status ? status : 1;
            }
        }
    }
    free(cq); free(qsc);
    return status;
}

/* ---------------------------------------------------------------- O9 ----- */
/* Page-literal single pass ([9-2] §2 segments 2 and 3), fp32, used only to
 * check that one pass equals three passes ([9-2] §3) and that the running max
 * never decreases ([9-2] §4).  Codes and stored steps in, fp32 out:
 *   per token: s = (sum over blocks of dot32_b * qsc_b) * ks * scale;
 *   if s > M: rescale S and acc by exp(M - s), M = s, weight 1;
 *   else weight exp(s - M);  S += weight;  acc += code_v * (weight * vs);
 *   finally out = acc / S.
 * m_trace (may be NULL) receives M after each token. */
void orc_single_pass(const int8_t *cq, const float *qsc,
                     const int8_t *ck, const float *ks,
                     const int8_t *cv, const float *vs,
                     int64_t n, int hd, float scale, float *out, float *m_trace)
{
    float *acc = (float *)calloc((size_t)hd, sizeof(float));
    float M = -1e9f, S = 0.0f;
    int nblk = hd / 32;
    for (int64_t t = 0; t < n; ++t) {
        float s = 0.0f;
        for (int blk = 0; blk < nblk; ++blk) {
            int32_t dot = 0;
            for (int i = 32 * blk; i < 32 * blk + 32; ++i)
                dot += (int32_t)cq[i] * (int32_t)ck[t * hd + i];
            s += (float)dot * qsc[blk];
        }
        s = s * ks[t] * scale;
        float w;
        if (s > M) {
            float f = expf(M - s);
            S *= f;
            for (int i = 0; i < hd; ++i) acc[i] *= f;
            M = s;
            w = 1.0f;
        } else {
            w = expf(s - M);
        }
        S += w;
        float wv = w * vs[t];
        for (int i = 0; i < hd; ++i) acc[i] += (float)cv[t * hd + i] * wv;
        if (m_trace) m_trace[t] = M;
    }
    for (int i = 0; i < hd; ++i) out[i] = (n > 0) ? acc[i] / S : 0.0f;
    free(acc);
}

/* ------------------------------------------------------------ O11 ------- */
/* Block-sparse decode ([10-1] §1: cut the history into 32-token blocks, find
 * the most relevant k blocks with a cheap probe, run exact attention over the
 * chosen blocks only; §2: defaults k = 32 blocks per head, 32 positions per
 * block, 8 probe samples per block with "max-dot fusion", and the sparse path
 * only for sequences longer than 2 blocks).  The page that details the probe
 * is not available; the readings taken here:
 *   - probe rows: 8 evenly spaced rows 0, 4, ..., 28 of each block (those
 *     below the sequence length);
 *   - a probe row's value is the q8 attention score of that row as [9-2] §2
 *     segment 2 defines it: the int32 block sums P_b of the query and key
 *     codes, s = (sum over blocks of P_b * qscale_b) * kscale * scale --
 *     evaluated here in double (every P_b * qscale_b is exact in double; the
 *     sum and the two products round once each, far below any fp32 ulp);
 *   - a block's importance: the maximum over its probe rows ("max-dot
 *     fusion");
 *   - selection per query head: the k blocks of highest importance, ties to
 *     the lower block index; nothing forced in; every block when the
 *     sequence has at most 2 blocks' worth of tokens or at most k blocks;
 *   - attention over every token of the chosen blocks (O4-O7 restricted to
 *     them).
 * An implementation that evaluates the score in lower precision may keep a
 * different set only among blocks whose importances lie within its rounding
 * of each other; the tests judge its kept set against these double scores. */
#define ORC_SPARSE_BLOCK 32
#define ORC_SPARSE_PROBES 8

/* The page's score of one key row against the quantized query, in double;
 * *mag (if not NULL) receives the same expression with every block term
 * taken by absolute value (the scale of the terms the sum cancels). */
static double orc_probe_score(const int8_t *cq, const float *qsc, const int8_t *ck, float ks, float scale,
                              double *mag)
{
    double s = 0.0, a = 0.0;
    for (int blk = 0; blk < 4; ++blk) {
        int64_t p = 0;
        for (int i = 32 * blk; i < 32 * blk + 32; ++i) p += (int64_t)cq[i] * (int64_t)ck[i];
        double x = (double)p * (double)qsc[blk];
        s += x;
        a += fabs(x);
    }
    if (mag) *mag = a * (double)ks * (double)scale;
    return s * (double)ks * (double)scale;
}

/* Importance of every block of one (b, h) of length n into score[0..nb) (and
 * mag[0..nb) if not NULL: the largest mag over the block's probe rows, which
 * bounds how far any row score can move under a rounding of its terms).
 * Returns 0, or -1 on a bad block id. */
static int orc_block_importance(int b, int kh, int nkv, int hd, int kv_bs, const int32_t *block_table,
                                int max_blocks_per_seq, int num_blocks, int64_t n, const int8_t *k_codes,
                                const float *k_step, const int8_t *cq, const float *qsc, float scale,
                                double *score, double *mag)
{
    int nb = (int)((n + ORC_SPARSE_BLOCK - 1) / ORC_SPARSE_BLOCK);
    for (int j = 0; j < nb; ++j) {
        double best = -INFINITY, best_mag = 0.0;
        for (int pr = 0; pr < ORC_SPARSE_PROBES; ++pr) {
            int64_t t = (int64_t)j * ORC_SPARSE_BLOCK + pr * (ORC_SPARSE_BLOCK / ORC_SPARSE_PROBES);
            if (t >= n) break;
            int64_t r = orc_row_of(block_table, max_blocks_per_seq, b, t, kv_bs, num_blocks);
            if (r < 0) return -1;
            double m;
            double sc = orc_probe_score(cq, qsc, k_codes + (r * nkv + kh) * hd, k_step[r * nkv + kh], scale, &m);
            if (sc > best) best = sc;
            if (m > best_mag) best_mag = m;
        }
        score[j] = best;
        if (mag) mag[j] = best_mag;
    }
    return 0;
}

/* Importance of every block of every (b, h): scores[b][h][j] for j <
 * ceil(seq_lens[b] / 32), -inf up to max_nb; mags (may be NULL) likewise,
 * 0 past the end.  Returns 0, or -1 on a bad length or block id. */
int orc_sparse_scores(int batch, int nq, int nkv, int hd, int kv_bs,
                      const int32_t *block_table, int max_blocks_per_seq,
                      const int32_t *seq_lens, int num_blocks,
                      const int8_t *k_codes, const float *k_step,
                      const float *q, float scale, int max_nb, double *scores, double *mags)
{
    int status = 0;
    for (int b = 0; b < batch; ++b) {
        int64_t n = seq_lens[b];
        for (int h = 0; h < nq; ++h) {
            double *o = scores + ((int64_t)b * nq + h) * max_nb;
            double *m = mags ? mags + ((int64_t)b * nq + h) * max_nb : NULL;
            for (int j = 0; j < max_nb; ++j) {
                o[j] = -INFINITY;
                if (m) m[j] = 0.0;
            }
            if (n < 0 || n > (int64_t)max_blocks_per_seq * kv_bs || (n + 31) / 32 > max_nb) { status = -1; continue; }
            int8_t cq[128];
            float qsc[4];
            orc_quantize_q(q + ((int64_t)b * nq + h) * hd, hd, cq, qsc);
            if (orc_block_importance(b, h / (nq / nkv), nkv, hd, kv_bs, block_table, max_blocks_per_seq,
                                     num_blocks, n, k_codes, k_step, cq, qsc, scale, o, m))
                status = -1;
        }
    }
    return status;
}

/* One (b, h): attention (O4-O7) over the tokens of the blocks sel[0..count)
 * of sequence b (32-token blocks; the last one ends at seq_lens[b]), taken in
 * the order given.  o = zeros when count is 0.  Returns 0, or -1 on a bad
 * length, block index or block id (o = zeros). */
static int orc_attend_blocks(int b, int h, int nq, int nkv, int hd, int kv_bs,
                             const int32_t *block_table, int max_blocks_per_seq,
                             const int32_t *seq_lens, int num_blocks,
                             const int8_t *k_codes, const int8_t *v_codes,
                             const float *k_step, const float *v_step,
                             const float *q_row, float scale, const int32_t *sel, int count, float *o)
{
    int kh = h / (nq / nkv);
    int64_t n = seq_lens[b];
    for (int i = 0; i < hd; ++i) o[i] = 0.0f;
    if (n < 0 || n > (int64_t)max_blocks_per_seq * kv_bs) return -1;
    int nb = (int)((n + ORC_SPARSE_BLOCK - 1) / ORC_SPARSE_BLOCK);
    int64_t m = 0;
    for (int c = 0; c < count; ++c) {
        if (sel[c] < 0 || sel[c] >= nb) return -1;
        int64_t t1 = (int64_t)(sel[c] + 1) * ORC_SPARSE_BLOCK;
        m += (t1 < n ? t1 : n) - (int64_t)sel[c] * ORC_SPARSE_BLOCK;
    }
    if (m == 0) return 0;
    int8_t cq[128];
    float qsc[4];
    orc_quantize_q(q_row, hd, cq, qsc);
    double *qh = (double *)malloc(sizeof(double) * (size_t)hd);
    double *kk = (double *)malloc(sizeof(double) * (size_t)(m * hd));
    double *vv = (double *)malloc(sizeof(double) * (size_t)(m * hd));
    double *oh = (double *)malloc(sizeof(double) * (size_t)hd);
    for (int i = 0; i < hd; ++i) qh[i] = (double)cq[i] * (double)qsc[i / 32];
    int rc = 0;
    int64_t u = 0;
    for (int c = 0; c < count && rc == 0; ++c) {
        for (int64_t t = (int64_t)sel[c] * ORC_SPARSE_BLOCK; t < (int64_t)(sel[c] + 1) * ORC_SPARSE_BLOCK && t < n; ++t) {
            int64_t r = orc_row_of(block_table, max_blocks_per_seq, b, t, kv_bs, num_blocks);
            if (r < 0) { rc = -1; break; }
            const int8_t *ck = k_codes + (r * nkv + kh) * hd;
            const int8_t *cv = v_codes + (r * nkv + kh) * hd;
            double dk = (double)k_step[r * nkv + kh], dv = (double)v_step[r * nkv + kh];
            for (int i = 0; i < hd; ++i) {
                kk[u * hd + i] = (double)ck[i] * dk;
                vv[u * hd + i] = (double)cv[i] * dv;
            }
            ++u;
        }
    }
    if (rc == 0) {
        orc_attend_dense(qh, kk, vv, m, hd, (double)scale, oh);
        for (int i = 0; i < hd; ++i) o[i] = (float)oh[i];
    }
    free(qh); free(kk); free(vv); free(oh);
    return rc;
}

/* One (b, h) of the block-sparse decode: the kept blocks (ascending) into
 * sel[0..count) and the attention over their tokens into o.  Returns count,
 * or -1 on a bad length or block id (o = zeros). */
static int orc_one_row_sparse(int b, int h, int nq, int nkv, int hd, int kv_bs,
                              const int32_t *block_table, int max_blocks_per_seq,
                              const int32_t *seq_lens, int num_blocks,
                              const int8_t *k_codes, const int8_t *v_codes,
                              const float *k_step, const float *v_step,
                              const float *q_row, float scale, int topk, float *o, int32_t *sel)
{
    int64_t n = seq_lens[b];
    for (int i = 0; i < hd; ++i) o[i] = 0.0f;
    if (n < 0 || n > (int64_t)max_blocks_per_seq * kv_bs) return -1;
    if (n == 0) return 0;
    int nb = (int)((n + ORC_SPARSE_BLOCK - 1) / ORC_SPARSE_BLOCK);
    int count = 0;
    if (n <= 2 * ORC_SPARSE_BLOCK || nb <= topk) {
        for (int j = 0; j < nb; ++j) sel[count++] = j;
    } else {
        int8_t cq[128];
        float qsc[4];
        orc_quantize_q(q_row, hd, cq, qsc);
        double *score = (double *)malloc(sizeof(double) * (size_t)nb);
        char *taken = (char *)calloc((size_t)nb, 1);
        if (orc_block_importance(b, h / (nq / nkv), nkv, hd, kv_bs, block_table, max_blocks_per_seq, num_blocks,
                                 n, k_codes, k_step, cq, qsc, scale, score, NULL)) {
            free(score);
            free(taken);
            return -1;
        }
        /* k rounds of "the highest importance not taken yet, lowest index on ties" */
        for (int round = 0; round < topk; ++round) {
            int arg = -1;
            for (int j = 0; j < nb; ++j)
                if (!taken[j] && (arg < 0 || score[j] > score[arg])) arg = j;
            taken[arg] = 1;
        }
        for (int j = 0; j < nb; ++j)
            if (taken[j]) sel[count++] = j;
        free(score);
        free(taken);
    }
    if (orc_attend_blocks(b, h, nq, nkv, hd, kv_bs, block_table, max_blocks_per_seq, seq_lens, num_blocks,
                          k_codes, v_codes, k_step, v_step, q_row, scale, sel, count, o))
        return -1;
    return count;
}

/* Every (b, h).  out: [batch][nq][hd]; sel (optional): [batch][nq][topk]
 * selected block indices ascending, -1 after the last.  Returns 0, or -1 if
 * any row had a bad length or block id. */
int orc_decode_attn_sparse(int batch, int nq, int nkv, int hd, int kv_bs,
                           const int32_t *block_table, int max_blocks_per_seq,
                           const int32_t *seq_lens, int num_blocks,
                           const int8_t *k_codes, const int8_t *v_codes,
                           const float *k_step, const float *v_step,
                           const float *q, float scale, int topk, float *out, int32_t *sel,
                           int nthreads)
{
    int status = 0;
    int64_t rows = (int64_t)batch * nq;
    if (nthreads < 1) nthreads = 1;
#pragma omp parallel for schedule(dynamic, 1) num_threads(nthreads)
    for (int64_t bh = 0; bh < rows; ++bh) {
        int b = (int)(bh / nq);
        int64_t n = seq_lens[b];
        int nb = n > 0 ? (int)((n + ORC_SPARSE_BLOCK - 1) / ORC_SPARSE_BLOCK) : 0;
        int32_t *s = (int32_t *)malloc(sizeof(int32_t) * (size_t)(nb > 0 ? nb : 1));
        int rc = orc_one_row_sparse(b, (int)(bh % nq), nq, nkv, hd, kv_bs, block_table, max_blocks_per_seq,
                                    seq_lens, num_blocks, k_codes, v_codes, k_step, v_step,
                                    q + bh * hd, scale, topk, out + bh * hd, s);
        if (sel) {
            int32_t *d = sel + bh * topk;
            for (int c = 0; c < topk; ++c) d[c] = (rc > 0 && c < rc) ? s[c] : -1;
        }
        free(s);
        if (rc < 0) {
#pragma omp atomic write
            status = -1;
        }
    }
    return status;
}

/* Attention over a given block set for every (b, h): sel[b][h][0..width)
 * lists block indices, ended by the first negative entry.  out:
 * [batch][nq][hd].  Returns 0, or -1 if any row had a bad length, block
 * index or block id (that row is zeros). */
int orc_decode_attn_blocks(int batch, int nq, int nkv, int hd, int kv_bs,
                           const int32_t *block_table, int max_blocks_per_seq,
                           const int32_t *seq_lens, int num_blocks,
                           const int8_t *k_codes, const int8_t *v_codes,
                           const float *k_step, const float *v_step,
                           const float *q, float scale, const int32_t *sel, int width, float *out,
                           int nthreads)
{
    int status = 0;
    int64_t rows = (int64_t)batch * nq;
    if (nthreads < 1) nthreads = 1;
#pragma omp parallel for schedule(dynamic, 1) num_threads(nthreads)
    for (int64_t bh = 0; bh < rows; ++bh) {
        const int32_t *s = sel + bh * width;
        int count = 0;
        while (count < width && s[count] >= 0) ++count;
        int rc = orc_attend_blocks((int)(bh / nq), (int)(bh % nq), nq, nkv, hd, kv_bs, block_table,
                                   max_blocks_per_seq, seq_lens, num_blocks, k_codes, v_codes, k_step, v_step,
                                   q + bh * hd, scale, s, count, out + bh * hd);
        if (rc) {
#pragma omp atomic write
            status = -1;
        }
    }
    return status;
}

/* ------------------------------------------------------------ O12 ------- */
/* Batched prefill attention over the q8 cache ([10-1] §1: a prefill batch of
 * nb new tokens scores against the whole history, O(nb x n); §2: the exact
 * batched path beside the block-sparse one).  The pages do not spell out the
 * masking inside the batch or the query quantization for many rows; the
 * readings taken here:
 *   - the nb_b = q_start[b + 1] - q_start[b] new tokens of sequence b are the
 *     last nb_b positions of its cache (appended before the call), so query
 *     row r (q_start[b] <= r < q_start[b + 1]) sits at position
 *     p = seq_lens[b] - nb_b + (r - q_start[b]);
 *   - causal: that row attends to positions 0..p (the history and the batch's
 *     earlier tokens and itself);
 *   - each query row is quantized on its own exactly like the decode query
 *     (O2), and its attention is the decode attention (O4-O8) over the first
 *     p + 1 positions.
 * q, out: [total_q][nq][hd] fp32, total_q = q_start[batch].  Returns 0, or -1
 * on a bad q_start, length or block id (rows of such a sequence are zeros;
 * nothing is written for a q_start range outside [0, total_q]). */
int orc_prefill_attn(int batch, int nq, int nkv, int hd, int kv_bs,
                     const int32_t *block_table, int max_blocks_per_seq,
                     const int32_t *seq_lens, int num_blocks,
                     const int8_t *k_codes, const int8_t *v_codes,
                     const float *k_step, const float *v_step,
                     const int32_t *q_start, int total_q,
                     const float *q, float scale, float *out, int nthreads)
{
    int status = 0;
    if (nthreads < 1) nthreads = 1;
    for (int b = 0; b < batch; ++b) {
        int32_t r0 = q_start[b], r1 = q_start[b + 1];
        int64_t n = seq_lens[b];
        if (r0 < 0 || r1 < r0 || r1 > total_q) { status = -1; continue; }
        int64_t nb = (int64_t)r1 - r0;
        int bad = n < nb || n > (int64_t)max_blocks_per_seq * kv_bs;
        if (bad) {
            status = -1;
            for (int64_t i = (int64_t)r0 * nq * hd; i < (int64_t)r1 * nq * hd; ++i) out[i] = 0.0f;
            continue;
        }
        int64_t rows = nb * nq;
#pragma omp parallel for schedule(dynamic, 1) num_threads(nthreads)
        for (int64_t rh = 0; rh < rows; ++rh) {
            int64_t r = r0 + rh / nq;
            int h = (int)(rh % nq);
            int64_t pos = n - nb + (r - r0);
            int rc = orc_one_row_n(b, h, nq, nkv, hd, kv_bs, block_table, max_blocks_per_seq, pos + 1,
                                   num_blocks, k_codes, v_codes, k_step, v_step,
                                   q + (r * nq + h) * hd, scale, out + (r * nq + h) * hd);
            if (rc) {
#pragma omp atomic write
                status = -1;
            }
        }
    }
    return status;
}

int orc_num_threads_available(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}
