/*
 * MLA paged-KV decode oracle -- TEST INFRASTRUCTURE ONLY.
 *
 * A plain, slow, obviously correct CPU definition of what the decode path
 * computes, used to check the GPU library.  Only the tests, the smoke check
 * and the benchmark's CPU-baseline leg may load this file's library.  It shares
 * no code, header, table or constant with the HIP library.
 *
 * All arithmetic is IEEE double.  bf16 and e4m3 inputs are widened exactly.
 *
 * What is computed (per request b, query row i < s_q, head h < h_q):
 *   - Multi-head latent attention in its decode form: every query head attends
 *     to one shared compressed latent row per cached token ("Was ist MLA?",
 *     MHA/MQA/GQA/MLA table, Novita AI page: MQA-style sharing of one KV
 *     stream by all query heads; MLA = latent vectors plus a decoupled RoPE
 *     part).  Each token's key is 576 values: 512 latent + 64 RoPE.  The value
 *     is the first 512 of them.
 *   - The cache is paged in blocks of 64 tokens and reached through a
 *     per-request block table (DeepSeek launch announcement quoted on the
 *     8bitnewsroom FlashMLA page; feature list of the aivengo.media page).
 *   - score_j = scale * <q, K_j>, lse = ln sum_j exp(score_j),
 *     out = sum_j softmax_j * K_j[0:512]   (textbook softmax attention; the
 *     pages never write the formula, this is the plain reading).
 *   - Causal rows (s_q > 1): query row i is the (s_q-1-i)-th newest token and
 *     sees the first L - (s_q - 1 - i) keys (bottom-right alignment).
 *   - A row that sees no key returns out = 0 and lse = -inf.
 *   - FP8 cache ("Key Contributions", DeepSeek KB page: 656 bytes per token,
 *     RoPE slice kept in BF16): a token record is 512 OCP E4M3FN codes, then
 *     four little-endian fp32 scales (one per 128-dim tile), then 64 bf16
 *     RoPE values.  Dequantised key = e4m3(code) * scale[d / 128].
 *   - Writing that record from a bf16 row (the cache writer): the pages give
 *     the record but not the quantiser; the plain reading used here maps each
 *     tile's absolute maximum to E4M3's largest finite value, 448:
 *     scale = amax / 448 (fp32), code = E4M3 nearest-even of clip(x / scale,
 *     +-448) (fp32 division), and an all-zero tile gets scale 0 and codes 0.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

enum { ORC_D_QK = 576, ORC_D_V = 512, ORC_PAGE = 64 };
enum { ORC_FP8_RECORD = 656, ORC_FP8_SCALES_AT = 512, ORC_FP8_ROPE_AT = 528 };

/* bf16 is the top half of an IEEE binary32. */
static double orc_bf16(uint16_t bits)
{
    uint32_t u = (uint32_t)bits << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

/* OCP E4M3FN: 1 sign, 4 exponent (bias 7), 3 mantissa bits; no infinities;
 * S.1111.111 is NaN; subnormals when the exponent field is 0. */
double mla_oracle_e4m3_value(uint8_t code)
{
    int sign = code >> 7;
    int e = (code >> 3) & 15;
    int m = code & 7;
    double mag;
    if (e == 15 && m == 7)
        return NAN;
    if (e == 0)
        mag = ldexp((double)m / 8.0, -6);
    else
        mag = ldexp(1.0 + (double)m / 8.0, e - 7);
    return sign ? -mag : mag;
}

/*
 * OCP E4M3FN encoding of a finite fp32 value with |x| <= 448: the nearest
 * representable value, ties to the even code (last mantissa bit 0).  Plain
 * search over the 127 non-negative finite codes, whose values increase with
 * the code; the sign bit is copied (so -0 encodes as 0x80).
 */
uint8_t mla_oracle_e4m3_encode(float x)
{
    static double value[127];
    static int have_values = 0;
    double a = fabs((double)x), best_d = INFINITY;
    int c, best = 0;
    if (!have_values) {  /* the code table, from the decoding definition */
        for (c = 0; c < 127; ++c)
            value[c] = mla_oracle_e4m3_value((uint8_t)c);
        have_values = 1;
    }
    for (c = 0; c < 127; ++c) {
        double d = fabs(value[c] - a);
        if (d < best_d || (d == best_d && (c & 1) == 0)) {
            best_d = d;
            best = c;
        }
    }
    return (uint8_t)(best | (signbit(x) ? 0x80 : 0));
}

/* One 576-dim bf16 row -> one 656-byte FP8 record (see the header). */
void mla_oracle_fp8_record_from_row(const uint16_t *row, uint8_t *rec)
{
    int t, d;
    for (t = 0; t < ORC_D_V / 128; ++t) {
        float amax = 0.f, scale;
        for (d = 128 * t; d < 128 * (t + 1); ++d) {
            float v = fabsf((float)orc_bf16(row[d]));
            if (v > amax) amax = v;
        }
        scale = amax / 448.0f;
        memcpy(rec + ORC_FP8_SCALES_AT + 4 * t, &scale, 4);
        for (d = 128 * t; d < 128 * (t + 1); ++d) {
            float x;
            if (!(scale > 0.f)) {
                rec[d] = 0;
                continue;
            }
            x = (float)orc_bf16(row[d]) / scale;
            if (x > 448.0f) x = 448.0f;
            if (x < -448.0f) x = -448.0f;
            rec[d] = mla_oracle_e4m3_encode(x);
        }
    }
    memcpy(rec + ORC_FP8_ROPE_AT, row + ORC_D_V, 2 * (ORC_D_QK - ORC_D_V));
}

/*
 * Cache writer.  k_new bf16 [batch][n_new][576]: row i of request b is the
 * token at position L_b - n_new + i of that request (seqlens already count
 * the new rows); rows at negative positions are skipped.  The token's page is
 * block_table[b][pos / 64], its slot pos % 64.  kind 0 copies the bf16 row
 * into a [pages][64][576] cache; kind 1 writes the FP8 record into a
 * [pages][64][656] cache.  Nothing else in the cache changes.
 */
void mla_oracle_kv_write(const uint16_t *k_new, int batch, int n_new, const int32_t *block_table,
                         int64_t bt_stride, const int32_t *seqlens, int kind, void *cache)
{
    int b, i;
    for (b = 0; b < batch; ++b)
        for (i = 0; i < n_new; ++i) {
            int64_t pos = (int64_t)seqlens[b] - n_new + i, phys;
            const uint16_t *row = k_new + ((int64_t)b * n_new + i) * ORC_D_QK;
            if (pos < 0) continue;
            phys = block_table[(int64_t)b * bt_stride + pos / ORC_PAGE];
            if (kind == 0)
                memcpy((uint16_t *)cache + (phys * ORC_PAGE + pos % ORC_PAGE) * ORC_D_QK, row,
                       2 * ORC_D_QK);
            else
                mla_oracle_fp8_record_from_row(
                    row, (uint8_t *)cache + (phys * ORC_PAGE + pos % ORC_PAGE) * ORC_FP8_RECORD);
        }
}

/* One cached token's 576-dim key, widened to double. */
static void orc_key(const void *cache, int kind, int64_t phys, int slot, double *k)
{
    int d;
    if (kind == 0) {
        const uint16_t *row = (const uint16_t *)cache + (phys * ORC_PAGE + slot) * ORC_D_QK;
        for (d = 0; d < ORC_D_QK; ++d)
            k[d] = orc_bf16(row[d]);
    } else {
        const uint8_t *rec = (const uint8_t *)cache + (phys * ORC_PAGE + slot) * ORC_FP8_RECORD;
        float scale[4];
        memcpy(scale, rec + ORC_FP8_SCALES_AT, sizeof scale);
        for (d = 0; d < ORC_D_V; ++d)
            k[d] = mla_oracle_e4m3_value(rec[d]) * (double)scale[d / 128];
        for (d = 0; d < ORC_D_QK - ORC_D_V; ++d) {
            uint16_t bits;
            memcpy(&bits, rec + ORC_FP8_ROPE_AT + 2 * d, 2);
            k[ORC_D_V + d] = orc_bf16(bits);
        }
    }
}

/* Number of keys query row i of a request with L cached tokens may see. */
static int64_t orc_visible(int64_t L, int s_q, int i, int causal)
{
    int64_t n = causal ? L - (int64_t)(s_q - 1 - i) : L;
    if (n < 0) n = 0;
    if (n > L) n = L;
    return n;
}

/*
 * Attention of one query row over keys [lo, hi) of its request (the window is
 * further clipped to the keys the row may see).  out: 512 doubles.
 */
static void orc_attend(const uint16_t *q, int s_q, int h_q, const void *cache, int kind,
                       const int32_t *block_table, int64_t bt_stride, const int32_t *seqlens,
                       double scale, int causal, int b, int i, int h, int64_t lo, int64_t hi,
                       double *out, double *lse)
{
    double qd[ORC_D_QK], kd[ORC_D_QK];
    const uint16_t *qrow = q + (((int64_t)b * s_q + i) * h_q + h) * ORC_D_QK;
    int64_t n = orc_visible(seqlens[b], s_q, i, causal);
    int64_t j, cnt;
    double *score, mx, z;
    int d;

    if (lo < 0) lo = 0;
    if (hi > n) hi = n;
    for (d = 0; d < ORC_D_V; ++d)
        out[d] = 0.0;
    if (hi <= lo) {
        *lse = -INFINITY;
        return;
    }
    for (d = 0; d < ORC_D_QK; ++d)
        qd[d] = orc_bf16(qrow[d]);

    cnt = hi - lo;
    score = (double *)malloc((size_t)cnt * sizeof(double));
    mx = -INFINITY;
    for (j = lo; j < hi; ++j) {
        int64_t phys = block_table[(int64_t)b * bt_stride + j / ORC_PAGE];
        double dot = 0.0;
        orc_key(cache, kind, phys, (int)(j % ORC_PAGE), kd);
        for (d = 0; d < ORC_D_QK; ++d)
            dot += qd[d] * kd[d];
        score[j - lo] = scale * dot;
        if (score[j - lo] > mx) mx = score[j - lo];
    }
    z = 0.0;
    for (j = lo; j < hi; ++j) {
        int64_t phys = block_table[(int64_t)b * bt_stride + j / ORC_PAGE];
        double w = exp(score[j - lo] - mx);
        z += w;
        orc_key(cache, kind, phys, (int)(j % ORC_PAGE), kd);
        for (d = 0; d < ORC_D_V; ++d)
            out[d] += w * kd[d];
    }
    for (d = 0; d < ORC_D_V; ++d)
        out[d] /= z;
    *lse = mx + log(z);
    free(score);
}

/*
 * Decode a list of query rows.
 *   q            bf16 bits [batch, s_q, h_q, 576]
 *   cache        kind 0: bf16 bits [num_pages, 64, 576];
 *                kind 1: bytes [num_pages, 64, 656] (FP8 records)
 *   block_table  int32 [batch, bt_stride]; logical block j of request b -> page
 *   seqlens      int32 [batch]; cached tokens per request (including the s_q
 *                tokens being decoded)
 *   rows         int32 [n_rows, 3] = (b, i, h)
 *   windows      NULL, or int64 [n_rows, 2] = key window [lo, hi) per row
 *   out          double [n_rows, 512];  lse double [n_rows] (natural log)
 * Returns the number of OpenMP threads used.
 */
int mla_oracle_decode_rows(const uint16_t *q, int s_q, int h_q, const void *cache, int kind,
                           const int32_t *block_table, int64_t bt_stride, const int32_t *seqlens,
                           double scale, int causal, const int32_t *rows, int64_t n_rows,
                           const int64_t *windows, double *out, double *lse)
{
    int threads = 1;
    int64_t r;
#ifdef _OPENMP
    threads = omp_get_max_threads();
#endif
#pragma omp parallel for schedule(dynamic, 1)
    for (r = 0; r < n_rows; ++r) {
        int b = rows[3 * r], i = rows[3 * r + 1], h = rows[3 * r + 2];
        int64_t lo = windows ? windows[2 * r] : 0;
        int64_t hi = windows ? windows[2 * r + 1] : (int64_t)seqlens[b];
        orc_attend(q, s_q, h_q, cache, kind, block_table, bt_stride, seqlens, scale, causal,
                   b, i, h, lo, hi, out + r * ORC_D_V, lse + r);
    }
    return threads;
}

/*
 * Sparse decode: query token i of request b attends only to the cached
 * tokens its list names (DeepSeek KB page, "Key Contributions": the FP8
 * cache serves a sparse decode kernel; the list itself comes from an indexer
 * the pages do not describe).  indices int32 [batch][s_q][topk] holds token
 * positions within the request; the list of query token (b, i) ends at its
 * first negative entry (lists shorter than topk are padded with negatives).
 * A listed position is used as given (a position listed twice counts twice).
 * Row (b, i, h) gets the textbook attention over the listed keys; a row whose
 * list is empty gets out = 0, lse = -inf.
 *   rows int32 [n_rows, 3] = (b, i, h); out double [n_rows, 512]; lse [n_rows]
 */
void mla_oracle_decode_sparse_rows(const uint16_t *q, int s_q, int h_q, const void *cache,
                                   int kind, const int32_t *block_table, int64_t bt_stride,
                                   const int32_t *indices, int topk, double scale,
                                   const int32_t *rows, int64_t n_rows, double *out, double *lse)
{
    int64_t r;
#pragma omp parallel for schedule(dynamic, 1)
    for (r = 0; r < n_rows; ++r) {
        int b = rows[3 * r], i = rows[3 * r + 1], h = rows[3 * r + 2];
        const int32_t *list = indices + ((int64_t)b * s_q + i) * topk;
        const uint16_t *qrow = q + (((int64_t)b * s_q + i) * h_q + h) * ORC_D_QK;
        double qd[ORC_D_QK], kd[ORC_D_QK], *o = out + r * ORC_D_V;
        double *score = (double *)malloc((size_t)(topk > 0 ? topk : 1) * sizeof(double));
        double mx = -INFINITY, z = 0.0;
        int k, d, n = 0;
        for (d = 0; d < ORC_D_V; ++d)
            o[d] = 0.0;
        for (d = 0; d < ORC_D_QK; ++d)
            qd[d] = orc_bf16(qrow[d]);
        for (k = 0; k < topk; ++k) {
            int64_t j = list[k], phys;
            double dot = 0.0;
            if (j < 0) break;
            phys = block_table[(int64_t)b * bt_stride + j / ORC_PAGE];
            orc_key(cache, kind, phys, (int)(j % ORC_PAGE), kd);
            for (d = 0; d < ORC_D_QK; ++d)
                dot += qd[d] * kd[d];
            score[n] = scale * dot;
            if (score[n] > mx) mx = score[n];
            ++n;
        }
        if (n == 0) {
            lse[r] = -INFINITY;
            free(score);
            continue;
        }
        n = 0;
        for (k = 0; k < topk; ++k) {
            int64_t j = list[k], phys;
            double w;
            if (j < 0) break;
            phys = block_table[(int64_t)b * bt_stride + j / ORC_PAGE];
            orc_key(cache, kind, phys, (int)(j % ORC_PAGE), kd);
            w = exp(score[n++] - mx);
            z += w;
            for (d = 0; d < ORC_D_V; ++d)
                o[d] += w * kd[d];
        }
        for (d = 0; d < ORC_D_V; ++d)
            o[d] /= z;
        lse[r] = mx + log(z);
        free(score);
    }
}

/*
 * Merge attention results computed over disjoint key sets of the same row.
 * Each part holds its own normalised output o_p and lse_p.  The merged lse is
 * ln sum_p exp(lse_p) and the merged output weights each part by
 * exp(lse_p - lse).  Parts with lse = -inf carry no keys and weigh 0.
 *   o_parts [n_parts, dv], lse_parts [n_parts] -> out [dv], *lse
 */
void mla_oracle_lse_merge(const double *o_parts, const double *lse_parts, int n_parts, int dv,
                          double *out, double *lse)
{
    double mx = -INFINITY, z = 0.0;
    int p, d;
    for (d = 0; d < dv; ++d)
        out[d] = 0.0;
    for (p = 0; p < n_parts; ++p)
        if (lse_parts[p] > mx) mx = lse_parts[p];
    if (mx == -INFINITY) {
        *lse = -INFINITY;
        return;
    }
    for (p = 0; p < n_parts; ++p)
        z += exp(lse_parts[p] - mx);
    *lse = mx + log(z);
    for (p = 0; p < n_parts; ++p) {
        double w = exp(lse_parts[p] - *lse);
        if (lse_parts[p] == -INFINITY) continue;
        for (d = 0; d < dv; ++d)
            out[d] += w * o_parts[(int64_t)p * dv + d];
    }
}

/* Dequantise one FP8 token record into 576 doubles (512 latent + 64 RoPE). */
void mla_oracle_fp8_record_values(const uint8_t *record, double *k)
{
    orc_key(record, 1, 0, 0, k);
}

int mla_oracle_fp8_record_bytes(void) { return ORC_FP8_RECORD; }
int mla_oracle_bf16_token_bytes(void) { return 2 * ORC_D_QK; }
