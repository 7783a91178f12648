/*
 * pafp8_oracle.c -- CPU oracle for FP8 (e4m3) paged decode attention.
 *
 * TEST INFRASTRUCTURE ONLY.  This file is a plain, slow, deliberately
 * unoptimised C implementation of what the GPU library computes.  It exists so
 * that tests/, the smoke check and the bench's CPU-baseline leg have an
 * independent result to compare against.  It shares no source, header, table
 * or helper with the HIP library, and no product code path may call it.
 *
 * Sources (the pages are translations/summaries of one post):
 *   [KVQ]  "Smaller, faster, safer: running Kimi and GLM at scale" (Cloudflare
 *          blog; translation at reed-read.pages.dev/article/2383), section
 *          "KV 缓存量化" (KV cache quantization): K/V are stored as FP8 e4m3,
 *          halving the cache versus BF16; the attention kernel converts the
 *          format when it reads.
 *   [KVP]  same post, section "共享 KV 缓存保护" (shared KV cache protection):
 *          every physical cache page carries a tag that changes whenever the
 *          page is reallocated; the server records, per request, which pages
 *          and tags it expects; the mapping is verified before decode reads the
 *          cache and a mismatching request is terminated.  The check is a
 *          separate batched pass, not fused into attention.
 *   [PAG]  remio.ai analysis of the same post, section "Bezpieczeństwo
 *          współdzielonego cache KV..." (shared KV cache safety): paged
 *          attention splits the cache into reusable blocks and maps each
 *          logical sequence onto physical pages; tags act like generation
 *          counters.
 *   [WQ]   same post, section "模型权重压缩" (model weight compression): GLM
 *          weights go from FP8 to INT4; decode reads the weights for every
 *          token, so fewer bytes decode faster; the weights are expanded
 *          before multiplying.
 *   [OFP8] The e4m3 format itself is not defined on the pages, which only name
 *          it.  The reading used here is the OCP 8-bit floating point "E4M3"
 *          encoding: 1 sign bit, 4 exponent bits with bias 7, 3 mantissa bits,
 *          no infinities, a single NaN mantissa pattern (S.1111.111), largest
 *          finite magnitude 448.
 *
 * Readings where the pages are silent:
 *   - encoding rounds to nearest, ties to the even code, and saturates
 *     magnitudes >= 448 (and infinities) to +-448; NaN encodes as 0x7F|sign;
 *   - quantisation is enc(f32(x) / scale) with an IEEE single-precision
 *     (correctly rounded) division;
 *   - scores use sm_scale supplied by the caller; query head h reads KV head
 *     h / G (consecutive query heads share a KV head);
 *   - a request whose status is non-zero yields out = 0 and lse = -inf and
 *     none of its pages are read;
 *   - when no status is supplied, a request with an invalid length or page id
 *     yields NaN outputs (nothing outside the pool is ever read); an empty
 *     request (length 0) yields out = 0, lse = -inf.
 *
 * Every floating-point result below is computed in fp64 from exactly decoded
 * inputs unless a step is defined in fp32 (the quantisation division).
 */
#include <math.h>
#ifdef _OPENMP
#include <omp.h>
#endif
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORACLE_REQ_TAG_MISMATCH 1
#define ORACLE_REQ_PAGE_OOB 2
#define ORACLE_REQ_BAD_LEN 4

/* ------------------------------------------------------------------------ */
/* O1. e4m3 decode, straight from the format definition [OFP8].              */
/*   exponent field 0      : subnormal, value = m * 2^-9                     */
/*   exponent field 1..15  : normal, value = (1 + m/8) * 2^(e - 7)            */
/*   exponent 15, m = 7    : NaN                                             */
/* ------------------------------------------------------------------------ */
double oracle_e4m3_decode(uint8_t code)
{
    int sign = (code >> 7) & 1;
    int e = (code >> 3) & 0xF;
    int m = code & 0x7;
    double mag;
    if (e == 15 && m == 7)
        return NAN;
    if (e == 0)
        mag = (double)m * ldexp(1.0, -9);
    else
        mag = (1.0 + (double)m / 8.0) * ldexp(1.0, e - 7);
    return sign ? -mag : mag;
}

/* ------------------------------------------------------------------------ */
/* O2a. e4m3 encode, brute-force form: the definition of round-to-nearest.   */
/* Search every non-negative finite code for the one closest to |x|; on an   */
/* exact tie keep the code whose last mantissa bit is 0 (ties-to-even).      */
/* ------------------------------------------------------------------------ */
uint8_t oracle_e4m3_encode_brute(float x)
{
    uint8_t sign = signbit(x) ? 0x80 : 0x00;
    double a, best_d = INFINITY;
    int c, best = 0;
    if (isnan(x))
        return (uint8_t)(0x7F | sign);
    a = fabs((double)x);
    if (a >= 448.0)
        return (uint8_t)(0x7E | sign);
    for (c = 0x00; c <= 0x7E; ++c) {
        double d = fabs(oracle_e4m3_decode((uint8_t)c) - a);
        if (d < best_d || (d == best_d && (c & 1) == 0)) {
            best = c;
            best_d = d;
        }
    }
    return (uint8_t)(best | sign);
}

/* ------------------------------------------------------------------------ */
/* O2b. e4m3 encode, arithmetic form (used for large sweeps).  Scales |x| so */
/* that one unit is the code spacing of its binade and rounds with rint()    */
/* (the default IEEE mode: nearest, ties to even).  Must agree with O2a.     */
/* ------------------------------------------------------------------------ */
uint8_t oracle_e4m3_encode(float x)
{
    uint8_t sign = signbit(x) ? 0x80 : 0x00;
    double a, q;
    int e2;
    if (isnan(x))
        return (uint8_t)(0x7F | sign);
    a = fabs((double)x);
    if (a >= 448.0)
        return (uint8_t)(0x7E | sign);
    if (a < ldexp(1.0, -6)) {
        /* subnormal binade: spacing 2^-9; rint(a * 512) in [0, 8] is the code
         * (8 is the smallest normal, code 0x08) */
        q = rint(a * 512.0);
        return (uint8_t)((int)q | sign);
    }
    /* a = f * 2^e2 with f in [0.5, 1): unbiased exponent E = e2 - 1 in [-6, 8] */
    frexp(a, &e2);
    {
        int E = e2 - 1;
        /* significand scaled to [8, 16): one unit = 2^(E-3), the code spacing */
        q = rint(ldexp(a, 3 - E));
        /* q == 16 carries into the next binade automatically */
        return (uint8_t)((((E + 7) << 3) + ((int)q - 8)) | sign);
    }
}

void oracle_e4m3_encode_array(const float *x, uint8_t *out, int64_t n)
{
    int64_t i;
#pragma omp parallel for schedule(static)
    for (i = 0; i < n; ++i)
        out[i] = oracle_e4m3_encode(x[i]);
}

void oracle_e4m3_encode_brute_array(const float *x, uint8_t *out, int64_t n)
{
    int64_t i;
#pragma omp parallel for schedule(static)
    for (i = 0; i < n; ++i)
        out[i] = oracle_e4m3_encode_brute(x[i]);
}

/* Encode the fp32 values whose bit patterns are first, first+1, ...,
 * first+n-1 (used for the all-patterns sweep). */
void oracle_e4m3_encode_bits_range(uint32_t first, int64_t n, uint8_t *out)
{
    int64_t i;
#pragma omp parallel for schedule(static)
    for (i = 0; i < n; ++i) {
        uint32_t bits = first + (uint32_t)i;
        float f;
        memcpy(&f, &bits, 4);
        out[i] = oracle_e4m3_encode(f);
    }
}

/* bf16 -> value: the upper 16 bits of an IEEE single. */
static float bf16_value(uint16_t h)
{
    uint32_t bits = (uint32_t)h << 16;
    float f;
    memcpy(&f, &bits, 4);
    return f;
}

/* ------------------------------------------------------------------------ */
/* O4. quantise one bf16 element with a per-head scale: enc(f32(x) / s).     */
/* The division is IEEE single precision (volatile keeps it a real float    */
/* division even if the compiler could fold it).                            */
/* ------------------------------------------------------------------------ */
uint8_t oracle_quantize(uint16_t x_bf16, float scale)
{
    volatile float num = bf16_value(x_bf16);
    volatile float den = scale;
    volatile float q = num / den;
    return oracle_e4m3_encode(q);
}

/* ------------------------------------------------------------------------ */
/* O5. addressing of token t of request b in the shared physical pool [PAG]. */
/*   page = page_table[b][t / P], slot = t mod P.                            */
/* Within a page, each KV head owns a K block and a V block of P*D elements  */
/* (e bytes each: 1 for e4m3, 2 for bf16), laid out as the library documents. */
/* Both blocks are cut into segments of SEG = min(P, 64/e) tokens.            */
/*   K: a token row of D*e bytes is R = D*e/16 chunks of 16 bytes, chunk      */
/*      c = q*KL + l with KL = R/4.  Token u of a segment, u = TG*s + 4j + a  */
/*      with TG = 16/e and a < 4, has chunk c at chunk position               */
/*      ((j*KL + l)*4 + q)*(4*NS) + 4s + a of the segment, NS = SEG/TG.       */
/*   V: a segment is [D][SEG]: element (u, d) at d*SEG + u.                   */
/* Offsets below are in elements from the start of the pool.                 */
/* ------------------------------------------------------------------------ */
static int64_t k_offset(int kv_dtype, int64_t page, int g, int slot, int d, int Hkv, int P, int D)
{
    int e = kv_dtype == 0 ? 1 : 2;
    int SEG = 64 / e < P ? 64 / e : P;
    int TG = 16 / e, NS = SEG / TG, R = D * e / 16, KL = R / 4;
    int seg = slot / SEG, u = slot % SEG;
    int sub = u / TG, w = u % TG, j = w / 4, a = w % 4;
    int byte = d * e, c = byte / 16, q = c / KL, l = c % KL;
    int64_t block = (page * Hkv + g) * (int64_t)P * D * e;            /* bytes */
    int64_t in_block = (int64_t)seg * SEG * D * e                     /* whole segments */
                       + ((int64_t)((j * KL + l) * 4 + q) * (4 * NS) + 4 * sub + a) * 16
                       + byte % 16;
    return (block + in_block) / e;
}

static int64_t v_offset(int kv_dtype, int64_t page, int g, int slot, int d, int Hkv, int P, int D)
{
    int e = kv_dtype == 0 ? 1 : 2;
    int SEG = 64 / e < P ? 64 / e : P;
    return (page * Hkv + g) * (int64_t)P * D + ((int64_t)(slot / SEG) * D + d) * SEG + slot % SEG;
}

int64_t oracle_k_offset(int kv_dtype, int64_t page, int g, int slot, int d, int Hkv, int P, int D)
{
    return k_offset(kv_dtype, page, g, slot, d, Hkv, P, D);
}

int64_t oracle_v_offset(int kv_dtype, int64_t page, int g, int slot, int d, int Hkv, int P, int D)
{
    return v_offset(kv_dtype, page, g, slot, d, Hkv, P, D);
}

/* ------------------------------------------------------------------------ */
/* O5'. write tokens into the pool.  Request b's source token j (j < count[b])
 * goes to position start[b] + j.  Source layout [B][T_src][Hkv][D] (bf16).
 * kv_dtype 0: e4m3 codes with per-head scales; 1: bf16 copied unchanged.
 * A request whose status is non-zero, or whose target page is outside the
 * table or the pool, is skipped.                                           */
/* ------------------------------------------------------------------------ */
void oracle_kv_write(int kv_dtype, int B, int maxP, int P, int Hkv, int D, int num_pages,
                     const int32_t *page_table, const int32_t *start, const int32_t *count,
                     int T_src, const int32_t *status,
                     const uint16_t *k_src, const uint16_t *v_src,
                     const float *k_scale, const float *v_scale,
                     void *k_pool, void *v_pool)
{
    int b, g;
    /* heads write disjoint bytes: one thread per head */
#pragma omp parallel for schedule(static) private(b)
    for (g = 0; g < Hkv; ++g) {
        for (b = 0; b < B; ++b) {
            int j;
            if (status && status[b] != 0)
                continue;
            for (j = 0; j < count[b]; ++j) {
                int64_t t = (int64_t)start[b] + j;
                int64_t pi = t / P;
                int slot = (int)(t % P), d;
                int32_t page;
                if (t < 0 || pi >= maxP)
                    continue;
                page = page_table[(int64_t)b * maxP + pi];
                if (page < 0 || page >= num_pages)
                    continue;
                for (d = 0; d < D; ++d) {
                    int64_t src = (((int64_t)b * T_src + j) * Hkv + g) * D + d;
                    int64_t ko = k_offset(kv_dtype, page, g, slot, d, Hkv, P, D);
                    int64_t vo = v_offset(kv_dtype, page, g, slot, d, Hkv, P, D);
                    if (kv_dtype == 0) {
                        ((uint8_t *)k_pool)[ko] = oracle_quantize(k_src[src], k_scale[g]);
                        ((uint8_t *)v_pool)[vo] = oracle_quantize(v_src[src], v_scale[g]);
                    } else {
                        ((uint16_t *)k_pool)[ko] = k_src[src];
                        ((uint16_t *)v_pool)[vo] = v_src[src];
                    }
                }
            }
        }
    }
}

/* Decode-step append: the new token sits at position context_lens[b] - 1.
 * Source layout [B][Hkv][D]. */
void oracle_kv_append(int kv_dtype, int B, int maxP, int P, int Hkv, int D, int num_pages,
                      const int32_t *page_table, const int32_t *context_lens,
                      const int32_t *status,
                      const uint16_t *k_new, const uint16_t *v_new,
                      const float *k_scale, const float *v_scale,
                      void *k_pool, void *v_pool)
{
    int b;
    for (b = 0; b < B; ++b) {
        int32_t start = context_lens[b] - 1, one = 1;
        if (context_lens[b] < 1 || (int64_t)context_lens[b] > (int64_t)maxP * P)
            continue;
        oracle_kv_write(kv_dtype, 1, maxP, P, Hkv, D, num_pages,
                        page_table + (int64_t)b * maxP, &start, &one, 1,
                        status ? status + b : NULL,
                        k_new + (int64_t)b * Hkv * D, v_new + (int64_t)b * Hkv * D,
                        k_scale, v_scale, k_pool, v_pool);
    }
}

/* ------------------------------------------------------------------------ */
/* O6. page-tag integrity check [KVP]: for every page covering the tokens of  */
/* request b, the physical page id must lie in the pool and its current tag   */
/* must equal the tag recorded for the request.  Flags are OR-ed.            */
/* ------------------------------------------------------------------------ */
void oracle_page_tag_check(int B, int maxP, int P, const int32_t *page_table,
                           const int32_t *context_lens, const uint32_t *expected_tags,
                           const uint32_t *page_tags, int num_pages, int32_t *status_out)
{
    int b;
    for (b = 0; b < B; ++b) {
        int32_t L = context_lens[b], st = 0;
        if (L < 1 || (int64_t)L > (int64_t)maxP * P) {
            st = ORACLE_REQ_BAD_LEN;
        } else {
            int n = (L + P - 1) / P, i;
            for (i = 0; i < n; ++i) {
                int32_t page = page_table[(int64_t)b * maxP + i];
                if (page < 0 || page >= num_pages)
                    st |= ORACLE_REQ_PAGE_OOB;
                else if (page_tags[page] != expected_tags[(int64_t)b * maxP + i])
                    st |= ORACLE_REQ_TAG_MISMATCH;
            }
        }
        status_out[b] = st;
    }
}

/* O6b: giving pages to new owners (Cloudflare, "Smaller, faster, safer",
 * section "共享 KV 缓存保护": a page's tag changes every time the page is
 * reallocated).  Entries are applied in list order: the page's tag moves on
 * by one (modulo 2^32) and an owner inside the table records the page and
 * the new tag.  Entries naming a page outside the pool change nothing. */
void oracle_page_tag_realloc(int n, const int32_t *page_ids, const int32_t *owner_req,
                             const int32_t *owner_slot, uint32_t *page_tags, int num_pages,
                             int32_t *page_table, uint32_t *expected_tags, int B, int maxP)
{
    int k;
    for (k = 0; k < n; ++k) {
        int32_t page = page_ids[k], b, i;
        if (page < 0 || page >= num_pages)
            continue;
        page_tags[page] = page_tags[page] + 1u;
        if (owner_req == NULL)
            continue;
        b = owner_req[k];
        i = owner_slot[k];
        if (b < 0 || b >= B || i < 0 || i >= maxP)
            continue;
        expected_tags[(int64_t)b * maxP + i] = page_tags[page];
        if (page_table != NULL)
            page_table[(int64_t)b * maxP + i] = page;
    }
}

/* exact value of element (token t, head g, dim d) of K or V, or NaN when the
 * token's page is not a valid page of the pool */
static double kv_value(int kv_dtype, int is_v, const void *pool, const float *scale,
                       const int32_t *pt_row, int maxP, int P, int Hkv, int D,
                       int num_pages, int64_t t, int g, int d, int *bad)
{
    int64_t pi = t / P;
    int slot = (int)(t % P);
    int32_t page;
    int64_t off;
    if (pi >= maxP) {
        *bad = 1;
        return NAN;
    }
    page = pt_row[pi];
    if (page < 0 || page >= num_pages) {
        *bad = 1;
        return NAN;
    }
    off = is_v ? v_offset(kv_dtype, page, g, slot, d, Hkv, P, D)
               : k_offset(kv_dtype, page, g, slot, d, Hkv, P, D);
    if (kv_dtype == 0)
        return oracle_e4m3_decode(((const uint8_t *)pool)[off]) * (double)scale[g];
    return (double)bf16_value(((const uint16_t *)pool)[off]);
}

/* ------------------------------------------------------------------------ */
/* O7. attention of one (request, query head) over tokens [t0, t1), fp64.     */
/*   s_t = sm_scale * sum_d q_d * k_t,d                                      */
/*   lse = log sum_t exp(s_t);  o = sum_t exp(s_t - lse) * v_t               */
/* Writes o[D] and lse.  An empty range gives o = 0, lse = -inf; a range     */
/* that touches an invalid page gives NaN.                                   */
/* ------------------------------------------------------------------------ */
static void attend_range(int kv_dtype, const void *k_pool, const void *v_pool,
                         const float *k_scale, const float *v_scale,
                         const int32_t *pt_row, int maxP, int P, int Hkv, int D, int num_pages,
                         const uint16_t *q_row, int g, double sm_scale,
                         int64_t t0, int64_t t1, double *o, double *lse)
{
    int64_t n = t1 - t0, t;
    int d, bad = 0;
    double *s, m = -INFINITY, sum = 0.0;
    for (d = 0; d < D; ++d)
        o[d] = 0.0;
    if (n <= 0) {
        *lse = -INFINITY;
        return;
    }
    s = (double *)malloc((size_t)n * sizeof(double));
    for (t = 0; t < n; ++t) {
        double acc = 0.0;
        for (d = 0; d < D; ++d)
            acc += (double)bf16_value(q_row[d]) *
                   kv_value(kv_dtype, 0, k_pool, k_scale, pt_row, maxP, P, Hkv, D, num_pages,
                            t0 + t, g, d, &bad);
        s[t] = sm_scale * acc;
        if (s[t] > m)
            m = s[t];
    }
    if (bad) {
        for (d = 0; d < D; ++d)
            o[d] = NAN;
        *lse = NAN;
        free(s);
        return;
    }
    for (t = 0; t < n; ++t)
        sum += exp(s[t] - m);
    *lse = m + log(sum);
    for (t = 0; t < n; ++t) {
        double p = exp(s[t] - *lse);
        for (d = 0; d < D; ++d)
            o[d] += p * kv_value(kv_dtype, 1, v_pool, v_scale, pt_row, maxP, P, Hkv, D,
                                 num_pages, t0 + t, g, d, &bad);
    }
    free(s);
}

/* Full decode attention for a batch.  q: bf16 [B][Hq][D]; out: fp64 [B][Hq][D];
 * lse: fp64 [B][Hq].  status may be NULL (no tracker). */
void oracle_paged_attention(int kv_dtype, int B, int Hq, int Hkv, int D, int P, int maxP,
                            int num_pages, const int32_t *page_table,
                            const int32_t *context_lens, const int32_t *status,
                            const uint16_t *q, const void *k_pool, const void *v_pool,
                            const float *k_scale, const float *v_scale, double sm_scale,
                            double *out, double *lse)
{
    int G = Hq / Hkv;
    int64_t bh;
#pragma omp parallel for schedule(dynamic, 1)
    for (bh = 0; bh < (int64_t)B * Hq; ++bh) {
        int b = (int)(bh / Hq), h = (int)(bh % Hq), d;
        int32_t L = context_lens[b];
        double *o = out + bh * D;
        if (status && status[b] != 0) {
            for (d = 0; d < D; ++d)
                o[d] = 0.0;
            lse[bh] = -INFINITY;
            continue;
        }
        if (L < 0 || (int64_t)L > (int64_t)maxP * P) {
            for (d = 0; d < D; ++d)
                o[d] = NAN;
            lse[bh] = NAN;
            continue;
        }
        attend_range(kv_dtype, k_pool, v_pool, k_scale, v_scale,
                     page_table + (int64_t)b * maxP, maxP, P, Hkv, D, num_pages,
                     q + bh * D, h / G, sm_scale, 0, L, o, &lse[bh]);
    }
}

/* Attention of one (b, h) restricted to tokens [t0, t1): a partial result. */
void oracle_attention_range(int kv_dtype, int Hq, int Hkv, int D, int P, int maxP,
                            int num_pages, const int32_t *page_table, int b, int h,
                            const uint16_t *q, const void *k_pool, const void *v_pool,
                            const float *k_scale, const float *v_scale, double sm_scale,
                            int64_t t0, int64_t t1, double *o, double *lse)
{
    int G = Hq / Hkv;
    attend_range(kv_dtype, k_pool, v_pool, k_scale, v_scale,
                 page_table + (int64_t)b * maxP, maxP, P, Hkv, D, num_pages,
                 q + ((int64_t)b * Hq + h) * D, h / G, sm_scale, t0, t1, o, lse);
}

/* ------------------------------------------------------------------------ */
/* O8. combine per-split partials (o_s, lse_s) of one softmax:               */
/*   LSE = log sum_s exp(lse_s),  out = sum_s exp(lse_s - LSE) * o_s          */
/* Splits with lse = -inf are empty and contribute nothing; if all are empty */
/* the result is out = 0, lse = -inf.  A non-zero status gives 0 / -inf.     */
/* part_o: fp32 [B][Hq][S][D]; part_lse: fp32 [B][Hq][S].                    */
/* ------------------------------------------------------------------------ */
void oracle_splitk_combine(int B, int Hq, int S, int D, const float *part_o,
                           const float *part_lse, const int32_t *status,
                           double *out, double *lse)
{
    int64_t bh;
    for (bh = 0; bh < (int64_t)B * Hq; ++bh) {
        int b = (int)(bh / Hq), s, d;
        double M = -INFINITY, sum = 0.0, LSE;
        double *o = out + bh * D;
        const float *pl = part_lse + bh * S;
        const float *po = part_o + bh * S * D;
        int has_nan = 0;
        for (d = 0; d < D; ++d)
            o[d] = 0.0;
        if (status && status[b] != 0) {
            lse[bh] = -INFINITY;
            continue;
        }
        for (s = 0; s < S; ++s) {
            if (isnan(pl[s]))
                has_nan = 1;
            else if ((double)pl[s] > M)
                M = pl[s];
        }
        if (has_nan) {
            for (d = 0; d < D; ++d)
                o[d] = NAN;
            lse[bh] = NAN;
            continue;
        }
        if (M == -INFINITY) {
            lse[bh] = -INFINITY;
            continue;
        }
        for (s = 0; s < S; ++s)
            sum += exp((double)pl[s] - M);
        LSE = M + log(sum);
        for (s = 0; s < S; ++s) {
            double w;
            if (pl[s] == -INFINITY)
                continue;
            w = exp((double)pl[s] - LSE);
            for (d = 0; d < D; ++d)
                o[d] += w * (double)po[(int64_t)s * D + d];
        }
        lse[bh] = LSE;
    }
}

int oracle_num_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* ------------------------------------------------------------------------
 * INT4 weight streaming (Cloudflare, "Smaller, faster, safer", section
 * "模型权重压缩" (model weight compression): GLM weights go from FP8 to INT4; decode reads
 * the weights for every token and expands them before multiplying).  The
 * pages give no grouping or zero point; the reading taken: symmetric signed
 * 4-bit integers, one bf16 scale per output row and 128 input features.
 * ------------------------------------------------------------------------ */

/* weight q[n][k] from the packed layout: 1024-byte blocks per (16 rows,
 * 128 features), ordered by row tile then group; inside a block, byte
 * 16*(16*kq + c) + 4*j + b holds row 16*nt + c, features
 * 128*g + 32*j + 8*kq + 2*b (low nibble) and the next one (high nibble) */
static int int4_weight(const uint8_t *packed, int K, int n, int k)
{
    int nt = n / 16, c = n % 16, g = k / 128, r = k % 128;
    int j = r / 32, kq = (r % 32) / 8, b = (r % 8) / 2, high = r % 2;
    int64_t byte = ((int64_t)nt * (K / 128) + g) * 1024 + (16 * kq + c) * 16 + 4 * j + b;
    int nib = high ? (packed[byte] >> 4) & 15 : packed[byte] & 15;
    return nib >= 8 ? nib - 16 : nib;
}

void oracle_int4_unpack(const uint8_t *packed, int N, int K, int8_t *q_out)
{
    int n, k;
    for (n = 0; n < N; ++n)
        for (k = 0; k < K; ++k)
            q_out[(int64_t)n * K + k] = (int8_t)int4_weight(packed, K, n, k);
}

/* y[m][n] = sum_k x[m][k] * q[n][k] * s[k / 128][n], in fp64 (exact inputs) */
void oracle_int4_gemv(int M, int N, int K, const uint16_t *x, const uint8_t *packed,
                      const uint16_t *scales, double *y)
{
    int64_t mn;
#ifdef _OPENMP
#pragma omp parallel for schedule(dynamic, 64)
#endif
    for (mn = 0; mn < (int64_t)M * N; ++mn) {
        int m = (int)(mn / N), n = (int)(mn % N), k;
        {
            double acc = 0.0;
            for (k = 0; k < K; ++k) {
                double xv = (double)bf16_value(x[(int64_t)m * K + k]);
                double sv = (double)bf16_value(scales[(int64_t)(k / 128) * N + n]);
                acc += xv * (double)int4_weight(packed, K, n, k) * sv;
            }
            y[(int64_t)m * N + n] = acc;
        }
    }
}

