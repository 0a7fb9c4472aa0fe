/*
 * Plain CPU oracle of the MiniMax-M3 MSA fused producer.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path may link, load or call
 * this file: only the test suite, the smoke check and the CPU-baseline leg of
 * the benchmark use it.  It shares no code, header, table or helper with the
 * HIP implementation in paged_kv_cache_msa_amd/csrc.
 *
 * What it computes (sources are the three pull-request pages):
 *   - "Fuse MiniMax-M3 QKV and index projection", AFTER figure and change list:
 *     one packed projection row [Q | K | V | index-Q | index-K] per token;
 *     Q/K normalisation and RoPE on Q, K, index-Q and index-K; compact Q and
 *     index-Q outputs; K, V and index-K written into paged HND caches (FP8),
 *     with padded or out-of-range cache slots contained (skipped).
 *   - "Fuse MiniMax-M3 MSA per-layer KV-cache writes into one kernel",
 *     sections "The problem", "The fix" and "Nsys trace": a token's cache
 *     location is page = slot / page_size, offset = slot % page_size, computed
 *     once per token, and K, V and index-K are written together.
 *   - "Wire in custom decode kernels for MinimaxM3", conflict-resolution
 *     commit notes: write slots are derived from the per-request block (page)
 *     table rather than a per-token slot buffer.
 *
 * The pages fix no arithmetic precision.  The readings used here (each one
 * IEEE-754 operation rounding once, round-to-nearest-even, no fused
 * multiply-add, denormals kept):
 *   inv_freq_i = 1 / theta^(2i/D)                                   (binary64)
 *   angle      = pos * inv_freq_i                                   (binary64)
 *   c_i, s_i   = (float)cos(angle), (float)sin(angle)               (binary64 libm, one rounding)
 *   ss         = sum_j a_j^2, ascending j                           (binary64)
 *   r          = (float)(1 / sqrt(ss / D + eps))                    (binary64, one final rounding)
 *   y_j        = (a_j * r) * w_j                                    (binary32, two roundings)
 *   o_i        = y_i * c_i - y_{i+D/2} * s_i                        (binary32, neox rotate-half)
 *   o_{i+D/2}  = y_{i+D/2} * c_i + y_i * s_i
 *   Q, index-Q outputs: bf16(o) for every token, padded or not.
 *   cache values: K and index-K use o, V uses the raw input a;
 *     fp8 cache: e4m3_satfinite(v * (float)(1 / scale)),  bf16 cache: bf16(v).
 *
 * Built with: gcc -O2 -std=c11 -ffp-contract=off -fno-fast-math -fopenmp
 * (on x86-64 every float operation rounds to binary32).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORC_OK 0
#define ORC_ERR_ARG 1
#define ORC_ERR_DUPLICATE_SLOT 2

#define ORC_FP8_E4M3 0
#define ORC_BF16 1

static float f32_of_bits(uint32_t u) { float f; memcpy(&f, &u, sizeof f); return f; }
static uint32_t bits_of_f32(float f) { uint32_t u; memcpy(&u, &f, sizeof u); return u; }

/* bf16 storage -> value: bf16 is the upper half of a binary32. */
static float bf16_value(uint16_t h) { return f32_of_bits((uint32_t)h << 16); }

/*
 * binary32 -> bf16 (1 sign, 8 exponent, 7 fraction bits), round to nearest,
 * ties to even, overflow to infinity.  A NaN keeps its sign and upper payload
 * and becomes quiet.  The value is rounded on the grid of its binade: a bf16
 * carries 8 significant bits, so for |v| in [2^(e-1), 2^e) the spacing is
 * 2^(e-8), and never finer than the subnormal spacing 2^-133.
 */
uint16_t msa_oracle_bf16(float v)
{
    uint32_t u = bits_of_f32(v);
    if (isnan(v)) return (uint16_t)((u >> 16) | 0x0040u);
    if (isinf(v) || v == 0.0f) return (uint16_t)(u >> 16);
    double d = (double)v;
    int e;
    frexp(fabs(d), &e);
    int qexp = e - 8;
    if (qexp < -133) qexp = -133;
    double r = ldexp(nearbyint(ldexp(d, -qexp)), qexp);   /* scalings exact; nearbyint is RNE */
    if (fabs(r) >= ldexp(1.0, 128)) return (uint16_t)((u >> 16 & 0x8000u) | 0x7f80u);
    return (uint16_t)(bits_of_f32((float)r) >> 16);       /* r has <= 8 significant bits: exact */
}

/*
 * binary32 -> OCP FP8 E4M3 ("E4M3FN": exponent bias 7, 3 fraction bits, no
 * infinities, S.1111.111 is NaN, largest finite 448 = 0x7E, smallest
 * subnormal 2^-9).  Round to nearest, ties to even; saturating: every
 * magnitude >= 448, infinities included, becomes +-448.  NaN -> S.1111.111.
 * The sign of zero is kept.  Normal spacing for |v| in [2^(e-1), 2^e) is
 * 2^(e-4); subnormal spacing 2^-9.
 */
uint8_t msa_oracle_e4m3(float v)
{
    uint8_t sign = signbit(v) ? 0x80u : 0x00u;
    if (isnan(v)) return (uint8_t)(sign | 0x7fu);
    double a = fabs((double)v);
    if (a >= 448.0) return (uint8_t)(sign | 0x7eu);
    if (a == 0.0) return sign;
    int e;
    frexp(a, &e);
    int qexp = e - 4;
    if (qexp < -9) qexp = -9;
    double r = ldexp(nearbyint(ldexp(a, -qexp)), qexp);   /* rounded magnitude, <= 448 */
    if (r == 0.0) return sign;
    if (r < ldexp(1.0, -6))                                /* subnormal: r = m * 2^-9 */
        return (uint8_t)(sign | (uint8_t)ldexp(r, 9));
    int er;
    double m = frexp(r, &er);                              /* r = m * 2^er, m in [0.5, 1) */
    int exp_field = er - 1 + 7;
    int frac = (int)ldexp(m * 2.0 - 1.0, 3);
    return (uint8_t)(sign | (uint8_t)(exp_field << 3) | (uint8_t)frac);
}

/*
 * binary64 -> bf16 in one rounding (round to nearest, ties to even, overflow
 * to infinity), on the same per-binade grid as above.  Rounding a binary64 sum
 * through binary32 first would round twice; this does not.  NaN -> the quiet
 * NaN 0x7fc0 with the sign.
 */
uint16_t msa_oracle_bf16_of_f64(double d)
{
    uint16_t sign = signbit(d) ? 0x8000u : 0x0000u;
    if (isnan(d)) return (uint16_t)(sign | 0x7fc0u);
    if (isinf(d)) return (uint16_t)(sign | 0x7f80u);
    if (d == 0.0) return sign;
    int e;
    frexp(fabs(d), &e);
    int qexp = e - 8;
    if (qexp < -133) qexp = -133;
    double r = ldexp(nearbyint(ldexp(d, -qexp)), qexp);   /* scalings exact; nearbyint is RNE */
    if (fabs(r) >= ldexp(1.0, 128)) return (uint16_t)(sign | 0x7f80u);
    if (r == 0.0) return sign;
    return (uint16_t)(bits_of_f32((float)r) >> 16);       /* r has <= 8 significant bits: exact */
}

void msa_oracle_encode_bf16(const float* v, int64_t n, uint16_t* out)
{
    for (int64_t i = 0; i < n; ++i) out[i] = msa_oracle_bf16(v[i]);
}

void msa_oracle_encode_e4m3(const float* v, int64_t n, uint8_t* out)
{
    for (int64_t i = 0; i < n; ++i) out[i] = msa_oracle_e4m3(v[i]);
}

/* RoPE coefficients for one position: c[i], s[i], i in [0, D/2). */
static void rope_coeffs(int32_t pos, double theta, int32_t head_dim, float* c, float* s)
{
    for (int32_t i = 0; i < head_dim / 2; ++i) {
        double inv_freq = 1.0 / pow(theta, (double)(2 * i) / (double)head_dim);
        double angle = (double)pos * inv_freq;
        c[i] = (float)cos(angle);
        s[i] = (float)sin(angle);
    }
}

/* Table of coefficients for n positions: cos_out/sin_out are [n, D/2]. */
void msa_oracle_rope_table(const int32_t* pos, int64_t n, double theta, int32_t head_dim,
                           float* cos_out, float* sin_out)
{
    for (int64_t t = 0; t < n; ++t)
        rope_coeffs(pos[t], theta, head_dim, cos_out + t * (head_dim / 2), sin_out + t * (head_dim / 2));
}

/* RMSNorm scale from a sum of squares. */
static float rms_scale_from_ss(double ss, int32_t head_dim, float eps)
{
    return (float)(1.0 / sqrt(ss / (double)head_dim + (double)eps));
}

void msa_oracle_rms_scale(const double* ss, int64_t n, int32_t head_dim, float eps, float* r_out)
{
    for (int64_t i = 0; i < n; ++i) r_out[i] = rms_scale_from_ss(ss[i], head_dim, eps);
}

/*
 * Cache slot of one token: page_table[seq][pos / P] * P + pos % P, or -1 when
 * the token is padded or its page lies outside the table or the pool.
 */
static int64_t token_slot(int32_t pos, int32_t seq, const int32_t* page_table, int64_t pt_stride,
                          int32_t num_seqs, int32_t max_pages, int32_t page_size, int64_t num_pages,
                          int64_t* page, int64_t* offset)
{
    if (seq < 0 || seq >= num_seqs || pos < 0) return -1;
    int32_t logical = pos / page_size;
    if (logical >= max_pages) return -1;
    int64_t pg = page_table[(int64_t)seq * pt_stride + logical];
    if (pg < 0 || pg >= num_pages) return -1;
    *page = pg;
    *offset = pos % page_size;
    return pg * page_size + pos % page_size;
}

void msa_oracle_slots(const int32_t* pos, const int32_t* seq, int64_t n, const int32_t* page_table,
                      int64_t pt_stride, int32_t num_seqs, int32_t max_pages, int32_t page_size,
                      int64_t num_pages, int64_t* slots)
{
    for (int64_t t = 0; t < n; ++t) {
        int64_t pg, off;
        slots[t] = token_slot(pos[t], seq[t], page_table, pt_stride, num_seqs, max_pages,
                              page_size, num_pages, &pg, &off);
    }
}

static int cmp_i64(const void* a, const void* b)
{
    int64_t x = *(const int64_t*)a, y = *(const int64_t*)b;
    return (x > y) - (x < y);
}

/* Streams of the packed row, in column order. */
enum { S_Q = 0, S_K = 1, S_V = 2, S_IQ = 3, S_IK = 4 };

/*
 * One token's five streams.  Writes:
 *   q_out  [hq,  D] bf16          iq_out [hiq, D] bf16
 *   k_rows [hkv, D], v_rows [hkv, D], ik_rows [hik, D]: cache codes (1 byte
 *   for fp8, 2 bytes for bf16), as they are to be stored in the cache.
 */
static void produce_token(const uint16_t* row, int32_t head_dim, int32_t hq, int32_t hkv, int32_t hiq,
                          int32_t hik, int32_t pos, const uint16_t* const w[4], float eps, double theta,
                          const int32_t dtype[3], const float inv_scale[3], uint16_t* q_out,
                          uint16_t* iq_out, void* rows[3], float* scratch)
{
    const int32_t half = head_dim / 2;
    float* c = scratch;
    float* s = c + half;
    float* a = s + half;
    float* y = a + head_dim;
    float* o = y + head_dim;
    rope_coeffs(pos, theta, head_dim, c, s);

    const int32_t counts[5] = { hq, hkv, hkv, hiq, hik };
    int32_t col = 0;
    for (int st = 0; st < 5; ++st) {
        for (int32_t h = 0; h < counts[st]; ++h, col += head_dim) {
            for (int32_t j = 0; j < head_dim; ++j) a[j] = bf16_value(row[col + j]);
            const float* v = a;
            if (st != S_V) {
                const uint16_t* wt = w[st == S_Q ? 0 : st == S_K ? 1 : st == S_IQ ? 2 : 3];
                double ss = 0.0;
                for (int32_t j = 0; j < head_dim; ++j) ss += (double)a[j] * (double)a[j];
                float r = rms_scale_from_ss(ss, head_dim, eps);
                for (int32_t j = 0; j < head_dim; ++j) y[j] = (a[j] * r) * bf16_value(wt[j]);
                for (int32_t i = 0; i < half; ++i) {
                    o[i] = y[i] * c[i] - y[i + half] * s[i];
                    o[i + half] = y[i + half] * c[i] + y[i] * s[i];
                }
                v = o;
            }
            if (st == S_Q || st == S_IQ) {
                uint16_t* dst = (st == S_Q ? q_out : iq_out) + (int64_t)h * head_dim;
                for (int32_t j = 0; j < head_dim; ++j) dst[j] = msa_oracle_bf16(v[j]);
            } else {
                int ci = st == S_K ? 0 : st == S_V ? 1 : 2;
                if (dtype[ci] == ORC_FP8_E4M3) {
                    uint8_t* dst = (uint8_t*)rows[ci] + (int64_t)h * head_dim;
                    for (int32_t j = 0; j < head_dim; ++j) dst[j] = msa_oracle_e4m3(v[j] * inv_scale[ci]);
                } else {
                    uint16_t* dst = (uint16_t*)rows[ci] + (int64_t)h * head_dim;
                    for (int32_t j = 0; j < head_dim; ++j) dst[j] = msa_oracle_bf16(v[j]);
                }
            }
        }
    }
}

static int check_common(int64_t T, int32_t head_dim, int32_t hq, int32_t hkv, int32_t hiq, int32_t hik,
                        int32_t page_size, const int32_t dtype[3])
{
    if (T < 0 || head_dim <= 0 || head_dim % 2 || hq < 0 || hkv < 0 || hiq < 0 || hik < 0 || page_size <= 0)
        return ORC_ERR_ARG;
    for (int i = 0; i < 3; ++i)
        if (dtype[i] != ORC_FP8_E4M3 && dtype[i] != ORC_BF16) return ORC_ERR_ARG;
    return ORC_OK;
}

static int check_unique(const int64_t* slots, int64_t T)
{
    int64_t* sorted = (int64_t*)malloc((size_t)(T > 0 ? T : 1) * sizeof(int64_t));
    if (!sorted) return ORC_ERR_ARG;
    int64_t m = 0;
    for (int64_t t = 0; t < T; ++t)
        if (slots[t] >= 0) sorted[m++] = slots[t];
    qsort(sorted, (size_t)m, sizeof(int64_t), cmp_i64);
    int rc = ORC_OK;
    for (int64_t i = 1; i < m; ++i)
        if (sorted[i] == sorted[i - 1]) rc = ORC_ERR_DUPLICATE_SLOT;
    free(sorted);
    return rc;
}

/*
 * Dense form: per-token cache rows instead of cache writes.
 *   x        bf16, row t at x + t * x_stride, W = (hq + 2 hkv + hiq + hik) * D columns used
 *   q_out    bf16 [T, hq, D];  iq_out bf16 [T, hiq, D]
 *   k_rows   [T, hkv, D], v_rows [T, hkv, D], ik_rows [T, hik, D] in cache codes
 *   slots    int64 [T], slot or -1
 * scales are the per-tensor dequantisation scales (fp8 caches only).
 * Rows are produced for every token; the caller uses slots to place them.
 */
int msa_oracle_produce_rows(const uint16_t* x, int64_t x_stride, int64_t T, int32_t head_dim,
                            int32_t hq, int32_t hkv, int32_t hiq, int32_t hik,
                            const int32_t* positions, const int32_t* seq_idx,
                            const int32_t* page_table, int64_t pt_stride, int32_t num_seqs,
                            int32_t max_pages, int32_t page_size, int64_t num_pages,
                            const uint16_t* w_q, const uint16_t* w_k, const uint16_t* w_iq,
                            const uint16_t* w_ik, float eps, double theta,
                            int32_t k_dtype, int32_t v_dtype, int32_t ik_dtype,
                            float k_scale, float v_scale, float ik_scale,
                            uint16_t* q_out, uint16_t* iq_out, void* k_rows, void* v_rows,
                            void* ik_rows, int64_t* slots, int32_t num_threads)
{
    const int32_t dtype[3] = { k_dtype, v_dtype, ik_dtype };
    int rc = check_common(T, head_dim, hq, hkv, hiq, hik, page_size, dtype);
    if (rc) return rc;
    const uint16_t* const w[4] = { w_q, w_k, w_iq, w_ik };
    const float inv_scale[3] = { 1.0f / k_scale, 1.0f / v_scale, 1.0f / ik_scale };
    const int32_t heads[3] = { hkv, hkv, hik };
    void* const base[3] = { k_rows, v_rows, ik_rows };
    if (num_threads < 1) num_threads = 1;

    #pragma omp parallel num_threads(num_threads)
    {
        float* scratch = (float*)malloc(sizeof(float) * (size_t)head_dim * 4);
        #pragma omp for schedule(static)
        for (int64_t t = 0; t < T; ++t) {
            int64_t pg, off;
            slots[t] = token_slot(positions[t], seq_idx[t], page_table, pt_stride, num_seqs, max_pages,
                                  page_size, num_pages, &pg, &off);
            void* rows[3];
            for (int ci = 0; ci < 3; ++ci) {
                int64_t esize = dtype[ci] == ORC_FP8_E4M3 ? 1 : 2;
                rows[ci] = (uint8_t*)base[ci] + t * heads[ci] * head_dim * esize;
            }
            produce_token(x + t * x_stride, head_dim, hq, hkv, hiq, hik, positions[t], w, eps, theta,
                          dtype, inv_scale, q_out + t * hq * head_dim, iq_out + t * hiq * head_dim,
                          rows, scratch);
        }
        free(scratch);
    }
    return check_unique(slots, T);
}

/*
 * Cache form: the same computation, with K, V and index-K written into paged
 * caches.  Cache element (page, head, token, d) lives at element offset
 * page * s_page + head * s_head + token * s_token + d from the cache base.
 * Only tokens with a valid slot write; nothing else in a cache changes.
 */
int msa_oracle_produce(const uint16_t* x, int64_t x_stride, int64_t T, int32_t head_dim,
                       int32_t hq, int32_t hkv, int32_t hiq, int32_t hik,
                       const int32_t* positions, const int32_t* seq_idx,
                       const int32_t* page_table, int64_t pt_stride, int32_t num_seqs,
                       int32_t max_pages, int32_t page_size, int64_t num_pages,
                       const uint16_t* w_q, const uint16_t* w_k, const uint16_t* w_iq,
                       const uint16_t* w_ik, float eps, double theta,
                       void* k_cache, int64_t k_sp, int64_t k_sh, int64_t k_st, int32_t k_dtype, float k_scale,
                       void* v_cache, int64_t v_sp, int64_t v_sh, int64_t v_st, int32_t v_dtype, float v_scale,
                       void* ik_cache, int64_t ik_sp, int64_t ik_sh, int64_t ik_st, int32_t ik_dtype, float ik_scale,
                       uint16_t* q_out, uint16_t* iq_out, int64_t* slots, int32_t num_threads)
{
    const int32_t dtype[3] = { k_dtype, v_dtype, ik_dtype };
    int rc = check_common(T, head_dim, hq, hkv, hiq, hik, page_size, dtype);
    if (rc) return rc;
    const int32_t heads[3] = { hkv, hkv, hik };
    int64_t esize[3];
    void* rows[3];
    for (int ci = 0; ci < 3; ++ci) {
        esize[ci] = dtype[ci] == ORC_FP8_E4M3 ? 1 : 2;
        rows[ci] = malloc((size_t)((T > 0 ? T : 1) * heads[ci] * head_dim * esize[ci] + 1));
    }
    if (!rows[0] || !rows[1] || !rows[2]) { free(rows[0]); free(rows[1]); free(rows[2]); return ORC_ERR_ARG; }
    rc = msa_oracle_produce_rows(x, x_stride, T, head_dim, hq, hkv, hiq, hik, positions, seq_idx,
                                 page_table, pt_stride, num_seqs, max_pages, page_size, num_pages,
                                 w_q, w_k, w_iq, w_ik, eps, theta, k_dtype, v_dtype, ik_dtype,
                                 k_scale, v_scale, ik_scale, q_out, iq_out, rows[0], rows[1], rows[2],
                                 slots, num_threads);
    if (rc == ORC_OK) {
        void* const cache[3] = { k_cache, v_cache, ik_cache };
        const int64_t sp[3] = { k_sp, v_sp, ik_sp }, sh[3] = { k_sh, v_sh, ik_sh }, stt[3] = { k_st, v_st, ik_st };
        for (int64_t t = 0; t < T; ++t) {
            if (slots[t] < 0) continue;
            int64_t pg = slots[t] / page_size, off = slots[t] % page_size;
            for (int ci = 0; ci < 3; ++ci)
                for (int32_t h = 0; h < heads[ci]; ++h) {
                    int64_t dst = pg * sp[ci] + h * sh[ci] + off * stt[ci];
                    int64_t src = (t * heads[ci] + h) * head_dim;
                    memcpy((uint8_t*)cache[ci] + dst * esize[ci], (uint8_t*)rows[ci] + src * esize[ci],
                           (size_t)(head_dim * esize[ci]));
                }
        }
    }
    for (int ci = 0; ci < 3; ++ci) free(rows[ci]);
    return rc;
}

/* ------------------------------------------------------------------------------------------------
 * Indexer (the downstream consumer of the index-K cache): proxy scores of index-Q against the
 * visible index-K keys, max-pooled over fixed token blocks, then the top-k blocks per query.
 * Pages: "Fuse MiniMax-M3 MSA per-layer KV-cache writes into one kernel", "Where this PR targets
 * at", step 4 (proxy-FMHA over index-K, max-reduce, top-16 of 128-token blocks); "Fuse MiniMax-M3
 * QKV and index projection", BEFORE/AFTER figures (score visible index-K, max-pool by block,
 * select top-k block IDs).  Reading: the score of key position p for query token t and index-Q
 * head h is the exact dot product iq[t,h,:] . ik[p,:] (binary64: every product of a bf16 and an
 * e4m3/bf16 value is exact, and so is the sum for any realistic range), times the index-K
 * dequantisation scale; visible = same sequence, 0 <= p <= pos_t, with a valid page.  Softmax
 * and 1/sqrt(D) are monotone per (t, h) and do not change the selection, so they are not applied.
 * ---------------------------------------------------------------------------------------------- */

/* OCP E4M3 code -> value (NaN for S.1111.111). */
static double e4m3_value(uint8_t c)
{
    int E = (c >> 3) & 15, M = c & 7;
    double mag;
    if (E == 15 && M == 7) return NAN;
    mag = E == 0 ? ldexp((double)M, -9) : ldexp((double)(8 + M), E - 10);
    return (c & 0x80) ? -mag : mag;
}

/*
 * block_scores [hiq, T, max_blocks]: for block b (positions [b*B, (b+1)*B)) the maximum over its
 * visible keys of the score; -inf when none is visible.  Padded tokens (no valid own slot) get -inf
 * everywhere.  Index-Q head h reads index-K head h / (hiq / hik).
 */
int msa_oracle_index_scores(const uint16_t* iq, int64_t T, int32_t hiq, int32_t head_dim,
                            const int32_t* positions, const int32_t* seq_idx, const int32_t* page_table,
                            int64_t pt_stride, int32_t num_seqs, int32_t max_pages, int32_t page_size,
                            int64_t num_pages, const void* ik_cache, int64_t sp, int64_t sh, int64_t st,
                            int32_t hik, int32_t ik_dtype, float ik_scale, int32_t block_tokens,
                            int32_t max_blocks, double* block_scores)
{
    if (T < 0 || hiq <= 0 || hik <= 0 || hiq % hik || head_dim <= 0 || page_size <= 0 || block_tokens <= 0 ||
        max_blocks < 0 || (ik_dtype != ORC_FP8_E4M3 && ik_dtype != ORC_BF16))
        return ORC_ERR_ARG;
    const int32_t group = hiq / hik;
    const double scale = ik_dtype == ORC_FP8_E4M3 ? (double)ik_scale : 1.0;
    for (int64_t i = 0; i < (int64_t)hiq * T * max_blocks; ++i) block_scores[i] = -INFINITY;
    for (int64_t t = 0; t < T; ++t) {
        int64_t pg, off;
        if (token_slot(positions[t], seq_idx[t], page_table, pt_stride, num_seqs, max_pages, page_size,
                       num_pages, &pg, &off) < 0)
            continue;
        const int32_t s = seq_idx[t];
        for (int32_t p = 0; p <= positions[t]; ++p) {
            int64_t kpg, koff;
            if (token_slot(p, s, page_table, pt_stride, num_seqs, max_pages, page_size, num_pages, &kpg, &koff) < 0)
                continue;
            const int32_t b = p / block_tokens;
            if (b >= max_blocks) continue;
            for (int32_t h = 0; h < hiq; ++h) {
                const int64_t base = kpg * sp + (int64_t)(h / group) * sh + koff * st;
                double dot = 0.0;
                for (int32_t j = 0; j < head_dim; ++j) {
                    double k = ik_dtype == ORC_FP8_E4M3 ? e4m3_value(((const uint8_t*)ik_cache)[base + j])
                                                        : (double)bf16_value(((const uint16_t*)ik_cache)[base + j]);
                    dot += (double)bf16_value(iq[(t * hiq + h) * head_dim + j]) * k;
                }
                const double score = dot * scale;
                double* dst = &block_scores[((int64_t)h * T + t) * max_blocks + b];
                if (score > *dst) *dst = score;
            }
        }
    }
    return ORC_OK;
}

/*
 * Top-k blocks of every (head, token) row of block_scores: ids [hiq, T, top_k] in descending score,
 * equal scores in ascending block index; blocks scored -inf are never selected; unused entries are
 * -1.  counts [hiq, T] (optional) = number of selected blocks.
 */
int msa_oracle_index_topk(const double* block_scores, int32_t hiq, int64_t T, int32_t max_blocks, int32_t top_k,
                          int32_t* ids, int32_t* counts)
{
    if (hiq <= 0 || T < 0 || max_blocks < 0 || top_k <= 0) return ORC_ERR_ARG;
    for (int64_t r = 0; r < (int64_t)hiq * T; ++r) {
        const double* row = block_scores + r * max_blocks;
        int32_t* out = ids + r * top_k;
        int32_t n = 0;
        for (int32_t k = 0; k < top_k; ++k) {
            int32_t best = -1;
            for (int32_t b = 0; b < max_blocks; ++b) {
                if (row[b] == -INFINITY || isnan(row[b])) continue;
                int taken = 0;
                for (int32_t i = 0; i < n; ++i) taken |= out[i] == b;
                if (taken) continue;
                if (best < 0 || row[b] > row[best]) best = b;   /* strict: the lower index wins ties */
            }
            if (best < 0) break;
            out[n++] = best;
        }
        for (int32_t k = n; k < top_k; ++k) out[k] = -1;
        if (counts) counts[r] = n;
    }
    return ORC_OK;
}

/*
 * The packed projection that feeds the producer (page "Fuse MiniMax-M3 QKV and
 * index projection", AFTER figure: one wider GEMM produces the row
 * [Q | K | V | index-Q | index-K] from the hidden states):
 *
 *   x[t, c] = bf16( sum_k h[t, k] * w[c, k] )      t < T, c < N, k < K
 *
 * h is bf16 [T, K] (row stride h_stride), w is bf16 [N, K] (one row per output
 * column, row stride w_stride), x is bf16 [T, N] (row stride x_stride).  Each
 * product of two bf16 values is exact in binary64; the sum runs in binary64 in
 * ascending k and is rounded once to bf16.  Optional outputs: the binary64 sum
 * itself and sum_k |h[t, k] * w[c, k]| (both [T, N] dense), from which a test
 * bounds what a binary32 accumulation in any order can reach.
 */
int msa_oracle_project(const uint16_t* h, int64_t h_stride, int64_t T, int64_t K,
                       const uint16_t* w, int64_t w_stride, int64_t N,
                       uint16_t* x_out, int64_t x_stride, double* sum_out, double* abs_out,
                       int32_t num_threads)
{
    if (T < 0 || K < 0 || N < 0 || h_stride < K || w_stride < K || x_stride < N) return ORC_ERR_ARG;
    if (num_threads < 1) num_threads = 1;
    #pragma omp parallel for num_threads(num_threads) schedule(static)
    for (int64_t t = 0; t < T; ++t) {
        const uint16_t* hr = h + t * h_stride;
        for (int64_t c = 0; c < N; ++c) {
            const uint16_t* wr = w + c * w_stride;
            double acc = 0.0, mag = 0.0;
            for (int64_t k = 0; k < K; ++k) {
                double p = (double)bf16_value(hr[k]) * (double)bf16_value(wr[k]);
                acc += p;
                mag += fabs(p);
            }
            x_out[t * x_stride + c] = msa_oracle_bf16_of_f64(acc);
            if (sum_out) sum_out[t * N + c] = acc;
            if (abs_out) abs_out[t * N + c] = mag;
        }
    }
    return ORC_OK;
}
