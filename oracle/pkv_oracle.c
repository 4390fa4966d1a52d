/*
 * Plain CPU oracle for paged decode attention and the KV append.
 *
 * TEST INFRASTRUCTURE.  Only the tests, the smoke check and the benchmark's
 * CPU-baseline leg may load this library.  It shares no code with the GPU
 * path: the layout, the slot arithmetic and the attention are written out
 * here again from the pages' definitions, in fp64, without blocking, fusion
 * or reordering beyond what the definitions state.
 *
 * Sources (all from the pages on PagedAttention):
 *  - "PagedAttention 详解：缓存的存储结构" (kefan.life), sections "Block Table",
 *    "软件地址翻译" (software address translation), "一个具体的例子" (worked
 *    example) and "写入新 K/V" (writing new K/V);
 *  - "vLLM 核心工程深度剖析" (ybb.press), section 3.1 (kernel signature and the
 *    four steps: table lookup, per-KV-head block loop, softmax, V-weighted sum);
 *  - "PagedAttention是什麼？" (yololab.net), FAQ: paging changes only where K/V
 *    are stored and read, never the attention result.
 *
 * Pool layouts (element type T, x = 16 / sizeof(T)):
 *   key   [num_blocks][Hkv][hs/x][B][x]   (the "cache structure" page's key layout)
 *   value [num_blocks][Hkv][hs][B]        (its value layout: block_size innermost)
 *
 * Readings of points the pages leave open (each is also listed with the
 * design notes): the query head h reads KV head h / (Hq/Hkv); a decode step
 * appends the token at position L-1 and then attends over all L tokens;
 * L == 0 yields a zero output; a negative slot is skipped; the context-split
 * merge is the exact log-sum-exp combination.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

enum { ORC_F32 = 0, ORC_BF16 = 1, ORC_FP8 = 2 };

/* ---- FP8 cache elements ---------------------------------------------------
 * The pages allow an FP8 cache element (the cache-structure page: x = 16 /
 * sizeof(cache_t), 16 for FP8) but fix neither the format nor a scale.  The
 * reading taken here: the E4M3 format of the OCP 8-bit floating-point
 * specification (sign bit, 4 exponent bits with bias 7, 3 mantissa bits; no
 * infinities; S.1111.111 is NaN; the exponent field 0 holds the subnormals
 * m * 2^-9), with one scale per pool: a value x is stored as the code
 * nearest to x * (1 / scale) (the product rounded to fp32 first) and read
 * back as code_value * scale. */

/* value of an E4M3 code */
double orc_fp8_decode(uint8_t c)
{
    int sign = c >> 7, e = (c >> 3) & 15, m = c & 7;
    double v;
    if (e == 15 && m == 7)
        return NAN;
    if (e == 0)
        v = m * ldexp(1.0, -9);                  /* subnormal: m/8 * 2^(1-7) */
    else
        v = (1.0 + m / 8.0) * ldexp(1.0, e - 7);
    return sign ? -v : v;
}

/* The E4M3 code nearest to v, found by trying every finite magnitude; a tie
 * goes to the code with the even mantissa; a magnitude above 448 (the
 * largest finite value) saturates to 448; NaN gives 0x7F. */
uint8_t orc_fp8_encode(float v)
{
    if (isnan(v))
        return 0x7F;
    uint8_t sign = signbit(v) ? 0x80 : 0x00;
    double a = fabs((double)v);
    if (a > 448.0)
        return sign | 0x7E;
    int best = 0;
    double best_err = INFINITY;
    for (int c = 0; c <= 0x7E; ++c) {
        double err = fabs(orc_fp8_decode((uint8_t)c) - a);
        if (err < best_err || (err == best_err && (c & 1) == 0 && (best & 1) == 1)) {
            best = c;
            best_err = err;
        }
    }
    return sign | (uint8_t)best;
}

/* ---- element access ------------------------------------------------------ */

static double orc_load(const void* base, size_t idx, int dtype)
{
    if (dtype == ORC_FP8)
        return orc_fp8_decode(((const uint8_t*)base)[idx]);
    if (dtype == ORC_F32)
        return (double)((const float*)base)[idx];
    /* bf16: the 16 stored bits are the upper half of an fp32 pattern */
    uint32_t bits = (uint32_t)((const uint16_t*)base)[idx] << 16;
    float f;
    memcpy(&f, &bits, sizeof f);
    return (double)f;
}

static void orc_copy_elem(void* dst, size_t di, const void* src, size_t si, int dtype)
{
    if (dtype == ORC_F32)
        memcpy((char*)dst + di * 4, (const char*)src + si * 4, 4);
    else
        memcpy((char*)dst + di * 2, (const char*)src + si * 2, 2);
}

/* ---- layout: where element d of token slot t of KV head h in block b sits */

/* Key pool: head_size is split into hs/x chunks of x contiguous elements;
 * the chunk index comes before the slot index (address translation section:
 * k_ptr = base + block*kv_block_stride + head*kv_head_stride + offset*x, and
 * successive x-chunks of one key are block_size*x elements apart). */
size_t orc_key_index(int64_t b, int64_t h, int64_t t, int64_t d,
                     int32_t Hkv, int32_t B, int32_t hs, int32_t x)
{
    int64_t kv_head_stride = (int64_t)hs * B;
    int64_t kv_block_stride = (int64_t)Hkv * kv_head_stride;
    return (size_t)(b * kv_block_stride + h * kv_head_stride
                    + (d / x) * ((int64_t)B * x) + t * x + d % x);
}

/* Value pool: v_ptr = base + block*kv_block_stride + head*kv_head_stride,
 * element = v_ptr + head_dim_idx*block_size + slot. */
size_t orc_value_index(int64_t b, int64_t h, int64_t t, int64_t d,
                       int32_t Hkv, int32_t B, int32_t hs)
{
    int64_t kv_head_stride = (int64_t)hs * B;
    int64_t kv_block_stride = (int64_t)Hkv * kv_head_stride;
    return (size_t)(b * kv_block_stride + h * kv_head_stride + d * B + t);
}

/* ---- slot mapping ("writing new K/V" section) ---------------------------- */

/* slot = block_tables[seq][pos / B] * B + pos % B */
int64_t orc_slot_of_position(const int32_t* table_row, int64_t pos, int32_t B)
{
    int64_t block_table_idx = pos / B;
    int64_t offset_in_block = pos % B;
    int64_t block_id = table_row[block_table_idx];
    return block_id * B + offset_in_block;
}

/* block_id = slot / B, offset = slot % B */
void orc_slot_split(int64_t slot, int32_t B, int64_t* block_id, int64_t* offset)
{
    *block_id = slot / B;
    *offset = slot % B;
}

/* Decode step: the new token of sequence s sits at position L_s - 1.
 * A sequence with L_s == 0 gets slot -1 (nothing to write). */
void orc_decode_slot_mapping(const int32_t* block_tables, const int32_t* seq_lens,
                             int32_t S, int32_t M, int32_t B, int64_t* slots)
{
    for (int32_t s = 0; s < S; ++s) {
        int64_t L = seq_lens[s];
        slots[s] = (L > 0) ? orc_slot_of_position(block_tables + (size_t)s * M, L - 1, B) : -1;
    }
}

/* Several new tokens per sequence: rows q_start[s] .. q_start[s+1]-1 are the
 * last n_s of sequence s's L_s tokens, so row i of s sits at position
 * L_s - n_s + i.  A row whose position falls outside 0 .. L_s - 1 gets -1. */
void orc_multi_token_slot_mapping(const int32_t* block_tables, const int32_t* seq_lens, const int32_t* q_start,
                                  int32_t S, int32_t M, int32_t B, int64_t* slots)
{
    for (int32_t s = 0; s < S; ++s) {
        int64_t L = seq_lens[s];
        int64_t n = (int64_t)q_start[s + 1] - q_start[s];
        for (int64_t i = 0; i < n; ++i) {
            int64_t pos = L - n + i;
            slots[q_start[s] + i] =
                (pos >= 0 && pos < L) ? orc_slot_of_position(block_tables + (size_t)s * M, pos, B) : -1;
        }
    }
}

/* ---- append: copy each new token's K and V into its slot ----------------- */

void orc_kv_append(const void* k, const void* v, const int64_t* slots, int32_t T,
                   int32_t Hkv, int32_t hs, int32_t B, int32_t dtype,
                   void* k_pool, void* v_pool)
{
    int32_t x = 16 / (dtype == ORC_F32 ? 4 : 2);
    for (int32_t i = 0; i < T; ++i) {
        if (slots[i] < 0)
            continue;
        int64_t b, off;
        orc_slot_split(slots[i], B, &b, &off);
        for (int32_t h = 0; h < Hkv; ++h)
            for (int32_t d = 0; d < hs; ++d) {
                size_t src = ((size_t)i * Hkv + h) * hs + d;
                orc_copy_elem(k_pool, orc_key_index(b, h, off, d, Hkv, B, hs, x), k, src, dtype);
                orc_copy_elem(v_pool, orc_value_index(b, h, off, d, Hkv, B, hs), v, src, dtype);
            }
    }
}

/* FP8 caches: element d of token i's key (value) is stored as
 * orc_fp8_encode((float)k * k_inv_scale) (the product in fp32); the source
 * is fp32 or bf16 (src_dtype).  Key layout with x = 16. */
void orc_kv_append_fp8(const void* k, const void* v, const int64_t* slots, int32_t T,
                       int32_t Hkv, int32_t hs, int32_t B, int32_t src_dtype,
                       float k_inv_scale, float v_inv_scale, uint8_t* k_pool, uint8_t* v_pool)
{
    for (int32_t i = 0; i < T; ++i) {
        if (slots[i] < 0)
            continue;
        int64_t b, off;
        orc_slot_split(slots[i], B, &b, &off);
        for (int32_t h = 0; h < Hkv; ++h)
            for (int32_t d = 0; d < hs; ++d) {
                size_t src = ((size_t)i * Hkv + h) * hs + d;
                float kq = (float)orc_load(k, src, src_dtype) * k_inv_scale;
                float vq = (float)orc_load(v, src, src_dtype) * v_inv_scale;
                k_pool[orc_key_index(b, h, off, d, Hkv, B, hs, 16)] = orc_fp8_encode(kq);
                v_pool[orc_value_index(b, h, off, d, Hkv, B, hs)] = orc_fp8_encode(vq);
            }
    }
}

/* codes of n values (fp32 or bf16) quantized with inv_scale, as in the append */
void orc_fp8_quantize(const void* src, int64_t n, int32_t src_dtype, float inv_scale, uint8_t* out)
{
    for (int64_t i = 0; i < n; ++i)
        out[i] = orc_fp8_encode((float)orc_load(src, (size_t)i, src_dtype) * inv_scale);
}

/* ---- attention ----------------------------------------------------------- */

typedef struct {
    const void* q; const void* k_pool; const void* v_pool;
    const int32_t* block_tables; const int32_t* seq_lens;
    int32_t S, Hq, Hkv, hs, B, M, dtype, x;
    double scale;
    int32_t kv_dtype;          /* element type of the pools (dtype: of q) */
    double k_scale, v_scale;   /* pool values are element * scale (1 unless FP8) */
} orc_problem;

/* Score of logical token t of sequence s for query head h of query row qr:
 * scale * sum_d q[qr,h,d] * K[t,d], where K[t] is found through the table. */
static double orc_score(const orc_problem* p, int32_t s, int64_t qr, int32_t h, int32_t kvh, int64_t t)
{
    int64_t block_idx = t / p->B;
    int64_t slot = t % p->B;
    int64_t block = p->block_tables[(size_t)s * p->M + block_idx];
    double dot = 0.0;
    for (int32_t d = 0; d < p->hs; ++d) {
        double qd = orc_load(p->q, ((size_t)qr * p->Hq + h) * p->hs + d, p->dtype);
        double kd = p->k_scale *
                    orc_load(p->k_pool, orc_key_index(block, kvh, slot, d, p->Hkv, p->B, p->hs, p->x), p->kv_dtype);
        dot += qd * kd;
    }
    return p->scale * dot;
}

static double orc_value(const orc_problem* p, int32_t s, int32_t kvh, int64_t t, int32_t d)
{
    int64_t block = p->block_tables[(size_t)s * p->M + t / p->B];
    return p->v_scale * orc_load(p->v_pool, orc_value_index(block, kvh, t % p->B, d, p->Hkv, p->B, p->hs),
                                 p->kv_dtype);
}

/* Softmax attention of query row qr, head h of sequence s over tokens [t0, t1):
 * m = max score, w_t = exp(score_t - m), l = sum w_t, o = sum w_t v_t / l.
 * `score` is scratch of length >= t1 - t0.  Returns 0 when the range is empty. */
static int orc_attend_range(const orc_problem* p, int32_t s, int64_t qr, int32_t h, int64_t t0, int64_t t1,
                            double* score, double* m_out, double* l_out, double* o)
{
    int32_t kvh = h / (p->Hq / p->Hkv);
    if (t1 <= t0) {
        for (int32_t d = 0; d < p->hs; ++d) o[d] = 0.0;
        *m_out = -INFINITY;
        *l_out = 0.0;
        return 0;
    }
    double m = -INFINITY;
    for (int64_t t = t0; t < t1; ++t) {
        score[t - t0] = orc_score(p, s, qr, h, kvh, t);
        if (score[t - t0] > m) m = score[t - t0];
    }
    double l = 0.0;
    for (int64_t t = t0; t < t1; ++t) {
        score[t - t0] = exp(score[t - t0] - m);
        l += score[t - t0];
    }
    /* o[d] accumulates w_t * v_t[d] in token order for every d */
    for (int32_t d = 0; d < p->hs; ++d) o[d] = 0.0;
    for (int64_t t = t0; t < t1; ++t)
        for (int32_t d = 0; d < p->hs; ++d)
            o[d] += score[t - t0] * orc_value(p, s, kvh, t, d);
    for (int32_t d = 0; d < p->hs; ++d) o[d] /= l;
    *m_out = m;
    *l_out = l;
    return 1;
}

static int orc_run_threads(int threads)
{
#ifdef _OPENMP
    return threads > 0 ? threads : omp_get_max_threads();
#else
    (void)threads;
    return 1;
#endif
}

/* Attention for selected (sequence, query head) units: unit u = s*Hq + h,
 * row i of `out` receives units[i].  units == NULL selects every unit in
 * order (out is then [S][Hq][hs]).  threads <= 0: OpenMP default.
 * Returns the number of threads used. */
static int32_t orc_x(int32_t dtype) { return dtype == ORC_F32 ? 4 : (dtype == ORC_BF16 ? 8 : 16); }

/* As orc_paged_attention_units, with pools of their own element type
 * (kv_dtype; FP8 values read as code_value * k_scale / v_scale). */
int orc_paged_attention_units_kv(const void* q, const void* k_pool, const void* v_pool,
                                 const int32_t* block_tables, const int32_t* seq_lens,
                                 int32_t S, int32_t Hq, int32_t Hkv, int32_t hs, int32_t B, int32_t M,
                                 int32_t dtype, int32_t kv_dtype, double k_scale, double v_scale,
                                 double scale, const int64_t* units, int64_t n_units, double* out, int threads)
{
    orc_problem p = { q, k_pool, v_pool, block_tables, seq_lens, S, Hq, Hkv, hs, B, M, dtype,
                      orc_x(kv_dtype), scale, kv_dtype, k_scale, v_scale };
    int64_t maxL = 0;
    for (int32_t s = 0; s < S; ++s)
        if (seq_lens[s] > maxL) maxL = seq_lens[s];
    int nt = orc_run_threads(threads);
    if (units == NULL)
        n_units = (int64_t)S * Hq;
#pragma omp parallel num_threads(nt)
    {
        double* score = (double*)malloc(sizeof(double) * (size_t)(maxL > 0 ? maxL : 1));
#pragma omp for schedule(dynamic, 1)
        for (int64_t i = 0; i < n_units; ++i) {
            int64_t u = units ? units[i] : i;
            int32_t s = (int32_t)(u / Hq), h = (int32_t)(u % Hq);
            double m, l;
            orc_attend_range(&p, s, s, h, 0, seq_lens[s], score, &m, &l, out + (size_t)i * hs);
        }
        free(score);
    }
    return nt;
}

int orc_paged_attention_units(const void* q, const void* k_pool, const void* v_pool,
                              const int32_t* block_tables, const int32_t* seq_lens,
                              int32_t S, int32_t Hq, int32_t Hkv, int32_t hs, int32_t B, int32_t M,
                              int32_t dtype, double scale, const int64_t* units, int64_t n_units,
                              double* out, int threads)
{
    return orc_paged_attention_units_kv(q, k_pool, v_pool, block_tables, seq_lens, S, Hq, Hkv, hs, B, M, dtype,
                                        dtype, 1.0, 1.0, scale, units, n_units, out, threads);
}

/* out[s][h][d], fp64, every unit. */
int orc_paged_attention(const void* q, const void* k_pool, const void* v_pool,
                        const int32_t* block_tables, const int32_t* seq_lens,
                        int32_t S, int32_t Hq, int32_t Hkv, int32_t hs, int32_t B, int32_t M,
                        int32_t dtype, double scale, double* out, int threads)
{
    return orc_paged_attention_units(q, k_pool, v_pool, block_tables, seq_lens, S, Hq, Hkv, hs, B, M,
                                     dtype, scale, NULL, 0, out, threads);
}

/* Context split: each P-token partition yields (m_p, l_p, o_p) with o_p
 * normalised by l_p; partitions that hold no token are skipped; the merge is
 * M = max m_p, w_p = l_p * exp(m_p - M), out = sum w_p o_p / sum w_p. */
int orc_paged_attention_split(const void* q, const void* k_pool, const void* v_pool,
                              const int32_t* block_tables, const int32_t* seq_lens,
                              int32_t S, int32_t Hq, int32_t Hkv, int32_t hs, int32_t B, int32_t M,
                              int32_t dtype, double scale, int32_t P, double* out, int threads)
{
    orc_problem p = { q, k_pool, v_pool, block_tables, seq_lens, S, Hq, Hkv, hs, B, M, dtype,
                      orc_x(dtype), scale, dtype, 1.0, 1.0 };
    int64_t maxL = 0;
    for (int32_t s = 0; s < S; ++s)
        if (seq_lens[s] > maxL) maxL = seq_lens[s];
    int64_t maxparts = (maxL + P - 1) / P;
    if (maxparts < 1) maxparts = 1;
    int nt = orc_run_threads(threads);
    int64_t units = (int64_t)S * Hq;
#pragma omp parallel num_threads(nt)
    {
        double* score = (double*)malloc(sizeof(double) * (size_t)P);
        double* pm = (double*)malloc(sizeof(double) * (size_t)maxparts);
        double* pl = (double*)malloc(sizeof(double) * (size_t)maxparts);
        double* po = (double*)malloc(sizeof(double) * (size_t)(maxparts * hs));
#pragma omp for schedule(dynamic, 1)
        for (int64_t u = 0; u < units; ++u) {
            int32_t s = (int32_t)(u / Hq), h = (int32_t)(u % Hq);
            int64_t L = seq_lens[s];
            int64_t nparts = (L + P - 1) / P;
            double* o = out + (size_t)u * hs;
            /* partials */
            for (int64_t k = 0; k < nparts; ++k) {
                int64_t t0 = k * P, t1 = (t0 + P < L) ? t0 + P : L;
                orc_attend_range(&p, s, s, h, t0, t1, score, &pm[k], &pl[k], po + k * hs);
            }
            /* merge */
            double Mx = -INFINITY;
            for (int64_t k = 0; k < nparts; ++k)
                if (pl[k] > 0.0 && pm[k] > Mx) Mx = pm[k];
            double W = 0.0;
            for (int32_t d = 0; d < hs; ++d) o[d] = 0.0;
            for (int64_t k = 0; k < nparts; ++k) {
                if (!(pl[k] > 0.0))
                    continue;
                double w = pl[k] * exp(pm[k] - Mx);
                W += w;
                for (int32_t d = 0; d < hs; ++d) o[d] += w * po[k * hs + d];
            }
            if (W > 0.0)
                for (int32_t d = 0; d < hs; ++d) o[d] /= W;
        }
        free(score);
        free(pm);
        free(pl);
        free(po);
    }
    return nt;
}

/* Several query tokens per sequence (chunked prefill, speculative decoding):
 * the query tokens of sequence s are rows q_start[s] .. q_start[s+1]-1 of q
 * ([rows][Hq][hs]); they are the last n_s = q_start[s+1] - q_start[s] of its
 * L_s = seq_lens[s] tokens, in order, so query row i of s sits at position
 * L_s - n_s + i and attends the tokens at positions 0 .. L_s - n_s + i (the
 * causal rule: a token sees itself and everything before it).  out has the
 * layout of q.  Pools of element type kv_dtype (FP8 read as code * scale). */
int orc_paged_multi_token_attention(const void* q, const int32_t* q_start, const void* k_pool, const void* v_pool,
                                const int32_t* block_tables, const int32_t* seq_lens, int32_t S, int32_t Hq,
                                int32_t Hkv, int32_t hs, int32_t B, int32_t M, int32_t dtype, int32_t kv_dtype,
                                double k_scale, double v_scale, double scale, double* out, int threads)
{
    orc_problem p = { q, k_pool, v_pool, block_tables, seq_lens, S, Hq, Hkv, hs, B, M, dtype,
                      orc_x(kv_dtype), scale, kv_dtype, k_scale, v_scale };
    int64_t maxL = 0;
    for (int32_t s = 0; s < S; ++s)
        if (seq_lens[s] > maxL) maxL = seq_lens[s];
    int64_t rows = q_start[S];
    int nt = orc_run_threads(threads);
#pragma omp parallel num_threads(nt)
    {
        double* score = (double*)malloc(sizeof(double) * (size_t)(maxL > 0 ? maxL : 1));
#pragma omp for schedule(dynamic, 1)
        for (int64_t u = 0; u < rows * Hq; ++u) {
            int64_t qr = u / Hq;
            int32_t h = (int32_t)(u % Hq);
            int32_t s = 0;
            while (q_start[s + 1] <= qr)
                ++s;
            int64_t n = q_start[s + 1] - q_start[s];
            int64_t pos = (int64_t)seq_lens[s] - n + (qr - q_start[s]);
            double m, l;
            orc_attend_range(&p, s, qr, h, 0, pos + 1, score, &m, &l, out + (size_t)u * hs);
        }
        free(score);
    }
    return nt;
}

int orc_max_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}
