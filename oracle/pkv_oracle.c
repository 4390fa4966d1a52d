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

enum { ORC_F32 = 0, ORC_BF16 = 1 };

/* ---- element access ------------------------------------------------------ */

static double orc_load(const void* base, size_t idx, int dtype)
{
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

/* ---- attention ----------------------------------------------------------- */

typedef struct {
    const void* q; const void* k_pool; const void* v_pool;
    const int32_t* block_tables; const int32_t* seq_lens;
    int32_t S, Hq, Hkv, hs, B, M, dtype, x;
    double scale;
} orc_problem;

/* Score of logical token t for query head h of sequence s:
 * scale * sum_d q[s,h,d] * K[t,d], where K[t] is found through the table. */
static double orc_score(const orc_problem* p, int32_t s, int32_t h, int32_t kvh, int64_t t)
{
    int64_t block_idx = t / p->B;
    int64_t slot = t % p->B;
    int64_t block = p->block_tables[(size_t)s * p->M + block_idx];
    double dot = 0.0;
    for (int32_t d = 0; d < p->hs; ++d) {
        double qd = orc_load(p->q, ((size_t)s * p->Hq + h) * p->hs + d, p->dtype);
        double kd = orc_load(p->k_pool, orc_key_index(block, kvh, slot, d, p->Hkv, p->B, p->hs, p->x), p->dtype);
        dot += qd * kd;
    }
    return p->scale * dot;
}

static double orc_value(const orc_problem* p, int32_t s, int32_t kvh, int64_t t, int32_t d)
{
    int64_t block = p->block_tables[(size_t)s * p->M + t / p->B];
    return orc_load(p->v_pool, orc_value_index(block, kvh, t % p->B, d, p->Hkv, p->B, p->hs), p->dtype);
}

/* Softmax attention of one (sequence, query head) over tokens [t0, t1):
 * m = max score, w_t = exp(score_t - m), l = sum w_t, o = sum w_t v_t / l.
 * `score` is scratch of length >= t1 - t0.  Returns 0 when the range is empty. */
static int orc_attend_range(const orc_problem* p, int32_t s, int32_t h, int64_t t0, int64_t t1,
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
        score[t - t0] = orc_score(p, s, h, kvh, t);
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
int orc_paged_attention_units(const void* q, const void* k_pool, const void* v_pool,
                              const int32_t* block_tables, const int32_t* seq_lens,
                              int32_t S, int32_t Hq, int32_t Hkv, int32_t hs, int32_t B, int32_t M,
                              int32_t dtype, double scale, const int64_t* units, int64_t n_units,
                              double* out, int threads)
{
    orc_problem p = { q, k_pool, v_pool, block_tables, seq_lens, S, Hq, Hkv, hs, B, M, dtype,
                      16 / (dtype == ORC_F32 ? 4 : 2), scale };
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
            orc_attend_range(&p, s, h, 0, seq_lens[s], score, &m, &l, out + (size_t)i * hs);
        }
        free(score);
    }
    return nt;
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
                      16 / (dtype == ORC_F32 ? 4 : 2), scale };
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
                orc_attend_range(&p, s, h, t0, t1, score, &pm[k], &pl[k], po + k * hs);
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

int orc_max_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}
