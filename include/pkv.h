/*
 * pkv.h — C ABI of the paged KV-cache decode library for AMD MI355X (gfx950).
 *
 * Two operations make up one decode step of PagedAttention:
 *   1. kv_cache_append: store each sequence's new key/value vectors in the
 *      slot the block allocator gave them (slot = block_id * B + offset);
 *   2. paged_decode_attention: for every sequence and query head, walk the
 *      sequence's block table to the physical blocks that hold its keys and
 *      values and compute softmax(scale * q K^T) V over its seq_len tokens.
 * pkv_decode_slot_mapping computes the slots of a decode step's new tokens
 * from the block tables and lengths.
 *
 * Sources: the pages on PagedAttention —
 *   "PagedAttention 详解：缓存的存储结构" (kefan.life): sections "Block Table",
 *     "软件地址翻译" (software address translation, the K/V layouts and the
 *     block_tables / seq_lens inputs), "一个具体的例子" (worked example) and
 *     "写入新 K/V" (slot_mapping and its split in the cache-write kernel);
 *   "vLLM 核心工程深度剖析" (ybb.press), section 3.1 (kernel signature: out,
 *     q, k_cache, v_cache, block_tables, context_lens, max blocks per
 *     sequence, scaling) and section 3.2;
 *   "PagedAttention是什麼？" (yololab.net), section on the kernel (grid over
 *     sequence, head and partition; partition reduction for long contexts).
 *
 * ---------------------------------------------------------------------------
 * Data layout (device memory, all buffers owned by the caller)
 * ---------------------------------------------------------------------------
 * Pool element type T is fp32 (PKV_F32), bfloat16 (PKV_BF16, 16-bit patterns)
 * or an FP8 code (PKV_FP8_E4M3, see below).  x = 16 / sizeof(T) elements form
 * one 16-byte chunk (4 for fp32, 8 for bf16, 16 for FP8: the cache-structure
 * page's x = 16 / sizeof(cache_t)).
 *
 *   key pool    [num_blocks][num_kv_heads][head_size / x][block_size][x]
 *   value pool  [num_blocks][num_kv_heads][head_size][block_size]
 *
 * so element d of token slot t of KV head h in block b sits at
 *   key:   ((b*Hkv + h)*(hs/x) + d/x)*(B*x) + t*x + d%x
 *   value: ((b*Hkv + h)*hs + d)*B + t
 * Each (block, KV head) tile is B*hs contiguous elements in both pools.
 *
 *   q, out        [num_seqs][num_q_heads][head_size], element type T (bf16 with FP8 pools;
 *                 out is fp32 when the descriptor's out_f32 is set)
 *   k, v (append) [num_tokens][num_kv_heads][head_size], element type T (bf16 with FP8 pools)
 *   block_tables  int32 [num_seqs][max_blocks_per_seq]
 *   seq_lens      int32 [num_seqs]
 *   slot_mapping  int64 [num_tokens]
 *
 * Query head h reads KV head h / (num_q_heads / num_kv_heads).
 * Token t of sequence s lives in block block_tables[s][t / B], slot t % B.
 * Table entries at index >= ceil(seq_len / B) and slots >= seq_len in the
 * last block are never read; they may hold anything, NaN included.
 * All q/out/k/v/pool pointers must be 16-byte aligned.
 *
 * FP8 pools.  The pages allow an FP8 cache element but fix no format or
 * scale.  Here: the E4M3 codes of the OCP 8-bit floating-point format (sign,
 * 4 exponent bits with bias 7, 3 mantissa bits, no infinities, 0x7F / 0xFF
 * NaN, largest finite 448), one scale per pool (cache->k_scale, v_scale).  An
 * append stores the code nearest to fp32(x * (1 / scale)) (ties to the even
 * mantissa; magnitudes beyond 448 saturate to 448); attention reads
 * code_value * scale.
 *
 * ---------------------------------------------------------------------------
 * Conventions
 * ---------------------------------------------------------------------------
 * - Every call is asynchronous on `stream` (a hipStream_t, passed as void*;
 *   NULL is the default stream).  Nothing is read back to the host, so
 *   seq_lens and block_tables stay on the device.
 * - The library allocates no device memory; the caller sizes the attention
 *   workspace with pkv_decode_workspace_bytes (attention) or
 *   pkv_decode_step_workspace_bytes (decode step), and the optional
 *   schedule buffer with pkv_decode_schedule_bytes.
 * - Arguments that can be checked on the host are checked before any launch;
 *   a failed check returns an error status and launches nothing.
 * - Device-side contract (not checked on the host): block IDs of used table
 *   entries lie in [0, num_blocks); 0 <= seq_len <= max_blocks_per_seq * B;
 *   slots of one append call are distinct.  A kernel that meets an
 *   out-of-range block ID or slot skips that block or token instead of
 *   touching memory outside the pools, and a seq_len above
 *   max_blocks_per_seq * B is treated as that maximum.
 * - Results are deterministic: the reduction order depends only on the
 *   logical token order, so relabelling physical blocks or sharing blocks
 *   between tables gives bit-identical outputs.
 */
#ifndef PKV_H
#define PKV_H

#include <stddef.h>
#include <stdint.h>

#if defined(__GNUC__) || defined(__clang__)
#define PKV_API __attribute__((visibility("default")))
#else
#define PKV_API
#endif

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    PKV_OK = 0,
    PKV_ERR_INVALID_ARG = -1,  /* null pointer, bad size, misaligned pointer */
    PKV_ERR_UNSUPPORTED = -2,  /* a shape or type this build has no kernel for */
    PKV_ERR_WORKSPACE = -3,    /* workspace missing or smaller than required */
    PKV_ERR_HIP = -4,          /* a HIP launch failed; see pkv_last_hip_error */
    PKV_ERR_OUT_OF_BLOCKS = -5 /* the block pool has no free block left */
} pkv_status;

typedef enum {
    PKV_F32 = 0,
    PKV_BF16 = 1,
    PKV_FP8_E4M3 = 2   /* pools only; q, out, k, v are bf16 */
} pkv_dtype;

/* Describes both pools (key and value share it). */
typedef struct {
    int32_t num_blocks;    /* physical blocks in each pool                     */
    int32_t num_kv_heads;  /* Hkv                                              */
    int32_t block_size;    /* B: token slots per block; 1, 8, 16, 32 or 64     */
                           /* (FP8 pools: 16, 32 or 64)                        */
    int32_t head_size;     /* hs: 64 or 128                                    */
    int32_t dtype;         /* pkv_dtype of the pools (and of q, out, k, v,     */
                           /* which are bf16 when the pools are FP8)           */
    float k_scale;         /* FP8 pools: key value = code * k_scale (> 0);     */
    float v_scale;         /* value = code * v_scale.  Ignored otherwise.      */
    int32_t out_f32;       /* element type of the attention output `out`:      */
                           /* 0 = the type of q (bf16 with bf16 and FP8 pools, */
                           /* rounded to nearest even); 1 = fp32, the value    */
                           /* that rounding would take.  With fp32 pools both  */
                           /* mean fp32.  Values other than 0 and 1 are       */
                           /* PKV_ERR_INVALID_ARG in every call; calls that    */
                           /* write no attention output otherwise ignore it.   */
} pkv_cache_desc;

/* Layout contract version; changes whenever the pool layout above changes. */
PKV_API int32_t pkv_layout_version(void);

/* Human-readable name of a status code (static storage). */
PKV_API const char* pkv_status_string(int32_t status);

/* Name of the HIP error behind the last PKV_ERR_HIP on this host thread. */
PKV_API const char* pkv_last_hip_error(void);

/*
 * Slot mapping of a decode step ("writing new K/V" section: slot =
 * block_tables[s][pos / B] * B + pos % B).  The new token of sequence s is
 * the last one, pos = seq_lens[s] - 1; sequences with seq_len <= 0, or whose
 * position falls outside the table row, get slot -1 (the append skips it).
 *   block_tables  device int32 [num_seqs][max_blocks_per_seq]
 *   seq_lens      device int32 [num_seqs]
 *   slot_mapping  device int64 [num_seqs], written
 * Errors: PKV_ERR_INVALID_ARG for null pointers or non-positive sizes.
 */
PKV_API pkv_status pkv_decode_slot_mapping(const int32_t* block_tables, const int32_t* seq_lens,
                                   int32_t num_seqs, int32_t max_blocks_per_seq,
                                   int32_t block_size, int64_t* slot_mapping, void* stream);

/*
 * KV append ("writing new K/V" section: the cache-write kernel splits each
 * slot into block_id = slot / B and offset = slot % B and stores the token's
 * key and value there).  Bit-exact copy, no type conversion: k, v and the
 * pools share cache->dtype.
 *   k, v          device T [num_tokens][num_kv_heads][head_size]
 *   slot_mapping  device int64 [num_tokens]; slot < 0 means skip the token
 *   k_cache, v_cache  device pools (layout above), written in place
 * num_tokens == 0 is a no-op.  Errors: PKV_ERR_INVALID_ARG (null pointer,
 * negative count, misaligned pointer, bad descriptor), PKV_ERR_UNSUPPORTED
 * (dtype, head_size or block_size without a kernel), PKV_ERR_HIP.
 */
PKV_API pkv_status kv_cache_append(const void* k, const void* v, const int64_t* slot_mapping,
                           int32_t num_tokens, const pkv_cache_desc* cache,
                           void* k_cache, void* v_cache, void* stream);

/*
 * Longest-first schedule of a decode batch: a device buffer that
 * pkv_decode_append can fill and paged_decode_attention can read.  It lists
 * the sequences in decreasing number of blocks (ties by index), with their
 * lengths and block-table rows in that order, so that the attention kernel
 * starts the longest sequences first and no long one is left running alone
 * at the end.  It also lists the chunks of the library's default
 * partitioning (partition_tokens == 0) by decreasing size (the full chunks
 * first, then the partial ones), so that an attention call with the default
 * partitioning on a large batch starts the largest chunks first.  This is a
 * scheduling aid of this library, not part of
 * the method: results are bit-identical with and without it.
 * Returns its size in bytes for these sizes (int32 order[S], lens[S] and
 * tables[S][max_blocks_per_seq], each rounded up to 16 bytes, a count padded
 * to 16 bytes and the chunk list uint32 [S][ceil(max_blocks_per_seq / 4)][2]),
 * or 0 when no schedule is used (num_seqs <= 1 or num_seqs > 4096).
 */
PKV_API size_t pkv_decode_schedule_bytes(int32_t num_seqs, int32_t max_blocks_per_seq);

/*
 * Decode-step append in one launch: for each sequence s the new token sits at
 * position seq_lens[s] - 1, its slot is block_tables[s][pos / B] * B + pos % B
 * (as in pkv_decode_slot_mapping), and k[s], v[s] are stored there exactly as
 * kv_cache_append would.  Sequences with seq_len <= 0 or a position outside
 * their table row are skipped.
 *   k, v          device T [num_seqs][num_kv_heads][head_size]
 *   block_tables  device int32 [num_seqs][max_blocks_per_seq]
 *   seq_lens      device int32 [num_seqs] (lengths including the new token)
 *   slot_mapping  device int64 [num_seqs] receiving the slots, or NULL
 *   schedule      device buffer of schedule_bytes >= pkv_decode_schedule_bytes
 *                 (16-byte aligned) that receives the batch's longest-first
 *                 schedule, or NULL (ignored when that size is 0)
 * A sequence's last block must not be shared with another sequence (the
 * copy-on-write rule: a shared block is copied before it is written).
 * Errors: as kv_cache_append; PKV_ERR_WORKSPACE for a schedule buffer that is
 * too small or misaligned.
 */
PKV_API pkv_status pkv_decode_append(const void* k, const void* v, const int32_t* block_tables,
                                     const int32_t* seq_lens, int32_t num_seqs, int32_t max_blocks_per_seq,
                                     const pkv_cache_desc* cache, void* k_cache, void* v_cache,
                                     int64_t* slot_mapping, int32_t* schedule, size_t schedule_bytes,
                                     void* stream);

/*
 * Context-partition length, in tokens, that paged_decode_attention will use
 * for these sizes.  partition_tokens > 0 requests that length (it must be a
 * multiple of block_size and at most 64 * block_size, and for blocks of
 * fewer than 16 tokens a multiple of 16 and at most 512); 0 lets the
 * library choose (512, or the whole table when shorter).  Returns 0 for
 * invalid sizes.
 */
PKV_API int32_t pkv_decode_partition_tokens(int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads,
                                    int32_t head_size, int32_t max_blocks_per_seq,
                                    int32_t block_size, int32_t partition_tokens);

/*
 * Bytes of device workspace paged_decode_attention needs for these sizes
 * (fp32 partial results per (sequence, query head, partition)).  Zero when
 * one partition covers max_blocks_per_seq * block_size tokens.
 */
PKV_API size_t pkv_decode_workspace_bytes(int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads,
                                  int32_t head_size, int32_t max_blocks_per_seq,
                                  int32_t block_size, int32_t partition_tokens);

/*
 * Paged decode attention (signature of the "vLLM engineering deep-dive"
 * page, section 3.1; partitioned long-context variant of the yololab page's
 * kernel section).  For each sequence s and query head h, with
 * kvh = h / (num_q_heads / num_kv_heads) and L = seq_lens[s]:
 *   out[s][h] = sum_t softmax_t(scale * q[s][h] . K[t]) * V[t],  t < L,
 * where K[t] and V[t] are slot t % B of block block_tables[s][t / B], KV
 * head kvh.  Accumulation is fp32; a bf16 output is rounded to nearest
 * even (cache->out_f32 = 1 writes the fp32 value instead, and then the bf16
 * output of the same call is exactly that value rounded to nearest even);
 * L == 0 gives a zero output.
 *   q             device T [num_seqs][num_q_heads][head_size]
 *   k_cache, v_cache  device pools (layout above)
 *   block_tables  device int32 [num_seqs][max_blocks_per_seq]
 *   seq_lens      device int32 [num_seqs]
 *   scale         softmax scale, positive and finite (else PKV_ERR_INVALID_ARG;
 *                 the same rule holds for every attention entry point below)
 *   out           device T (fp32 with cache->out_f32) [num_seqs][num_q_heads][head_size], written
 *   workspace     device scratch of workspace_bytes >= pkv_decode_workspace_bytes(...)
 *                 (may be NULL when that size is 0); contents are overwritten
 *   partition_tokens  0 = library's choice, else as in pkv_decode_partition_tokens
 *   schedule      the longest-first schedule that pkv_decode_append wrote for
 *                 these same block_tables and seq_lens (schedule_bytes as
 *                 there), or NULL: then a batch of up to 64 sequences is
 *                 ranked by the kernel itself and a larger one is attended
 *                 in batch order.  A schedule that does not match the tables
 *                 and lengths gives wrong results.
 * Calls that share a workspace must be ordered on one stream.
 * Errors: PKV_ERR_INVALID_ARG, PKV_ERR_UNSUPPORTED (head_size not 64/128,
 * block_size not 1/8/16/32/64 or below 16 with FP8 pools, num_q_heads / num_kv_heads not in 1..16 or not an
 * integer), PKV_ERR_WORKSPACE (workspace or schedule too small or
 * misaligned), PKV_ERR_HIP.
 */
PKV_API pkv_status paged_decode_attention(const void* q, const void* k_cache, const void* v_cache,
                                  const int32_t* block_tables, const int32_t* seq_lens,
                                  int32_t num_seqs, int32_t num_q_heads, int32_t max_blocks_per_seq,
                                  const pkv_cache_desc* cache, float scale, void* out,
                                  void* workspace, size_t workspace_bytes,
                                  int32_t partition_tokens, const int32_t* schedule,
                                  size_t schedule_bytes, void* stream);

/*
 * Bytes of device workspace paged_decode_step needs: the attention's
 * (pkv_decode_workspace_bytes), rounded up to 256, plus the longest-first
 * schedule (pkv_decode_schedule_bytes).  Zero only when both are zero.
 */
PKV_API size_t pkv_decode_step_workspace_bytes(int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads,
                                               int32_t head_size, int32_t max_blocks_per_seq,
                                               int32_t block_size, int32_t partition_tokens);

/*
 * One whole decode step in one call: for each sequence s, the new token
 * new_k[s], new_v[s] is stored in the slot of position seq_lens[s] - 1
 * (pkv_decode_append), and the attention of paged_decode_attention is
 * computed over all seq_lens[s] tokens, the new one included.  The result,
 * the pools and slot_mapping are bit-identical to calling those two
 * functions in that order.  Every argument is validated before anything is
 * launched, so a rejected call changes nothing.
 *   - Batches of up to 64 sequences: one launch (plus the chunk merge where
 *     sequences span several chunks).  The attention ranks the batch longest
 *     first itself and takes each new token from new_k / new_v; work-groups
 *     of the same launch, after the attention's, store the new tokens.
 *   - Larger batches: the append launch, which also writes the batch's
 *     longest-first schedule into the workspace (see
 *     pkv_decode_schedule_bytes), then the attention launch, which reads it.
 * new_k / new_v must not overlap the pools (they are read while the pools
 * are written).
 *   new_k, new_v  device T [num_seqs][num_kv_heads][head_size]
 *   slot_mapping  device int64 [num_seqs] receiving the slots, or NULL
 *   workspace     device scratch of workspace_bytes >=
 *                 pkv_decode_step_workspace_bytes(...), 16-byte aligned
 *   other arguments as paged_decode_attention
 * Errors: as paged_decode_attention; new_k / new_v must be non-null and
 * 16-byte aligned.
 */
PKV_API pkv_status paged_decode_step(const void* q, const void* new_k, const void* new_v, void* k_cache,
                                     void* v_cache, const int32_t* block_tables, const int32_t* seq_lens,
                                     int32_t num_seqs, int32_t num_q_heads, int32_t max_blocks_per_seq,
                                     const pkv_cache_desc* cache, float scale, void* out,
                                     int64_t* slot_mapping, void* workspace, size_t workspace_bytes,
                                     int32_t partition_tokens, void* stream);

/*
 * The decode step of paged_decode_step for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation): the same launches and the same
 * results, bit for bit, with the workspace taken from a device array inside
 * the library instead of a caller buffer.  The array holds
 * PKV_STATIC_SCRATCH_BYTES on every GPU the library runs on, until the
 * process ends; the call uses the current device's copy (stream must belong
 * to the current device) and allocates nothing (no hipMalloc, no allocating
 * library routine).  All calls on one GPU share that array and each leaves
 * its contents behind: calls that may overlap on one GPU (different streams,
 * or different host threads without ordering) race and must not be issued;
 * calls ordered on one stream are safe.  Nothing in it needs clearing
 * between calls.
 *   arguments as paged_decode_step, without workspace / workspace_bytes
 * Errors: as paged_decode_step; PKV_ERR_WORKSPACE when
 * pkv_decode_step_workspace_bytes(...) for these sizes exceeds
 * PKV_STATIC_SCRATCH_BYTES; PKV_ERR_UNSUPPORTED on a device index >= 64.
 */
#define PKV_STATIC_SCRATCH_BYTES ((size_t)32 << 20)

PKV_API pkv_status paged_decode_step_static(const void* q, const void* new_k, const void* new_v, void* k_cache,
                                            void* v_cache, const int32_t* block_tables, const int32_t* seq_lens,
                                            int32_t num_seqs, int32_t num_q_heads, int32_t max_blocks_per_seq,
                                            const pkv_cache_desc* cache, float scale, void* out,
                                            int64_t* slot_mapping, int32_t partition_tokens, void* stream);

/*
 * ---------------------------------------------------------------------------
 * Several query tokens per sequence: chunked prefill, prefill of the tokens a
 * prefix-cache lookup missed, and the draft tokens of speculative decoding
 * ---------------------------------------------------------------------------
 *
 * The pages name these users of the paged cache ("vLLM 核心工程深度剖析",
 * section 6.1 chunked prefill and section 9 speculative decoding; the
 * cache-structure page, "分配与增长": prefill computes only the tokens that
 * missed the cache and attends over the hit blocks as they are).  The rule
 * used here: the query rows of sequence s are rows q_start[s] ..
 * q_start[s+1]-1 of q, of out and of the new k/v; they are the LAST
 * n_s = q_start[s+1] - q_start[s] of its seq_lens[s] = L_s tokens, so row i
 * sits at position L_s - n_s + i, and it attends to the tokens at positions
 * 0 .. L_s - n_s + i (itself and everything before it).
 *
 * Caller contract: q_start (int32 [num_seqs + 1], device) is nondecreasing
 * from 0 to num_q_rows, 1 <= n_s <= max_q_len and n_s <= L_s for every
 * sequence that has query rows.  The kernels never access memory outside
 * the arguments when it is broken: a sequence whose rows fall outside
 * 0 .. num_q_rows - 1 is skipped, rows past max_q_len are not computed, and
 * a row whose position is negative (n_s > L_s) attends to nothing and gets
 * zeros.  q and out: [num_q_rows][num_q_heads][head_size] in the query
 * type; new k/v: [num_q_rows][num_kv_heads][head_size].  A call with no
 * query rows (num_q_rows or max_q_len 0: every sequence sits the step out)
 * launches nothing and returns PKV_OK after the shape checks; q, out and
 * the new rows may then be null.
 */

/*
 * partition_tokens of the multi-token calls may also be PKV_PARTITION_NONE:
 * the unpartitioned kernel, whose work-groups take 128 rows each and walk
 * the whole visible context with the keys and values staged in LDS (no
 * workspace; bf16 and FP8 pools with blocks of 16 tokens or more, else
 * PKV_ERR_UNSUPPORTED).  With 0 the library picks it when every (sequence,
 * KV head) has at least 64 rows and the batch gives it at least 512
 * work-groups, and the partitioned kernel otherwise; a positive length
 * always selects the partitioned kernel.  Both compute the same rule.
 */
#define PKV_PARTITION_NONE (-1)

/*
 * Which kernel paged_multi_token_attention runs for these sizes: 1 for the
 * unpartitioned kernel, 0 for the partitioned one, -1 for sizes it rejects
 * (invalid descriptor or head counts, or PKV_PARTITION_NONE where the
 * unpartitioned kernel is not supported).
 */
PKV_API int32_t pkv_multi_token_kernel(int32_t num_seqs, int32_t num_q_heads, int32_t max_q_len,
                                       const pkv_cache_desc* cache, int32_t partition_tokens);

/*
 * Bytes of device workspace paged_multi_token_attention needs with the
 * partitioned kernel (0 when each sequence's table fits one chunk of
 * partitions; the unpartitioned kernel needs none): one fp32 partial per
 * (sequence, KV head, tile of 16 (row, group member) pairs, chunk, tile row).
 * max_q_len <= 0 or an invalid shape gives 0.
 */
PKV_API size_t pkv_multi_token_workspace_bytes(int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads,
                                               int32_t head_size, int32_t max_q_len, int32_t max_blocks_per_seq,
                                               int32_t block_size, int32_t partition_tokens);

/*
 * Bytes of device workspace of paged_multi_token_step with the batch's
 * longest-first schedule: the attention partials
 * (pkv_multi_token_workspace_bytes; none with PKV_PARTITION_NONE), rounded
 * up to 256, plus the schedule (pkv_decode_schedule_bytes); just the
 * partials when no schedule applies (num_seqs outside 2 .. 4096).
 */
PKV_API size_t pkv_multi_token_step_workspace_bytes(int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads,
                                                    int32_t head_size, int32_t max_q_len,
                                                    int32_t max_blocks_per_seq, int32_t block_size,
                                                    int32_t partition_tokens);

/*
 * slot_mapping[q_start[s] + i] = slot of position L_s - n_s + i (the slot
 * rule of pkv_decode_slot_mapping), or -1 when that position lies outside
 * 0 .. L_s - 1 or past the table row.  Rows of no sequence are not written.
 *   schedule  device buffer of schedule_bytes >= pkv_decode_schedule_bytes
 *             receiving the batch's longest-first schedule (the layout
 *             pkv_decode_append writes, from block_tables and seq_lens), or
 *             NULL; ignored when that size is 0
 * Asynchronous on `stream`.  PKV_ERR_UNSUPPORTED for num_seqs > 65535;
 * PKV_ERR_WORKSPACE for a schedule buffer that is too small or not 16-byte
 * aligned.
 */
PKV_API pkv_status pkv_multi_token_slot_mapping(const int32_t* block_tables, const int32_t* seq_lens,
                                                const int32_t* q_start, int32_t num_seqs, int32_t num_q_rows,
                                                int32_t max_q_len, int32_t max_blocks_per_seq,
                                                int32_t block_size, int64_t* slot_mapping, int32_t* schedule,
                                                size_t schedule_bytes, void* stream);

/*
 * Stores new_k / new_v of every query row (rule above) in the slot of its
 * position, bit for bit as kv_cache_append with pkv_multi_token_slot_mapping
 * would (FP8 pools: the same quantization), but block by block: the rows
 * that land in one block are written together, so the value rows of the
 * block are written along their length instead of one element per token.
 * Rows whose position is negative, past the table row or in a block outside
 * the pool are skipped.  Asynchronous on `stream`.  PKV_ERR_UNSUPPORTED for
 * num_seqs > 65535.
 */
PKV_API pkv_status pkv_multi_token_append(const void* k, const void* v, const int32_t* q_start, int32_t num_q_rows,
                                          int32_t max_q_len, const int32_t* block_tables, const int32_t* seq_lens,
                                          int32_t num_seqs, int32_t max_blocks_per_seq, const pkv_cache_desc* cache,
                                          void* k_cache, void* v_cache, void* stream);

/*
 * Causal paged attention of every query row (rule above) over its
 * sequence's cached tokens, read through block_tables as in
 * paged_decode_attention (same pools, scale, partition_tokens and workspace
 * rules; workspace of pkv_multi_token_workspace_bytes).  The tokens of the
 * query rows themselves must already be in the cache (kv_cache_append with
 * pkv_multi_token_slot_mapping, or paged_multi_token_step).  schedule:
 * the longest-first schedule pkv_multi_token_slot_mapping (or
 * pkv_decode_append) wrote for these same block_tables and seq_lens, or
 * NULL, as in paged_decode_attention (both kernels start the longest
 * sequences first with it; the results are bit-identical either way).
 * PKV_ERR_UNSUPPORTED for max_q_len > 65535 or num_seqs > 65535.
 */
PKV_API pkv_status paged_multi_token_attention(const void* q, const int32_t* q_start, int32_t num_q_rows,
                                               int32_t max_q_len, const void* k_cache, const void* v_cache,
                                               const int32_t* block_tables, const int32_t* seq_lens,
                                               int32_t num_seqs, int32_t num_q_heads, int32_t max_blocks_per_seq,
                                               const pkv_cache_desc* cache, float scale, void* out,
                                               void* workspace, size_t workspace_bytes, int32_t partition_tokens,
                                               const int32_t* schedule, size_t schedule_bytes, void* stream);

/*
 * One multi-token step: slot mapping of the rows into slot_mapping (int64
 * [num_q_rows], device, required), append of new_k/new_v of every row
 * (pkv_multi_token_append), then paged_multi_token_attention.  Three kernels in
 * stream order; every argument is checked before the first, so a rejected
 * call changes nothing.  With a workspace of
 * pkv_multi_token_step_workspace_bytes the slot mapping launch also writes
 * the batch's longest-first schedule there and the partitioned attention
 * reads it; a workspace of pkv_multi_token_workspace_bytes runs the step
 * without one (bit-identical results).
 */
PKV_API pkv_status paged_multi_token_step(const void* q, const void* new_k, const void* new_v, void* k_cache,
                                          void* v_cache, const int32_t* q_start, int32_t num_q_rows,
                                          int32_t max_q_len, const int32_t* block_tables, const int32_t* seq_lens,
                                          int32_t num_seqs, int32_t num_q_heads, int32_t max_blocks_per_seq,
                                          const pkv_cache_desc* cache, float scale, void* out,
                                          int64_t* slot_mapping, void* workspace, size_t workspace_bytes,
                                          int32_t partition_tokens, void* stream);

/*
 * ---------------------------------------------------------------------------
 * Block copy and the host block pool (copy-on-write and fork)
 * ---------------------------------------------------------------------------
 */

/*
 * Block copy ("PagedAttention 笔记" page, copy-on-write section: "copy P8 ->
 * P11" before the writer's token goes into P11): for each pair
 * (src, dst) = (pairs[2i], pairs[2i+1]), every element of block src of both
 * pools (all KV heads, all slots) is copied to block dst, bit for bit.
 *   pairs      device int32 [num_pairs][2]
 *   k_cache, v_cache  device pools (layout above)
 * Device-side contract (not checked on the host): the dst blocks of one call
 * are distinct and none of them is also a src of the call; a pair with a
 * block outside [0, num_blocks) is skipped.
 * Errors: PKV_ERR_INVALID_ARG (null or misaligned pointer, bad descriptor,
 * num_pairs < 0), PKV_ERR_UNSUPPORTED, PKV_ERR_HIP.
 */
PKV_API pkv_status pkv_copy_blocks(const int32_t* pairs, int32_t num_pairs, const pkv_cache_desc* cache,
                                   void* k_cache, void* v_cache, void* stream);

/*
 * Host block pool: the bookkeeping of the block allocator of the
 * "vLLM 核心工程深度剖析" page (section 2.2: a free list used as a stack,
 * one reference count per block and one block table per sequence; a new
 * block only when the sequence's last block is full; blocks return to the
 * free list when their count reaches zero; running out is an error), its
 * fork (section 4.1: the child shares every block of the parent, one more
 * reference each) and the copy-on-write rule of the "PagedAttention 笔记"
 * page (a block referenced by more than one sequence is never written: the
 * writer takes a new block, the shared block is copied into it with
 * pkv_copy_blocks, the writer's table entry points at the copy and the
 * shared block loses a reference).
 * Host memory only; the pool touches no device memory.  One pool must not be
 * used from two threads at once.  Sequences are named by caller-chosen
 * 64-bit ids.
 */
typedef struct pkv_block_pool pkv_block_pool;

/* A pool of num_blocks blocks of block_size tokens, all free; the free list
 * is 0 .. num_blocks-1 and its last entry is handed out first.  NULL for
 * non-positive sizes or when host memory runs out. */
PKV_API pkv_block_pool* pkv_pool_create(int32_t num_blocks, int32_t block_size);

/* As pkv_pool_create, with the free list given (count distinct blocks in
 * [0, num_blocks); the last one is handed out first; blocks not listed are
 * never handed out).  NULL for an invalid list. */
PKV_API pkv_block_pool* pkv_pool_create_with_free_list(int32_t num_blocks, int32_t block_size,
                                                       const int32_t* free_list, int32_t count);

PKV_API void pkv_pool_destroy(pkv_block_pool* pool);

/* A new sequence holding num_tokens tokens: ceil(num_tokens / block_size)
 * blocks from the free list, in table order.  PKV_ERR_OUT_OF_BLOCKS when the
 * free list is too short (nothing changes); PKV_ERR_INVALID_ARG for a known
 * id or a negative count. */
PKV_API pkv_status pkv_pool_add_sequence(pkv_block_pool* pool, int64_t seq, int64_t num_tokens);

/* Reserves the slot of the next token of each of num_seqs distinct
 * sequences (position L = the sequence's length, which becomes L + 1) and
 * returns it in slots[i] = table[L / B] * B + L % B.  A full last block gets
 * a new block after it; a shared last block is replaced by a new one, and
 * the pair (shared, new) that pkv_copy_blocks must copy before the token is
 * written is appended to copies (host int32 [num_seqs][2], *num_copies
 * pairs).  Everything is checked first: PKV_ERR_OUT_OF_BLOCKS or
 * PKV_ERR_INVALID_ARG (unknown or repeated id) leave the pool unchanged. */
PKV_API pkv_status pkv_pool_append_slots(pkv_block_pool* pool, const int64_t* seqs, int32_t num_seqs,
                                         int64_t* slots, int32_t* copies, int32_t* num_copies);

/* The child (a new id) gets the parent's table and length; every block gains
 * a reference. */
PKV_API pkv_status pkv_pool_fork(pkv_block_pool* pool, int64_t parent, int64_t child);

/* Drops one reference on each block of the sequence (in table order) and
 * returns blocks whose count reaches zero to the end of the free list. */
PKV_API pkv_status pkv_pool_free(pkv_block_pool* pool, int64_t seq);

/* Queries: free blocks; a block's reference count (-1 if out of range); a
 * sequence's length (-1 if unknown); a sequence's table (returns its number
 * of blocks, -1 if unknown, and copies at most capacity entries to out). */
PKV_API int32_t pkv_pool_num_free(const pkv_block_pool* pool);
PKV_API int32_t pkv_pool_ref_count(const pkv_block_pool* pool, int32_t block);
PKV_API int64_t pkv_pool_seq_len(const pkv_block_pool* pool, int64_t seq);
PKV_API int32_t pkv_pool_block_table(const pkv_block_pool* pool, int64_t seq, int32_t* out, int32_t capacity);

/* Writes the kernel inputs for a batch: block_tables (host int32
 * [num_seqs][max_blocks_per_seq], padded with pad_block) and seq_lens (host
 * int32 [num_seqs]).  PKV_ERR_INVALID_ARG for an unknown id or a table longer
 * than max_blocks_per_seq (nothing is written then). */
PKV_API pkv_status pkv_pool_export(const pkv_block_pool* pool, const int64_t* seqs, int32_t num_seqs,
                                   int32_t max_blocks_per_seq, int32_t pad_block, int32_t* block_tables,
                                   int32_t* seq_lens);

/*
 * ---------------------------------------------------------------------------
 * Contract check (debugging aid)
 * ---------------------------------------------------------------------------
 *
 * The kernels contain a broken device-side contract (they skip an
 * out-of-pool block or slot and clamp a length) but do not report it.
 * pkv_validate reports it.  The rules checked, from the pages:
 *   - a used table entry (index < ceil(L / B)) names a block inside the pool
 *     and 0 <= L <= max_blocks_per_seq * B (the table walk of the cache-
 *     structure page, "软件地址翻译" / "Block Table");
 *   - the slots of one append are distinct and inside the pool (the cache-
 *     structure page, "写入新 K/V": each new token has its own slot);
 *   - no slot lies in a block that more than one sequence references
 *     ("PagedAttention 笔记", "写时复制是正确性的边界": a shared block is only
 *     read; a writer copies it first, pkv_copy_blocks).
 * Counts are exact; each "first" field is the smallest offending index, or
 * -1 when there is none.
 */
typedef struct {
    int64_t bad_seq_lens;         /* sequences with seq_len < 0 or > max_blocks_per_seq * B        */
    int64_t bad_block_ids;        /* used table entries outside [0, num_blocks)                    */
    int64_t bad_slots;            /* slots >= num_blocks * B (negative slots are skips, not errors) */
    int64_t duplicate_slots;      /* tokens whose slot (>= 0) equals an earlier token's slot       */
    int64_t shared_block_writes;  /* tokens whose slot lies in a block with ref_counts > 1         */
    int64_t first_bad_seq_len;    /* sequence index                                                */
    int64_t first_bad_block_id;   /* s * max_blocks_per_seq + i of table entry i of sequence s      */
    int64_t first_bad_slot;       /* token index                                                   */
    int64_t first_duplicate_slot; /* token index (the later token of a repeated slot)              */
    int64_t first_shared_block_write; /* token index                                               */
} pkv_validate_report;

/*
 * Checks the inputs of an attention call, an append or a decode step:
 *   block_tables  device int32 [num_seqs][max_blocks_per_seq]
 *   seq_lens      device int32 [num_seqs]
 *   slot_mapping  device int64 [num_tokens]: the slots of an append; or NULL
 *                 (num_tokens ignored): the decode step's slots, one per
 *                 sequence, by the rule of pkv_decode_slot_mapping (token
 *                 index = sequence index)
 *   ref_counts    device int32 [cache->num_blocks], each block's number of
 *                 referencing sequences (pkv_pool_ref_count), or NULL to skip
 *                 the shared-block rule
 *   report        device pkv_validate_report, 8-byte aligned, written
 * Only the tables, lengths, slots and counts are read, never the pools.
 * Asynchronous on `stream` (three launches; the report is complete when the
 * stream reaches it); a duplicate check compares every pair of slots, so the
 * cost grows with num_tokens squared (a debugging aid, not for the hot path).
 * Errors: PKV_ERR_INVALID_ARG (null report, a null array that the sizes
 * need, negative sizes, misaligned report, bad descriptor),
 * PKV_ERR_UNSUPPORTED (as for the descriptor), PKV_ERR_HIP.
 */
PKV_API pkv_status pkv_validate(const int32_t* block_tables, const int32_t* seq_lens, int32_t num_seqs,
                                int32_t max_blocks_per_seq, const int64_t* slot_mapping, int32_t num_tokens,
                                const int32_t* ref_counts, const pkv_cache_desc* cache, pkv_validate_report* report,
                                void* stream);

/*
 * ---------------------------------------------------------------------------
 * Measurement aid
 * ---------------------------------------------------------------------------
 *
 * Streaming-read probe: reads `bytes` of the device buffer `buf` once with
 * `work_groups` work-groups of 256 threads (each the next contiguous share,
 * eight 16-byte non-temporal loads in flight per thread), so that a caller
 * timing it gets the GPU's practical read bandwidth, the ceiling of the
 * bandwidth-bound kernels above.  Not part of the attention method.
 *   buf          device buffer, 16-byte aligned; bytes a multiple of 16
 *   out          device buffer of 4 bytes; a thread writes 0x9E3779B9 there
 *                when the XOR of the 32-bit words it read equals that value
 *                (so that no load can be dropped), and nothing otherwise
 *   work_groups  1 .. 1048576
 * Asynchronous on `stream`.  PKV_ERR_INVALID_ARG for a null or misaligned
 * pointer, a size that is not a multiple of 16, or work_groups out of range.
 */
PKV_API pkv_status pkv_probe_stream_read(const void* buf, size_t bytes, void* out, int32_t work_groups,
                                         void* stream);

/*
 * Gather-read probe: reads num_tiles whole tiles of tile_bytes each, tile t
 * from buf0 (t even) or buf1 (t odd) at byte offset tile_offsets[t], with
 * `work_groups` work-groups of 256 threads (each wave the next contiguous
 * share of the list, eight 16-byte non-temporal loads in flight per thread).
 * With the key and value tiles of a pool's blocks listed in turn (one
 * (block, KV head) tile of each per entry pair, as block_tables and
 * seq_lens select them: the cache-structure page's block-table translation)
 * it gives the rate of the paged access pattern on its own, every address
 * known in advance: the ceiling of decode attention on that pool, below the
 * streaming probe's.  Not part of the attention method.
 *   buf0, buf1     device buffers of bytes0, bytes1 bytes, 16-byte aligned
 *   tile_offsets   device int64 [num_tiles]; a tile at a negative offset, an
 *                  offset that is not a multiple of 16, or reaching past its
 *                  buffer is skipped (never read)
 *   tile_bytes     a multiple of 1024, 1024 .. 1048576
 *   out            device buffer of 4 bytes, written as by pkv_probe_stream_read
 *   work_groups    1 .. 1048576
 * Asynchronous on `stream`.  PKV_ERR_INVALID_ARG for a null or misaligned
 * buffer, tile_bytes or work_groups out of range, or a negative num_tiles.
 */
PKV_API pkv_status pkv_probe_gather_read(const void* buf0, size_t bytes0, const void* buf1, size_t bytes1,
                                         const int64_t* tile_offsets, int64_t num_tiles, int32_t tile_bytes,
                                         void* out, int32_t work_groups, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* PKV_H */
