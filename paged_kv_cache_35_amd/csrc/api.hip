// C-ABI entry points: host-side validation, workspace sizing, partition
// choice and dispatch to the kernels.  The contract is documented in
// include/pkv.h.
#include <string.h>

#include <atomic>
#include <cmath>
#include <mutex>

#include "../../include/pkv.h"
#include "pkv_internal.h"

namespace {

thread_local hipError_t g_last_hip_error = hipSuccess;

pkv_status hip_status(hipError_t e)
{
    if (e == hipSuccess)
        return PKV_OK;
    g_last_hip_error = e;
    return PKV_ERR_HIP;
}

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

int elem_bytes(int32_t dtype) { return dtype == PKV_F32 ? 4 : (dtype == PKV_FP8_E4M3 ? 1 : 2); }

size_t round_up(size_t n, size_t a) { return (n + a - 1) / a * a; }

// Library choice of the context-partition length: kDefaultPartitionTokens
// (512: 32 blocks at B = 16, 16 at B = 32), at most 64 blocks (one block ID
// per lane of the wave; blocks of fewer than 16 tokens: 512 tokens, the
// IDs in windows of 64), or one partition when the table is shorter.
// Blocks of fewer than 16 tokens are read in 16-token units that must not
// straddle two partitions: the length is then a multiple of 16.
constexpr int64_t kDefaultPartitionTokens = 512;
int32_t resolve_partition_tokens(int32_t max_blocks_per_seq, int32_t block_size, int32_t requested)
{
    if (requested < 0 || max_blocks_per_seq <= 0 || block_size <= 0)
        return 0;
    // a wave's list holds at most 64 blocks, or 512 tokens' worth of blocks
    // of fewer than 16 tokens (kept in windows of 64 by the kernel)
    const int64_t max_blocks = block_size < 16 ? 512 / block_size : 64;
    if (requested > 0) {
        if (requested % block_size != 0 || requested / block_size > max_blocks ||
            (block_size < 16 && requested % 16 != 0))
            return 0;
        return requested;
    }
    const int64_t whole = (int64_t)max_blocks_per_seq * block_size;
    const int64_t dflt =
        kDefaultPartitionTokens < max_blocks * block_size ? kDefaultPartitionTokens : max_blocks * block_size;
    return (int32_t)(whole < dflt ? whole : dflt);
}

// Longest-first schedule: int32 order [S], lens [S], tables [S][M] (each
// rounded up to 16 bytes), the chunk count (padded to 16 bytes) and the chunk
// list [S][ceil(M / 4)] of (rank and chunk, sequence) pairs (a chunk has at
// least 4 blocks: one per wave).
size_t schedule_items_capacity(int32_t num_seqs, int32_t max_blocks_per_seq)
{
    return (size_t)num_seqs * (((size_t)max_blocks_per_seq + 3) / 4);
}

pkv::AppendArgs::Schedule schedule_parts(void* schedule, int32_t num_seqs, int32_t max_blocks_per_seq,
                                         int32_t block_size)
{
    char* base = (char*)schedule;
    const size_t vec = round_up((size_t)num_seqs * 4, 16);
    char* after_tables = base + 2 * vec + round_up((size_t)num_seqs * max_blocks_per_seq * 4, 16);
    const int32_t P = resolve_partition_tokens(max_blocks_per_seq, block_size, 0);  // the library's default
    return {(int32_t*)base, (int32_t*)(base + vec), (int32_t*)(base + 2 * vec), (int32_t*)after_tables,
            (uint32_t*)(after_tables + 16), (P / block_size) * pkv::kDecodeWaves};
}

// Validates a pool descriptor; returns PKV_OK or the status to report.
pkv_status check_cache(const pkv_cache_desc* c)
{
    if (!c)
        return PKV_ERR_INVALID_ARG;
    if (c->num_blocks <= 0 || c->num_kv_heads <= 0 || c->block_size <= 0 || c->head_size <= 0)
        return PKV_ERR_INVALID_ARG;
    if (c->dtype != PKV_F32 && c->dtype != PKV_BF16 && c->dtype != PKV_FP8_E4M3)
        return PKV_ERR_UNSUPPORTED;
    if (c->dtype == PKV_FP8_E4M3 &&
        !(c->k_scale > 0.f && c->v_scale > 0.f && std::isfinite(c->k_scale) && std::isfinite(c->v_scale)))
        return PKV_ERR_INVALID_ARG;
    if (c->head_size != 64 && c->head_size != 128)
        return PKV_ERR_UNSUPPORTED;
    const int32_t B = c->block_size;
    if (B != 1 && B != 8 && B != 16 && B != 32 && B != 64)
        return PKV_ERR_UNSUPPORTED;
    if (c->dtype == PKV_FP8_E4M3 && B < 16)
        return PKV_ERR_UNSUPPORTED;
    if (c->out_f32 != 0 && c->out_f32 != 1)
        return PKV_ERR_INVALID_ARG;
    return PKV_OK;
}


}  // namespace

extern "C" {

int32_t pkv_layout_version(void) { return 2; }

const char* pkv_status_string(int32_t status)
{
    switch (status) {
    case PKV_OK: return "PKV_OK";
    case PKV_ERR_INVALID_ARG: return "PKV_ERR_INVALID_ARG";
    case PKV_ERR_UNSUPPORTED: return "PKV_ERR_UNSUPPORTED";
    case PKV_ERR_WORKSPACE: return "PKV_ERR_WORKSPACE";
    case PKV_ERR_HIP: return "PKV_ERR_HIP";
    case PKV_ERR_OUT_OF_BLOCKS: return "PKV_ERR_OUT_OF_BLOCKS";
    default: return "PKV_UNKNOWN_STATUS";
    }
}

const char* pkv_last_hip_error(void) { return hipGetErrorName(g_last_hip_error); }

pkv_status pkv_decode_slot_mapping(const int32_t* block_tables, const int32_t* seq_lens, int32_t num_seqs,
                                   int32_t max_blocks_per_seq, int32_t block_size, int64_t* slot_mapping,
                                   void* stream)
{
    if (num_seqs < 0 || max_blocks_per_seq <= 0 || block_size <= 0)
        return PKV_ERR_INVALID_ARG;
    if (num_seqs == 0)
        return PKV_OK;
    if (!block_tables || !seq_lens || !slot_mapping)
        return PKV_ERR_INVALID_ARG;
    return hip_status(pkv::launch_slot_mapping(block_tables, seq_lens, num_seqs, max_blocks_per_seq, block_size,
                                               slot_mapping, (hipStream_t)stream));
}

namespace {

pkv::AppendArgs append_args(const void* k, const void* v, int64_t* slot_mapping, const int32_t* block_tables,
                            const int32_t* seq_lens, int32_t max_blocks_per_seq, int32_t num_tokens,
                            const pkv_cache_desc* cache, void* k_cache, void* v_cache,
                            pkv::AppendArgs::Schedule sched = {})
{
    pkv::AppendArgs a;
    a.sched = sched;
    a.k = k;
    a.v = v;
    a.slot_mapping = slot_mapping;
    a.block_tables = block_tables;
    a.seq_lens = seq_lens;
    a.max_blocks_per_seq = max_blocks_per_seq;
    a.k_cache = k_cache;
    a.v_cache = v_cache;
    a.num_tokens = num_tokens;
    a.num_kv_heads = cache->num_kv_heads;
    a.head_size = cache->head_size;
    a.block_size = cache->block_size;
    a.num_blocks = cache->num_blocks;
    a.elem_bytes = elem_bytes(cache->dtype);
    // FP8: both sides of the append multiply by the fp32 reciprocal of the scale
    a.k_inv_scale = cache->dtype == PKV_FP8_E4M3 ? 1.0f / cache->k_scale : 1.0f;
    a.v_inv_scale = cache->dtype == PKV_FP8_E4M3 ? 1.0f / cache->v_scale : 1.0f;
    return a;
}

pkv_status append_common(const void* k, const void* v, int64_t* slot_mapping, const int32_t* block_tables,
                         const int32_t* seq_lens, int32_t max_blocks_per_seq, int32_t num_tokens,
                         const pkv_cache_desc* cache, void* k_cache, void* v_cache, void* stream,
                         pkv::AppendArgs::Schedule sched = {})
{
    const pkv::AppendArgs a = append_args(k, v, slot_mapping, block_tables, seq_lens, max_blocks_per_seq, num_tokens,
                                          cache, k_cache, v_cache, sched);
    return hip_status(pkv::launch_append(a, (hipStream_t)stream));
}

}  // namespace

pkv_status kv_cache_append(const void* k, const void* v, const int64_t* slot_mapping, int32_t num_tokens,
                           const pkv_cache_desc* cache, void* k_cache, void* v_cache, void* stream)
{
    if (num_tokens < 0)
        return PKV_ERR_INVALID_ARG;
    pkv_status st = check_cache(cache);
    if (st != PKV_OK)
        return st;
    if (!k_cache || !v_cache || !aligned16(k_cache) || !aligned16(v_cache))
        return PKV_ERR_INVALID_ARG;
    if (num_tokens == 0)
        return PKV_OK;
    if (!k || !v || !slot_mapping || !aligned16(k) || !aligned16(v))
        return PKV_ERR_INVALID_ARG;
    // the kernel only reads slot_mapping when no block table is given
    return append_common(k, v, const_cast<int64_t*>(slot_mapping), nullptr, nullptr, 0, num_tokens, cache, k_cache,
                         v_cache, stream);
}

size_t pkv_decode_schedule_bytes(int32_t num_seqs, int32_t max_blocks_per_seq)
{
    if (num_seqs <= 1 || num_seqs > pkv::kScheduleMaxSeqs || max_blocks_per_seq <= 0)
        return 0;
    return 2 * round_up((size_t)num_seqs * 4, 16) + round_up((size_t)num_seqs * max_blocks_per_seq * 4, 16) + 16 +
           schedule_items_capacity(num_seqs, max_blocks_per_seq) * 8;
}

pkv_status pkv_decode_append(const void* k, const void* v, const int32_t* block_tables, const int32_t* seq_lens,
                             int32_t num_seqs, int32_t max_blocks_per_seq, const pkv_cache_desc* cache,
                             void* k_cache, void* v_cache, int64_t* slot_mapping, int32_t* schedule,
                             size_t schedule_bytes, void* stream)
{
    if (num_seqs < 0 || max_blocks_per_seq <= 0)
        return PKV_ERR_INVALID_ARG;
    pkv_status st = check_cache(cache);
    if (st != PKV_OK)
        return st;
    if (!k_cache || !v_cache || !aligned16(k_cache) || !aligned16(v_cache))
        return PKV_ERR_INVALID_ARG;
    if (num_seqs == 0)
        return PKV_OK;
    if (!k || !v || !block_tables || !seq_lens || !aligned16(k) || !aligned16(v))
        return PKV_ERR_INVALID_ARG;
    pkv::AppendArgs::Schedule sched = {};
    const size_t sb = pkv_decode_schedule_bytes(num_seqs, max_blocks_per_seq);
    if (schedule && sb > 0) {
        if (schedule_bytes < sb || !aligned16(schedule))
            return PKV_ERR_WORKSPACE;
        sched = schedule_parts(schedule, num_seqs, max_blocks_per_seq, cache->block_size);
    }
    return append_common(k, v, slot_mapping, block_tables, seq_lens, max_blocks_per_seq, num_seqs, cache, k_cache,
                         v_cache, stream, sched);
}

int32_t pkv_decode_partition_tokens(int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads,
                                    int32_t head_size, int32_t max_blocks_per_seq, int32_t block_size,
                                    int32_t partition_tokens)
{
    if (num_seqs < 0 || num_q_heads <= 0 || num_kv_heads <= 0 || head_size <= 0)
        return 0;
    return resolve_partition_tokens(max_blocks_per_seq, block_size, partition_tokens);
}

size_t pkv_decode_workspace_bytes(int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads, int32_t head_size,
                                  int32_t max_blocks_per_seq, int32_t block_size, int32_t partition_tokens)
{
    const int32_t P = pkv_decode_partition_tokens(num_seqs, num_q_heads, num_kv_heads, head_size,
                                                  max_blocks_per_seq, block_size, partition_tokens);
    if (P <= 0)
        return 0;
    // one fp32 partial (o[hs], m, l) per (sequence, query head, chunk of
    // kDecodeWaves partitions); none when one chunk covers the table
    const int64_t cb = (int64_t)(P / block_size) * pkv::kDecodeWaves;
    const int64_t chunks = (max_blocks_per_seq + cb - 1) / cb;
    if (chunks <= 1)
        return 0;
    return (size_t)num_seqs * num_q_heads * chunks * ((size_t)head_size + 2) * sizeof(float);
}

size_t pkv_decode_step_workspace_bytes(int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads,
                                       int32_t head_size, int32_t max_blocks_per_seq, int32_t block_size,
                                       int32_t partition_tokens)
{
    const size_t attn = pkv_decode_workspace_bytes(num_seqs, num_q_heads, num_kv_heads, head_size,
                                                   max_blocks_per_seq, block_size, partition_tokens);
    if (pkv_decode_partition_tokens(num_seqs, num_q_heads, num_kv_heads, head_size, max_blocks_per_seq,
                                    block_size, partition_tokens) <= 0)
        return 0;
    return round_up(attn, 256) + pkv_decode_schedule_bytes(num_seqs, max_blocks_per_seq);
}

namespace {

// The chunk list serves batches above kLptMaxSeqs sequences (smaller ones
// are launched with each sequence's chunks consecutive in the grid, which
// needs no list); its launch is one-dimensional: one work-group per (KV
// head, row tile, possible chunk), kept below 2^24 work-groups of 256
// threads.
bool listed_grid_fits(const pkv::DecodeArgs& a)
{
    return a.num_seqs > pkv::kLptMaxSeqs &&
           (int64_t)a.num_kv_heads * a.row_tiles * a.num_seqs * a.max_parts < (int64_t)1 << 24;
}

// Points the attention launch at a schedule written for the same tables and
// lengths: order, lengths and table rows always; the chunk list only with
// the default partitioning it was written for, on large batches.
void use_schedule(pkv::DecodeArgs& a, const pkv::AppendArgs::Schedule& p, int32_t partition_tokens)
{
    a.sched_order = p.order;
    a.sched_lens = p.lens;
    a.sched_tables = p.tables;
    if (partition_tokens == 0 && listed_grid_fits(a)) {
        a.sched_count = p.count;
        a.sched_items = p.items;
    }
}

// A caller's schedule buffer: PKV_OK with *used set when it is given and a
// schedule applies to this batch, PKV_ERR_WORKSPACE when it is too small or
// misaligned.
pkv_status caller_schedule(const int32_t* schedule, size_t schedule_bytes, int32_t num_seqs,
                           int32_t max_blocks_per_seq, int32_t block_size, pkv::AppendArgs::Schedule& p, bool& used)
{
    used = false;
    const size_t sb = pkv_decode_schedule_bytes(num_seqs, max_blocks_per_seq);
    if (!schedule || sb == 0)
        return PKV_OK;
    if (schedule_bytes < sb || !aligned16(schedule))
        return PKV_ERR_WORKSPACE;
    p = schedule_parts(const_cast<int32_t*>(schedule), num_seqs, max_blocks_per_seq, block_size);
    used = true;
    return PKV_OK;
}

// Validates the attention arguments and fills the launch description; no
// GPU work.  PKV_OK with *nothing_to_do set when num_seqs == 0.
pkv_status attention_args(const void* q, const void* k_cache, const void* v_cache, const int32_t* block_tables,
                          const int32_t* seq_lens, int32_t num_seqs, int32_t num_q_heads, int32_t max_blocks_per_seq,
                          const pkv_cache_desc* cache, float scale, void* out, void* workspace,
                          size_t workspace_bytes, int32_t partition_tokens, pkv::DecodeArgs& a, bool& nothing_to_do,
                          bool check_workspace = true)
{
    nothing_to_do = false;
    if (num_seqs < 0 || num_q_heads <= 0 || max_blocks_per_seq <= 0)
        return PKV_ERR_INVALID_ARG;
    pkv_status st = check_cache(cache);
    if (st != PKV_OK)
        return st;
    // the kernels keep the running maximum of raw scores, which needs a
    // positive scale
    if (!(scale > 0.f) || !std::isfinite(scale))
        return PKV_ERR_INVALID_ARG;
    const int32_t Hkv = cache->num_kv_heads;
    if (num_q_heads % Hkv != 0)
        return PKV_ERR_INVALID_ARG;
    const int32_t G = num_q_heads / Hkv;
    if (G > 16)
        return PKV_ERR_UNSUPPORTED;
    if ((int64_t)max_blocks_per_seq * cache->block_size > INT32_MAX)
        return PKV_ERR_INVALID_ARG;
    if (num_seqs == 0) {
        nothing_to_do = true;
        return PKV_OK;
    }
    if (!q || !k_cache || !v_cache || !block_tables || !seq_lens || !out)
        return PKV_ERR_INVALID_ARG;
    if (!aligned16(q) || !aligned16(k_cache) || !aligned16(v_cache) || !aligned16(out))
        return PKV_ERR_INVALID_ARG;
    const int32_t P = resolve_partition_tokens(max_blocks_per_seq, cache->block_size, partition_tokens);
    if (P <= 0)
        return PKV_ERR_INVALID_ARG;
    const int32_t pb = P / cache->block_size;
    const int32_t parts = (max_blocks_per_seq + pb * pkv::kDecodeWaves - 1) / (pb * pkv::kDecodeWaves);
    if (num_seqs > 65535 || parts > 65535)
        return PKV_ERR_UNSUPPORTED;
    const size_t need = pkv_decode_workspace_bytes(num_seqs, num_q_heads, Hkv, cache->head_size,
                                                   max_blocks_per_seq, cache->block_size, partition_tokens);
    if (check_workspace && need > 0 && (!workspace || workspace_bytes < need || !aligned16(workspace)))
        return PKV_ERR_WORKSPACE;

    a.step_append = {};
    a.sched_order = nullptr;
    a.sched_lens = nullptr;
    a.sched_tables = nullptr;
    a.sched_count = nullptr;
    a.sched_items = nullptr;
    a.q_start = nullptr;
    a.num_q_rows = num_seqs;
    a.max_q_len = 1;
    a.row_tiles = 1;
    a.q = q;
    a.k_cache = k_cache;
    a.v_cache = v_cache;
    a.block_tables = block_tables;
    a.seq_lens = seq_lens;
    a.out = out;
    a.out_f32 = cache->out_f32;
    const size_t units = (size_t)num_seqs * num_q_heads * parts;
    a.ws_o = need > 0 ? (float*)workspace : nullptr;
    a.ws_ml = need > 0 ? (float*)workspace + units * cache->head_size : nullptr;
    a.num_seqs = num_seqs;
    a.num_q_heads = num_q_heads;
    a.num_kv_heads = Hkv;
    a.head_size = cache->head_size;
    a.block_size = cache->block_size;
    a.max_blocks_per_seq = max_blocks_per_seq;
    a.num_blocks = cache->num_blocks;
    a.dtype = cache->dtype;
    a.partition_blocks = pb;
    a.max_parts = parts;
    // A requested partition length is honoured literally (each wave owns one
    // contiguous partition); the library's own choice deals each chunk's
    // blocks round-robin to the waves, which balances sequences that end
    // inside a chunk.  Both compute the same attention.
    a.interleave = partition_tokens == 0 ? 1 : 0;
    a.scale = scale;
    a.k_scale = cache->dtype == PKV_FP8_E4M3 ? cache->k_scale : 1.0f;
    a.v_scale = cache->dtype == PKV_FP8_E4M3 ? cache->v_scale : 1.0f;
    return PKV_OK;
}

}  // namespace

pkv_status paged_decode_attention(const void* q, const void* k_cache, const void* v_cache,
                                  const int32_t* block_tables, const int32_t* seq_lens, int32_t num_seqs,
                                  int32_t num_q_heads, int32_t max_blocks_per_seq, const pkv_cache_desc* cache,
                                  float scale, void* out, void* workspace, size_t workspace_bytes,
                                  int32_t partition_tokens, const int32_t* schedule, size_t schedule_bytes,
                                  void* stream)
{
    pkv::DecodeArgs a;
    bool nothing_to_do;
    const pkv_status st = attention_args(q, k_cache, v_cache, block_tables, seq_lens, num_seqs, num_q_heads,
                                         max_blocks_per_seq, cache, scale, out, workspace, workspace_bytes,
                                         partition_tokens, a, nothing_to_do);
    if (st != PKV_OK || nothing_to_do)
        return st;
    pkv::AppendArgs::Schedule p;
    bool used;
    const pkv_status ss = caller_schedule(schedule, schedule_bytes, num_seqs, max_blocks_per_seq, cache->block_size,
                                          p, used);
    if (ss != PKV_OK)
        return ss;
    if (used)
        use_schedule(a, p, partition_tokens);
    return hip_status(pkv::launch_decode(a, (hipStream_t)stream));
}

size_t pkv_multi_token_workspace_bytes(int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads,
                                       int32_t head_size, int32_t max_q_len, int32_t max_blocks_per_seq,
                                       int32_t block_size, int32_t partition_tokens)
{
    if (num_kv_heads <= 0 || max_q_len <= 0 || num_q_heads % num_kv_heads != 0)
        return 0;
    const int32_t P = pkv_decode_partition_tokens(num_seqs, num_q_heads, num_kv_heads, head_size,
                                                  max_blocks_per_seq, block_size, partition_tokens);
    if (P <= 0)
        return 0;
    // one fp32 partial (o[hs], m, l) per (sequence, KV head, 16-row tile,
    // chunk, tile row); none when one chunk covers the table
    const int64_t cb = (int64_t)(P / block_size) * pkv::kDecodeWaves;
    const int64_t chunks = (max_blocks_per_seq + cb - 1) / cb;
    if (chunks <= 1)
        return 0;
    const int64_t G = num_q_heads / num_kv_heads;
    const int64_t tiles = ((int64_t)max_q_len * G + 15) / 16;
    return (size_t)num_seqs * num_kv_heads * tiles * chunks * 16 * ((size_t)head_size + 2) * sizeof(float);
}

pkv_status pkv_multi_token_slot_mapping(const int32_t* block_tables, const int32_t* seq_lens,
                                        const int32_t* q_start, int32_t num_seqs, int32_t num_q_rows,
                                        int32_t max_q_len, int32_t max_blocks_per_seq, int32_t block_size,
                                        int64_t* slot_mapping, int32_t* schedule, size_t schedule_bytes,
                                        void* stream)
{
    if (num_seqs < 0 || num_q_rows < 0 || max_q_len < 0 || max_blocks_per_seq <= 0 || block_size <= 0)
        return PKV_ERR_INVALID_ARG;
    if (num_seqs == 0 || num_q_rows == 0 || max_q_len == 0)
        return PKV_OK;
    if (!block_tables || !seq_lens || !q_start || !slot_mapping)
        return PKV_ERR_INVALID_ARG;
    if (num_seqs > 65535)
        return PKV_ERR_UNSUPPORTED;
    pkv::AppendArgs::Schedule sched = {};
    bool used;
    const pkv_status ss = caller_schedule(schedule, schedule_bytes, num_seqs, max_blocks_per_seq, block_size, sched,
                                          used);
    if (ss != PKV_OK)
        return ss;
    return hip_status(pkv::launch_multi_token_slot_mapping(block_tables, seq_lens, q_start, num_seqs, num_q_rows,
                                                           max_q_len, max_blocks_per_seq, block_size, slot_mapping,
                                                           sched, (hipStream_t)stream));
}

pkv_status pkv_multi_token_append(const void* k, const void* v, const int32_t* q_start, int32_t num_q_rows,
                                  int32_t max_q_len, const int32_t* block_tables, const int32_t* seq_lens,
                                  int32_t num_seqs, int32_t max_blocks_per_seq, const pkv_cache_desc* cache,
                                  void* k_cache, void* v_cache, void* stream)
{
    if (num_seqs < 0 || num_q_rows < 0 || max_q_len < 0 || max_blocks_per_seq <= 0)
        return PKV_ERR_INVALID_ARG;
    const pkv_status st = check_cache(cache);
    if (st != PKV_OK)
        return st;
    if (!k_cache || !v_cache || !aligned16(k_cache) || !aligned16(v_cache))
        return PKV_ERR_INVALID_ARG;
    if (num_seqs == 0 || num_q_rows == 0 || max_q_len == 0)
        return PKV_OK;
    if (!k || !v || !q_start || !block_tables || !seq_lens || !aligned16(k) || !aligned16(v))
        return PKV_ERR_INVALID_ARG;
    if (num_seqs > 65535 || (int64_t)max_q_len / cache->block_size + 2 > 65535)
        return PKV_ERR_UNSUPPORTED;
    const pkv::AppendArgs a = append_args(k, v, nullptr, block_tables, seq_lens, max_blocks_per_seq, num_q_rows,
                                          cache, k_cache, v_cache);
    return hip_status(pkv::launch_multi_token_append(a, q_start, num_seqs, num_q_rows, max_q_len, (hipStream_t)stream));
}

namespace {

// The library's choice for a multi-token call (partition_tokens == 0): the
// prefill kernel when every (sequence, KV head) has at least 64 rows (query
// tokens x group size) and the batch gives it at least 512 work-groups (two
// per compute unit); otherwise the partitioned decode kernel, which splits
// long contexts over work-groups.  A requested partition length always
// selects the partitioned kernel.
constexpr int64_t kPrefillMinRows = 64;
constexpr int64_t kPrefillMinGroups = 512;

bool picks_prefill_sizes(int32_t dtype, int32_t block_size, int32_t head_size, int64_t num_seqs,
                         int64_t num_q_heads, int64_t num_kv_heads, int64_t max_q_len, int32_t partition_tokens)
{
    if (partition_tokens == PKV_PARTITION_NONE)
        return true;
    const int64_t G = num_q_heads / num_kv_heads;
    const int64_t wgs = pkv::prefill_work_groups(num_seqs, num_q_heads, num_kv_heads, max_q_len);
    return partition_tokens == 0 && pkv::prefill_shape_supported(dtype, block_size, head_size) &&
           max_q_len * G >= kPrefillMinRows && wgs >= kPrefillMinGroups && wgs <= INT32_MAX;
}

bool picks_prefill(const pkv::DecodeArgs& a, int32_t partition_tokens)
{
    return picks_prefill_sizes(a.dtype, a.block_size, a.head_size, a.num_seqs, a.num_q_heads, a.num_kv_heads,
                               a.max_q_len, partition_tokens);
}

hipError_t launch_multi_token(const pkv::DecodeArgs& a, int32_t partition_tokens, hipStream_t stream)
{
    return picks_prefill(a, partition_tokens) ? pkv::launch_prefill(a, stream) : pkv::launch_decode(a, stream);
}

// attention_args plus the query-row description of a multi-token call.
pkv_status multi_token_args(const void* q, const int32_t* q_start, int32_t num_q_rows, int32_t max_q_len,
                            const void* k_cache, const void* v_cache, const int32_t* block_tables,
                            const int32_t* seq_lens, int32_t num_seqs, int32_t num_q_heads,
                            int32_t max_blocks_per_seq, const pkv_cache_desc* cache, float scale, void* out,
                            void* workspace, size_t workspace_bytes, int32_t partition_tokens, pkv::DecodeArgs& a,
                            bool& nothing_to_do)
{
    if (num_q_rows < 0 || max_q_len < 0)
        return PKV_ERR_INVALID_ARG;
    // No query rows (every sequence sits this step out): nothing to compute
    // or append, and q, out and the new rows may be empty (null).  The
    // shapes and the pool descriptor are still checked, as for an empty
    // batch.
    if (num_q_rows == 0 || max_q_len == 0)
        return attention_args(q, k_cache, v_cache, block_tables, seq_lens, 0, num_q_heads, max_blocks_per_seq, cache,
                              scale, out, workspace, workspace_bytes, 0, a, nothing_to_do, false);
    // PKV_PARTITION_NONE: the unpartitioned (prefill) kernel, no workspace
    const bool unpartitioned = partition_tokens == PKV_PARTITION_NONE;
    const int32_t P = unpartitioned ? 0 : partition_tokens;
    // the decode workspace is never larger than the multi-token one, so the
    // decode check in attention_args passes whenever the check below does
    const size_t need = unpartitioned ? 0
                                      : pkv_multi_token_workspace_bytes(
                                            num_seqs, num_q_heads, cache ? cache->num_kv_heads : 0,
                                            cache ? cache->head_size : 0, max_q_len > 0 ? max_q_len : 1,
                                            max_blocks_per_seq, cache ? cache->block_size : 0, P);
    pkv_status st = attention_args(q, k_cache, v_cache, block_tables, seq_lens, num_seqs, num_q_heads,
                                   max_blocks_per_seq, cache, scale, out, workspace,
                                   need > workspace_bytes ? 0 : workspace_bytes, P, a, nothing_to_do, !unpartitioned);
    if (st != PKV_OK || nothing_to_do)
        return st;
    if (!q_start)
        return PKV_ERR_INVALID_ARG;
    const int64_t G = num_q_heads / cache->num_kv_heads;
    const int64_t tiles = ((int64_t)max_q_len * G + 15) / 16;
    if (max_q_len > 65535 || tiles * cache->num_kv_heads > INT32_MAX)
        return PKV_ERR_UNSUPPORTED;
    if (need > 0 && (!workspace || workspace_bytes < need || !aligned16(workspace)))
        return PKV_ERR_WORKSPACE;
    a.q_start = q_start;
    a.num_q_rows = num_q_rows;
    a.max_q_len = max_q_len;
    a.row_tiles = (int32_t)tiles;
    const size_t units = (size_t)num_seqs * cache->num_kv_heads * tiles * a.max_parts * 16;
    a.ws_o = need > 0 ? (float*)workspace : nullptr;
    a.ws_ml = need > 0 ? (float*)workspace + units * cache->head_size : nullptr;
    if (unpartitioned && (!pkv::prefill_supported(a) || pkv::prefill_work_groups(a) > INT32_MAX))
        return PKV_ERR_UNSUPPORTED;
    return PKV_OK;
}

}  // namespace

pkv_status paged_multi_token_attention(const void* q, const int32_t* q_start, int32_t num_q_rows, int32_t max_q_len,
                                       const void* k_cache, const void* v_cache, const int32_t* block_tables,
                                       const int32_t* seq_lens, int32_t num_seqs, int32_t num_q_heads,
                                       int32_t max_blocks_per_seq, const pkv_cache_desc* cache, float scale,
                                       void* out, void* workspace, size_t workspace_bytes, int32_t partition_tokens,
                                       const int32_t* schedule, size_t schedule_bytes, void* stream)
{
    pkv::DecodeArgs a;
    bool nothing_to_do;
    const pkv_status st = multi_token_args(q, q_start, num_q_rows, max_q_len, k_cache, v_cache, block_tables,
                                           seq_lens, num_seqs, num_q_heads, max_blocks_per_seq, cache, scale, out,
                                           workspace, workspace_bytes, partition_tokens, a, nothing_to_do);
    if (st != PKV_OK || nothing_to_do)
        return st;
    pkv::AppendArgs::Schedule p;
    bool used;
    const pkv_status ss = caller_schedule(schedule, schedule_bytes, num_seqs, max_blocks_per_seq, cache->block_size,
                                          p, used);
    if (ss != PKV_OK)
        return ss;
    if (used)
        use_schedule(a, p, partition_tokens);
    return hip_status(launch_multi_token(a, partition_tokens, (hipStream_t)stream));
}

int32_t pkv_multi_token_kernel(int32_t num_seqs, int32_t num_q_heads, int32_t max_q_len,
                               const pkv_cache_desc* cache, int32_t partition_tokens)
{
    if (check_cache(cache) != PKV_OK || num_seqs < 0 || num_q_heads <= 0 || max_q_len < 0 ||
        num_q_heads % cache->num_kv_heads != 0 || partition_tokens < PKV_PARTITION_NONE)
        return -1;
    if (partition_tokens == PKV_PARTITION_NONE &&
        !pkv::prefill_shape_supported(cache->dtype, cache->block_size, cache->head_size))
        return -1;
    return picks_prefill_sizes(cache->dtype, cache->block_size, cache->head_size, num_seqs, num_q_heads,
                               cache->num_kv_heads, max_q_len, partition_tokens)
               ? 1
               : 0;
}

size_t pkv_multi_token_step_workspace_bytes(int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads,
                                            int32_t head_size, int32_t max_q_len, int32_t max_blocks_per_seq,
                                            int32_t block_size, int32_t partition_tokens)
{
    if (num_kv_heads <= 0 || max_q_len <= 0 || num_q_heads % num_kv_heads != 0)
        return 0;
    const size_t attn = pkv_multi_token_workspace_bytes(num_seqs, num_q_heads, num_kv_heads, head_size, max_q_len,
                                                        max_blocks_per_seq, block_size, partition_tokens);
    if (partition_tokens != PKV_PARTITION_NONE &&
        pkv_decode_partition_tokens(num_seqs, num_q_heads, num_kv_heads, head_size, max_blocks_per_seq, block_size,
                                    partition_tokens) <= 0)
        return attn;
    const size_t sb = pkv_decode_schedule_bytes(num_seqs, max_blocks_per_seq);
    return sb == 0 ? attn : round_up(attn, 256) + sb;
}

pkv_status paged_multi_token_step(const void* q, const void* new_k, const void* new_v, void* k_cache,
                                  void* v_cache, const int32_t* q_start, int32_t num_q_rows, int32_t max_q_len,
                                  const int32_t* block_tables, const int32_t* seq_lens, int32_t num_seqs,
                                  int32_t num_q_heads, int32_t max_blocks_per_seq, const pkv_cache_desc* cache,
                                  float scale, void* out, int64_t* slot_mapping, void* workspace,
                                  size_t workspace_bytes, int32_t partition_tokens, void* stream)
{
    // every argument is checked before the first launch, so a rejected call
    // changes nothing
    pkv::DecodeArgs a;
    bool nothing_to_do;
    pkv_status st = multi_token_args(q, q_start, num_q_rows, max_q_len, k_cache, v_cache, block_tables, seq_lens,
                                     num_seqs, num_q_heads, max_blocks_per_seq, cache, scale, out, workspace,
                                     workspace_bytes, partition_tokens, a, nothing_to_do);
    if (st != PKV_OK || nothing_to_do)
        return st;
    if (!new_k || !new_v || !slot_mapping || !aligned16(new_k) || !aligned16(new_v))
        return PKV_ERR_INVALID_ARG;
    if (num_seqs > 65535)
        return PKV_ERR_UNSUPPORTED;
    // With room for it (pkv_multi_token_step_workspace_bytes), the slot
    // mapping launch writes the longest-first schedule after the attention
    // partials and the attention launch reads it (either kernel); a
    // workspace of pkv_multi_token_workspace_bytes runs the same step
    // without it.
    pkv::AppendArgs::Schedule sched = {};
    const size_t attn = partition_tokens == PKV_PARTITION_NONE
                            ? 0
                            : pkv_multi_token_workspace_bytes(num_seqs, num_q_heads, cache->num_kv_heads,
                                                              cache->head_size, max_q_len, max_blocks_per_seq,
                                                              cache->block_size, partition_tokens);
    const size_t sb = pkv_decode_schedule_bytes(num_seqs, max_blocks_per_seq);
    if (sb > 0 && workspace && workspace_bytes >= round_up(attn, 256) + sb) {
        sched = schedule_parts((char*)workspace + round_up(attn, 256), num_seqs, max_blocks_per_seq,
                               cache->block_size);
        use_schedule(a, sched, partition_tokens);
    }
    st = hip_status(pkv::launch_multi_token_slot_mapping(block_tables, seq_lens, q_start, num_seqs, num_q_rows,
                                                         max_q_len, max_blocks_per_seq, cache->block_size,
                                                         slot_mapping, sched, (hipStream_t)stream));
    if (st != PKV_OK)
        return st;
    const pkv::AppendArgs ap = append_args(new_k, new_v, nullptr, block_tables, seq_lens, max_blocks_per_seq,
                                           num_q_rows, cache, k_cache, v_cache);
    st = hip_status(pkv::launch_multi_token_append(ap, q_start, num_seqs, num_q_rows, max_q_len, (hipStream_t)stream));
    if (st != PKV_OK)
        return st;
    return hip_status(launch_multi_token(a, partition_tokens, (hipStream_t)stream));
}

pkv_status paged_decode_step(const void* q, const void* new_k, const void* new_v, void* k_cache, void* v_cache,
                             const int32_t* block_tables, const int32_t* seq_lens, int32_t num_seqs,
                             int32_t num_q_heads, int32_t max_blocks_per_seq, const pkv_cache_desc* cache,
                             float scale, void* out, int64_t* slot_mapping, void* workspace,
                             size_t workspace_bytes, int32_t partition_tokens, void* stream)
{
    // every argument is checked before the append, so a rejected call
    // changes nothing
    pkv::DecodeArgs a;
    bool nothing_to_do;
    pkv_status st = attention_args(q, k_cache, v_cache, block_tables, seq_lens, num_seqs, num_q_heads,
                                   max_blocks_per_seq, cache, scale, out, workspace, workspace_bytes,
                                   partition_tokens, a, nothing_to_do);
    if (st != PKV_OK || nothing_to_do)
        return st;
    if (!new_k || !new_v || !aligned16(new_k) || !aligned16(new_v))
        return PKV_ERR_INVALID_ARG;
    const size_t need = pkv_decode_step_workspace_bytes(num_seqs, num_q_heads, cache->num_kv_heads,
                                                        cache->head_size, max_blocks_per_seq, cache->block_size,
                                                        partition_tokens);
    if (need > 0 && (!workspace || workspace_bytes < need || !aligned16(workspace)))
        return PKV_ERR_WORKSPACE;
    if (num_seqs <= pkv::kLptMaxSeqs) {
        // one launch: the attention ranks the batch itself and takes the new
        // tokens from new_k / new_v, and work-groups after its own store them
        // (plus the chunk merge launch, where there is one)
        const pkv::AppendArgs ap = append_args(new_k, new_v, slot_mapping, block_tables, seq_lens, max_blocks_per_seq,
                                               num_seqs, cache, k_cache, v_cache);
        const int32_t chunks = cache->num_kv_heads * cache->head_size / (16 / ap.elem_bytes);  // 16-byte key chunks
        a.step_append = {new_k, new_v, k_cache, v_cache, slot_mapping,
                         (chunks + pkv::kStoreThreads - 1) / pkv::kStoreThreads, ap.k_inv_scale, ap.v_inv_scale};
        return hip_status(pkv::launch_decode(a, (hipStream_t)stream));
    }
    // the append launch writes the longest-first schedule after the
    // attention partials; the attention launch reads it
    pkv::AppendArgs::Schedule sched = {};
    if (pkv_decode_schedule_bytes(num_seqs, max_blocks_per_seq) > 0) {
        const size_t attn = pkv_decode_workspace_bytes(num_seqs, num_q_heads, cache->num_kv_heads,
                                                       cache->head_size, max_blocks_per_seq, cache->block_size,
                                                       partition_tokens);
        sched = schedule_parts((char*)workspace + round_up(attn, 256), num_seqs, max_blocks_per_seq,
                               cache->block_size);
        use_schedule(a, sched, partition_tokens);
    }
    st = append_common(new_k, new_v, slot_mapping, block_tables, seq_lens, max_blocks_per_seq, num_seqs, cache,
                       k_cache, v_cache, stream, sched);
    if (st != PKV_OK)
        return st;
    return hip_status(pkv::launch_decode(a, (hipStream_t)stream));
}

}  // extern "C"

namespace {

// Workspace of paged_decode_step_static: a file-scope device array, one copy
// per GPU (each at its own address), held until the process ends.  In host
// code the name `scratch` is only a stand-in for the symbol: its device
// address comes from hipGetSymbolAddress, called once per device with that
// device current, and only that address is ever handed to a kernel.
static __device__ __align__(256) unsigned char scratch[PKV_STATIC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::atomic<void*> g_scratch_ptr[kMaxDevices];
std::mutex g_scratch_mutex;

// The current device's copy of `scratch` (looked up on the first call on
// each device).
pkv_status device_scratch(void** ptr)
{
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess)
        return hip_status(e);
    if (dev < 0 || dev >= kMaxDevices)
        return PKV_ERR_UNSUPPORTED;
    void* p = g_scratch_ptr[dev].load(std::memory_order_acquire);
    if (!p) {
        std::lock_guard<std::mutex> lock(g_scratch_mutex);
        p = g_scratch_ptr[dev].load(std::memory_order_relaxed);
        if (!p) {
            e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
            if (e != hipSuccess)
                return hip_status(e);
            if (!p)
                return PKV_ERR_HIP;
            g_scratch_ptr[dev].store(p, std::memory_order_release);
        }
    }
    *ptr = p;
    return PKV_OK;
}

}  // namespace

extern "C" {

pkv_status paged_decode_step_static(const void* q, const void* new_k, const void* new_v, void* k_cache,
                                    void* v_cache, const int32_t* block_tables, const int32_t* seq_lens,
                                    int32_t num_seqs, int32_t num_q_heads, int32_t max_blocks_per_seq,
                                    const pkv_cache_desc* cache, float scale, void* out, int64_t* slot_mapping,
                                    int32_t partition_tokens, void* stream)
{
    // the sizes are checked here only as far as the workspace needs them;
    // paged_decode_step checks everything else before its first launch
    if (num_seqs < 0 || num_q_heads <= 0 || max_blocks_per_seq <= 0)
        return PKV_ERR_INVALID_ARG;
    const pkv_status st = check_cache(cache);
    if (st != PKV_OK)
        return st;
    const size_t need = pkv_decode_step_workspace_bytes(num_seqs, num_q_heads, cache->num_kv_heads,
                                                        cache->head_size, max_blocks_per_seq, cache->block_size,
                                                        partition_tokens);
    if (need > PKV_STATIC_SCRATCH_BYTES)
        return PKV_ERR_WORKSPACE;
    void* ws = nullptr;
    if (need > 0) {
        const pkv_status ss = device_scratch(&ws);
        if (ss != PKV_OK)
            return ss;
    }
    // nothing in the step needs the workspace cleared: the append launch
    // writes the whole schedule and each chunk partial is written before the
    // merge reads it
    return paged_decode_step(q, new_k, new_v, k_cache, v_cache, block_tables, seq_lens, num_seqs, num_q_heads,
                             max_blocks_per_seq, cache, scale, out, slot_mapping, ws, need > 0 ? need : 0,
                             partition_tokens, stream);
}

pkv_status pkv_copy_blocks(const int32_t* pairs, int32_t num_pairs, const pkv_cache_desc* cache, void* k_cache,
                           void* v_cache, void* stream)
{
    if (num_pairs < 0)
        return PKV_ERR_INVALID_ARG;
    const pkv_status st = check_cache(cache);
    if (st != PKV_OK)
        return st;
    if (!k_cache || !v_cache || !aligned16(k_cache) || !aligned16(v_cache))
        return PKV_ERR_INVALID_ARG;
    if (num_pairs == 0)
        return PKV_OK;
    if (!pairs)
        return PKV_ERR_INVALID_ARG;
    if (num_pairs > INT32_MAX / 2)
        return PKV_ERR_UNSUPPORTED;
    const int64_t block_bytes =
        (int64_t)cache->num_kv_heads * cache->block_size * cache->head_size * elem_bytes(cache->dtype);
    return hip_status(pkv::launch_copy_blocks(pairs, num_pairs, cache->num_blocks, block_bytes, k_cache, v_cache,
                                              (hipStream_t)stream));
}

pkv_status pkv_validate(const int32_t* block_tables, const int32_t* seq_lens, int32_t num_seqs,
                        int32_t max_blocks_per_seq, const int64_t* slot_mapping, int32_t num_tokens,
                        const int32_t* ref_counts, const pkv_cache_desc* cache, pkv_validate_report* report,
                        void* stream)
{
    if (!report || ((uintptr_t)report & 7u) != 0 || num_seqs < 0 || max_blocks_per_seq <= 0)
        return PKV_ERR_INVALID_ARG;
    const pkv_status st = check_cache(cache);
    if (st != PKV_OK)
        return st;
    if (num_seqs > 0 && (!block_tables || !seq_lens))
        return PKV_ERR_INVALID_ARG;
    if (slot_mapping && num_tokens < 0)
        return PKV_ERR_INVALID_ARG;
    return hip_status(pkv::launch_validate(block_tables, seq_lens, num_seqs, max_blocks_per_seq, slot_mapping,
                                           slot_mapping ? num_tokens : 0, ref_counts, cache->block_size,
                                           cache->num_blocks, report, (hipStream_t)stream));
}

pkv_status pkv_probe_stream_read(const void* buf, size_t bytes, void* out, int32_t work_groups, void* stream)
{
    if (!buf || !out || !aligned16(buf) || bytes % 16 != 0 || work_groups < 1 || work_groups > (1 << 20))
        return PKV_ERR_INVALID_ARG;
    if (bytes == 0)
        return PKV_OK;
    return hip_status(pkv::launch_stream_read(buf, bytes, out, work_groups, (hipStream_t)stream));
}

pkv_status pkv_probe_gather_read(const void* buf0, size_t bytes0, const void* buf1, size_t bytes1,
                                 const int64_t* tile_offsets, int64_t num_tiles, int32_t tile_bytes, void* out,
                                 int32_t work_groups, void* stream)
{
    if (!buf0 || !buf1 || !out || !aligned16(buf0) || !aligned16(buf1) || num_tiles < 0 ||
        work_groups < 1 || work_groups > (1 << 20) || tile_bytes < 1024 || tile_bytes > (1 << 20) ||
        tile_bytes % 1024 != 0 || (num_tiles > 0 && !tile_offsets))
        return PKV_ERR_INVALID_ARG;
    if (num_tiles == 0)
        return PKV_OK;
    return hip_status(pkv::launch_gather_read(buf0, bytes0, buf1, bytes1, tile_offsets, num_tiles, tile_bytes, out,
                                              work_groups, (hipStream_t)stream));
}

}  // extern "C"
