// Internal launch interface between the C-ABI entry points (api.hip) and
// the kernel translation units.  Not part of the public ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace pkv {

// Waves per work-group of the partition kernel: each wave attends over one
// context partition and the work-group merges its NW partitions, so one
// work-group covers a chunk of NW partitions.
constexpr int kDecodeWaves = 4;

// A stand-alone attention call on up to this many sequences is scheduled
// longest first by the attention kernel itself (each work-group ranks all
// lengths: O(S^2 / threads) work, which outweighs the gain on larger batches).
constexpr int kLptMaxSeqs = 64;
constexpr int kStoreThreads = 256;  // threads of a work-group that stores new tokens (kv_store.h)
// The decode step's append launch writes a longest-first schedule for
// batches of up to this many sequences (each of its work-groups reads all
// lengths once).
constexpr int kScheduleMaxSeqs = 4096;

// Problem description shared by the decode launchers; every field has been
// validated on the host before a launcher sees it.
struct DecodeArgs {
    const void* q;
    const void* k_cache;
    const void* v_cache;
    const int32_t* block_tables;
    const int32_t* seq_lens;
    void* out;
    int32_t out_f32;  // bf16 queries: 1 = out holds fp32 (the value before rounding to bf16)
    // Longest-first schedule written by the decode step's append launch (all
    // null otherwise): work-group row y attends sequence order[y], whose
    // length and table row are lens[y] and tables[y].
    const int32_t* sched_order;
    const int32_t* sched_lens;
    const int32_t* sched_tables;
    // With the schedule's chunk list (default partitioning only): one
    // work-group per listed chunk and KV head, all chunks of the longest
    // sequence first (null: one work-group per (KV head, rank, chunk)).
    const int32_t* sched_count;
    const uint32_t* sched_items;
    // Several query tokens per sequence (null: one each, row s): rows
    // q_start[s] .. q_start[s+1]-1 of q and out, at most max_q_len of them.
    const int32_t* q_start;
    int32_t num_q_rows;  // rows of q and out
    int32_t max_q_len;
    int32_t row_tiles;   // 16-row MFMA tiles per (sequence, KV head): ceil(max_q_len * G / 16); 1 without q_start
    // fp32 chunk partials, null when max_parts == 1; rows per block RPB = G
    // (one query row per sequence) or 16 (q_start set)
    float* ws_o;    // [S][Hkv][row_tiles][max_parts][RPB][hs]
    float* ws_ml;   // [S][Hkv][row_tiles][max_parts][RPB][2] (running max in log2 units, sum)
    int32_t num_seqs;
    int32_t num_q_heads;
    int32_t num_kv_heads;
    int32_t head_size;
    int32_t block_size;
    int32_t max_blocks_per_seq;
    int32_t num_blocks;
    int32_t dtype;            // pkv_dtype
    int32_t partition_blocks; // blocks per context partition (<= 64, or <= 512 tokens of B < 16), one wave each
    int32_t max_parts;        // chunks per sequence: ceil(max_blocks_per_seq / (partition_blocks * kDecodeWaves))
    int32_t interleave;       // 1: a chunk's blocks dealt round-robin to its waves;
                              // 0: one contiguous partition per wave
    float scale;
    float k_scale, v_scale;   // FP8 pools: stored code * scale (1 otherwise)
    // Decode step in one launch (k null otherwise; one query row per
    // sequence): after the attention's work-groups come `groups` work-groups
    // per sequence that store its new token k[s], v[s] in the slot of
    // position seq_lens[s] - 1 (store_token in kv_store.h), and the attention
    // takes that token from k / v instead of the pools, which those
    // work-groups may not have written yet.
    struct StepAppend {
        const void* k;
        const void* v;
        void* k_cache;          // the pools (written)
        void* v_cache;
        int64_t* slot_mapping;  // receives the slots, or null
        int32_t groups;         // store work-groups per token
        float k_inv_scale, v_inv_scale;  // FP8 pools: code = E4M3(fp32(x * inv_scale))
    } step_append;
};

hipError_t launch_decode(const DecodeArgs& a, hipStream_t stream);

// Streaming-read probe (probe.hip): reads bytes (a multiple of 16) of buf
// with work_groups work-groups; out receives at most one 4-byte marker.
hipError_t launch_stream_read(const void* buf, size_t bytes, void* out, int32_t work_groups, hipStream_t stream);
hipError_t launch_gather_read(const void* buf0, size_t bytes0, const void* buf1, size_t bytes1,
                              const int64_t* tile_offsets, int64_t num_tiles, int32_t tile_bytes, void* out,
                              int32_t work_groups, hipStream_t stream);

// Multi-token attention with many rows per (sequence, KV head): the
// prefill kernel (prefill.hip) takes 128 rows per work-group over the whole
// visible context, no partitions and no workspace.  Supported for bf16 and
// FP8 pools with blocks of 16 tokens or more.
bool prefill_shape_supported(int32_t dtype, int32_t block_size, int32_t head_size);
bool prefill_supported(const DecodeArgs& a);
int64_t prefill_work_groups(int64_t num_seqs, int64_t num_q_heads, int64_t num_kv_heads, int64_t max_q_len);
int64_t prefill_work_groups(const DecodeArgs& a);
hipError_t launch_prefill(const DecodeArgs& a, hipStream_t stream);

struct AppendArgs {
    const void* k;
    const void* v;
    // Slots: read from slot_mapping, or (block_tables != null) computed as the
    // decode slot of each sequence and written to slot_mapping if non-null.
    int64_t* slot_mapping;
    const int32_t* block_tables;
    const int32_t* seq_lens;
    int32_t max_blocks_per_seq;
    void* k_cache;
    void* v_cache;
    int32_t num_tokens;
    int32_t num_kv_heads;
    int32_t head_size;
    int32_t block_size;
    int32_t num_blocks;
    int32_t elem_bytes;  // pool element: 1 (FP8 codes, bf16 input), 2 or 4
    float k_inv_scale, v_inv_scale;  // FP8 pools: code = E4M3(fp32(x * inv_scale))
    // Decode step only (block_tables != null): when sched.order is non-null,
    // the launch also writes the longest-first schedule of the batch.
    struct Schedule {
        int32_t* order;  // [num_tokens] sequence of rank y
        int32_t* lens;   // [num_tokens] seq_lens[order[y]]
        int32_t* tables; // [num_tokens][max_blocks_per_seq] block_tables[order[y]]
        // The chunks of the library's default partitioning (chunk_blocks
        // blocks each, the last one partial; at least one per sequence) by
        // decreasing size: items[2k] = y | (chunk << 16) with y the
        // sequence's rank, items[2k + 1] = order[y]; count = their number.
        int32_t* count;
        uint32_t* items; // [num_tokens * ceil(max_blocks_per_seq / 4)][2]
        int32_t chunk_blocks;
    } sched;
};

hipError_t launch_append(const AppendArgs& a, hipStream_t stream);

// Append of the rows of a multi-token call (a.block_tables, a.seq_lens set;
// a.slot_mapping unused): the rows landing in one block are written together.
hipError_t launch_multi_token_append(const AppendArgs& a, const int32_t* q_start, int32_t num_seqs, int32_t num_q_rows,
                                     int32_t max_q_len, hipStream_t stream);

// Copies whole blocks (block_bytes per pool) for num_pairs (src, dst) pairs.
hipError_t launch_copy_blocks(const int32_t* pairs, int32_t num_pairs, int32_t num_blocks, int64_t block_bytes,
                              void* k_cache, void* v_cache, hipStream_t stream);

// Slots of the query rows of a multi-token call: row q_start[s] + i of
// sequence s gets the slot of position L - n + i (-1 when that position is
// outside the sequence or its table row).
hipError_t launch_multi_token_slot_mapping(const int32_t* block_tables, const int32_t* seq_lens,
                                           const int32_t* q_start, int32_t num_seqs, int32_t num_q_rows,
                                           int32_t max_q_len, int32_t max_blocks_per_seq, int32_t block_size,
                                           int64_t* slot_mapping, const AppendArgs::Schedule& sched,
                                           hipStream_t stream);

// Contract check (validate.hip): fills the pkv_validate_report at report_buf.
hipError_t launch_validate(const int32_t* block_tables, const int32_t* seq_lens, int32_t num_seqs,
                           int32_t max_blocks_per_seq, const int64_t* slot_mapping, int32_t num_tokens,
                           const int32_t* ref_counts, int32_t block_size, int32_t num_blocks, void* report_buf,
                           hipStream_t stream);

hipError_t launch_slot_mapping(const int32_t* block_tables, const int32_t* seq_lens, int32_t num_seqs,
                               int32_t max_blocks_per_seq, int32_t block_size, int64_t* slot_mapping,
                               hipStream_t stream);

}  // namespace pkv
