// Decode-step slot mapping and the KV append kernels.
//
// Slot arithmetic and the per-token store are in kv_store.h (the "writing
// new K/V" section of the "cache structure" page).
#include <type_traits>

#include "kv_store.h"
#include "pkv_internal.h"

namespace pkv {

__global__ void decode_slot_mapping_kernel(const int32_t* __restrict__ block_tables,
                                           const int32_t* __restrict__ seq_lens, int32_t num_seqs,
                                           int32_t max_blocks_per_seq, int32_t block_size,
                                           int64_t* __restrict__ slot_mapping)
{
    const int32_t s = blockIdx.x * blockDim.x + threadIdx.x;
    if (s < num_seqs)
        slot_mapping[s] = decode_slot(block_tables, seq_lens, s, max_blocks_per_seq, block_size);
}


constexpr int kAppendThreads = kStoreThreads;

// Longest-first schedule of a decode batch (written by the decode step's
// append launch, read by its attention launch): sequence i goes to rank
//   y = #{ j : blocks(j) > blocks(i), or blocks(j) == blocks(i) and j < i },
// a permutation of 0..S-1 (blocks = ceil(clamped length / B)).  The
// work-group of sequence i writes order[y] = i, lens[y] = seq_lens[i] and
// copies its block-table row to tables[y], so that an attention work-group
// finds its sequence, length and row from y alone, with no dependent load.
// It also places its chunks (of the default partitioning) in the chunk list
// (see write_schedule), so that the attention launch starts the largest
// chunks first.
//
// The loads (every length, the row) do not depend on the rank, so they are
// issued when the work-group starts, together with the token's loads; the
// first kSchedRegs * 256 lengths and row entries are held in registers and
// the rest, if any, read at the end.
constexpr int kSchedRegs = 4;

struct SchedulePrefetch {
    int32_t len[kSchedRegs];
    int32_t row[kSchedRegs];
};

__device__ __forceinline__ void prefetch_schedule(SchedulePrefetch& p, int32_t i, int32_t S,
                                                  const int32_t* __restrict__ seq_lens,
                                                  const int32_t* __restrict__ block_tables, int32_t M)
{
    const int32_t* src = block_tables + (int64_t)i * M;
#pragma unroll
    for (int t = 0; t < kSchedRegs; ++t) {
        const int j = threadIdx.x + t * kAppendThreads;
        p.len[t] = j < S ? seq_lens[j] : 0;
        p.row[t] = j < M ? src[j] : 0;
    }
}

__device__ void write_schedule(const SchedulePrefetch& p, int32_t i, int32_t S,
                               const int32_t* __restrict__ seq_lens, const int32_t* __restrict__ block_tables,
                               int32_t M, int32_t B, const AppendArgs::Schedule& sc)
{
    constexpr int NW = kAppendThreads / 64;
    __shared__ int sm_part[6][NW];
    const int64_t cap = (int64_t)M * B;
    auto blocks_of = [&](int32_t L) {
        const int64_t Lc = L < 0 ? 0 : (L > cap ? cap : L);
        return (Lc + B - 1) / B;
    };
    // Chunks of the default partitioning: floor(k / CB) full chunks of CB
    // blocks and, when blocks remain (or the sequence is empty: its zero
    // output is written by the work-group of its one chunk), one partial
    // chunk of k % CB blocks.  The chunk list is ordered by decreasing size
    // (longest processing time first): every full chunk, by sequence index,
    // then the partial chunks by decreasing size, ties by sequence index.
    const int64_t CB = sc.chunk_blocks;
    const int32_t Li = seq_lens[i];
    const int64_t ki = blocks_of(Li);
    const int64_t full_i = ki / CB, rem_i = ki % CB;
    const bool part_i = rem_i > 0 || ki == 0;
    int acc[6] = {0, 0, 0, 0, 0, 0};  // rank, full before, full all, larger partials, equal partials before, chunks
    auto count = [&](int j, int32_t Lj) __attribute__((always_inline)) {
        const int64_t kj = blocks_of(Lj);
        const int64_t fj = kj / CB, rj = kj % CB;
        const bool pj = rj > 0 || kj == 0;
        acc[0] += (kj > ki || (kj == ki && j < i)) ? 1 : 0;
        acc[1] += j < i ? (int)fj : 0;
        acc[2] += (int)fj;
        acc[3] += (pj && rj > rem_i) ? 1 : 0;
        acc[4] += (pj && rj == rem_i && j < i) ? 1 : 0;
        acc[5] += (int)fj + (pj ? 1 : 0);
    };
#pragma unroll
    for (int t = 0; t < kSchedRegs; ++t) {
        const int j = threadIdx.x + t * kAppendThreads;
        if (j < S)
            count(j, p.len[t]);
    }
    for (int j = threadIdx.x + kSchedRegs * kAppendThreads; j < S; j += kAppendThreads)
        count(j, seq_lens[j]);
#pragma unroll
    for (int a = 0; a < 6; ++a) {
#pragma unroll
        for (int o = 32; o > 0; o >>= 1)
            acc[a] += __shfl_xor(acc[a], o);
        if ((threadIdx.x & 63) == 0)
            sm_part[a][threadIdx.x >> 6] = acc[a];
    }
    __syncthreads();
    int tot[6] = {0, 0, 0, 0, 0, 0};
#pragma unroll
    for (int a = 0; a < 6; ++a)
#pragma unroll
        for (int k = 0; k < NW; ++k)
            tot[a] += sm_part[a][k];
    const int y = tot[0];
    uint2* items = reinterpret_cast<uint2*>(sc.items);
    for (int c = threadIdx.x; c < (int)full_i; c += kAppendThreads) {
        uint2 it;
        it.x = (uint32_t)y | ((uint32_t)c << 16);
        it.y = (uint32_t)i;
        items[tot[1] + c] = it;
    }
    if (threadIdx.x == 0 && part_i) {
        uint2 it;
        it.x = (uint32_t)y | ((uint32_t)full_i << 16);
        it.y = (uint32_t)i;
        items[tot[2] + tot[3] + tot[4]] = it;
    }
    if (threadIdx.x == 0 && i == 0)
        *sc.count = tot[5];
    int32_t* __restrict__ order = sc.order;
    int32_t* __restrict__ lens = sc.lens;
    int32_t* __restrict__ tables = sc.tables;
    if (threadIdx.x == 0) {
        order[y] = i;
        lens[y] = Li;
    }
    int32_t* dst = tables + (int64_t)y * M;
#pragma unroll
    for (int t = 0; t < kSchedRegs; ++t) {
        const int m = threadIdx.x + t * kAppendThreads;
        if (m < M)
            dst[m] = p.row[t];
    }
    // the rest of a long row: four independent loads in flight per thread
    const int32_t* src = block_tables + (int64_t)i * M;
    for (int m0 = threadIdx.x + kSchedRegs * kAppendThreads; m0 < M; m0 += 4 * kAppendThreads) {
        int32_t v[4];
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            const int m = m0 + k * kAppendThreads;
            v[k] = m < M ? src[m] : 0;
        }
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            const int m = m0 + k * kAppendThreads;
            if (m < M)
                dst[m] = v[k];
        }
    }
}

// Slots of the query rows of a multi-token call: row i of sequence s (n
// rows) holds position L - n + i; rows outside 0 .. L - 1 or past the table
// row get -1.  One work-group per sequence.  With sched.order set (multi-token
// step), each work-group also writes its sequence's entry of the
// longest-first schedule (write_schedule), whatever its rows.
__global__ __launch_bounds__(kAppendThreads) void multi_token_slot_mapping_kernel(
    const int32_t* __restrict__ block_tables, const int32_t* __restrict__ seq_lens,
    const int32_t* __restrict__ q_start, int32_t num_q_rows, int32_t max_q_len, int32_t max_blocks_per_seq,
    int32_t block_size, int64_t* __restrict__ slot_mapping, AppendArgs::Schedule sched)
{
    const int32_t s = blockIdx.x;
    const bool sched_wg = sched.order != nullptr;
    SchedulePrefetch pre;
    if (sched_wg)
        prefetch_schedule(pre, s, gridDim.x, seq_lens, block_tables, max_blocks_per_seq);
    const int32_t qs0 = q_start[s];
    const int32_t qs1 = q_start[s + 1];
    int32_t n = qs1 - qs0;
    if (qs0 < 0 || n < 0 || qs1 > num_q_rows)
        n = 0;  // rows of no valid range: none written
    n = n < max_q_len ? n : max_q_len;
    const int32_t L = seq_lens[s];
    for (int32_t i = threadIdx.x; i < n; i += blockDim.x) {
        const int64_t pos = (int64_t)L - n + i;
        const int64_t idx = pos >= 0 ? pos / block_size : -1;
        int64_t slot = -1;
        if (pos >= 0 && pos < L && idx < max_blocks_per_seq) {
            const int64_t block = block_tables[(int64_t)s * max_blocks_per_seq + idx];
            slot = block < 0 ? -1 : block * block_size + (pos - idx * block_size);
        }
        slot_mapping[qs0 + i] = slot;
    }
    if (sched_wg)
        write_schedule(pre, s, gridDim.x, seq_lens, block_tables, max_blocks_per_seq, block_size, sched);
}

// Token i = blockIdx.x, part blockIdx.y of its K/V (store_token).
// FROM_TABLE: the slot is the decode slot of sequence i (computed from
// block_tables / seq_lens and also written to slot_mapping); otherwise it is
// read from slot_mapping.  With sched.order set (decode step), the first
// work-group of each sequence also writes its entry of the longest-first
// schedule (write_schedule).
template <typename E, bool FROM_TABLE>
__global__ __launch_bounds__(kAppendThreads) void kv_append_kernel(
    const u32x4* __restrict__ k, const u32x4* __restrict__ v, int64_t* __restrict__ slot_mapping,
    const int32_t* __restrict__ block_tables, const int32_t* __restrict__ seq_lens, int32_t max_blocks_per_seq,
    u32x4* __restrict__ k_cache, E* __restrict__ v_cache, int32_t num_kv_heads, int32_t head_size,
    int32_t block_size, int32_t num_blocks, AppendArgs::Schedule sched, float k_inv_scale, float v_inv_scale)
{
    const int32_t i = blockIdx.x;
    const bool sched_wg = FROM_TABLE && sched.order && blockIdx.y == 0;  // uniform per work-group
    SchedulePrefetch pre;
    if (sched_wg)
        prefetch_schedule(pre, i, gridDim.x, seq_lens, block_tables, max_blocks_per_seq);
    store_token<E, FROM_TABLE>(i, blockIdx.y, k, v, slot_mapping, block_tables, seq_lens, max_blocks_per_seq,
                               k_cache, v_cache, num_kv_heads, head_size, block_size, num_blocks, k_inv_scale,
                               v_inv_scale);
    if (sched_wg)
        write_schedule(pre, i, gridDim.x, seq_lens, block_tables, max_blocks_per_seq, block_size, sched);
}

hipError_t launch_slot_mapping(const int32_t* block_tables, const int32_t* seq_lens, int32_t num_seqs,
                               int32_t max_blocks_per_seq, int32_t block_size, int64_t* slot_mapping,
                               hipStream_t stream)
{
    const int threads = 256;
    const int blocks = (num_seqs + threads - 1) / threads;
    hipLaunchKernelGGL(decode_slot_mapping_kernel, dim3(blocks), dim3(threads), 0, stream, block_tables,
                       seq_lens, num_seqs, max_blocks_per_seq, block_size, slot_mapping);
    return hipGetLastError();
}

hipError_t launch_multi_token_slot_mapping(const int32_t* block_tables, const int32_t* seq_lens,
                                           const int32_t* q_start, int32_t num_seqs, int32_t num_q_rows,
                                           int32_t max_q_len, int32_t max_blocks_per_seq, int32_t block_size,
                                           int64_t* slot_mapping, const AppendArgs::Schedule& sched,
                                           hipStream_t stream)
{
    hipLaunchKernelGGL(multi_token_slot_mapping_kernel, dim3(num_seqs), dim3(kAppendThreads), 0, stream,
                       block_tables, seq_lens, q_start, num_q_rows, max_q_len, max_blocks_per_seq, block_size,
                       slot_mapping, sched);
    return hipGetLastError();
}

template <typename E, bool FROM_TABLE>
static void launch_append_typed(const AppendArgs& a, dim3 grid, dim3 block, hipStream_t stream)
{
    hipLaunchKernelGGL((kv_append_kernel<E, FROM_TABLE>), grid, block, 0, stream, (const u32x4*)a.k,
                       (const u32x4*)a.v, a.slot_mapping, a.block_tables, a.seq_lens, a.max_blocks_per_seq,
                       (u32x4*)a.k_cache, (E*)a.v_cache, a.num_kv_heads, a.head_size, a.block_size, a.num_blocks,
                       a.sched, a.k_inv_scale, a.v_inv_scale);
}

template <bool FROM_TABLE>
static hipError_t launch_append_impl(const AppendArgs& a, hipStream_t stream)
{
    const int32_t nchunks = a.num_kv_heads * a.head_size / (16 / a.elem_bytes);
    const dim3 grid(a.num_tokens, (nchunks + kAppendThreads - 1) / kAppendThreads), block(kAppendThreads);
    if (a.elem_bytes == 1)
        launch_append_typed<uint8_t, FROM_TABLE>(a, grid, block, stream);
    else if (a.elem_bytes == 2)
        launch_append_typed<uint16_t, FROM_TABLE>(a, grid, block, stream);
    else
        launch_append_typed<uint32_t, FROM_TABLE>(a, grid, block, stream);
    return hipGetLastError();
}

hipError_t launch_append(const AppendArgs& a, hipStream_t stream)
{
    return a.block_tables ? launch_append_impl<true>(a, stream) : launch_append_impl<false>(a, stream);
}

// Append of the query rows of a multi-token call, block by block.  The rows
// of sequence s are its last n tokens (positions L - n .. L - 1), so the
// rows that land in one block are consecutive slots of it: work-group
// (segment g, KV head h, sequence s) writes the rows of the g-th block they
// touch.  Keys go out as 16-byte chunks, consecutive tokens side by side in
// a chunk row; values are staged through LDS ([token][hs], rows read whole)
// and written along the block's [hs][B] rows, consecutive tokens side by
// side, instead of one scattered element per token.  The slots are those of
// pkv_multi_token_slot_mapping and the bytes those of kv_cache_append
// (FP8: the same quantize16 / single-code conversion).  Rows whose position
// is negative, past the table row or in a block outside the pool are
// skipped.
template <typename E>
__global__ __launch_bounds__(kAppendThreads) void multi_token_append_kernel(
    const uint8_t* __restrict__ k, const uint8_t* __restrict__ v, const int32_t* __restrict__ block_tables,
    const int32_t* __restrict__ seq_lens, const int32_t* __restrict__ q_start, int32_t num_q_rows,
    int32_t max_q_len, int32_t M, u32x4* __restrict__ k_cache, E* __restrict__ v_cache, int32_t Hkv,
    int32_t hs, int32_t B, int32_t num_blocks, float k_inv_scale, float v_inv_scale)
{
    constexpr bool Q8 = sizeof(E) == 1;
    constexpr int X = 16 / sizeof(E);             // pool elements per 16-byte chunk
    constexpr int IB = Q8 ? 2 : (int)sizeof(E);    // input bytes per element (bf16 for FP8 pools)
    extern __shared__ __attribute__((aligned(16))) uint8_t vs_raw[];  // [B][hs * IB + 4]
    const int g = blockIdx.x, h = blockIdx.y, s = blockIdx.z;
    const int qs0 = q_start[s], qs1 = q_start[s + 1];
    int n = qs1 - qs0;
    if (qs0 < 0 || n < 0 || qs1 > num_q_rows)
        return;
    n = n < max_q_len ? n : max_q_len;
    const int L = seq_lens[s];
    const int P0 = L - n;  // position of row 0
    const int first = P0 > 0 ? P0 : 0;
    const int b = first / B + g;  // table index of this segment's block
    const int seg0 = b * B > first ? b * B : first;
    const int seg1 = (b + 1) * B < L ? (b + 1) * B : L;
    if (n <= 0 || seg0 >= seg1 || b >= M)
        return;
    const int64_t id = block_tables[(int64_t)s * M + b];
    if (id < 0 || id >= num_blocks)
        return;
    const int cnt = seg1 - seg0, off0 = seg0 - b * B;
    const int64_t row0 = qs0 + (seg0 - P0);
    const int64_t in_row = (int64_t)Hkv * hs * IB;  // bytes of one input row
    const int CH = hs / X;                          // key chunks per head
    const int row_bytes = hs * IB + 4;              // LDS row, padded

    // keys: chunk f of token j, token fastest
    for (int it = threadIdx.x; it < CH * cnt; it += kAppendThreads) {
        const int f = it / cnt, j = it - f * cnt;
        const uint8_t* src = k + (row0 + j) * in_row + ((int64_t)h * hs + (int64_t)f * X) * IB;
        u32x4 val;
        if constexpr (Q8) {
            const u32x4 in[2] = {*(const u32x4*)src, *(const u32x4*)(src + 16)};
            val = quantize16(in, k_inv_scale);
        } else {
            val = *(const u32x4*)src;
        }
        __builtin_nontemporal_store(val, &k_cache[((id * Hkv + h) * CH + f) * B + off0 + j]);
    }
    // values: stage the rows, then write along the block rows
    const int pieces = hs * IB / 16;
    for (int it = threadIdx.x; it < cnt * pieces; it += kAppendThreads) {
        const int j = it / pieces, pc = it - j * pieces;
        const u32x4 val = *(const u32x4*)(v + (row0 + j) * in_row + (int64_t)h * hs * IB + pc * 16);
        uint32_t* dst = (uint32_t*)(vs_raw + j * row_bytes + pc * 16);
        dst[0] = val[0];
        dst[1] = val[1];
        dst[2] = val[2];
        dst[3] = val[3];
    }
    __syncthreads();
    E* vdst = v_cache + (id * Hkv + h) * (int64_t)hs * B + off0;
    for (int it = threadIdx.x; it < hs * cnt; it += kAppendThreads) {
        const int d = it / cnt, j = it - d * cnt;
        const uint8_t* e = vs_raw + j * row_bytes + d * IB;
        E out;
        if constexpr (Q8)
            out = quantize1(*(const uint16_t*)e, v_inv_scale);
        else
            out = *(const E*)e;
        __builtin_nontemporal_store(out, &vdst[(int64_t)d * B + j]);
    }
}

hipError_t launch_multi_token_append(const AppendArgs& a, const int32_t* q_start, int32_t num_seqs, int32_t num_q_rows,
                                     int32_t max_q_len, hipStream_t stream)
{
    // segments: the blocks max_q_len consecutive positions can touch
    const int segs = (max_q_len + a.block_size - 1) / a.block_size + 1;
    const dim3 grid(segs, a.num_kv_heads, num_seqs);
    const int ib = a.elem_bytes == 1 ? 2 : a.elem_bytes;
    const size_t lds = (size_t)a.block_size * (a.head_size * ib + 4);
    switch (a.elem_bytes) {
    case 1:
        hipLaunchKernelGGL(multi_token_append_kernel<uint8_t>, grid, dim3(kAppendThreads), lds, stream,
                           (const uint8_t*)a.k, (const uint8_t*)a.v, a.block_tables, a.seq_lens, q_start, num_q_rows,
                           max_q_len, a.max_blocks_per_seq, (u32x4*)a.k_cache, (uint8_t*)a.v_cache, a.num_kv_heads,
                           a.head_size, a.block_size, a.num_blocks, a.k_inv_scale, a.v_inv_scale);
        break;
    case 2:
        hipLaunchKernelGGL(multi_token_append_kernel<uint16_t>, grid, dim3(kAppendThreads), lds, stream,
                           (const uint8_t*)a.k, (const uint8_t*)a.v, a.block_tables, a.seq_lens, q_start, num_q_rows,
                           max_q_len, a.max_blocks_per_seq, (u32x4*)a.k_cache, (uint16_t*)a.v_cache, a.num_kv_heads,
                           a.head_size, a.block_size, a.num_blocks, a.k_inv_scale, a.v_inv_scale);
        break;
    default:
        hipLaunchKernelGGL(multi_token_append_kernel<uint32_t>, grid, dim3(kAppendThreads), lds, stream,
                           (const uint8_t*)a.k, (const uint8_t*)a.v, a.block_tables, a.seq_lens, q_start, num_q_rows,
                           max_q_len, a.max_blocks_per_seq, (u32x4*)a.k_cache, (uint32_t*)a.v_cache, a.num_kv_heads,
                           a.head_size, a.block_size, a.num_blocks, a.k_inv_scale, a.v_inv_scale);
    }
    return hipGetLastError();
}

}  // namespace pkv
