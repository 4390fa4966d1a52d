// Decode-step slot mapping and the KV append kernel.
//
// Slot arithmetic follows the "writing new K/V" section of the "cache
// structure" page: slot = block_id * B + offset, split back by the cache
// write as block_id = slot / B and offset = slot % B.  The copy is bit-exact
// (16-byte moves for keys, element moves for values; no float arithmetic).
#include "pkv_internal.h"

namespace pkv {

// One thread per sequence: the new token sits at position L - 1.
__global__ void decode_slot_mapping_kernel(const int32_t* __restrict__ block_tables,
                                           const int32_t* __restrict__ seq_lens, int32_t num_seqs,
                                           int32_t max_blocks_per_seq, int32_t block_size,
                                           int64_t* __restrict__ slot_mapping)
{
    const int32_t s = blockIdx.x * blockDim.x + threadIdx.x;
    if (s >= num_seqs)
        return;
    const int32_t L = seq_lens[s];
    int64_t slot = -1;
    if (L > 0) {
        const int32_t pos = L - 1;
        const int32_t idx = pos / block_size;
        if (idx < max_blocks_per_seq) {
            const int64_t block = block_tables[(int64_t)s * max_blocks_per_seq + idx];
            if (block >= 0)
                slot = block * block_size + (pos - idx * block_size);
        }
    }
    slot_mapping[s] = slot;
}

// One work-group per new token.  Keys move in 16-byte chunks: chunk f of KV
// head h is the x elements [f*x, f*x + x) of the head vector and lands at
// ((b*Hkv + h)*(hs/x) + f)*B*x + off*x.  Values are read in 16-byte chunks
// and scattered one element per head dim to ((b*Hkv + h)*hs + d)*B + off.
template <typename E>
__global__ __launch_bounds__(256) void kv_append_kernel(const uint4* __restrict__ k, const uint4* __restrict__ v,
                                                        const int64_t* __restrict__ slot_mapping,
                                                        uint4* __restrict__ k_cache, E* __restrict__ v_cache,
                                                        int32_t num_kv_heads, int32_t head_size,
                                                        int32_t block_size, int32_t num_blocks)
{
    constexpr int X = 16 / sizeof(E);
    const int32_t i = blockIdx.x;
    const int64_t slot = slot_mapping[i];
    if (slot < 0)
        return;
    const int64_t b = slot / block_size;
    const int32_t off = (int32_t)(slot - b * block_size);
    if (b >= num_blocks)
        return;  // out-of-range slot: skipped, never written
    const int32_t chunks_per_head = head_size / X;
    const int32_t nchunks = num_kv_heads * chunks_per_head;
    const uint4* ksrc = k + (int64_t)i * nchunks;
    const uint4* vsrc = v + (int64_t)i * nchunks;
    for (int32_t ci = threadIdx.x; ci < nchunks; ci += blockDim.x) {
        const int32_t h = ci / chunks_per_head;
        const int32_t f = ci - h * chunks_per_head;
        // key: one 16-byte chunk per thread
        const int64_t kdst = ((b * num_kv_heads + h) * chunks_per_head + f) * block_size + off;
        k_cache[kdst] = ksrc[ci];
        // value: X consecutive head dims, block_size elements apart in the pool
        union {
            uint4 u;
            E e[X];
        } val;
        val.u = vsrc[ci];
        E* vdst = v_cache + ((b * num_kv_heads + h) * head_size + (int64_t)f * X) * block_size + off;
#pragma unroll
        for (int e = 0; e < X; ++e)
            vdst[(int64_t)e * block_size] = val.e[e];
    }
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

hipError_t launch_append(const AppendArgs& a, hipStream_t stream)
{
    const dim3 grid(a.num_tokens), block(256);
    if (a.elem_bytes == 2)
        hipLaunchKernelGGL(kv_append_kernel<uint16_t>, grid, block, 0, stream, (const uint4*)a.k,
                           (const uint4*)a.v, a.slot_mapping, (uint4*)a.k_cache, (uint16_t*)a.v_cache,
                           a.num_kv_heads, a.head_size, a.block_size, a.num_blocks);
    else
        hipLaunchKernelGGL(kv_append_kernel<uint32_t>, grid, block, 0, stream, (const uint4*)a.k,
                           (const uint4*)a.v, a.slot_mapping, (uint4*)a.k_cache, (uint32_t*)a.v_cache,
                           a.num_kv_heads, a.head_size, a.block_size, a.num_blocks);
    return hipGetLastError();
}

}  // namespace pkv
