// Debug check of the device-side contract of the attention and append
// calls: block IDs of used table entries inside the pool, lengths within the
// table, distinct slots in one append, and no slot in a block that more than
// one sequence references (the copy-on-write rule of the "PagedAttention 笔记"
// page: a shared block is read-only, a writer copies it first).  The kernels
// themselves only contain such violations; this pass reports them.  It reads
// the tables, lengths, slots and reference counts, never the pools.
#include "../../include/pkv.h"
#include "pkv_internal.h"

namespace pkv {

constexpr int kValidateThreads = 256;

// Report fields as unsigned 64-bit words for the atomics: five counts, then
// five "first offender" indices kept as minima (all ones = none = -1).
struct ReportWords {
    unsigned long long count[5];
    unsigned long long first[5];
};
static_assert(sizeof(ReportWords) == sizeof(pkv_validate_report), "report layout");
enum { kBadLen = 0, kBadBlock = 1, kBadSlot = 2, kDupSlot = 3, kSharedWrite = 4 };

__global__ void validate_init_kernel(ReportWords* __restrict__ rep)
{
    if (threadIdx.x < 5) {
        rep->count[threadIdx.x] = 0ull;
        rep->first[threadIdx.x] = ~0ull;
    }
}

// Adds the wave's offenders to field f: one atomic per wave for the count,
// one for the smallest index.
__device__ __forceinline__ void report(ReportWords* rep, int f, bool bad, int64_t index)
{
    const uint64_t mask = __ballot(bad);
    if (mask == 0)
        return;
    unsigned long long idx = bad ? (unsigned long long)index : ~0ull;
    for (int o = 32; o > 0; o >>= 1) {
        const unsigned long long other = __shfl_xor(idx, o);
        idx = other < idx ? other : idx;
    }
    if ((threadIdx.x & 63) == __builtin_ctzll(mask)) {
        atomicAdd(&rep->count[f], (unsigned long long)__builtin_popcountll(mask));
        atomicMin(&rep->first[f], idx);
    }
}

// Lengths and used table entries: entry e = s * M + i, one per thread
// (grid-stride).  An entry is used when i < ceil(L / B) with L clamped to
// 0 .. M * B, as the attention kernels read it.
__global__ __launch_bounds__(kValidateThreads) void validate_tables_kernel(
    const int32_t* __restrict__ block_tables, const int32_t* __restrict__ seq_lens, int32_t S, int32_t M,
    int32_t B, int32_t num_blocks, ReportWords* __restrict__ rep)
{
    const int64_t total = (int64_t)S * M;
    const int64_t cap = (int64_t)M * B;
    const int64_t stride = (int64_t)gridDim.x * kValidateThreads;
    // every lane runs the same number of iterations (the ballots need the whole wave)
    for (int64_t base = (int64_t)blockIdx.x * kValidateThreads; base < total; base += stride) {
        const int64_t e = base + threadIdx.x;
        bool bad_len = false, bad_id = false;
        if (e < total) {
            const int32_t s = (int32_t)(e / M);
            const int32_t i = (int32_t)(e - (int64_t)s * M);
            const int64_t L = seq_lens[s];
            if (i == 0)
                bad_len = L < 0 || L > cap;
            const int64_t Lc = L < 0 ? 0 : (L > cap ? cap : L);
            if (i < (Lc + B - 1) / B) {
                const int32_t id = block_tables[e];
                bad_id = id < 0 || id >= num_blocks;
            }
        }
        report(rep, kBadLen, bad_len, e / M);
        report(rep, kBadBlock, bad_id, e);
    }
}

// The slot of token t: slot_mapping[t], or (slot_mapping null) the decode
// step's slot of sequence t, the rule of pkv_decode_slot_mapping.
__device__ __forceinline__ int64_t validate_slot(const int64_t* __restrict__ slot_mapping,
                                                 const int32_t* __restrict__ block_tables,
                                                 const int32_t* __restrict__ seq_lens, int32_t t, int32_t M,
                                                 int32_t B)
{
    if (slot_mapping)
        return slot_mapping[t];
    const int32_t L = seq_lens[t];
    if (L <= 0)
        return -1;
    const int32_t idx = (L - 1) / B;
    if (idx >= M)
        return -1;
    const int64_t id = block_tables[(int64_t)t * M + idx];
    return id < 0 ? -1 : id * B + (L - 1 - idx * B);
}

// Slots: token t = blockIdx.x * 256 + threadIdx.x.  A slot at or past the
// pool's end is out of range; one inside a block with ref_counts > 1 writes
// a shared block; one equal to the slot of an earlier token repeats it
// (checked against every earlier token, 256 at a time through LDS).
// Negative slots are skips, not errors.
__global__ __launch_bounds__(kValidateThreads) void validate_slots_kernel(
    const int64_t* __restrict__ slot_mapping, const int32_t* __restrict__ block_tables,
    const int32_t* __restrict__ seq_lens, int32_t T, int32_t M, int32_t B, int32_t num_blocks,
    const int32_t* __restrict__ ref_counts, ReportWords* __restrict__ rep)
{
    __shared__ int64_t tile[kValidateThreads];
    const int32_t t = blockIdx.x * kValidateThreads + threadIdx.x;
    const int64_t slot = t < T ? validate_slot(slot_mapping, block_tables, seq_lens, t, M, B) : -1;
    const bool in_pool = slot >= 0 && slot / B < num_blocks;
    report(rep, kBadSlot, slot >= 0 && !in_pool, t);
    bool shared = false;
    if (in_pool && ref_counts)
        shared = ref_counts[slot / B] > 1;
    report(rep, kSharedWrite, shared, t);
    bool dup = false;
    const int32_t t0 = blockIdx.x * kValidateThreads;
    for (int32_t j0 = 0; j0 <= t0; j0 += kValidateThreads) {
        const int32_t j = j0 + threadIdx.x;
        __syncthreads();
        tile[threadIdx.x] = j < T ? validate_slot(slot_mapping, block_tables, seq_lens, j, M, B) : -1;
        __syncthreads();
        const int32_t n = j0 + kValidateThreads <= t ? kValidateThreads : t - j0;  // earlier tokens only
        if (slot >= 0)
            for (int32_t k = 0; k < n; ++k)
                dup |= tile[k] == slot;
    }
    report(rep, kDupSlot, dup, t);
}

hipError_t launch_validate(const int32_t* block_tables, const int32_t* seq_lens, int32_t num_seqs,
                           int32_t max_blocks_per_seq, const int64_t* slot_mapping, int32_t num_tokens,
                           const int32_t* ref_counts, int32_t block_size, int32_t num_blocks, void* report_buf,
                           hipStream_t stream)
{
    ReportWords* rep = static_cast<ReportWords*>(report_buf);
    hipLaunchKernelGGL(validate_init_kernel, dim3(1), dim3(64), 0, stream, rep);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess)
        return e;
    const int64_t entries = (int64_t)num_seqs * max_blocks_per_seq;
    if (entries > 0) {
        const int64_t groups = (entries + kValidateThreads - 1) / kValidateThreads;
        hipLaunchKernelGGL(validate_tables_kernel, dim3((unsigned)(groups < 4096 ? groups : 4096)),
                           dim3(kValidateThreads), 0, stream, block_tables, seq_lens, num_seqs, max_blocks_per_seq,
                           block_size, num_blocks, rep);
        e = hipGetLastError();
        if (e != hipSuccess)
            return e;
    }
    // slots: the call's slot_mapping, or the decode step's slot of each sequence
    const int32_t T = slot_mapping ? num_tokens : num_seqs;
    if (T > 0) {
        hipLaunchKernelGGL(validate_slots_kernel, dim3((T + kValidateThreads - 1) / kValidateThreads),
                           dim3(kValidateThreads), 0, stream, slot_mapping, block_tables, seq_lens, T,
                           max_blocks_per_seq, block_size, num_blocks, ref_counts, rep);
        e = hipGetLastError();
    }
    return e;
}

}  // namespace pkv
