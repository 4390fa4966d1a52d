// Read probes: measurement aids, not part of the attention method.
//
// Streaming-read probe: the rate at which the GPU reads a large buffer that
// no kernel has touched recently, the practical ceiling of the library's
// bandwidth-bound kernels (decode attention reads each key and value byte
// once).  Work-group b reads the b-th contiguous share of the buffer; each
// thread keeps eight independent 16-byte non-temporal loads in flight and
// folds the words it read into one value by XOR, which it stores only when
// it equals a marker, so that no load can be dropped.
//
// Gather-read probe: see gather_read_kernel below.
#include "pkv_internal.h"

namespace pkv {

namespace {

typedef unsigned int u32x4v __attribute__((ext_vector_type(4)));
constexpr int kProbeThreads = 256;
constexpr int kProbeDepth = 8;

__global__ __launch_bounds__(kProbeThreads) void stream_read_kernel(const u32x4v* __restrict__ p, size_t n,
                                                                     unsigned* __restrict__ out)
{
    const size_t per = (n + gridDim.x - 1) / gridDim.x;
    const size_t lo = (size_t)blockIdx.x * per;
    const size_t hi = lo + per < n ? lo + per : n;
    u32x4v acc = {0u, 0u, 0u, 0u};
    size_t i = lo + threadIdx.x;
    for (; i + (kProbeDepth - 1) * kProbeThreads < hi; i += kProbeDepth * kProbeThreads) {
        u32x4v t[kProbeDepth];
#pragma unroll
        for (int k = 0; k < kProbeDepth; ++k)
            t[k] = __builtin_nontemporal_load(p + i + k * kProbeThreads);
#pragma unroll
        for (int k = 0; k < kProbeDepth; ++k)
            acc ^= t[k];
    }
    for (; i < hi; i += kProbeThreads)
        acc ^= p[i];
    const unsigned x = acc.x ^ acc.y ^ acc.z ^ acc.w;
    if (x == 0x9E3779B9u)
        out[0] = x;
}

// Gather-read probe: the rate at which the GPU reads a list of whole tiles
// at arbitrary places of two buffers (a pool's key and value tiles through
// its block tables), with every tile's address known in advance: the paged
// access pattern of decode attention without its per-item chains (length,
// table row, first loads), its arithmetic or its merge.
//
// Each wave takes the next contiguous share of the tile list; tile t lies
// in buffer t % 2 at byte offset offs[t].  Tile offsets are read 64 at a time
// (one per lane, the next 64 already in flight) and broadcast by lane
// exchange; each lane keeps kProbeDepth 16-byte non-temporal loads in
// flight, lane l reading words l, l + 64, ... of each tile (tile_words is a
// multiple of 64).  A tile outside its buffer, or at a negative offset or
// one that is not a multiple of 16, is skipped.  The words read are folded
// by XOR as in the streaming probe.
__global__ __launch_bounds__(kProbeThreads) void gather_read_kernel(
    const char* __restrict__ b0, const char* __restrict__ b1, size_t n0, size_t n1,
    const int64_t* __restrict__ offs, int64_t ntiles, int32_t tile_words, unsigned* __restrict__ out)
{
    const int lane = threadIdx.x & 63;
    const int64_t waves = (int64_t)gridDim.x * (kProbeThreads / 64);
    const int64_t wid = (int64_t)blockIdx.x * (kProbeThreads / 64) + (threadIdx.x >> 6);
    const int64_t per = (ntiles + waves - 1) / waves;
    const int64_t t_lo = wid * per;
    const int64_t t_hi = t_lo + per < ntiles ? t_lo + per : ntiles;
    if (t_lo >= t_hi)
        return;  // uniform per wave; the kernel has no barrier
    const int64_t tile_bytes = (int64_t)tile_words * 16;
    // offsets of tiles tb .. tb + 63 (cur) and tb + 64 .. tb + 127 (next)
    int64_t tb = t_lo;
    int64_t cur = tb + lane < t_hi ? offs[tb + lane] : -1;
    int64_t nxt = tb + 64 + lane < t_hi ? offs[tb + 64 + lane] : -1;
    const int64_t g_end = (t_hi - t_lo) * tile_words;  // words of this wave's tiles
    u32x4v acc = {0u, 0u, 0u, 0u};
    for (int64_t g = 0; g < g_end; g += 64 * kProbeDepth) {
        if (t_lo + g / tile_words >= tb + 64) {  // uniform: the window moves on by 64 tiles
            tb += 64;
            cur = nxt;
            nxt = tb + 64 + lane < t_hi ? offs[tb + 64 + lane] : -1;
        }
        u32x4v t[kProbeDepth];
#pragma unroll
        for (int k = 0; k < kProbeDepth; ++k) {
            t[k] = (u32x4v){0u, 0u, 0u, 0u};
            const int64_t gk = g + 64 * k;  // uniform
            if (gk < g_end) {
                const int64_t tile = t_lo + gk / tile_words;  // at most kProbeDepth tiles past tb: in cur or nxt
                const int64_t d = tile - tb;
                const int64_t off = d < 64 ? __shfl(cur, (int)d) : __shfl(nxt, (int)(d - 64));
                const char* base = (tile & 1) ? b1 : b0;
                const size_t n = (tile & 1) ? n1 : n0;
                if (off >= 0 && (off & 15) == 0 && (size_t)off + (size_t)tile_bytes <= n)
                    t[k] = __builtin_nontemporal_load(reinterpret_cast<const u32x4v*>(base + off) + gk % tile_words + lane);
            }
        }
#pragma unroll
        for (int k = 0; k < kProbeDepth; ++k)
            acc ^= t[k];
    }
    const unsigned x = acc.x ^ acc.y ^ acc.z ^ acc.w;
    if (x == 0x9E3779B9u)
        out[0] = x;
}

}  // namespace

hipError_t launch_gather_read(const void* buf0, size_t bytes0, const void* buf1, size_t bytes1,
                              const int64_t* tile_offsets, int64_t num_tiles, int32_t tile_bytes, void* out,
                              int32_t work_groups, hipStream_t stream)
{
    hipLaunchKernelGGL(gather_read_kernel, dim3(work_groups), dim3(kProbeThreads), 0, stream, (const char*)buf0,
                       (const char*)buf1, bytes0, bytes1, tile_offsets, num_tiles, tile_bytes / 16, (unsigned*)out);
    return hipGetLastError();
}

hipError_t launch_stream_read(const void* buf, size_t bytes, void* out, int32_t work_groups, hipStream_t stream)
{
    hipLaunchKernelGGL(stream_read_kernel, dim3(work_groups), dim3(kProbeThreads), 0, stream,
                       (const u32x4v*)buf, bytes / 16, (unsigned*)out);
    return hipGetLastError();
}

}  // namespace pkv
