// Paged decode attention for gfx950: block-table walk, MFMA scores, online
// softmax, MFMA value sum, and the log-sum-exp merge of context partitions.
//
// What is computed follows the pages on PagedAttention: the kernel signature
// and its four steps in section 3.1 of the "vLLM engineering deep-dive" page
// (look up each logical block's physical block, loop over the blocks of one
// KV head, softmax, value-weighted sum), the address translation of the
// "cache structure" page (block_tables[s][t / B], slot t % B), and the grid
// over (sequence, head, partition) with a partition reduction for long
// contexts from the yololab page's kernel section.
//
// How it maps onto CDNA4:
//  * One work-group per (KV head, sequence, context partition); its NW waves
//    take the partition's blocks round-robin, so every (block, KV head) tile
//    is read from HBM exactly once for all G = Hq/Hkv query heads.
//  * The key tile is the A operand of v_mfma_f32_16x16x32_bf16 (16 token
//    rows x 32 head dims; 8 bf16 per lane).  With the key layout
//    [hs/x][B][x] one 16-byte load per lane covers 16 tokens x 4 chunks:
//    1 KiB of contiguous memory per wave load at B = 16.  The G query heads
//    (padded to 16) are the B operand, held in registers for the whole
//    partition.  The result lands as S^T: lane (r, c) holds the scores of
//    tokens 4r..4r+3 for query head c.
//  * That register layout is exactly the A operand of
//    v_mfma_f32_16x16x16_bf16 (16 heads x 16 tokens), so the probabilities
//    feed the value MFMA without any lane exchange.  The value layout
//    [hs][B] puts 4 consecutive tokens of one head dim in 8 bytes: the B
//    operand of that MFMA is one 8-byte load per lane, 512 contiguous bytes
//    per wave load.  Probabilities are split into bf16 hi + lo parts (two
//    MFMAs), so the value sum keeps fp32-level precision.
//  * fp32 caches use v_mfma_f32_16x16x4_f32 with the same operand roles.
//  * Online softmax in log2 units with a lazy rescale: the running maximum
//    is only raised (and the accumulators rescaled) when a tile's maximum
//    exceeds it by more than kRescaleSlack, which keeps rescaling off the
//    common path; the result is exact either way.
//  * Masked slots (t >= seq_len) get score -inf and their value operand is
//    zeroed by selection, so stale or NaN pool contents never reach a sum.
#include <math.h>

#include "pkv_internal.h"

namespace pkv {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kRescaleSlack = 8.0f;  // log2 units: probabilities stay <= 256

template <typename T>
struct Ops;

// bf16: per 16-token sub-tile, HS/32 key operands (16 B) and HS/16 value
// operands (8 B) per lane.
template <>
struct Ops<__bf16> {
    template <int HS>
    struct KReg {
        bf16x8 v[HS / 32];
    };
    template <int HS>
    struct VReg {
        bf16x4 v[HS / 16];
    };
    template <int HS>
    struct QReg {
        bf16x8 v[HS / 32];
    };
};

// fp32: HS/16 key operands (16 B = 4 head dims) and HS/16 value operands
// (16 B = 4 tokens) per lane.
template <>
struct Ops<float> {
    template <int HS>
    struct KReg {
        f32x4 v[HS / 16];
    };
    template <int HS>
    struct VReg {
        f32x4 v[HS / 16];
    };
    template <int HS>
    struct QReg {
        f32x4 v[HS / 16];
    };
};

template <typename T, int HS, int BS>
struct TileRegs {
    static constexpr int MT = BS / 16;
    typename Ops<T>::template KReg<HS> k[MT];
    typename Ops<T>::template VReg<HS> v[MT];
};

__device__ __forceinline__ float to_float(__bf16 x) { return (float)x; }
__device__ __forceinline__ float to_float(float x) { return x; }
__device__ __forceinline__ void store_elem(__bf16* p, float x) { *p = (__bf16)x; }
__device__ __forceinline__ void store_elem(float* p, float x) { *p = x; }

// Issue the loads of one (block, KV head) tile.  `tile_k`/`tile_v` point at
// the tile's first element; lane = 16*r + c.
template <typename T, int HS, int BS>
__device__ __forceinline__ void load_tile(TileRegs<T, HS, BS>& t, const T* __restrict__ tile_k,
                                          const T* __restrict__ tile_v, int r, int c)
{
#pragma unroll
    for (int mt = 0; mt < BS / 16; ++mt) {
        if constexpr (sizeof(T) == 2) {
#pragma unroll
            for (int i = 0; i < HS / 32; ++i)  // chunk 4i + r of token 16mt + c
                t.k[mt].v[i] = *(const bf16x8*)(tile_k + ((4 * i + r) * BS + 16 * mt + c) * 8);
        } else {
#pragma unroll
            for (int i = 0; i < HS / 16; ++i)
                t.k[mt].v[i] = *(const f32x4*)(tile_k + ((4 * i + r) * BS + 16 * mt + c) * 4);
        }
#pragma unroll
        for (int i = 0; i < HS / 16; ++i) {  // head dim 16i + c, tokens 16mt + 4r .. +3
            if constexpr (sizeof(T) == 2)
                t.v[mt].v[i] = *(const bf16x4*)(tile_v + (16 * i + c) * BS + 16 * mt + 4 * r);
            else
                t.v[mt].v[i] = *(const f32x4*)(tile_v + (16 * i + c) * BS + 16 * mt + 4 * r);
        }
    }
}

// Scores S^T for one 16-token sub-tile: element j of the result is token
// 4r + j of the sub-tile, query head c.
template <typename T, int HS>
__device__ __forceinline__ f32x4 tile_scores(const typename Ops<T>::template KReg<HS>& k,
                                             const typename Ops<T>::template QReg<HS>& q)
{
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    if constexpr (sizeof(T) == 2) {
#pragma unroll
        for (int i = 0; i < HS / 32; ++i)
            acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(k.v[i], q.v[i], acc, 0, 0, 0);
    } else {
#pragma unroll
        for (int i = 0; i < HS / 16; ++i)
#pragma unroll
            for (int e = 0; e < 4; ++e)
                acc = __builtin_amdgcn_mfma_f32_16x16x4f32(k.v[i][e], q.v[i][e], acc, 0, 0, 0);
    }
    return acc;
}

// O += P V for one 16-token sub-tile; p[j] is the probability of token
// 4r + j for query head c; O[i] element j is head 4r + j, head dim 16i + c.
template <typename T, int HS>
__device__ __forceinline__ void tile_pv(f32x4 (&O)[HS / 16], const float (&p)[4],
                                        const typename Ops<T>::template VReg<HS>& v)
{
    if constexpr (sizeof(T) == 2) {
        bf16x4 hi, lo;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const __bf16 h = (__bf16)p[j];
            hi[j] = h;
            lo[j] = (__bf16)(p[j] - (float)h);
        }
#pragma unroll
        for (int i = 0; i < HS / 16; ++i) {
            O[i] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(hi, v.v[i], O[i], 0, 0, 0);
            O[i] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(lo, v.v[i], O[i], 0, 0, 0);
        }
    } else {
#pragma unroll
        for (int i = 0; i < HS / 16; ++i)
#pragma unroll
            for (int j = 0; j < 4; ++j)
                O[i] = __builtin_amdgcn_mfma_f32_16x16x4f32(p[j], v.v[i][j], O[i], 0, 0, 0);
    }
}

template <typename T, int HS, int BS>
__device__ __forceinline__ void zero_masked_values(TileRegs<T, HS, BS>& t, int tok0, int L, int r)
{
#pragma unroll
    for (int mt = 0; mt < BS / 16; ++mt)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const bool keep = tok0 + 16 * mt + 4 * r + j < L;
#pragma unroll
            for (int i = 0; i < HS / 16; ++i)
                t.v[mt].v[i][j] = keep ? t.v[mt].v[i][j] : (T)0.f;
        }
}

template <typename T, int HS, int BS, int NW>
__global__ __launch_bounds__(NW * 64) void paged_decode_partition_kernel(
    const T* __restrict__ q, const T* __restrict__ k_cache, const T* __restrict__ v_cache,
    const int32_t* __restrict__ block_tables, const int32_t* __restrict__ seq_lens, int32_t Hq, int32_t Hkv,
    int32_t M, int32_t num_blocks, int32_t PB, int32_t max_parts, float qscale, T* __restrict__ out,
    float* __restrict__ ws_o, float* __restrict__ ws_ml)
{
    constexpr int MT = BS / 16;
    constexpr int TILE = HS * BS;  // elements per (block, KV head) tile
    const int kvh = blockIdx.x;
    const int s = blockIdx.y;
    const int part = blockIdx.z;
    const int lane = threadIdx.x & 63;
    const int w = threadIdx.x >> 6;
    const int r = lane >> 4;
    const int c = lane & 15;
    const int G = Hq / Hkv;

    int L = seq_lens[s];
    L = L < 0 ? 0 : (L > M * BS ? M * BS : L);
    if (L == 0) {
        if (part == 0)
            for (int idx = threadIdx.x; idx < G * HS; idx += NW * 64)
                store_elem(out + ((int64_t)s * Hq + (int64_t)kvh * G) * HS + idx, 0.f);
        return;
    }
    const int nblk = (L + BS - 1) / BS;
    const int b0 = part * PB;
    if (b0 >= nblk)
        return;
    const int nb_part = (nblk - b0 < PB) ? nblk - b0 : PB;
    const int nparts = (nblk + PB - 1) / PB;

    // physical block IDs of this partition, one per lane (PB <= 64)
    const int32_t id_lane = lane < nb_part ? block_tables[(int64_t)s * M + b0 + lane] : 0;

    // query operand: head c of this KV head's group (zero for padding rows)
    typename Ops<T>::template QReg<HS> qr;
    {
        const bool real = c < G;
        const T* qh = q + ((int64_t)s * Hq + (int64_t)kvh * G + (real ? c : 0)) * HS;
        if constexpr (sizeof(T) == 2) {
#pragma unroll
            for (int i = 0; i < HS / 32; ++i) {
                bf16x8 v = *(const bf16x8*)(qh + 32 * i + 8 * r);
                qr.v[i] = real ? v : (bf16x8)(__bf16)0.f;
            }
        } else {
#pragma unroll
            for (int i = 0; i < HS / 16; ++i) {
                f32x4 v = *(const f32x4*)(qh + 16 * i + 4 * r);
                qr.v[i] = real ? v : (f32x4)0.f;
            }
        }
    }

    f32x4 O[HS / 16];
#pragma unroll
    for (int i = 0; i < HS / 16; ++i)
        O[i] = (f32x4)0.f;
    float m_run = -INFINITY;  // running max for head c, log2 units
    float l_part = 0.f;       // sum of probabilities of this lane's tokens

    const int64_t head_off = (int64_t)kvh * TILE;
    const int64_t block_stride = (int64_t)Hkv * TILE;

    auto tile_ptr_ok = [&](int j, const T*& tk, const T*& tv) -> bool {
        int32_t id = __builtin_amdgcn_readlane(id_lane, j);
        const bool ok = (uint32_t)id < (uint32_t)num_blocks;
        id = ok ? id : 0;
        tk = k_cache + (int64_t)id * block_stride + head_off;
        tv = v_cache + (int64_t)id * block_stride + head_off;
        return ok;
    };

    auto compute = [&](TileRegs<T, HS, BS>& t, int j, bool ok) {
        if (!ok)
            return;  // out-of-range block ID: the tile contributes nothing
        const int tok0 = (b0 + j) * BS;
        const bool partial = tok0 + BS > L;
        float sc[MT][4];
        float mx = -INFINITY;
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
            const f32x4 S = tile_scores<T, HS>(t.k[mt], qr);
#pragma unroll
            for (int jj = 0; jj < 4; ++jj) {
                float v = S[jj] * qscale;
                if (partial)
                    v = (tok0 + 16 * mt + 4 * r + jj < L) ? v : -INFINITY;
                sc[mt][jj] = v;
                mx = fmaxf(mx, v);
            }
        }
        if (partial)
            zero_masked_values<T, HS, BS>(t, tok0, L, r);
        mx = fmaxf(mx, __shfl_xor(mx, 16));
        mx = fmaxf(mx, __shfl_xor(mx, 32));
        if (__ballot(mx > m_run + kRescaleSlack) != 0) {
            const float m_new = fmaxf(m_run, mx);
            const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
            m_run = m_new;
            l_part *= alpha;
            float a_row[4];
#pragma unroll
            for (int jj = 0; jj < 4; ++jj)
                a_row[jj] = __shfl(alpha, 4 * r + jj);
#pragma unroll
            for (int i = 0; i < HS / 16; ++i)
#pragma unroll
                for (int jj = 0; jj < 4; ++jj)
                    O[i][jj] *= a_row[jj];
        }
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
            float p[4];
#pragma unroll
            for (int jj = 0; jj < 4; ++jj) {
                p[jj] = __builtin_amdgcn_exp2f(sc[mt][jj] - m_run);
                l_part += p[jj];
            }
            tile_pv<T, HS>(O, p, t.v[mt]);
        }
    };

    // software pipeline: the next tile's loads are in flight while the
    // current tile is computed
    TileRegs<T, HS, BS> ta, tb;
    const T* tk;
    const T* tv;
    int j = w;
    bool ok_a = false, ok_b = false;
    if (j < nb_part) {
        ok_a = tile_ptr_ok(j, tk, tv);
        load_tile<T, HS, BS>(ta, tk, tv, r, c);
    }
    while (j < nb_part) {
        if (j + NW < nb_part) {
            ok_b = tile_ptr_ok(j + NW, tk, tv);
            load_tile<T, HS, BS>(tb, tk, tv, r, c);
        }
        compute(ta, j, ok_a);
        j += NW;
        if (j >= nb_part)
            break;
        if (j + NW < nb_part) {
            ok_a = tile_ptr_ok(j + NW, tk, tv);
            load_tile<T, HS, BS>(ta, tk, tv, r, c);
        }
        compute(tb, j, ok_b);
        j += NW;
    }

    // ---- merge the waves' partial states (log-sum-exp) ----
    float l_tot = l_part + __shfl_xor(l_part, 16);
    l_tot += __shfl_xor(l_tot, 32);

    __shared__ float sm_o[NW][16][HS];
    __shared__ float sm_m[NW][16];
    __shared__ float sm_l[NW][16];
    if (r == 0) {
        sm_m[w][c] = m_run;
        sm_l[w][c] = l_tot;
    }
#pragma unroll
    for (int i = 0; i < HS / 16; ++i)
#pragma unroll
        for (int jj = 0; jj < 4; ++jj)
            sm_o[w][4 * r + jj][16 * i + c] = O[i][jj];
    __syncthreads();

    for (int idx = threadIdx.x; idx < G * HS; idx += NW * 64) {
        const int g = idx / HS;
        const int d = idx - g * HS;
        float mx = -INFINITY;
#pragma unroll
        for (int ww = 0; ww < NW; ++ww)
            if (sm_l[ww][g] > 0.f)
                mx = fmaxf(mx, sm_m[ww][g]);
        float lsum = 0.f, acc = 0.f;
#pragma unroll
        for (int ww = 0; ww < NW; ++ww)
            if (sm_l[ww][g] > 0.f) {
                const float f = __builtin_amdgcn_exp2f(sm_m[ww][g] - mx);
                lsum += sm_l[ww][g] * f;
                acc += sm_o[ww][g][d] * f;
            }
        const float o = lsum > 0.f ? acc / lsum : 0.f;
        const int64_t hrow = (int64_t)s * Hq + (int64_t)kvh * G + g;
        if (nparts == 1) {
            store_elem(out + hrow * HS + d, o);
        } else {
            const int64_t u = hrow * max_parts + part;
            ws_o[u * HS + d] = o;
            if (d == 0) {
                ws_ml[2 * u] = mx;
                ws_ml[2 * u + 1] = lsum;
            }
        }
    }
}

// Merge of the context partitions of one (sequence, query head):
// M = max m_p, w_p = l_p * 2^(m_p - M), out = sum w_p o_p / sum w_p
// (o_p is already normalised by l_p).  Sequences with one partition were
// written by the partition kernel and are skipped here.
template <typename T, int HS>
__global__ __launch_bounds__(64) void paged_decode_reduce_kernel(const int32_t* __restrict__ seq_lens, int32_t M,
                                                                 int32_t BS, int32_t PB, int32_t Hq,
                                                                 int32_t max_parts, const float* __restrict__ ws_o,
                                                                 const float* __restrict__ ws_ml,
                                                                 T* __restrict__ out)
{
    const int h = blockIdx.x;
    const int s = blockIdx.y;
    int L = seq_lens[s];
    L = L < 0 ? 0 : (L > M * BS ? M * BS : L);
    const int nblk = (L + BS - 1) / BS;
    const int nparts = (nblk + PB - 1) / PB;
    if (nparts <= 1)
        return;
    const int64_t u0 = ((int64_t)s * Hq + h) * max_parts;
    float mx = -INFINITY;
    for (int p = 0; p < nparts; ++p)
        mx = fmaxf(mx, ws_ml[2 * (u0 + p)]);
    float wsum = 0.f;
    float acc[HS / 64];
#pragma unroll
    for (int i = 0; i < HS / 64; ++i)
        acc[i] = 0.f;
    for (int p = 0; p < nparts; ++p) {
        const float f = ws_ml[2 * (u0 + p) + 1] * __builtin_amdgcn_exp2f(ws_ml[2 * (u0 + p)] - mx);
        wsum += f;
#pragma unroll
        for (int i = 0; i < HS / 64; ++i)
            acc[i] += f * ws_o[(u0 + p) * HS + threadIdx.x + 64 * i];
    }
#pragma unroll
    for (int i = 0; i < HS / 64; ++i)
        store_elem(out + ((int64_t)s * Hq + h) * HS + threadIdx.x + 64 * i, acc[i] / wsum);
}

template <typename T, int HS, int BS>
static hipError_t launch_typed(const DecodeArgs& a, hipStream_t stream)
{
    constexpr int NW = 4;
    const dim3 grid(a.num_kv_heads, a.num_seqs, a.max_parts);
    hipLaunchKernelGGL((paged_decode_partition_kernel<T, HS, BS, NW>), grid, dim3(NW * 64), 0, stream,
                       (const T*)a.q, (const T*)a.k_cache, (const T*)a.v_cache, a.block_tables, a.seq_lens,
                       a.num_q_heads, a.num_kv_heads, a.max_blocks_per_seq, a.num_blocks, a.partition_blocks,
                       a.max_parts, a.scale * kLog2e, (T*)a.out, a.ws_o, a.ws_ml);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || a.max_parts <= 1)
        return e;
    hipLaunchKernelGGL((paged_decode_reduce_kernel<T, HS>), dim3(a.num_q_heads, a.num_seqs), dim3(64), 0, stream,
                       a.seq_lens, a.max_blocks_per_seq, BS, a.partition_blocks, a.num_q_heads, a.max_parts,
                       a.ws_o, a.ws_ml, (T*)a.out);
    return hipGetLastError();
}

template <typename T>
static hipError_t launch_dtype(const DecodeArgs& a, hipStream_t stream)
{
    if (a.head_size == 128)
        return a.block_size == 16 ? launch_typed<T, 128, 16>(a, stream) : launch_typed<T, 128, 32>(a, stream);
    return a.block_size == 16 ? launch_typed<T, 64, 16>(a, stream) : launch_typed<T, 64, 32>(a, stream);
}

hipError_t launch_decode(const DecodeArgs& a, hipStream_t stream)
{
    return a.dtype == 1 ? launch_dtype<__bf16>(a, stream) : launch_dtype<float>(a, stream);
}

}  // namespace pkv
