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

#include <algorithm>
#include <type_traits>

#include "attn_common.h"
#include "kv_store.h"
#include "pkv_internal.h"

namespace pkv {


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

// Operand registers of one 16-token sub-tile (a block of B = 32 holds two).
template <typename T, int HS>
struct TileRegs {
    typename Ops<T>::template KReg<HS> k;
    typename Ops<T>::template VReg<HS> v;
};

// bf16 blocks of 32 tokens are handled as one 32-token unit: two key
// M-tiles and a value operand of 8 tokens per lane (v_mfma_f32_16x16x32_bf16
// with the tokens as the reduction dimension).  Each value load then covers
// a whole 64-byte [hs][32] row segment: 1 KiB contiguous per wave load.
template <int HS>
struct WideRegs {
    Ops<__bf16>::KReg<HS> k[2];
    bf16x8 v[HS / 16];
};

// K/V tiles are read exactly once per call: streaming (non-temporal) loads
// keep them from displacing reusable lines (queries, tables, partials).
template <typename V>
__device__ __forceinline__ V load_stream(const V* p)
{
    return __builtin_nontemporal_load(p);
}

// Address of one lane's operand: a wave-uniform base (the tile pointer plus
// the offset that does not depend on the lane, which stays in scalar
// registers) plus the lane's own unsigned byte offset.  Written this way the
// loads take the scalar-base + 32-bit vector-offset form, so a unit's loads
// share one or two offset registers instead of a 64-bit address each.
template <typename E>
__device__ __forceinline__ const E* lane_at(const E* base, int uniform_elems, uint32_t lane_bytes)
{
    return reinterpret_cast<const E*>(reinterpret_cast<const char*>(base + uniform_elems) + lane_bytes);
}

// Issue the loads of 16-token sub-tile m of one (block, KV head) tile.
// `tile_k`/`tile_v` point at the tile's first element; lane = 16*r + c.
template <typename T, int HS, int BS>
__device__ __forceinline__ void load_tile(TileRegs<T, HS>& t, const T* __restrict__ tile_k,
                                          const T* __restrict__ tile_v, int m, int r, int c)
{
    // (bf16 keeps plain element offsets here: the scalar-base form saves
    // nothing at 16 tokens and costs the head-size-64 variants a wave)
    if constexpr (sizeof(T) == 2) {
#pragma unroll
        for (int i = 0; i < HS / 32; ++i)  // chunk 4i + r of token 16m + c
            t.k.v[i] = load_stream((const bf16x8*)(tile_k + ((4 * i + r) * BS + 16 * m + c) * 8));
#pragma unroll
        for (int i = 0; i < HS / 16; ++i)  // head dim 16i + c, tokens 16m + 4r .. +3
            t.v.v[i] = load_stream((const bf16x4*)(tile_v + (16 * i + c) * BS + 16 * m + 4 * r));
    } else {
        const uint32_t k_lane = (uint32_t)(r * BS + c) * 16u;
        const uint32_t v_lane = (uint32_t)(c * BS + 4 * r) * 4u;
#pragma unroll
        for (int i = 0; i < HS / 16; ++i)
            t.k.v[i] = load_stream((const f32x4*)lane_at(tile_k, (4 * i * BS + 16 * m) * 4, k_lane));
#pragma unroll
        for (int i = 0; i < HS / 16; ++i)
            t.v.v[i] = load_stream((const f32x4*)lane_at(tile_v, 16 * i * BS + 16 * m, v_lane));
    }
}

// Blocks smaller than the 16-token unit (B = 1, 2, 4 or 8; bf16 or fp32):
// the unit's tokens come from 16 / B consecutive blocks of the wave's
// partition, so each lane fetches its own block IDs from the wave's list
// (ids: lane j holds block j; ds_bpermute): key token c of the unit, value
// tokens 4r .. 4r+3 (one block when B >= 4, else one element per token).
// An ID outside the pool reads block 0, and the returned 16-bit mask has the
// bits of that block's tokens clear (valid_blocks: bit j set when ID j is
// inside the pool), so that compute masks them.
template <typename T, int HS, int BS>
__device__ __forceinline__ int load_small(TileRegs<T, HS>& t, const T* __restrict__ k_cache,
                                          const T* __restrict__ v_cache, int64_t block_stride, int64_t head_off,
                                          int32_t ids, uint64_t valid_blocks, int32_t num_blocks, int u, int r, int c)
{
    static_assert(BS < 16 && 16 % BS == 0, "small-block path");
    constexpr int X = 16 / (int)sizeof(T);
    using KV = typename std::conditional<sizeof(T) == 2, bf16x8, f32x4>::type;
    using VV = typename std::conditional<sizeof(T) == 2, bf16x4, f32x4>::type;
    auto block_at = [&](int j) __attribute__((always_inline)) -> int64_t {
        const int32_t id = __shfl(ids, j);
        return ((uint32_t)id < (uint32_t)num_blocks ? id : 0) * block_stride + head_off;
    };
    const int tk = 16 * u + c;
    const T* kp = k_cache + block_at(tk / BS) + (tk % BS) * X;
#pragma unroll
    for (int i = 0; i < HS / (4 * X); ++i)  // chunk 4i + r of token c
        t.k.v[i] = load_stream((const KV*)(kp + (4 * i + r) * BS * X));
    if constexpr (BS >= 4) {
        const int tv = 16 * u + 4 * r;
        const T* vp = v_cache + block_at(tv / BS) + tv % BS;
#pragma unroll
        for (int i = 0; i < HS / 16; ++i)
            t.v.v[i] = load_stream((const VV*)(vp + (16 * i + c) * BS));
    } else {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int tv = 16 * u + 4 * r + j;
            const T* vp = v_cache + block_at(tv / BS) + tv % BS;
#pragma unroll
            for (int i = 0; i < HS / 16; ++i)
                t.v.v[i][j] = load_stream(vp + (16 * i + c) * BS);
        }
    }
    int tmask = 0;
#pragma unroll
    for (int k = 0; k < 16 / BS; ++k) {
        const int j = (16 * u) / BS + k;
        if (j >= 64 || ((valid_blocks >> j) & 1))
            tmask |= ((1 << BS) - 1) << (k * BS);
    }
    return tmask;
}

// 32-token unit m of a block of BS >= 32 tokens (tokens 32m .. 32m+31).
// With BS = 64 a unit reads half of each value row and the next unit the
// other half: those loads go through the caches normally (a streaming load
// of half a line left the other half to be fetched from HBM again).
template <typename V>
__device__ __forceinline__ V load_value_part(const V* p, bool whole_rows)
{
    return whole_rows ? load_stream(p) : *p;
}

template <int HS, int BS>
__device__ __forceinline__ void load_wide(WideRegs<HS>& t, const __bf16* __restrict__ tile_k,
                                          const __bf16* __restrict__ tile_v, int m, int r, int c)
{
    // key chunk 4i + r of token 32m + 16mp + c; value head dim 16i + c,
    // tokens 32m + 8r .. +7 (lane parts in bytes)
    const uint32_t k_lane = (uint32_t)(r * BS + c) * 16u;
    const uint32_t v_lane = (uint32_t)(c * BS + 8 * r) * 2u;
#pragma unroll
    for (int mp = 0; mp < 2; ++mp)
#pragma unroll
        for (int i = 0; i < HS / 32; ++i)
            t.k[mp].v[i] = load_stream((const bf16x8*)lane_at(tile_k, (4 * i * BS + 32 * m + 16 * mp) * 8, k_lane));
#pragma unroll
    for (int i = 0; i < HS / 16; ++i)
        t.v[i] = load_value_part((const bf16x8*)lane_at(tile_v, 16 * i * BS + 32 * m, v_lane), BS == 32);
}

// FP8 (E4M3) caches, bf16 queries: one 16-token sub-tile as raw codes.
// Keys: chunk 4i + r of token 16m + c, i < HS/64 (16 head dims per 16-byte
// chunk, key layout [hs/16][B][16]); one wave load is 16 tokens x 4 chunks,
// 1 KiB contiguous.  The 16 dims of a chunk feed two score MFMAs (dims
// 8h .. 8h+7 of chunk 4i + r go to MFMA 2i + h), and the query operand is
// loaded in the same order (see the query load): a dot product does not
// depend on the order of its terms.  Values: the 4 codes of tokens
// 16m + 4r .. +3 of head dim 16i + c (one 4-byte load per lane, 256 bytes
// contiguous per wave load).
template <int HS>
struct Fp8Regs {
    u32x4 k[HS / 64];
    unsigned v[HS / 16];
};

template <int HS, int BS>
__device__ __forceinline__ void load_fp8(Fp8Regs<HS>& t, const uint8_t* __restrict__ tile_k,
                                         const uint8_t* __restrict__ tile_v, int m, int r, int c)
{
    const uint32_t k_lane = (uint32_t)(r * BS + c) * 16u;
    const uint32_t v_lane = (uint32_t)(c * BS + 4 * r);
#pragma unroll
    for (int i = 0; i < HS / 64; ++i)
        t.k[i] = load_stream((const u32x4*)lane_at(tile_k, (4 * i * BS + 16 * m) * 16, k_lane));
#pragma unroll
    for (int i = 0; i < HS / 16; ++i)
        t.v[i] = load_stream((const unsigned*)lane_at(tile_v, 16 * i * BS + 16 * m, v_lane));
}

template <int HS>
__device__ __forceinline__ void fp8_to_operands(const Fp8Regs<HS>& raw, TileRegs<__bf16, HS>& t)
{
    typedef unsigned u32x2 __attribute__((ext_vector_type(2)));
#pragma unroll
    for (int i = 0; i < HS / 64; ++i)
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            unsigned a, b, c, d;
            fp8x4_to_bf16(raw.k[i][2 * h], a, b);
            fp8x4_to_bf16(raw.k[i][2 * h + 1], c, d);
            const u32x4 w = {a, b, c, d};
            t.k.v[2 * i + h] = __builtin_bit_cast(bf16x8, w);
        }
#pragma unroll
    for (int i = 0; i < HS / 16; ++i) {
        unsigned a, b;
        fp8x4_to_bf16(raw.v[i], a, b);
        const u32x2 w = {a, b};
        t.v.v[i] = __builtin_bit_cast(bf16x4, w);
    }
}

// FP8 pools with B >= 32: 32-token units, like the bf16 32-token path.  Key
// M-tile mp holds tokens 16mp .. 16mp+15 (chunk 4i + r of token 16mp + c;
// two 128-byte lines per lane group); the value operand is 8 codes per lane,
// tokens 8r .. 8r+7 of head dim 16i + c (the four lane groups read the dim's
// whole 32-byte row).
template <int HS>
struct Fp8WideRegs {
    u32x4 k[2][HS / 64];
    unsigned v[HS / 16][2];
};

template <int HS, int BS>
__device__ __forceinline__ void load_fp8_wide(Fp8WideRegs<HS>& t, const uint8_t* __restrict__ tile_k,
                                              const uint8_t* __restrict__ tile_v, int m, int r, int c)
{
    typedef unsigned u32x2 __attribute__((ext_vector_type(2)));
    const uint32_t k_lane = (uint32_t)(r * BS + c) * 16u;
    const uint32_t v_lane = (uint32_t)(c * BS + 8 * r);
#pragma unroll
    for (int mp = 0; mp < 2; ++mp)
#pragma unroll
        for (int i = 0; i < HS / 64; ++i)
            t.k[mp][i] = load_stream((const u32x4*)lane_at(tile_k, (4 * i * BS + 32 * m + 16 * mp) * 16, k_lane));
#pragma unroll
    for (int i = 0; i < HS / 16; ++i) {
        const u32x2 w = load_value_part((const u32x2*)lane_at(tile_v, 16 * i * BS + 32 * m, v_lane), BS == 32);
        t.v[i][0] = w[0];
        t.v[i][1] = w[1];
    }
}

template <int HS>
__device__ __forceinline__ void fp8_wide_to_operands(const Fp8WideRegs<HS>& raw, WideRegs<HS>& t)
{
#pragma unroll
    for (int mp = 0; mp < 2; ++mp)
#pragma unroll
        for (int i = 0; i < HS / 64; ++i)
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                unsigned a, b, c, d;
                fp8x4_to_bf16(raw.k[mp][i][2 * h], a, b);
                fp8x4_to_bf16(raw.k[mp][i][2 * h + 1], c, d);
                const u32x4 w = {a, b, c, d};
                t.k[mp].v[2 * i + h] = __builtin_bit_cast(bf16x8, w);
            }
#pragma unroll
    for (int i = 0; i < HS / 16; ++i) {
        unsigned a, b, c, d;
        fp8x4_to_bf16(raw.v[i][0], a, b);
        fp8x4_to_bf16(raw.v[i][1], c, d);
        const u32x4 w = {a, b, c, d};
        t.v[i] = __builtin_bit_cast(bf16x8, w);
    }
}

// Decode step in one launch: the unit's token p (the sequence's new token)
// is replaced by its K/V as the step's input holds them (sk, sv: head_size
// elements each, the input type), in the operand layout of each unit
// shape.  For FP8 pools the codes are formed as the store forms them
// (quantize16, quantize1 with the same inverse scales), so the attention
// reads the same bytes it would read from the pools after the store.
// Sets element (or byte) j of a value operand where j is wave-uniform.
template <int N, typename V, typename E>
__device__ __forceinline__ void set_elem(V& v, int j, E x)
{
#pragma unroll
    for (int e = 0; e < N; ++e)
        if (e == j)
            v[e] = x;
}

__device__ __forceinline__ unsigned set_byte(unsigned w, int j, unsigned code)
{
    return (w & ~(0xFFu << (8 * j))) | (code << (8 * j));
}

// 16-token unit, bf16 or fp32 (TileRegs): key chunk 4i + r of token c,
// value tokens 4r .. 4r + 3 of head dim 16i + c.
template <typename T, int HS>
__device__ __forceinline__ void patch_token(TileRegs<T, HS>& t, const T* sk, const T* sv, int p, int r, int c,
                                            float, float)
{
    constexpr int X = 16 / (int)sizeof(T);
    using KV = typename std::conditional<sizeof(T) == 2, bf16x8, f32x4>::type;
    if (c == p) {
#pragma unroll
        for (int i = 0; i < HS / (4 * X); ++i)
            t.k.v[i] = *(const KV*)(sk + (4 * i + r) * X);
    }
    if (r == p / 4) {
#pragma unroll
        for (int i = 0; i < HS / 16; ++i)
            set_elem<4>(t.v.v[i], p & 3, sv[16 * i + c]);
    }
}

// 32-token unit, bf16 (WideRegs): key chunk 4i + r of token 16mp + c, value
// tokens 8r .. 8r + 7 of head dim 16i + c.
template <int HS>
__device__ __forceinline__ void patch_token(WideRegs<HS>& t, const __bf16* sk, const __bf16* sv, int p, int r,
                                            int c, float, float)
{
    if (c == (p & 15)) {
#pragma unroll
        for (int i = 0; i < HS / 32; ++i) {
            const bf16x8 x = *(const bf16x8*)(sk + (4 * i + r) * 8);
            if (p < 16)
                t.k[0].v[i] = x;
            else
                t.k[1].v[i] = x;
        }
    }
    if (r == (p >> 3)) {
#pragma unroll
        for (int i = 0; i < HS / 16; ++i)
            set_elem<8>(t.v[i], p & 7, sv[16 * i + c]);
    }
}

// 16-token unit of FP8 codes (Fp8Regs): key chunk 4i + r (16 dims) of token
// c, value codes of tokens 4r .. 4r + 3 of head dim 16i + c.
template <int HS>
__device__ __forceinline__ void patch_token(Fp8Regs<HS>& t, const __bf16* sk, const __bf16* sv, int p, int r,
                                            int c, float k_inv, float v_inv)
{
    if (c == p) {
#pragma unroll
        for (int i = 0; i < HS / 64; ++i) {
            const u32x4 in[2] = {*(const u32x4*)(sk + (4 * i + r) * 16), *(const u32x4*)(sk + (4 * i + r) * 16 + 8)};
            t.k[i] = quantize16(in, k_inv);
        }
    }
    if (r == p / 4) {
#pragma unroll
        for (int i = 0; i < HS / 16; ++i)
            t.v[i] = set_byte(t.v[i], p & 3, quantize1(__builtin_bit_cast(uint16_t, sv[16 * i + c]), v_inv));
    }
}

// 32-token unit of FP8 codes (Fp8WideRegs): key chunk 4i + r of token
// 16mp + c, value codes of tokens 8r .. 8r + 7 of head dim 16i + c.
template <int HS>
__device__ __forceinline__ void patch_token(Fp8WideRegs<HS>& t, const __bf16* sk, const __bf16* sv, int p, int r,
                                            int c, float k_inv, float v_inv)
{
    if (c == (p & 15)) {
#pragma unroll
        for (int i = 0; i < HS / 64; ++i) {
            const u32x4 in[2] = {*(const u32x4*)(sk + (4 * i + r) * 16), *(const u32x4*)(sk + (4 * i + r) * 16 + 8)};
            const u32x4 code = quantize16(in, k_inv);
            if (p < 16)
                t.k[0][i] = code;
            else
                t.k[1][i] = code;
        }
    }
    if (r == (p >> 3)) {
#pragma unroll
        for (int i = 0; i < HS / 16; ++i) {
            const unsigned code = quantize1(__builtin_bit_cast(uint16_t, sv[16 * i + c]), v_inv);
            if ((p & 7) < 4)
                t.v[i][0] = set_byte(t.v[i][0], p & 3, code);
            else
                t.v[i][1] = set_byte(t.v[i][1], p & 3, code);
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

// Zero the value operand of tokens at or beyond L (tok0 = the sub-tile's
// first token), so stale or NaN slots never enter the value sum.
template <typename T, int HS>
__device__ __forceinline__ void zero_masked_values(TileRegs<T, HS>& t, int tok0, int L, int r, int tmask)
{
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const bool keep = tok0 + 4 * r + j < L && ((tmask >> (4 * r + j)) & 1);
#pragma unroll
        for (int i = 0; i < HS / 16; ++i)
            t.v.v[i][j] = keep ? t.v.v[i][j] : (T)0.f;
    }
}

// Occupancy targets (waves per SIMD) for bf16 queries: three with 16-token
// units (<= 168 VGPRs, including the MFMA accumulators), two with 32-token
// units (<= 256), for bf16 and FP8 pools alike.  Exceptions, where these
// targets would spill: one-token blocks (per-token value loads) run two;
// bf16 pools with 64-token blocks and head size 128 run one; FP8 pools with
// several query tokens per sequence (per-row causal limits) one less.  The
// fp32 variants (larger operands) are left unconstrained.
constexpr int decode_waves_per_eu(int elem, int HS, int BS, bool F8, bool MQ)
{
    if (elem != 2)
        return 1;
    int w = BS == 1 ? 2 : (BS <= 16 ? 3 : 2);
    if (F8 && MQ)
        w -= 1;
    return w < 1 ? 1 : w;
}
#define PKV_OCCUPANCY __attribute__((amdgpu_waves_per_eu(decode_waves_per_eu(sizeof(T), HS, BS, F8, MQ))))

// T: element type of q and out (and of the pools unless F8).  F8: the pools
// hold E4M3 codes (T is bf16); keys are read as code * k_scale (folded into
// qscale) and values as code * v_scale (oscale, applied to the output).
//
// MQ: several query tokens per sequence (a prefill chunk, or the draft
// tokens of speculative decoding).  Sequence s has the n = q_start[s+1] -
// q_start[s] query rows q_start[s] .. q_start[s+1]-1 of q and out; they are
// its last n tokens, so row i sits at position L - n + i and attends the
// tokens at positions 0 .. L - n + i (causal).  The (row, group member)
// pairs rho = i * G + g form the MFMA tile's rows, 16 per tile: work-group
// x = kvh * RT + rt takes rows 16 rt .. 16 rt + 15 of KV head kvh.  Without
// MQ, sequence s has the one query row s at position L - 1 and the tile's
// rows are the G heads of the group.
template <typename T, int HS, int BS, int NW, bool F8, bool MQ>
__global__ __launch_bounds__(NW * 64) PKV_OCCUPANCY void paged_decode_partition_kernel(
    const T* __restrict__ q, const typename std::conditional<F8, uint8_t, T>::type* __restrict__ k_cache,
    const typename std::conditional<F8, uint8_t, T>::type* __restrict__ v_cache,
    const int32_t* __restrict__ block_tables,
    const int32_t* __restrict__ seq_lens, int32_t Hq, int32_t Hkv,
    int32_t M, int32_t num_blocks, int32_t PB, int32_t max_parts, int32_t interleave, int32_t lpt, float qscale,
    const int32_t* __restrict__ sched_order, const int32_t* __restrict__ sched_lens,
    const int32_t* __restrict__ sched_tables, float oscale, void* __restrict__ out, int32_t out_f32,
    float* __restrict__ ws_o, float* __restrict__ ws_ml, const int32_t* __restrict__ q_start, int32_t num_q_rows,
    int32_t max_q_len, int32_t RT, const int32_t* __restrict__ sched_count, const uint32_t* __restrict__ sched_items,
    int32_t rank_in_z, DecodeArgs::StepAppend sa)
{
    using C = typename std::conditional<F8, uint8_t, T>::type;  // pool element type
    static_assert(!F8 || sizeof(T) == 2, "FP8 pools are read with bf16 queries");
    constexpr bool kWide = sizeof(T) == 2 && BS >= 32;  // 32-token units (see WideRegs, Fp8WideRegs)
    constexpr bool kSmall = BS < 16;                    // several blocks per unit (see load_small)
    static_assert(!(kSmall && F8), "FP8 pools need blocks of at least 16 tokens");
    constexpr int UT = kWide ? 32 : 16;                 // tokens per pipeline unit
    constexpr int PER = kSmall ? 1 : BS / UT;           // units per block
    constexpr int TILE = HS * BS;                       // elements per (block, KV head) tile
    __shared__ __attribute__((aligned(16))) float sm_out[NW][16 * HS];  // partition results, for the merge
    __shared__ float sm_m[NW][16];
    __shared__ float sm_l[NW][16];
    __shared__ int sm_pick;
    static_assert(kLptMaxSeqs <= NW * 16 * HS && kLptMaxSeqs <= 256,
                  "the length ranking reuses the merge buffer and keeps the index in 8 bits");

    // Work-group -> (KV head, row tile, rank y, chunk).  With the schedule's
    // chunk list (1-D grid, large batches): work-group x takes (KV head, row
    // tile) pair x % HR of listed chunk x / HR (HR = Hkv, times the row tiles
    // with MQ), so the largest chunks start first,
    // whichever sequence they belong to, and the unused work-groups (chunks
    // past the list's end) come last.  Otherwise blockIdx.x covers the KV
    // heads (and row tiles) and y, z the ranks and chunks: rank in z (chunks
    // of one sequence consecutive) for small batches, where few work-groups
    // find themselves past their sequence's end, rank in y otherwise.
    // Decode step in one launch (sa.k set): a 1-D grid whose first
    // S * Hkv * max_parts work-groups are the attention's, in the order of
    // the 3-D grid (KV head, then chunk, then rank), followed by sa.groups
    // work-groups per sequence that store its new token.  Placed last, the
    // stores fill the slots the attention's tail leaves free (placed first,
    // they delayed the attention's first work-groups).
    // S_grid: the sequences of this launch.
    int kvh, rt = 0, yr, chunk, s_listed = 0, S_grid;
    if (!MQ && sa.k) {
        static_assert(NW * 64 == kStoreThreads, "a store work-group is one attention work-group");
        const int per_seq = Hkv * max_parts;
        S_grid = (int)(gridDim.x / (unsigned)(per_seq + sa.groups));
        const int bx = blockIdx.x;
        if (bx >= S_grid * per_seq) {  // uniform: before any barrier
            using E = typename std::conditional<F8, uint8_t,
                                                typename std::conditional<sizeof(T) == 2, uint16_t, uint32_t>::type>::type;
            const int t = bx - S_grid * per_seq;
            store_token<E, true>(t / sa.groups, t % sa.groups, (const u32x4*)sa.k, (const u32x4*)sa.v,
                                 sa.slot_mapping, block_tables, seq_lens, M, (u32x4*)sa.k_cache, (E*)sa.v_cache, Hkv,
                                 HS, BS, num_blocks, sa.k_inv_scale, sa.v_inv_scale);
            return;
        }
        kvh = bx % Hkv;
        const int rest = bx / Hkv;
        chunk = rest % max_parts;
        yr = rest / max_parts;
    } else if (sched_items) {
        const int HR = MQ ? Hkv * RT : Hkv;  // (KV head, row tile) pairs
        const int item = blockIdx.x / HR;
        const int xr = blockIdx.x - item * HR;
        kvh = MQ ? xr / RT : xr;
        rt = MQ ? xr - kvh * RT : 0;
        if (item >= *sched_count)
            return;  // uniform, before any barrier
        const uint2 it = reinterpret_cast<const uint2*>(sched_items)[item];
        yr = (int)(it.x & 0xFFFFu);
        chunk = (int)(it.x >> 16);
        s_listed = (int)it.y;  // the sequence of rank yr, without another dependent load
        // a list that does not belong to this launch (caller error) must not
        // send a work-group outside its sequences or chunks
        S_grid = (int)(gridDim.x / ((unsigned)HR * max_parts));
        if (yr >= S_grid || chunk >= max_parts || (unsigned)s_listed >= (unsigned)S_grid)
            return;
    } else {
        kvh = MQ ? blockIdx.x / RT : blockIdx.x;
        rt = MQ ? blockIdx.x - kvh * RT : 0;  // row tile
        yr = rank_in_z ? blockIdx.z : blockIdx.y;
        chunk = rank_in_z ? blockIdx.y : blockIdx.z;
        S_grid = (int)(rank_in_z ? gridDim.z : gridDim.y);
    }
    const int lane = threadIdx.x & 63;
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // wave index, kept scalar
    const int part = chunk * NW + w;                                   // this wave's partition
    const int r = lane >> 4;
    const int c = lane & 15;
    const int G = Hq / Hkv;

    // Longest sequences first.  Work-groups start roughly in blockIdx order,
    // so a long sequence that happens to sit at the end of the batch would
    // run alone after everything else has finished.  Instead, blockIdx.y = y
    // takes the sequence of rank y in decreasing length (ties by index).
    // Each sequence's result does not depend on which work-group computes it.
    // - Decode step: its append launch has written the order, and the lengths
    //   and table rows in that order, so y alone addresses all three.
    // - Stand-alone call on a small batch (lpt): every work-group ranks the
    //   batch in LDS (the merge buffer, unused until the merge) by the key
    //   (blocks << 8) | (255 - index), distinct per sequence, and keeps the
    //   one of rank y.  Only the first chunk of each sequence is placed
    //   this way (later chunks take sequence y): a work-group of a later
    //   chunk learns that its sequence has no such chunk from one length
    //   load.
    int s = yr;
    bool s_ok = true;  // false: a schedule entry outside the batch
    if (sched_order) {
        // schedule given (decode step): rank y's sequence, length and table
        // row are read below from y alone.  An order that does not belong
        // to this batch (caller error) must not send the work-group to a
        // sequence outside it: q and q_start are read at sequence 0 instead
        // and the work-group takes the empty-sequence exit below without
        // storing anything.  (A return of its own here costs the FP8
        // variants registers: the compiler then holds the prologue's loads
        // back.)
        s = sched_items ? s_listed : sched_order[yr];
        s_ok = (unsigned)s < (unsigned)S_grid;
        s = s_ok ? s : 0;
    } else if (lpt && chunk == 0) {
        const int S = S_grid;  // <= kLptMaxSeqs = 64, M < 2^23 (checked on the host)
        unsigned* sm_key = reinterpret_cast<unsigned*>(&sm_out[0][0]);
        const int cap = M * BS;
        for (int i = threadIdx.x; i < S; i += NW * 64) {
            const int v = seq_lens[i];
            const int Lc = v < 0 ? 0 : (v > cap ? cap : v);
            sm_key[i] = ((unsigned)((Lc + BS - 1) / BS) << 8) | (unsigned)(255 - i);
        }
        __syncthreads();
        for (int cand = threadIdx.x; cand < S; cand += NW * 64) {
            const unsigned key = sm_key[cand];
            int rank = 0;
            const uint4* keys4 = reinterpret_cast<const uint4*>(sm_key);
            for (int j4 = 0; j4 < (S + 3) / 4; ++j4) {  // keys past S are never read: S % 4 handled below
                const uint4 k4 = keys4[j4];
                const int j = 4 * j4;
                rank += (k4.x > key) ? 1 : 0;
                rank += (j + 1 < S && k4.y > key) ? 1 : 0;
                rank += (j + 2 < S && k4.z > key) ? 1 : 0;
                rank += (j + 3 < S && k4.w > key) ? 1 : 0;
            }
            if (rank == yr)
                sm_pick = cand;
        }
        __syncthreads();
        s = sm_pick;
    }

    // This wave's blocks: base, base + stride, ... (nb_w of them, <= PB).
    // Contiguous mode: partition `part` = PB consecutive blocks.  Interleaved
    // mode: the chunk's blocks dealt round-robin to the NW waves, which keeps
    // the waves balanced when a sequence ends inside the chunk.  With several
    // units per block (B = 64) the units are dealt instead, so that a short
    // sequence's few blocks still spread over all waves: unit k of the chunk
    // goes to wave k % NW, which then holds part w % PER of every
    // (NW / PER)-th block (its list has up to PER * PB blocks, at most 64).
    // A wave with no blocks still joins the work-group merge below.
    // (Blocks smaller than a unit always use contiguous partitions: a unit's
    // tokens are then consecutive.)
    const int cb0 = chunk * NW * PB;
    const bool ilv = !kSmall && interleave;
    constexpr bool kUnitDeal = !kSmall && PER > 1 && NW % PER == 0;
    const bool deal = kUnitDeal && ilv && PB * PER <= 64;  // uniform
    const int base = deal ? cb0 + w / PER : (ilv ? cb0 + w : part * PB);
    const int stride = deal ? NW / PER : (ilv ? NW : 1);
    const int wpart = deal ? w % PER : 0;  // the part of each block this wave takes (unit dealing)
    const int nlist = deal ? PB * PER : PB;  // entries of this wave's block list
    // Physical block IDs of this wave's blocks, one per lane (the first 64;
    // small blocks keep the rest in windows, below); the tile loop
    // broadcasts them with readlane.  Loaded for all nlist lanes
    // within the table row, without waiting for the sequence length, so
    // that this load and the length load are in flight together; entries
    // past the sequence's blocks are never used.
    const int tb = base + lane * stride;
    const int32_t* trow = sched_order ? sched_tables + (int64_t)yr * M : block_tables + (int64_t)s * M;
    const int32_t id_lane = (lane < nlist && tb < M) ? trow[tb] : 0;
    // Blocks of fewer than 16 tokens: a partition of up to 512 tokens holds
    // more than 64 blocks (B = 1), so its list is kept in windows of 64
    // entries, window k in idw[k] (idw[0] = id_lane), all loaded here; the
    // tile loop moves to the next window by shifting them down.
    constexpr int NWIN = kSmall ? 512 / (64 * BS) : 1;
    int32_t idw[NWIN];
    idw[0] = id_lane;
#pragma unroll
    for (int k = 1; k < NWIN; ++k) {
        const int e = 64 * k + lane;  // list entry
        idw[k] = (e < nlist && base + e < M) ? trow[base + e] : 0;
    }
    // The length is loaded next, before anything waits (the query-row bounds
    // below may end the work-group), so that both loads are in flight at once.
    const int L_in = sched_order ? sched_lens[yr] : seq_lens[s];

    // Query rows: qs0 .. qs0 + n - 1 (MQ), else row s alone.  Rows outside
    // 0 .. num_q_rows - 1 or beyond max_q_len are never read or written.
    int qs0 = s, n = 1;
    if constexpr (MQ) {
        qs0 = q_start[s];
        const int qs1 = q_start[s + 1];
        n = qs1 - qs0;
        if (qs0 < 0 || n < 0 || qs1 > num_q_rows)
            n = 0;
        n = n < max_q_len ? n : max_q_len;
    }
    const int nrows = n * G;  // (row, group member) pairs
    const int tile_rows = MQ ? (nrows - 16 * rt < 16 ? nrows - 16 * rt : 16) : G;  // this tile's real rows
    if constexpr (MQ) {
        if (tile_rows <= 0)
            return;  // uniform: before any barrier
    }

    const int L = (L_in < 0 || !s_ok) ? 0 : (L_in > M * BS ? M * BS : L_in);
    // row rho of the tile, as (query row, head) of out
    auto out_row = [&](int rho) __attribute__((always_inline)) -> int64_t {
        const int i = rho / G;
        return ((int64_t)(qs0 + i) * Hq + (int64_t)kvh * G + (rho - i * G)) * HS;
    };
    if (L == 0) {
        if (chunk == 0 && w == 0 && s_ok) {
            if constexpr (MQ) {
                for (int idx = lane; idx < tile_rows * HS; idx += 64)
                    store_out<T>(out, out_row(16 * rt + idx / HS) + idx % HS, 0.f, out_f32);
            } else {
                for (int idx = lane; idx < G * HS; idx += 64)
                    store_out<T>(out, ((int64_t)s * Hq + (int64_t)kvh * G) * HS + idx, 0.f, out_f32);
            }
        }
        return;
    }
    const int nblk = (L + BS - 1) / BS;
    if (cb0 >= nblk)
        return;  // the whole work-group is past the end (uniform: before any barrier)
    const int nchunks = (nblk + NW * PB - 1) / (NW * PB);
    const int cnb = (nblk - cb0 < NW * PB) ? nblk - cb0 : NW * PB;
    const int nb_w = deal ? (cnb > w / PER ? (cnb - w / PER + stride - 1) / stride : 0)
                     : ilv ? (cnb > w ? (cnb - w + NW - 1) / NW : 0)
                           : (base >= nblk ? 0 : ((nblk - base < PB) ? nblk - base : PB));

    // query operand: row c of the tile.  Rows past the tile's real rows are
    // padding: they repeat a real row (head c % G without MQ), and their
    // results are never stored.  (Loading real rows rather than zeroing them
    // keeps the query registers free of any use before the tile loop, so the
    // first tile's loads are issued while the query loads are in flight.)
    // Lq: this lane's row sees the tokens below Lq; Lmin: the least of those
    // over the tile (the first query row's limit; L without MQ).
    const int rho_c = MQ ? (16 * rt + c) % nrows : c % G;
    const int Lq = MQ ? L - n + rho_c / G + 1 : L;
    const int Lmin = MQ ? L - n + (16 * rt) / G + 1 : L;
    typename Ops<T>::template QReg<HS> qr;
    {
        const T* qh = q + (MQ ? out_row(rho_c) : ((int64_t)s * Hq + (int64_t)kvh * G + c % G) * HS);
        if constexpr (F8) {
            // operand 2i + h holds dims (4i + r)*16 + 8h .. +7 (the FP8 key order)
#pragma unroll
            for (int i = 0; i < HS / 64; ++i)
#pragma unroll
                for (int h = 0; h < 2; ++h)
                    qr.v[2 * i + h] = *(const bf16x8*)(qh + (4 * i + r) * 16 + 8 * h);
        } else if constexpr (sizeof(T) == 2) {
#pragma unroll
            for (int i = 0; i < HS / 32; ++i)
                qr.v[i] = *(const bf16x8*)(qh + 32 * i + 8 * r);
        } else {
#pragma unroll
            for (int i = 0; i < HS / 16; ++i)
                qr.v[i] = *(const f32x4*)(qh + 16 * i + 4 * r);
        }
    }

    // Decode step in one launch: the new token (position L - 1) comes from
    // sa.k / sa.v.  It is patched in only where the store writes it: the
    // length inside the table row (L == L_in) and the unit's block inside the
    // pool (checked with the unit).  Each wave of the chunk holding it copies
    // it to the end of the wave's own slice of the merge buffer, which only
    // the merge uses again, after the tile loop; no other wave reads the
    // copy, so it needs no barrier.
    const bool patch = !MQ && sa.k != nullptr && L == L_in;
    const int tokp = L - 1;
    const bool stash = patch && tokp / BS >= cb0 && tokp / BS < cb0 + NW * PB;
    T* const st = reinterpret_cast<T*>(&sm_out[w][16 * HS]) - 2 * HS;  // key, then value
    constexpr int kStashWords = 2 * HS * (int)sizeof(T) / 4;           // 64, 128 or 256
    uint32_t stw[kStashWords / 64];
    if (stash) {
        const int64_t row = ((int64_t)s * Hkv + kvh) * HS;
        const uint32_t* srck = reinterpret_cast<const uint32_t*>(static_cast<const T*>(sa.k) + row);
        const uint32_t* srcv = reinterpret_cast<const uint32_t*>(static_cast<const T*>(sa.v) + row);
#pragma unroll
        for (int k = 0; k < kStashWords / 64; ++k) {
            const int idx = lane + 64 * k;
            stw[k] = idx < kStashWords / 2 ? srck[idx] : srcv[idx - kStashWords / 2];
        }
    }

    f32x4 O[HS / 16];
#pragma unroll
    for (int i = 0; i < HS / 16; ++i)
        O[i] = (f32x4)0.f;
    // running max for head c, log2 units; finite start so that a fully
    // masked tile gives exp2(-inf - m_run) = 0 rather than NaN
    float m_run = -1e30f;
    float l_part = 0.f;       // sum of probabilities of this lane's tokens

    const int64_t head_off = (int64_t)kvh * TILE;
    const int64_t block_stride = (int64_t)Hkv * TILE;

    auto tile_ptr_ok = [&](int j, const C*& tk, const C*& tv) __attribute__((always_inline)) -> bool {
        int32_t id = __builtin_amdgcn_readlane(id_lane, j);
        const bool ok = (uint32_t)id < (uint32_t)num_blocks;
        id = ok ? id : 0;
        tk = k_cache + (int64_t)id * block_stride + head_off;
        tv = v_cache + (int64_t)id * block_stride + head_off;
        return ok;
    };

    // Online-softmax update shared by both unit shapes: mx is this lane's
    // maximum over its valid scores (log2 units).  Raises the running maximum
    // only when mx exceeds it by more than kRescaleSlack.
    auto update_max = [&](float mx) __attribute__((always_inline)) {
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
    };

    // One 16-token sub-tile: scores, online softmax update, value sum.
    // tok0 is the sub-tile's first token; an out-of-range block ID was
    // replaced by block 0 and its tokens are all masked (valid below Lt), so
    // the loaded registers are consumed on every path.
    // Scores of tokens at or past the lane's row limit (Lq, or tok0 for an
    // invalid block) are masked; values are zeroed from the sequence end on
    // (Lv), where the slots may hold anything.
    // Small blocks: tmask marks the unit's tokens whose block ID is inside
    // the pool (ok: all of them).
    auto compute = [&](TileRegs<T, HS>& t, int tok0, bool ok, int tmask) __attribute__((always_inline)) {
        const int Lt = (kSmall || ok) ? Lq : tok0;
        const int Lv = (kSmall || ok) ? L : tok0;
        const bool partial = tok0 + 16 > ((kSmall || ok) ? Lmin : tok0) || (kSmall && !ok);
        const f32x4 S = tile_scores<T, HS>(t.k, qr);
        float sc[4];
        float mx = -INFINITY;
#pragma unroll
        for (int jj = 0; jj < 4; ++jj)
            sc[jj] = S[jj] * qscale;
        if (partial) {
            asm volatile("");  // a real branch: most tiles need no masking
#pragma unroll
            for (int jj = 0; jj < 4; ++jj)
                sc[jj] = (tok0 + 4 * r + jj < Lt && ((tmask >> (4 * r + jj)) & 1)) ? sc[jj] : -INFINITY;
        }
#pragma unroll
        for (int jj = 0; jj < 4; ++jj)
            mx = fmaxf(mx, sc[jj]);
        if (partial)
            zero_masked_values<T, HS>(t, tok0, Lv, r, tmask);
        update_max(mx);
        float p[4];
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
            p[jj] = __builtin_amdgcn_exp2f(sc[jj] - m_run);
            l_part += p[jj];
        }
        tile_pv<T, HS>(O, p, t.v);
    };

    // One 32-token unit (bf16, B = 32): element jj of M-tile mp's scores is
    // token 16mp + 4r + jj; value element e of a lane is token 8r + e (the
    // probabilities are moved to that order by to_value_order).
    auto compute_wide = [&](WideRegs<HS>& t, int tok0, bool ok) __attribute__((always_inline)) {
        if constexpr (kWide) {
            const int Lt = ok ? Lq : tok0;
            const int Lv = ok ? L : tok0;
            const bool partial = tok0 + 32 > (ok ? Lmin : tok0);
            float sc[8];
            float mx = -INFINITY;
#pragma unroll
            for (int mp = 0; mp < 2; ++mp) {
                const f32x4 S = tile_scores<__bf16, HS>(t.k[mp], qr);
#pragma unroll
                for (int jj = 0; jj < 4; ++jj)
                    sc[4 * mp + jj] = S[jj] * qscale;
            }
            if (partial) {
                asm volatile("");  // a real branch: most units need no masking
#pragma unroll
                for (int mp = 0; mp < 2; ++mp)
#pragma unroll
                    for (int jj = 0; jj < 4; ++jj)
                        sc[4 * mp + jj] = (tok0 + 16 * mp + 4 * r + jj < Lt) ? sc[4 * mp + jj] : -INFINITY;
            }
#pragma unroll
            for (int k = 0; k < 8; ++k)
                mx = fmaxf(mx, sc[k]);
            if (partial) {
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const bool keep = tok0 + 8 * r + e < Lv;
#pragma unroll
                    for (int i = 0; i < HS / 16; ++i)
                        t.v[i][e] = keep ? t.v[i][e] : (__bf16)0.f;
                }
            }
            update_max(mx);
            float pv[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                pv[e] = __builtin_amdgcn_exp2f(sc[e] - m_run);
                l_part += pv[e];
            }
#pragma unroll
            for (int jj = 0; jj < 4; ++jj)
                to_value_order(pv[jj], pv[4 + jj]);  // pv[e] is now token 8r + e
            bf16x8 hi, lo;
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const __bf16 hb = (__bf16)pv[e];
                hi[e] = hb;
                lo[e] = (__bf16)(pv[e] - (float)hb);
            }
#pragma unroll
            for (int i = 0; i < HS / 16; ++i) {
                O[i] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(hi, t.v[i], O[i], 0, 0, 0);
                O[i] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(lo, t.v[i], O[i], 0, 0, 0);
            }
        }
    };

    // Software pipeline over the partition's units (UT tokens each): unit u
    // is part part_of(u) of list block j_of(u).  The next unit's
    // loads are in flight while the current one is computed.  The
    // steady-state loop always prefetches and the last one or two units are
    // peeled, so every compute is preceded by exactly one batch of loads and
    // the memory-counter waits stay precise.
    using Regs = typename std::conditional<
        F8, typename std::conditional<kWide, Fp8WideRegs<HS>, Fp8Regs<HS>>::type,
        typename std::conditional<kWide, WideRegs<HS>, TileRegs<T, HS>>::type>::type;
    // 0 for a wave past the end
    const int nunits = kSmall ? (nb_w * BS + UT - 1) / UT : (deal ? nb_w : nb_w * PER);
    // unit u: block j_of(u) of this wave's list, part part_of(u) of it
    auto j_of = [&](int u) __attribute__((always_inline)) { return deal ? u : u / PER; };
    auto part_of = [&](int u) __attribute__((always_inline)) { return deal ? wpart : u % PER; };
    // small blocks: bit j set when block j of the current window is inside the pool
    uint64_t valid_blocks = kSmall ? __ballot((uint32_t)id_lane < (uint32_t)num_blocks) : 0;
    int cur_win = 0;  // the window idw[0] holds (small blocks)
    // returns the unit's token mask (all 16 bits when every block is valid,
    // 0 for an invalid block of B >= 16)
    auto issue = [&](Regs& t, int u) __attribute__((always_inline)) -> int {
        if constexpr (kSmall) {
            // a window is 64 blocks, 4 * BS units; units are issued in
            // increasing order, so the next window is at most one step away
            constexpr int UPW = 4 * BS;
            if (NWIN > 1 && u / UPW != cur_win) {  // uniform
#pragma unroll
                for (int k = 0; k + 1 < NWIN; ++k)
                    idw[k] = idw[k + 1];
                ++cur_win;
                valid_blocks = __ballot((uint32_t)idw[0] < (uint32_t)num_blocks);
            }
            return load_small<T, HS, BS>(t, k_cache, v_cache, (int64_t)Hkv * TILE, (int64_t)kvh * TILE, idw[0],
                                         valid_blocks, num_blocks, u - cur_win * UPW, r, c);
        } else {
            const int j = j_of(u);
            const int m = part_of(u);
            const C* tk;
            const C* tv;
            const bool ok = tile_ptr_ok(j, tk, tv);
            if constexpr (F8 && kWide)
                load_fp8_wide<HS, BS>(t, tk, tv, m, r, c);
            else if constexpr (F8)
                load_fp8<HS, BS>(t, tk, tv, m, r, c);
            else if constexpr (kWide)
                load_wide<HS, BS>(t, tk, tv, m, r, c);
            else
                load_tile<T, HS, BS>(t, tk, tv, m, r, c);
            return ok ? 0xFFFF : 0;
        }
    };
    auto first_token = [&](int u) __attribute__((always_inline)) {
        return kSmall ? base * BS + UT * u : (base + j_of(u) * stride) * BS + UT * part_of(u);
    };
    auto run = [&](Regs& t, int u, int tmask) __attribute__((always_inline)) {
        const int tok0 = first_token(u);
        if constexpr (!MQ) {
            const int p = tokp - tok0;  // the new token's place in the unit
            if (patch && p >= 0 && p < UT && ((tmask >> (kSmall ? p : 0)) & 1))  // uniform
                patch_token(t, st, st + HS, p, r, c, sa.k_inv_scale, sa.v_inv_scale);
        }
        const bool ok = tmask == 0xFFFF;
        if constexpr (F8 && kWide) {
            WideRegs<HS> op;  // the raw codes as bf16 operands
            fp8_wide_to_operands<HS>(t, op);
            compute_wide(op, tok0, ok);
        } else if constexpr (kWide) {
            compute_wide(t, tok0, ok);
        } else if constexpr (F8) {
            TileRegs<__bf16, HS> op;  // the raw codes as bf16 operands
            fp8_to_operands<HS>(t, op);
            compute(op, tok0, ok, 0xFFFF);
        } else {
            compute(t, tok0, ok, kSmall ? tmask : 0xFFFF);
        }
    };
    if (nunits > 0) {
        Regs ta, tb;
        int ok_a = issue(ta, 0);
        if (stash) {  // after the first unit's loads, so that they are not held back
            uint32_t* sw = reinterpret_cast<uint32_t*>(st);
#pragma unroll
            for (int k = 0; k < kStashWords / 64; ++k)
                sw[lane + 64 * k] = stw[k];
            __builtin_amdgcn_wave_barrier();
        }
        int ok_b = 0;
        int u = 0;
        for (; u + 2 < nunits; u += 2) {
            ok_b = issue(tb, u + 1);
            run(ta, u, ok_a);
            ok_a = issue(ta, u + 2);
            run(tb, u + 1, ok_b);
        }
        if (u + 1 < nunits) {
            ok_b = issue(tb, u + 1);
            run(ta, u, ok_a);
            run(tb, u + 1, ok_b);
        } else {
            run(ta, u, ok_a);
        }
    }

    // ---- merge the work-group's partitions (log-sum-exp) ----
    // Each wave stages its partition's normalised tile_rows x HS result and
    // the (m, l) of each row in LDS; the work-group then combines them with
    // weights l_w * 2^(m_w - M) and writes one block per (sequence, KV head,
    // row tile, chunk): the final output when the sequence has a single
    // chunk, otherwise a partial for the chunk merge kernel.
    float l_tot = l_part + __shfl_xor(l_part, 16);
    l_tot += __shfl_xor(l_tot, 32);
    if (r == 0) {
        sm_m[w][c] = m_run;
        sm_l[w][c] = l_tot;
    }
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) {
        const int g = 4 * r + jj;  // tile row
        const float l_g = __shfl(l_tot, g);
        const float inv = l_g > 0.f ? oscale / l_g : 0.f;  // oscale: 1, or the FP8 value scale
        if (g < tile_rows) {
#pragma unroll
            for (int i = 0; i < HS / 16; ++i)
                sm_out[w][g * HS + 16 * i + c] = O[i][jj] * inv;
        }
    }
    // LDS-only barrier: the merge exchanges nothing through global memory
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");

    // partial blocks: [S][Hkv][RT][max_parts] of RPB rows each
    constexpr int RPB_MQ = 16;
    const int RPB = MQ ? RPB_MQ : G;
    const int64_t blk = (((int64_t)s * Hkv + kvh) * (MQ ? RT : 1) + rt) * max_parts + chunk;
    for (int e = threadIdx.x; e < tile_rows * HS / 4; e += NW * 64) {  // 4 consecutive elements of tile row g
        const int g = (4 * e) / HS;
        float mx = -INFINITY;
#pragma unroll
        for (int ww = 0; ww < NW; ++ww)
            if (sm_l[ww][g] > 0.f)
                mx = fmaxf(mx, sm_m[ww][g]);
        float lsum = 0.f;
        f32x4 acc = (f32x4)0.f;
#pragma unroll
        for (int ww = 0; ww < NW; ++ww)
            if (sm_l[ww][g] > 0.f) {
                const float f = sm_l[ww][g] * __builtin_amdgcn_exp2f(sm_m[ww][g] - mx);
                lsum += f;
                acc += f * *(const f32x4*)(&sm_out[ww][4 * e]);
            }
        const float inv = lsum > 0.f ? 1.f / lsum : 0.f;
        acc *= inv;
        if (nchunks == 1) {
            // without MQ the group's G heads are adjacent rows of out
            store_out4<T>(out,
                          MQ ? out_row(16 * rt + g) + (4 * e) % HS : ((int64_t)s * Hq + (int64_t)kvh * G) * HS + 4 * e,
                          acc, out_f32);
        } else {
            *(f32x4*)(ws_o + blk * RPB * HS + 4 * e) = acc;
            if ((4 * e) % HS == 0) {
                float2 ml;
                ml.x = mx;
                ml.y = lsum;
                *(float2*)(ws_ml + (blk * RPB + g) * 2) = ml;
            }
        }
    }
}

// Merge of the context partitions of one (sequence, query head):
// M = max m_p, w_p = l_p * 2^(m_p - M), out = sum w_p o_p / sum w_p
// (o_p is already normalised by l_p; partitions whose tiles were all masked
// carry l_p = 0 and get weight 0).  Sequences with one partition were
// written by the partition kernel and are skipped here.
//
// A long context has dozens to hundreds of partitions per head, so the work
// is spread over the work-group in one pass: thread t takes head dims
// 4 (t % (HS/4)) .. + 3 of partitions t / (HS/4), + R, + 2R, ... (R groups of
// HS/4 threads), loading kMergeBatch partitions' (m, l) and 16-byte o at a
// time with no load waiting on another, and keeps its own running maximum
// (acc and the weight sum rescaled when it rises, as in the online softmax).
// The R groups' (m, weight sum, acc) are then combined by the same rule
// through LDS.  The result equals the formula above up to the order of the
// fp32 sums.
constexpr int kMergeThreads = 256;
constexpr int kMergeBatch = 4;

// Persistent over (sequence rank, query head) pairs: work-group b takes
// pairs b, b + gridDim.x, ...  Rank y is the y-th sequence of the
// longest-first schedule when one is given (the sequences that span several
// chunks come first, so the work spreads over the first work-groups), else
// sequence y.  Pairs of single-chunk sequences are skipped.
constexpr int kMergeGroups = 2048;

template <typename T, int HS>
__global__ __launch_bounds__(kMergeThreads) void paged_decode_reduce_kernel(
    const int32_t* __restrict__ seq_lens, const int32_t* __restrict__ sched_order,
    const int32_t* __restrict__ sched_lens, int32_t S, int32_t M, int32_t BS, int32_t CB, int32_t Hq, int32_t Hkv,
    int32_t max_parts, const float* __restrict__ ws_o, const float* __restrict__ ws_ml, void* __restrict__ out,
    int32_t out_f32)
{
    constexpr int Q = HS / 4;               // threads per partition row (4 head dims each)
    constexpr int R = kMergeThreads / Q;    // partition groups
    __shared__ float sm_m[R][Q], sm_l[R][Q];
    __shared__ f32x4 sm_acc[R][Q];
    const int G = Hq / Hkv;
    const int q4 = threadIdx.x % Q;
    const int grp = threadIdx.x / Q;
    const int64_t pairs = (int64_t)S * Hq;
    for (int64_t pr = blockIdx.x; pr < pairs; pr += gridDim.x) {
        const int y = (int)(pr / Hq);
        const int h = (int)(pr - (int64_t)y * Hq);
        const int s = sched_order ? sched_order[y] : y;
        if ((unsigned)s >= (unsigned)S)
            continue;  // an order that does not belong to this batch: uniform, before any barrier
        int L = sched_order ? sched_lens[y] : seq_lens[s];
        L = L < 0 ? 0 : (L > M * BS ? M * BS : L);
        const int nblk = (L + BS - 1) / BS;
        const int nparts = (nblk + CB - 1) / CB;  // chunks of CB blocks
        if (nparts <= 1)
            continue;  // uniform: the partition kernel wrote this output
        // chunk p of head h = kvh * G + g: row g of block (s, kvh, p)
        const int kvh = h / G;
        const int g = h - kvh * G;
        const int64_t u0 = ((int64_t)s * Hkv + kvh) * max_parts;

        float m_t = -INFINITY, l_t = 0.f;
        f32x4 acc = (f32x4)0.f;
        for (int p0 = grp; p0 < nparts; p0 += kMergeBatch * R) {
            float2 ml[kMergeBatch];
            f32x4 o[kMergeBatch];
#pragma unroll
            for (int k = 0; k < kMergeBatch; ++k) {
                const int p = p0 + k * R;
                ml[k] = make_float2(0.f, 0.f);
                o[k] = (f32x4)0.f;
                if (p < nparts) {
                    const int64_t row = (u0 + p) * G + g;
                    ml[k] = *reinterpret_cast<const float2*>(ws_ml + 2 * row);
                    o[k] = *reinterpret_cast<const f32x4*>(ws_o + row * HS + 4 * q4);
                }
            }
#pragma unroll
            for (int k = 0; k < kMergeBatch; ++k) {
                if (ml[k].y > 0.f) {  // l_p > 0 (never true past nparts)
                    if (ml[k].x > m_t) {  // the running maximum rises: rescale what was summed
                        const float f = __builtin_amdgcn_exp2f(m_t - ml[k].x);  // 0 while m_t is -inf
                        acc *= f;
                        l_t *= f;
                        m_t = ml[k].x;
                    }
                    const float wgt = ml[k].y * __builtin_amdgcn_exp2f(ml[k].x - m_t);
                    acc += wgt * o[k];
                    l_t += wgt;
                }
            }
        }
        sm_m[grp][q4] = m_t;
        sm_l[grp][q4] = l_t;
        sm_acc[grp][q4] = acc;
        __syncthreads();
        if (threadIdx.x < Q) {
            float mx = -INFINITY;
#pragma unroll
            for (int k = 0; k < R; ++k)
                if (sm_l[k][q4] > 0.f)
                    mx = fmaxf(mx, sm_m[k][q4]);
            float wsum = 0.f;
            f32x4 tot = (f32x4)0.f;
#pragma unroll
            for (int k = 0; k < R; ++k)
                if (sm_l[k][q4] > 0.f) {
                    const float f = __builtin_amdgcn_exp2f(sm_m[k][q4] - mx);
                    wsum += sm_l[k][q4] * f;
                    tot += f * sm_acc[k][q4];
                }
            const float inv = wsum > 0.f ? 1.f / wsum : 0.f;
            store_out4<T>(out, ((int64_t)s * Hq + h) * HS + 4 * q4, tot * inv, out_f32);
        }
        __syncthreads();  // the LDS slots are reused by the next pair
    }
}

// Chunk merge for launches with few chunks per sequence (at most
// kFewChunks): one wave per (sequence rank, query head) pair, persistent over
// the pairs, each lane taking 4 consecutive head dims, loading every chunk's
// (m, l) and partial at once and summing the chunks in increasing order; no
// LDS, no barrier.  (With many chunks, the work-group
// of the kernel above spreads a pair's chunks over its threads instead.)
constexpr int kFewChunks = 8;
constexpr int kFewMergeWaves = 8192;

template <typename T, int HS>
__global__ __launch_bounds__(64) void paged_decode_reduce_few_kernel(
    const int32_t* __restrict__ seq_lens, const int32_t* __restrict__ sched_order,
    const int32_t* __restrict__ sched_lens, int32_t S, int32_t M, int32_t BS, int32_t CB, int32_t Hq, int32_t Hkv,
    int32_t max_parts, const float* __restrict__ ws_o, const float* __restrict__ ws_ml, void* __restrict__ out,
    int32_t out_f32)
{
    constexpr int Q = HS / 4;  // lanes with work: 4 head dims each
    const int G = Hq / Hkv;
    const int64_t pairs = (int64_t)S * Hq;
    for (int64_t pr = blockIdx.x; pr < pairs; pr += gridDim.x) {
        const int y = (int)(pr / Hq);
        const int h = (int)(pr - (int64_t)y * Hq);
        const int s = sched_order ? sched_order[y] : y;
        if ((unsigned)s >= (unsigned)S)
            continue;  // an order that does not belong to this batch
        int L = sched_order ? sched_lens[y] : seq_lens[s];
        L = L < 0 ? 0 : (L > M * BS ? M * BS : L);
        const int nblk = (L + BS - 1) / BS;
        const int nparts = (nblk + CB - 1) / CB;  // chunks of CB blocks
        if (nparts <= 1 || threadIdx.x >= Q)
            continue;  // single chunk: the partition kernel wrote this output
        const int kvh = h / G;
        const int g = h - kvh * G;
        const int d = 4 * threadIdx.x;
        const int64_t u0 = ((int64_t)s * Hkv + kvh) * max_parts;
        // every chunk's (m, l) and 16-byte partial in flight at once
        float2 ml[kFewChunks];
        f32x4 o[kFewChunks];
#pragma unroll
        for (int p = 0; p < kFewChunks; ++p) {
            ml[p] = make_float2(0.f, 0.f);
            o[p] = (f32x4)0.f;
            if (p < nparts) {
                const int64_t row = (u0 + p) * G + g;
                ml[p] = *(const float2*)(ws_ml + 2 * row);
                o[p] = *(const f32x4*)(ws_o + row * HS + d);
            }
        }
        float mx = -INFINITY;
#pragma unroll
        for (int p = 0; p < kFewChunks; ++p)
            if (ml[p].y > 0.f)
                mx = fmaxf(mx, ml[p].x);
        float wsum = 0.f;
        f32x4 acc = (f32x4)0.f;
#pragma unroll
        for (int p = 0; p < kFewChunks; ++p) {  // in increasing chunk order
            const float wgt = ml[p].y > 0.f ? ml[p].y * __builtin_amdgcn_exp2f(ml[p].x - mx) : 0.f;
            wsum += wgt;
            acc += wgt * o[p];
        }
        f32x4 res;
#pragma unroll
        for (int k = 0; k < 4; ++k)
            res[k] = wsum > 0.f ? acc[k] / wsum : 0.f;
        store_out4<T>(out, ((int64_t)s * Hq + h) * HS + d, res, out_f32);
    }
}

// Chunk merge for several query rows per sequence: one work-group per
// (row tile, KV head, sequence), 16 threads per tile row, each owning 8
// consecutive head dims (two 16-byte loads per partial).  The row's running
// maxima are reduced over the chunks first, then every thread accumulates
// its dims over all chunks with weights l_p * 2^(m_p - M).
template <typename T, int HS>
__global__ __launch_bounds__(256) void paged_multi_token_reduce_kernel(
    const int32_t* __restrict__ seq_lens, int32_t M, int32_t BS, int32_t CB, int32_t Hq, int32_t Hkv,
    int32_t max_parts, const float* __restrict__ ws_o, const float* __restrict__ ws_ml, void* __restrict__ out,
    int32_t out_f32, const int32_t* __restrict__ q_start, int32_t num_q_rows, int32_t max_q_len, int32_t RT)
{
    static_assert(HS % 16 == 0 && HS / 16 <= 8, "16 threads per row, at most 8 dims each");
    constexpr int DPT = HS / 16;  // head dims per thread
    const int rt = blockIdx.x, kvh = blockIdx.y, s = blockIdx.z;
    const int G = Hq / Hkv;
    const int qs0 = q_start[s], qs1 = q_start[s + 1];
    int n = qs1 - qs0;
    if (qs0 < 0 || n < 0 || qs1 > num_q_rows)
        return;
    n = n < max_q_len ? n : max_q_len;
    int L = seq_lens[s];
    L = L < 0 ? 0 : (L > M * BS ? M * BS : L);
    const int nblk = (L + BS - 1) / BS;
    const int nparts = (nblk + CB - 1) / CB;
    if (nparts <= 1 || 16 * rt >= n * G)
        return;  // one chunk: the partition kernel wrote the rows
    const int rl = threadIdx.x / 16;          // tile row
    const int q = threadIdx.x % 16;           // dims q*DPT .. q*DPT + DPT - 1
    const int rho = 16 * rt + rl;
    const bool live = rho < n * G;
    const int64_t blk0 = (((int64_t)s * Hkv + kvh) * RT + rt) * max_parts;  // block of chunk 0
    float mx = -INFINITY;
    for (int p = q; p < nparts; p += 16) {
        const float2 ml = *(const float2*)(ws_ml + ((blk0 + p) * 16 + rl) * 2);
        if (ml.y > 0.f)
            mx = fmaxf(mx, ml.x);
    }
#pragma unroll
    for (int o = 8; o > 0; o >>= 1)
        mx = fmaxf(mx, __shfl_xor(mx, o, 16));
    float acc[DPT];
#pragma unroll
    for (int k = 0; k < DPT; ++k)
        acc[k] = 0.f;
    float wsum = 0.f;
    for (int p = 0; p < nparts; ++p) {
        const float2 ml = *(const float2*)(ws_ml + ((blk0 + p) * 16 + rl) * 2);
        const float wgt = ml.y > 0.f ? ml.y * __builtin_amdgcn_exp2f(ml.x - mx) : 0.f;
        wsum += wgt;
        const float* src = ws_o + ((blk0 + p) * 16 + rl) * HS + q * DPT;
#pragma unroll
        for (int k = 0; k < DPT; k += 4) {
            const f32x4 v = *(const f32x4*)(src + k);
            acc[k] += wgt * v[0];
            acc[k + 1] += wgt * v[1];
            acc[k + 2] += wgt * v[2];
            acc[k + 3] += wgt * v[3];
        }
    }
    if (!live)
        return;
    const float inv = wsum > 0.f ? 1.f / wsum : 0.f;
    const int i = rho / G;
    const int64_t dst = ((int64_t)(qs0 + i) * Hq + (int64_t)kvh * G + (rho - i * G)) * HS + q * DPT;
#pragma unroll
    for (int k = 0; k < DPT; k += 4)
        store_out4<T>(out, dst + k, (f32x4){acc[k] * inv, acc[k + 1] * inv, acc[k + 2] * inv, acc[k + 3] * inv},
                      out_f32);
}

template <typename T, int HS, int BS, bool F8, bool MQ>
static hipError_t launch_typed(const DecodeArgs& a, hipStream_t stream)
{
    constexpr int NW = kDecodeWaves;
    using C = typename std::conditional<F8, uint8_t, T>::type;
    const bool listed = a.sched_items != nullptr;
    const int rank_in_z = a.num_seqs <= kLptMaxSeqs ? 1 : 0;
    const int64_t HR = (int64_t)a.num_kv_heads * (MQ ? a.row_tiles : 1);  // (KV head, row tile) pairs
    const bool fused = !MQ && a.step_append.k != nullptr;
    const dim3 grid = fused ? dim3((unsigned)(a.num_seqs * (HR * a.max_parts + a.step_append.groups)))
                      : listed      ? dim3((unsigned)(HR * a.num_seqs * a.max_parts))
                      : rank_in_z ? dim3((unsigned)HR, a.max_parts, a.num_seqs)
                                  : dim3((unsigned)HR, a.num_seqs, a.max_parts);
    const float qscale = a.scale * kLog2e * (F8 ? a.k_scale : 1.0f);
    hipLaunchKernelGGL((paged_decode_partition_kernel<T, HS, BS, NW, F8, MQ>), grid, dim3(NW * 64), 0, stream,
                       (const T*)a.q, (const C*)a.k_cache, (const C*)a.v_cache, a.block_tables, a.seq_lens,
                       a.num_q_heads, a.num_kv_heads, a.max_blocks_per_seq, a.num_blocks, a.partition_blocks,
                       a.max_parts, a.interleave,
                       (a.num_seqs <= kLptMaxSeqs && a.max_blocks_per_seq < (1 << 23)) ? 1 : 0, qscale,
                       a.sched_order, a.sched_lens, a.sched_tables, F8 ? a.v_scale : 1.0f, a.out, a.out_f32, a.ws_o,
                       a.ws_ml, a.q_start, a.num_q_rows, a.max_q_len, a.row_tiles, a.sched_count, a.sched_items,
                       rank_in_z, a.step_append);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || a.max_parts <= 1)
        return e;  // one chunk per sequence: the partition kernel wrote the output
    if constexpr (MQ)
        hipLaunchKernelGGL((paged_multi_token_reduce_kernel<T, HS>), dim3(a.row_tiles, a.num_kv_heads, a.num_seqs),
                           dim3(256), 0, stream, a.seq_lens, a.max_blocks_per_seq, BS, a.partition_blocks * NW,
                           a.num_q_heads, a.num_kv_heads, a.max_parts, a.ws_o, a.ws_ml, a.out, a.out_f32, a.q_start,
                           a.num_q_rows, a.max_q_len, a.row_tiles);
    else if (a.max_parts <= kFewChunks)
        hipLaunchKernelGGL((paged_decode_reduce_few_kernel<T, HS>),
                           dim3((unsigned)std::min<int64_t>((int64_t)a.num_q_heads * a.num_seqs, kFewMergeWaves)),
                           dim3(64), 0, stream, a.seq_lens, a.sched_order, a.sched_lens, a.num_seqs,
                           a.max_blocks_per_seq, BS, a.partition_blocks * NW, a.num_q_heads, a.num_kv_heads,
                           a.max_parts, a.ws_o, a.ws_ml, a.out, a.out_f32);
    else
        hipLaunchKernelGGL((paged_decode_reduce_kernel<T, HS>),
                           dim3((unsigned)std::min<int64_t>((int64_t)a.num_q_heads * a.num_seqs, kMergeGroups)),
                           dim3(kMergeThreads), 0, stream, a.seq_lens, a.sched_order, a.sched_lens, a.num_seqs,
                           a.max_blocks_per_seq, BS, a.partition_blocks * NW, a.num_q_heads, a.num_kv_heads,
                           a.max_parts, a.ws_o, a.ws_ml, a.out, a.out_f32);
    return hipGetLastError();
}

template <typename T, int HS, int BS, bool F8>
static hipError_t launch_rows(const DecodeArgs& a, hipStream_t stream)
{
    return a.q_start ? launch_typed<T, HS, BS, F8, true>(a, stream) : launch_typed<T, HS, BS, F8, false>(a, stream);
}

template <typename T, int HS, bool F8>
static hipError_t launch_block(const DecodeArgs& a, hipStream_t stream)
{
    switch (a.block_size) {
    case 16: return launch_rows<T, HS, 16, F8>(a, stream);
    case 32: return launch_rows<T, HS, 32, F8>(a, stream);
    case 64: return launch_rows<T, HS, 64, F8>(a, stream);
    default:
        if constexpr (F8) {
            return hipErrorInvalidValue;  // rejected on the host: FP8 pools need B >= 16
        } else {
            return a.block_size == 8 ? launch_rows<T, HS, 8, F8>(a, stream) : launch_rows<T, HS, 1, F8>(a, stream);
        }
    }
}

template <typename T, bool F8>
static hipError_t launch_dtype(const DecodeArgs& a, hipStream_t stream)
{
    return a.head_size == 128 ? launch_block<T, 128, F8>(a, stream) : launch_block<T, 64, F8>(a, stream);
}

hipError_t launch_decode(const DecodeArgs& a, hipStream_t stream)
{
    switch (a.dtype) {
    case 1: return launch_dtype<__bf16, false>(a, stream);  // PKV_BF16
    case 2: return launch_dtype<__bf16, true>(a, stream);   // PKV_FP8_E4M3
    default: return launch_dtype<float, false>(a, stream);
    }
}

}  // namespace pkv
