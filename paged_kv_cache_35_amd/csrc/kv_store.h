// Storing one token's K/V into the pools, shared by the append launch
// (append.hip) and the attention launch of a fused decode step (decode.hip).
//
// Slot arithmetic follows the "writing new K/V" section of the "cache
// structure" page: slot = block_tables[s][pos / B] * B + pos % B, split back
// by the cache write as block_id = slot / B and offset = slot % B.  The copy
// is bit-exact for bf16 and fp32 pools (16-byte moves for keys, element
// moves for values); FP8 pools get the E4M3 code of each value (quantize16,
// quantize1).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "pkv_internal.h"

namespace pkv {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

// Slot of the newest token of a sequence (position L - 1), or -1 when the
// sequence is empty or the position falls outside its table row.
__device__ __forceinline__ int64_t decode_slot(const int32_t* __restrict__ block_tables,
                                               const int32_t* __restrict__ seq_lens, int32_t s,
                                               int32_t max_blocks_per_seq, int32_t block_size)
{
    const int32_t L = seq_lens[s];
    if (L <= 0)
        return -1;
    const int32_t pos = L - 1;
    const int32_t idx = pos / block_size;
    if (idx >= max_blocks_per_seq)
        return -1;
    const int64_t block = block_tables[(int64_t)s * max_blocks_per_seq + idx];
    return block < 0 ? -1 : block * block_size + (pos - idx * block_size);
}

// FP8 pools: the E4M3 codes of 16 bf16 values times inv_scale, as one
// 16-byte chunk.  The product is formed in fp32 and clamped to +-448 (the
// largest finite E4M3 magnitude), then v_cvt_pk_fp8_f32 rounds it to the
// nearest code, ties to the even mantissa (checked against the reference
// encoder on every tie and subnormal; without the clamp the conversion
// would give NaN from 464 up).
__device__ __forceinline__ u32x4 quantize16(const u32x4 (&in)[2], float inv_scale)
{
    u32x4 out;
#pragma unroll
    for (int w = 0; w < 4; ++w) {  // output word w: bf16 elements 4w .. 4w+3
        float f[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const unsigned word = in[w / 2][2 * (w % 2) + e / 2];
            const unsigned bits = (e & 1) ? (word & 0xFFFF0000u) : (word << 16);
            const float x = __builtin_bit_cast(float, bits) * inv_scale;
            f[e] = fminf(fmaxf(x, -448.0f), 448.0f);
        }
        int code = __builtin_amdgcn_cvt_pk_fp8_f32(f[0], f[1], 0, false);
        code = __builtin_amdgcn_cvt_pk_fp8_f32(f[2], f[3], code, true);
        out[w] = (unsigned)code;
    }
    return out;
}

// The E4M3 code of one bf16 value times inv_scale: the same product, clamp
// and rounding as one element of quantize16.
__device__ __forceinline__ uint8_t quantize1(uint16_t bf16_bits, float inv_scale)
{
    const float x = fminf(fmaxf(__builtin_bit_cast(float, (uint32_t)bf16_bits << 16) * inv_scale, -448.0f), 448.0f);
    return (uint8_t)(__builtin_amdgcn_cvt_pk_fp8_f32(x, x, 0, false) & 0xFF);
}

// Token i's K/V, part yy (of ceil(Hkv * hs / X / kStoreThreads)), stored by
// the kStoreThreads threads of one work-group.  E: pool element (uint8_t
// for FP8 codes with bf16 input, uint16_t for bf16, uint32_t for fp32).
// Keys: each thread moves one 16-byte chunk (chunk ci = yy * kStoreThreads
// + threadIdx.x of the token's Hkv * hs / X chunks); chunk f of KV head h
// lands at ((b*Hkv + h)*(hs/X) + f)*B*X + off*X.  Values: the same
// work-group moves the same X * kStoreThreads elements of the token's
// Hkv * hs, one element per thread and store, consecutive threads on
// consecutive head dims: element d of head h lands at ((b*Hkv + h)*hs + d)*B
// + off, so the 64 stores of a wave fall B elements apart and share cache
// lines (4 per 128-byte line at B = 16, bf16), where one 16-byte chunk per
// thread would send each store of the wave to 64 different lines.  The
// token's data is loaded before the slot is known, so the loads overlap the
// slot lookup.  FROM_TABLE: the slot is the decode slot of sequence i
// (computed from block_tables / seq_lens and also written to slot_mapping
// when that is non-null); otherwise it is read from slot_mapping.  A
// negative or out-of-range slot skips the token.
//
// The stores cover only part of each 32-byte sector (16 of 32 bytes of a key
// sector, 1, 2 or 4 bytes of a value row), and the memory system merges them
// with the old contents.  Writing whole sectors instead (reading the
// neighbouring bytes first) makes the append faster on its own, but the
// attention that follows slows down by more than that gain.
template <typename E, bool FROM_TABLE>
__device__ __forceinline__ void store_token(int32_t i, int32_t yy, const u32x4* __restrict__ k,
                                            const u32x4* __restrict__ v, int64_t* __restrict__ slot_mapping,
                                            const int32_t* __restrict__ block_tables,
                                            const int32_t* __restrict__ seq_lens, int32_t max_blocks_per_seq,
                                            u32x4* __restrict__ k_cache, E* __restrict__ v_cache,
                                            int32_t num_kv_heads, int32_t head_size, int32_t block_size,
                                            int32_t num_blocks, float k_inv_scale, float v_inv_scale)
{
    constexpr int X = 16 / sizeof(E);
    constexpr bool Q8 = sizeof(E) == 1;  // FP8 pools: bf16 input, 2 input pieces per pool chunk
    constexpr int IN = Q8 ? 2 : 1;
    using VIn = typename std::conditional<Q8, uint16_t, E>::type;  // one input value element
    const int32_t nchunks = num_kv_heads * (head_size / X);
    const int32_t nelem = num_kv_heads * head_size;
    const int32_t ci = yy * kStoreThreads + threadIdx.x;
    const int32_t e0 = yy * kStoreThreads * X + threadIdx.x;  // first value element
    const bool active = ci < nchunks;
    u32x4 kin[IN];
    VIn vin[X];
#pragma unroll
    for (int p = 0; p < IN; ++p) {
        kin[p] = (u32x4){0u, 0u, 0u, 0u};
        if (active)
            kin[p] = k[((int64_t)i * nchunks + ci) * IN + p];
    }
    const VIn* vrow = reinterpret_cast<const VIn*>(v) + (int64_t)i * nelem;
#pragma unroll
    for (int e = 0; e < X; ++e) {
        const int32_t idx = e0 + e * kStoreThreads;
        vin[e] = idx < nelem ? vrow[idx] : (VIn)0;
    }
    int64_t slot;
    if constexpr (FROM_TABLE) {
        slot = decode_slot(block_tables, seq_lens, i, max_blocks_per_seq, block_size);
        if (yy == 0 && threadIdx.x == 0 && slot_mapping)
            slot_mapping[i] = slot;
    } else {
        slot = slot_mapping[i];
    }
    if (slot >= 0 && slot / block_size < num_blocks) {  // out-of-range slot: skipped, never written
        const int64_t b = slot / block_size;
        const int32_t off = (int32_t)(slot - b * block_size);
        // streaming stores: the written lines are not re-read by this launch
        if (active) {
            const int32_t cph = head_size / X;  // key chunks per head
            const int32_t h = ci / cph, f = ci - h * cph;
            u32x4 kval;
            if constexpr (Q8)
                kval = quantize16(kin, k_inv_scale);
            else
                kval = kin[0];
            __builtin_nontemporal_store(kval, &k_cache[((b * num_kv_heads + h) * cph + f) * block_size + off]);
        }
#pragma unroll
        for (int e = 0; e < X; ++e) {
            const int32_t idx = e0 + e * kStoreThreads;
            if (idx < nelem) {
                E val;
                if constexpr (Q8)
                    val = quantize1(vin[e], v_inv_scale);
                else
                    val = vin[e];
                // element idx = h * hs + d of the token sits at ((b*Hkv + h)*hs + d)*B + off
                __builtin_nontemporal_store(val, &v_cache[(b * num_kv_heads * head_size + idx) * block_size + off]);
            }
        }
    }
}

}  // namespace pkv
