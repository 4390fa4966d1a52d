// Device helpers shared by the attention kernels (decode.hip, prefill.hip).
#pragma once

#include <hip/hip_runtime.h>

namespace pkv {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));


constexpr float kLog2e = 1.4426950408889634f;
constexpr float kRescaleSlack = 8.0f;  // log2 units: probabilities stay <= 256

// Key row c of M-tile mp of a 32-token unit holds token 16*mp + c, so each
// key load reads 16 consecutive 16-byte chunks (256 contiguous bytes per
// lane group: whole 128-byte lines for the streaming loads).  The score
// layout then gives lane group r tokens 4r .. 4r+3 (M-tile 0) and
// 16+4r .. 16+4r+3 (M-tile 1), while the value MFMA wants tokens
// 8r .. 8r+7 in lane group r; to_value_order moves the probabilities there.
//
// With X_r / Y_r the four values of lane group r from M-tile 0 / 1, lane
// group r needs (X_{2r}, X_{2r+1}) for r < 2 and (Y_{2r-4}, Y_{2r-3}) for
// r >= 2.  v_permlane32_swap exchanges lane groups 2,3 of its first operand
// with groups 0,1 of its second: (X0 X1 Y0 Y1), (X2 X3 Y2 Y3).
// v_permlane16_swap exchanges odd groups of the first with even groups of
// the second: (X0 X2 Y0 Y2), (X1 X3 Y1 Y3) -- the first and second four
// tokens of each lane group.
//
// Written as inline assembly because the compiler at hand, given the two
// swap builtins chained, keeps only the first result of the second swap
// (the second comes back as a copy of the first).  Both registers are read
// and written in place; the s_nop 1 before each swap gives the two wait
// states the swaps need after a vector write of their operands, and the one
// after covers a read of their results.
__device__ __forceinline__ void to_value_order(float& x, float& y)
{
    asm volatile(
        "s_nop 1\n\t"
        "v_permlane32_swap_b32 %0, %1\n\t"
        "s_nop 1\n\t"
        "v_permlane16_swap_b32 %0, %1\n\t"
        "s_nop 1"
        : "+v"(x), "+v"(y));
}

// Maximum over the four lane groups (lanes c, c + 16, c + 32, c + 48) of
// each column c, with the same two lane-group swaps (no LDS round trip):
// after v_permlane32_swap of two copies, lane l holds x[l] and x[l ^ 32];
// after v_permlane16_swap of two copies of that maximum, x[l ^ 16] joins.
// (IEEE maximum: a NaN among the inputs gives NaN.)
__device__ __forceinline__ float max_over_lane_groups(float x)
{
    float a = x, b = x;
    asm volatile("s_nop 1\n\tv_permlane32_swap_b32 %0, %1\n\ts_nop 1" : "+v"(a), "+v"(b));
    float c = __builtin_elementwise_maximum(a, b), d = c;
    asm volatile("s_nop 1\n\tv_permlane16_swap_b32 %0, %1\n\ts_nop 1" : "+v"(c), "+v"(d));
    return __builtin_elementwise_maximum(c, d);
}

// Output elements.  With bf16 queries the output is bf16, rounded to
// nearest even, or, when out_f32 is set, the fp32 value that rounding would
// take (so that the kernel's own error can be seen apart from the output
// rounding).  fp32 queries always give fp32.  i indexes elements of the
// output's own type; store_out4 needs i to be a multiple of 4.
template <typename T>
__device__ __forceinline__ void store_out(void* out, int64_t i, float x, bool out_f32)
{
    if (sizeof(T) == 4 || out_f32)
        static_cast<float*>(out)[i] = x;
    else
        static_cast<__bf16*>(out)[i] = (__bf16)x;
}

template <typename T>
__device__ __forceinline__ void store_out4(void* out, int64_t i, f32x4 x, bool out_f32)
{
    if (sizeof(T) == 4 || out_f32) {
        *reinterpret_cast<f32x4*>(static_cast<float*>(out) + i) = x;
    } else {
        bf16x4 v;
#pragma unroll
        for (int k = 0; k < 4; ++k)
            v[k] = (__bf16)x[k];
        *reinterpret_cast<bf16x4*>(static_cast<__bf16*>(out) + i) = v;
    }
}

// Four E4M3 codes (one dword) to four bf16.  Every E4M3 value (at most 4
// significant bits, exponents 2^-9 .. 2^8) is exact in bf16, and gfx950
// converts two codes to two packed bf16 in one instruction
// (v_cvt_scalef32_pk_bf16_fp8; a scale of 1.0 leaves the values as they
// are).  Element e of the result is code e (byte e of w).
__device__ __forceinline__ void fp8x4_to_bf16(unsigned w, unsigned& lo, unsigned& hi)
{
    lo = __builtin_bit_cast(unsigned, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, false));  // codes 0, 1
    hi = __builtin_bit_cast(unsigned, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, true));   // codes 2, 3
}

}  // namespace pkv
