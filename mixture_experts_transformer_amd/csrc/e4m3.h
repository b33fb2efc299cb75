// OCP E4M3 conversion helpers shared by the kernels that quantise (per-tensor
// quantisation, the gated activation's quantisation, the permute's E4M3 row
// copy).  Internal to libmoe.
#pragma once

#include "common.h"

namespace moe {

// E4M3 codes of float32 values by the hardware conversion (v_cvt_pk_fp8_f32:
// OCP E4M3, the nearest code with ties to the even mantissa), with the two rules
// it does not apply by itself: magnitudes above 448 saturate to +-448 first (from
// 464 up the nearest code would not be finite; between 448 and 464 it is 448
// anyway), and a NaN, which the conversion encodes as 0xFF, becomes 0x7F.  After
// saturation only NaN gives a byte with all seven low bits set, so adding 1 to
// each byte's low seven bits carries into bit 7 exactly for NaN bytes, whose sign
// bit is then cleared.
__device__ __forceinline__ float e4m3_sat(float x) {
    return fabsf(x) > 448.0f ? copysignf(448.0f, x) : x;   // NaN passes unchanged
}
__device__ __forceinline__ uint32_t e4m3_nan_fix(uint32_t w) {
    return w & ~(((w & 0x7F7F7F7Fu) + 0x01010101u) & 0x80808080u);
}
__device__ __forceinline__ uint32_t e4m3_pack4(float a, float b, float c, float d) {
    const int w = __builtin_amdgcn_cvt_pk_fp8_f32(e4m3_sat(a), e4m3_sat(b), 0, false);
    return e4m3_nan_fix(
        (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(e4m3_sat(c), e4m3_sat(d), w, true));
}
__device__ __forceinline__ uint32_t e4m3_code(float x) {
    return e4m3_pack4(x, 0.0f, 0.0f, 0.0f) & 0xFFu;
}

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

template <typename T> __device__ __forceinline__ float elem_f32(const T* p, int64_t i);
template <> __device__ __forceinline__ float elem_f32<float>(const float* p, int64_t i) {
    return p[i];
}
template <> __device__ __forceinline__ float elem_f32<bf16_t>(const bf16_t* p, int64_t i) {
    return bf16_to_f32(p[i].bits);
}
// element e of a group of 16 held in 16-byte vectors (no address taken, so the
// vectors stay in registers)
template <typename T> __device__ __forceinline__ float group_elem(const u32x4* in, int e);
template <> __device__ __forceinline__ float group_elem<float>(const u32x4* in, int e) {
    return __uint_as_float(in[e >> 2][e & 3]);
}
template <> __device__ __forceinline__ float group_elem<bf16_t>(const u32x4* in, int e) {
    return bf16_to_f32((u16)(in[e >> 3][(e >> 1) & 3] >> (16 * (e & 1))));
}

// max |.| over the block (256 threads) folded into *amax_bits with one atomic;
// non-negative floats order as their bit patterns.  Every thread must call it.
__device__ __forceinline__ void block_amax(float m, uint32_t* amax_bits) {
    __shared__ float red[4];
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) m = fmaxf(m, __shfl_xor(m, off, 64));
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = m;
    __syncthreads();
    if (threadIdx.x == 0)
        atomicMax(amax_bits, __float_as_uint(fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]))));
}

// 1 / s rounded to float32 (IEEE division), 1 without a scale
__device__ __forceinline__ float inv_of(const float* scale) {
    return scale ? 1.0f / scale[0] : 1.0f;
}

}  // namespace moe
