// Weighted combine as an ordered gather (Marin weekly summary of September 14:
// replacing an atomic scatter-add with an ordered gather made repeated scoring
// bitwise exact).  One wave per output row: for j = 0..k-1 in order, the row
// slot_row[t*k+j] of Y (if kept) is read in 16-byte chunks and accumulated with
// weight w[t*k+j] in float32; a dropped slot contributes nothing and the other
// weights are not renormalised (launch blog, section 4).  With
// MOE_COMBINE_KEEP_UNROUTED a row with no kept slot is left untouched (the
// unpermute of a receiver pool whose padding rows must survive).
#include "common.h"
#include "kernels.h"

namespace moe {

namespace {

constexpr int kMaxChunks = 8;     // 16-byte chunks per lane held in registers

template <typename T>
__device__ __forceinline__ void unpack(const uint4& u, float* v);
template <>
__device__ __forceinline__ void unpack<float>(const uint4& u, float* v) {
    v[0] = __uint_as_float(u.x); v[1] = __uint_as_float(u.y);
    v[2] = __uint_as_float(u.z); v[3] = __uint_as_float(u.w);
}
template <>
__device__ __forceinline__ void unpack<bf16_t>(const uint4& u, float* v) {
    const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
    for (int i = 0; i < 4; i++) {
        v[2 * i] = __uint_as_float(w[i] << 16);
        v[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
    }
}
template <typename T>
__device__ __forceinline__ uint4 pack(const float* v);
template <>
__device__ __forceinline__ uint4 pack<float>(const float* v) {
    return make_uint4(__float_as_uint(v[0]), __float_as_uint(v[1]), __float_as_uint(v[2]),
                      __float_as_uint(v[3]));
}
template <>
__device__ __forceinline__ uint4 pack<bf16_t>(const float* v) {
    uint4 u;
    u.x = (uint32_t)f32_to_bf16(v[0]) | ((uint32_t)f32_to_bf16(v[1]) << 16);
    u.y = (uint32_t)f32_to_bf16(v[2]) | ((uint32_t)f32_to_bf16(v[3]) << 16);
    u.z = (uint32_t)f32_to_bf16(v[4]) | ((uint32_t)f32_to_bf16(v[5]) << 16);
    u.w = (uint32_t)f32_to_bf16(v[6]) | ((uint32_t)f32_to_bf16(v[7]) << 16);
    return u;
}

template <typename T>
__global__ __launch_bounds__(256) void combine_kernel(const char* Y, const int32_t* slot_row,
                                                      const float* w, int64_t n_tok, int k,
                                                      int64_t row_bytes, char* out, int flags) {
    constexpr int kPer = 16 / sizeof(typename Elem<T>::store_t);   // elements per chunk
    const int lane = threadIdx.x & 63;
    const int64_t t = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    if (t >= n_tok) return;
    const int64_t nchunk = row_bytes / 16;
    bool any = false;
    for (int j = 0; j < k; j++) any |= slot_row[t * k + j] >= 0;
    if (!any && (flags & MOE_COMBINE_KEEP_UNROUTED)) return;
    // chunks handled by this lane: lane, lane + 64, ... (kMaxChunks per pass)
    for (int64_t c0 = 0; c0 < nchunk; c0 += 64 * kMaxChunks) {
        float acc[kMaxChunks][kPer];
#pragma unroll
        for (int q = 0; q < kMaxChunks; q++)
#pragma unroll
            for (int e = 0; e < kPer; e++) acc[q][e] = 0.0f;
        for (int j = 0; j < k; j++) {
            const int row = slot_row[t * k + j];
            if (row < 0) continue;
            const float wj = w ? w[t * k + j] : 1.0f;
            const char* src = Y + (int64_t)row * row_bytes;
            uint4 u[kMaxChunks];
#pragma unroll
            for (int q = 0; q < kMaxChunks; q++) {
                const int64_t c = c0 + lane + 64 * q;
                if (c < nchunk) u[q] = *(const uint4*)(src + c * 16);
            }
#pragma unroll
            for (int q = 0; q < kMaxChunks; q++) {
                const int64_t c = c0 + lane + 64 * q;
                if (c < nchunk) {
                    float v[kPer];
                    unpack<T>(u[q], v);
#pragma unroll
                    for (int e = 0; e < kPer; e++) acc[q][e] += wj * v[e];
                }
            }
        }
#pragma unroll
        for (int q = 0; q < kMaxChunks; q++) {
            const int64_t c = c0 + lane + 64 * q;
            if (c < nchunk) *(uint4*)(out + t * row_bytes + c * 16) = pack<T>(acc[q]);
        }
    }
}

}  // namespace

hipError_t launch_combine(const void* Y, moe_dtype dt, const int32_t* slot_row, const float* w,
                          int64_t T, int k, int64_t width, void* out, int flags, hipStream_t s) {
    if (T == 0) return hipSuccess;
    const int64_t blocks = (T + 3) / 4;
    if (dt == MOE_BF16)
        hipLaunchKernelGGL(combine_kernel<bf16_t>, dim3((unsigned)blocks), dim3(256), 0, s,
                           (const char*)Y, slot_row, w, T, k, width * 2, (char*)out, flags);
    else
        hipLaunchKernelGGL(combine_kernel<float>, dim3((unsigned)blocks), dim3(256), 0, s,
                           (const char*)Y, slot_row, w, T, k, width * 4, (char*)out, flags);
    return hipGetLastError();
}

}  // namespace moe
