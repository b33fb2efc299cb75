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

// Rows whose loads one wave keeps in flight together, and 16-byte chunks per
// lane per pass: 4 x 3 KB per wave in flight with 98 VGPRs (measured against
// 8 x 2 and 8 x 3 at the 535B shape; all within 4%).
constexpr int kRowsInFlight = 4;
constexpr int kChunksPerPass = 3;

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

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

// One wave per output row.  Lane j < k holds assignment j's row and weight, read
// once; the wave takes them in order with readlane.  The row is done in passes
// of C 16-byte chunks per lane; in each pass the loads of J assignments' rows
// are all issued before any is accumulated, so a wave keeps J * C KB of reads
// in flight.  Accumulation stays in j order.  Every Y row is read once and every
// output row written once, so both go through non-temporal accesses (14% faster
// than cached ones at the 535B shape).
template <typename T, int J, int C>
__global__ __launch_bounds__(256) void combine_kernel(const char* Y, const int32_t* slot_row,
                                                      const float* w, int64_t n_tok, int k,
                                                      int64_t row_bytes, char* out, int flags) {
    constexpr int kPer = 16 / sizeof(typename Elem<T>::store_t);   // elements per chunk
    const int lane = threadIdx.x & 63;
    const int64_t t = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    if (t >= n_tok) return;
    int my_row = -1;
    float my_w = 0.0f;
    if (lane < k) {
        my_row = slot_row[t * k + lane];
        my_w = w ? w[t * k + lane] : 1.0f;
    }
    if (__ballot(my_row >= 0) == 0 && (flags & MOE_COMBINE_KEEP_UNROUTED)) return;
    const int64_t nchunk = row_bytes / 16;
    for (int64_t c0 = 0; c0 < nchunk; c0 += 64 * C) {
        float acc[C][kPer];
#pragma unroll
        for (int q = 0; q < C; q++)
#pragma unroll
            for (int e = 0; e < kPer; e++) acc[q][e] = 0.0f;
        for (int j0 = 0; j0 < k; j0 += J) {
            uint4 u[J][C];
#pragma unroll
            for (int jj = 0; jj < J; jj++) {
                const int j = j0 + jj;
                const int row = j < k ? __builtin_amdgcn_readlane(my_row, j) : -1;
                if (row >= 0) {
                    // lanes past the row's end re-read its last chunk (unused)
                    const char* src = Y + (int64_t)row * row_bytes;
#pragma unroll
                    for (int q = 0; q < C; q++) {
                        const int64_t c = min(c0 + lane + 64 * q, nchunk - 1);
                        const u32x4 x = __builtin_nontemporal_load((const u32x4*)(src + c * 16));
                        u[jj][q] = make_uint4(x[0], x[1], x[2], x[3]);
                    }
                }
            }
#pragma unroll
            for (int jj = 0; jj < J; jj++) {
                const int j = j0 + jj;
                const int row = j < k ? __builtin_amdgcn_readlane(my_row, j) : -1;
                if (row >= 0) {
                    const float wj = __int_as_float(
                        __builtin_amdgcn_readlane(__float_as_int(my_w), j));
#pragma unroll
                    for (int q = 0; q < C; q++) {
                        float v[kPer];
                        unpack<T>(u[jj][q], v);
#pragma unroll
                        for (int e = 0; e < kPer; e++) acc[q][e] += wj * v[e];
                    }
                }
            }
        }
#pragma unroll
        for (int q = 0; q < C; q++) {
            const int64_t c = c0 + lane + 64 * q;
            if (c < nchunk) {
                const uint4 pk = pack<T>(acc[q]);
                const u32x4 x = {pk.x, pk.y, pk.z, pk.w};
                __builtin_nontemporal_store(x, (u32x4*)(out + t * row_bytes + c * 16));
            }
        }
    }
}

template <typename T>
void launch_t(const void* Y, const int32_t* slot_row, const float* w, int64_t T_, int k,
              int64_t row_bytes, void* out, int flags, hipStream_t s) {
    const int64_t blocks = (T_ + 3) / 4;
    if (k == 1)
        hipLaunchKernelGGL((combine_kernel<T, 1, 8>), dim3((unsigned)blocks), dim3(256), 0, s,
                           (const char*)Y, slot_row, w, T_, k, row_bytes, (char*)out, flags);
    else
        hipLaunchKernelGGL((combine_kernel<T, kRowsInFlight, kChunksPerPass>),
                           dim3((unsigned)blocks), dim3(256), 0, s, (const char*)Y, slot_row, w,
                           T_, k, row_bytes, (char*)out, flags);
}

}  // namespace

hipError_t launch_combine(const void* Y, moe_dtype dt, const int32_t* slot_row, const float* w,
                          int64_t T, int k, int64_t width, void* out, int flags, hipStream_t s) {
    if (T == 0) return hipSuccess;
    if (dt == MOE_BF16)
        launch_t<bf16_t>(Y, slot_row, w, T, k, width * 2, out, flags, s);
    else
        launch_t<float>(Y, slot_row, w, T, k, width * 4, out, flags, s);
    return hipGetLastError();
}

}  // namespace moe
