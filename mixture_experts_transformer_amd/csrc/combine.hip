// Weighted combine as an ordered gather (Marin weekly summary of September 14:
// replacing an atomic scatter-add with an ordered gather made repeated scoring
// bitwise exact).  One wave per output row: for j = 0..k-1 in order, the row
// slot_row[t*k+j] of Y (if kept) is read in 16-byte chunks and accumulated with
// weight w[t*k+j] in float32; a dropped slot contributes nothing and the other
// weights are not renormalised (launch blog, section 4).  With
// MOE_COMBINE_KEEP_UNROUTED a row with no kept slot is left untouched (the
// unpermute of a receiver pool whose padding rows must survive).
#include <algorithm>

#include "common.h"
#include "kernels.h"

namespace moe {

namespace {

// Rows whose loads one wave keeps in flight together (k > 1): 4 rows of C
// 16-byte chunks per lane.
constexpr int kRowsInFlight = 4;

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

template <typename T>
__device__ __forceinline__ void unpack(const u32x4& u, float* v);
template <>
__device__ __forceinline__ void unpack<float>(const u32x4& u, float* v) {
#pragma unroll
    for (int i = 0; i < 4; i++) v[i] = __uint_as_float(u[i]);
}
template <>
__device__ __forceinline__ void unpack<bf16_t>(const u32x4& u, float* v) {
#pragma unroll
    for (int i = 0; i < 4; i++) {
        v[2 * i] = __uint_as_float(u[i] << 16);
        v[2 * i + 1] = __uint_as_float(u[i] & 0xffff0000u);
    }
}
template <typename T>
__device__ __forceinline__ u32x4 pack(const float* v);
template <>
__device__ __forceinline__ u32x4 pack<float>(const float* v) {
    const u32x4 u = {__float_as_uint(v[0]), __float_as_uint(v[1]), __float_as_uint(v[2]),
                     __float_as_uint(v[3])};
    return u;
}
template <>
__device__ __forceinline__ u32x4 pack<bf16_t>(const float* v) {
    const u32x4 u = {pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]), pack_bf16x2(v[4], v[5]),
                     pack_bf16x2(v[6], v[7])};
    return u;
}

// One wave per (output row t, segment g of 64 * C 16-byte chunks of the row):
// splitting a row over several waves keeps every wave short, so the last waves
// of the launch leave little of the chip idle.  Lane j < k holds assignment j's
// row and weight; the wave takes them in order with readlane.  The loads of J
// assignments' segments are all issued before any is accumulated, so a wave
// keeps J * C KB of reads in flight; accumulation stays in j order.  Every Y row
// is read once and every output row written once, so both go through
// non-temporal accesses.
template <typename T, int J, int C>
__global__ __launch_bounds__(256) void combine_kernel(const char* Y, const int32_t* slot_row,
                                                      const float* w, int64_t n_tok, int k,
                                                      int64_t row_bytes, int nseg, char* out,
                                                      int flags) {
    constexpr int kPer = 16 / sizeof(typename Elem<T>::store_t);   // elements per chunk
    const int lane = threadIdx.x & 63;
    const int64_t wv = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    const int64_t t = wv / nseg;
    if (t >= n_tok) return;
    const int64_t c0 = (wv - t * nseg) * (64 * C);
    int my_row = -1;
    float my_w = 0.0f;
    if (lane < k) {
        my_row = slot_row[t * k + lane];
        my_w = w ? w[t * k + lane] : 1.0f;
    }
    if (__ballot(my_row >= 0) == 0 && (flags & MOE_COMBINE_KEEP_UNROUTED)) return;
    const int64_t nchunk = row_bytes / 16;
    float acc[C][kPer];
#pragma unroll
    for (int q = 0; q < C; q++)
#pragma unroll
        for (int e = 0; e < kPer; e++) acc[q][e] = 0.0f;
    for (int j0 = 0; j0 < k; j0 += J) {
        u32x4 u[J][C];
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
                    u[jj][q] = __builtin_nontemporal_load((const u32x4*)(src + c * 16));
                }
            }
        }
#pragma unroll
        for (int jj = 0; jj < J; jj++) {
            const int j = j0 + jj;
            const int row = j < k ? __builtin_amdgcn_readlane(my_row, j) : -1;
            if (row >= 0) {
                const float wj = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(my_w), j));
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
        if (c < nchunk)
            __builtin_nontemporal_store(pack<T>(acc[q]), (u32x4*)(out + t * row_bytes + c * 16));
    }
}

// Chunks per lane for a row of nchunk 16-byte chunks: among the candidates (in
// decreasing order), the one that leaves the fewest idle lane slots over the
// row's segments (the larger on a tie).
template <int N>
int chunks_for(int64_t nchunk, const int (&cand)[N]) {
    int best = cand[0];
    int64_t waste = -1;
    for (int c : cand) {
        const int64_t per = 64 * (int64_t)c;
        const int64_t w = (nchunk + per - 1) / per * per - nchunk;
        if (waste < 0 || w < waste) {
            waste = w;
            best = c;
        }
    }
    return best;
}

template <typename T, int J, int C>
void launch_jc(const void* Y, const int32_t* slot_row, const float* w, int64_t T_, int k,
               int64_t row_bytes, void* out, int flags, hipStream_t s) {
    const int64_t nchunk = row_bytes / 16;
    const int nseg = (int)std::max<int64_t>(1, (nchunk + 64 * C - 1) / (64 * C));
    const int64_t blocks = (T_ * nseg + 3) / 4;
    hipLaunchKernelGGL((combine_kernel<T, J, C>), dim3((unsigned)blocks), dim3(256), 0, s,
                       (const char*)Y, slot_row, w, T_, k, row_bytes, nseg, (char*)out, flags);
}

template <typename T>
void launch_t(const void* Y, const int32_t* slot_row, const float* w, int64_t T_, int k,
              int64_t row_bytes, void* out, int flags, hipStream_t s) {
    const int64_t nchunk = row_bytes / 16;
    if (k == 1) {
        // one row per output row: a plain gather, 4 to 8 chunks per lane
        static const int cand[] = {8, 6, 4};
        switch (chunks_for(nchunk, cand)) {
            case 4: launch_jc<T, 1, 4>(Y, slot_row, w, T_, k, row_bytes, out, flags, s); break;
            case 6: launch_jc<T, 1, 6>(Y, slot_row, w, T_, k, row_bytes, out, flags, s); break;
            default: launch_jc<T, 1, 8>(Y, slot_row, w, T_, k, row_bytes, out, flags, s);
        }
    } else {
        // 2 or 3 chunks (4 would never leave fewer idle lanes than 2)
        static const int cand[] = {3, 2};
        if (chunks_for(nchunk, cand) == 2)
            launch_jc<T, kRowsInFlight, 2>(Y, slot_row, w, T_, k, row_bytes, out, flags, s);
        else
            launch_jc<T, kRowsInFlight, 3>(Y, slot_row, w, T_, k, row_bytes, out, flags, s);
    }
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
