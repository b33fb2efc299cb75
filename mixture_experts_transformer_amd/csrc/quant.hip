// Per-tensor quantisation to OCP E4M3 for the fp8 expert GEMMs (Marin: Week of
// July 6th summary, the fp8 compute-lane paragraph: E4M3 in the forward, with
// delayed scaling, i.e. a scale the caller derives from the amax history).
//
//   q[i] = E4M3(x[i] * inv_scale)   the product rounded to float32 first;
//   amax = max |x[i]|               (optional; the value the history records)
//
// and the same quantisation fused with the expert MLP's gated activation
// (h = silu(g) u from a [g | u] row), which feeds the E4M3 down projection.
//
// HBM-bound: each thread converts 16 elements per pass (16-byte output stores,
// 32 or 64 bytes of input), grid-strided; the tail past a multiple of 16 is done
// element by element.
#include "common.h"
#include "kernels.h"

namespace moe {

namespace {

// E4M3 code of a float32 value, from the format's definition: sign, 4 exponent
// bits with bias 7, 3 mantissa bits, subnormal steps of 2^-9 below 2^-6.  The
// nearest code, ties to the even mantissa (rintf rounds half to even, and the
// scalings by powers of two are exact); magnitudes from 464 (the midpoint of 448
// and the next step, 480) up and infinities saturate to 448; NaN gives 0x7F.
__device__ __forceinline__ uint32_t e4m3_code(float x) {
    const uint32_t u = __float_as_uint(x);
    const uint32_t sign = (u >> 24) & 0x80u;
    const float a = fabsf(x);
    if (a != a) return 0x7Fu;
    if (a >= 464.0f) return sign | 0x7Eu;
    if (a < 0.015625f) return sign | (uint32_t)rintf(a * 512.0f);   // 0..8 (8 = 2^-6)
    int e = (int)((u >> 23) & 0xFFu) - 127;                          // a is a normal float
    float r = rintf(ldexpf(a, 3 - e));                               // 8..16
    if (r == 16.0f) {
        e += 1;
        r = 8.0f;
    }
    return sign | (uint32_t)(((e + 7) << 3) | ((int)r - 8));
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

__global__ void zero_u32_kernel(uint32_t* p) { *p = 0u; }

template <typename T>
__global__ __launch_bounds__(256) void quantize_kernel(const T* x, int64_t n, float inv,
                                                       uint8_t* q, uint32_t* amax_bits) {
    constexpr int kIn = 16 * (int)sizeof(T) / 16;          // 16-byte input vectors per group
    const int64_t groups = n / 16;
    float m = 0.0f;
    for (int64_t g = (int64_t)blockIdx.x * 256 + threadIdx.x; g < groups;
         g += (int64_t)gridDim.x * 256) {
        u32x4 in[kIn];
#pragma unroll
        for (int j = 0; j < kIn; j++)
            in[j] = __builtin_nontemporal_load((const u32x4*)(x + g * 16) + j);
        u32x4 out = {0u, 0u, 0u, 0u};
#pragma unroll
        for (int e = 0; e < 16; e++) {
            const float f = group_elem<T>(in, e);
            m = fmaxf(m, fabsf(f));                           // NaN does not win
            out[e >> 2] |= e4m3_code(f * inv) << (8 * (e & 3));
        }
        __builtin_nontemporal_store(out, (u32x4*)(q + g * 16));
    }
    if (blockIdx.x == 0) {
        for (int64_t i = groups * 16 + threadIdx.x; i < n; i += 256) {
            const float f = elem_f32<T>(x, i);
            m = fmaxf(m, fabsf(f));
            q[i] = (uint8_t)e4m3_code(f * inv);
        }
    }
    if (amax_bits) {
#pragma unroll
        for (int off = 32; off > 0; off >>= 1) m = fmaxf(m, __shfl_xor(m, off, 64));
        // non-negative floats order as their bit patterns
        if ((threadIdx.x & 63) == 0) atomicMax(amax_bits, __float_as_uint(m));
    }
}

// Gated activation of the expert MLP, quantised for the E4M3 down projection:
// for the rows r < offsets[E] (clamped to R_phys) of gu = [g | u] (2H wide),
//   h = silu(g) * u in float32,  hq[r, c] = E4M3(h * inv),  amax = max |h|.
// One thread per 16 consecutive columns of a row: two 32- or 64-byte loads (the
// gate and the up half), one 16-byte store.  rows * H / 16 < 2^31 (host-checked).
template <typename T>
__global__ __launch_bounds__(256) void swiglu_quantize_kernel(const T* gu, const int32_t* offsets,
                                                              int E, int64_t R_phys, int H16,
                                                              float inv, uint8_t* hq,
                                                              uint32_t* amax_bits) {
    constexpr int kIn = 16 * (int)sizeof(T) / 16;
    int64_t rows = offsets[E];
    rows = rows < 0 ? 0 : rows > R_phys ? R_phys : rows;
    const uint32_t groups = (uint32_t)rows * (uint32_t)H16;
    const int64_t H = (int64_t)H16 * 16;
    float m = 0.0f;
    for (uint32_t g = blockIdx.x * 256u + threadIdx.x; g < groups; g += gridDim.x * 256u) {
        const uint32_t r = g / (uint32_t)H16;
        const int64_t c = (int64_t)(g - r * (uint32_t)H16) * 16;
        const T* gate = gu + (int64_t)r * 2 * H + c;
        u32x4 gv[kIn], uv[kIn];
#pragma unroll
        for (int j = 0; j < kIn; j++) {
            gv[j] = __builtin_nontemporal_load((const u32x4*)gate + j);
            uv[j] = __builtin_nontemporal_load((const u32x4*)(gate + H) + j);
        }
        u32x4 out = {0u, 0u, 0u, 0u};
#pragma unroll
        for (int e = 0; e < 16; e++) {
            const float h = silu_f(group_elem<T>(gv, e)) * group_elem<T>(uv, e);
            m = fmaxf(m, fabsf(h));
            out[e >> 2] |= e4m3_code(h * inv) << (8 * (e & 3));
        }
        *(u32x4*)(hq + (int64_t)r * H + c) = out;
    }
    if (amax_bits) {
#pragma unroll
        for (int off = 32; off > 0; off >>= 1) m = fmaxf(m, __shfl_xor(m, off, 64));
        if ((threadIdx.x & 63) == 0) atomicMax(amax_bits, __float_as_uint(m));
    }
}

}  // namespace

hipError_t launch_swiglu_quantize_e4m3(const void* gu, moe_dtype dt, const int32_t* offsets,
                                       int E, int64_t R_phys, int64_t H, float inv_scale,
                                       uint8_t* hq, float* amax, hipStream_t s) {
    uint32_t* ab = (uint32_t*)amax;
    if (ab) hipLaunchKernelGGL(zero_u32_kernel, dim3(1), dim3(1), 0, s, ab);
    if (R_phys <= 0) return hipGetLastError();
    const int H16 = (int)(H / 16);
    int64_t grid = (R_phys * H16 + 255) / 256;
    if (grid > 4096) grid = 4096;
    if (dt == MOE_BF16)
        hipLaunchKernelGGL(swiglu_quantize_kernel<bf16_t>, dim3((unsigned)grid), dim3(256), 0, s,
                           (const bf16_t*)gu, offsets, E, R_phys, H16, inv_scale, hq, ab);
    else
        hipLaunchKernelGGL(swiglu_quantize_kernel<float>, dim3((unsigned)grid), dim3(256), 0, s,
                           (const float*)gu, offsets, E, R_phys, H16, inv_scale, hq, ab);
    return hipGetLastError();
}

hipError_t launch_quantize_e4m3(const void* x, moe_dtype dt, int64_t n, float inv_scale,
                                uint8_t* q, float* amax, hipStream_t s) {
    uint32_t* ab = (uint32_t*)amax;
    if (ab) hipLaunchKernelGGL(zero_u32_kernel, dim3(1), dim3(1), 0, s, ab);
    if (n <= 0) return hipGetLastError();
    const int64_t groups = n / 16;
    int64_t grid = (groups + 255) / 256;
    if (grid < 1) grid = 1;
    if (grid > 4096) grid = 4096;
    if (dt == MOE_BF16)
        hipLaunchKernelGGL(quantize_kernel<bf16_t>, dim3((unsigned)grid), dim3(256), 0, s,
                           (const bf16_t*)x, n, inv_scale, q, ab);
    else
        hipLaunchKernelGGL(quantize_kernel<float>, dim3((unsigned)grid), dim3(256), 0, s,
                           (const float*)x, n, inv_scale, q, ab);
    return hipGetLastError();
}

}  // namespace moe
