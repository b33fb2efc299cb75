// Per-tensor quantisation to OCP E4M3 for the fp8 expert GEMMs (Marin: Week of
// July 6th summary, the fp8 compute-lane paragraph: E4M3 in the forward, with
// delayed scaling, i.e. a scale the caller derives from the amax history).
//
//   q[i] = E4M3(x[i] * inv)   inv = 1 / s rounded to float32, s the dequantisation
//                             scale (device memory); the product rounded to float32;
//   amax = max |x[i]|         (optional; the value the history records)
//
// and the same quantisation fused with the expert MLP's gated activation
// (h = silu(g) u from a [g | u] row), which feeds the E4M3 down projection.
//
// HBM-bound: each thread converts 16 elements per pass (16-byte output stores,
// 32 or 64 bytes of input), grid-strided; the tail past a multiple of 16 is done
// element by element.
#include "common.h"
#include "e4m3.h"
#include "kernels.h"

namespace moe {

namespace {

__global__ void zero_u32_kernel(uint32_t* p) { *p = 0u; }

// Grid cap of the grid-strided quantising kernels: each block folds its amax into
// the result with one atomic, so fewer, longer-lived blocks mean fewer atomics on
// one address.
constexpr int64_t kQuantBlocks = 2048;


template <typename T>
__global__ __launch_bounds__(256) void quantize_kernel(const T* x, int64_t n, const float* scale,
                                                       uint8_t* q, uint32_t* amax_bits) {
    constexpr int kIn = 16 * (int)sizeof(T) / 16;          // 16-byte input vectors per group
    const float inv = inv_of(scale);
    const int64_t groups = n / 16;
    const int64_t stride = (int64_t)gridDim.x * 256;
    float m = 0.0f;
    // two groups per pass, both loaded before either is converted
    for (int64_t g = (int64_t)blockIdx.x * 256 + threadIdx.x; g < groups; g += 2 * stride) {
        const bool two = g + stride < groups;
        u32x4 in[2][kIn];
#pragma unroll
        for (int j = 0; j < kIn; j++) {
            in[0][j] = __builtin_nontemporal_load((const u32x4*)(x + g * 16) + j);
            if (two) in[1][j] = __builtin_nontemporal_load((const u32x4*)(x + (g + stride) * 16) + j);
        }
#pragma unroll
        for (int t = 0; t < 2; t++) {
            if (t == 1 && !two) break;
            float p[16];
#pragma unroll
            for (int e = 0; e < 16; e++) {
                const float f = group_elem<T>(in[t], e);
                m = fmaxf(m, fabsf(f));                       // NaN does not win
                p[e] = f * inv;
            }
            u32x4 out;
#pragma unroll
            for (int j = 0; j < 4; j++)
                out[j] = e4m3_pack4(p[4 * j], p[4 * j + 1], p[4 * j + 2], p[4 * j + 3]);
            __builtin_nontemporal_store(out, (u32x4*)(q + (g + t * stride) * 16));
        }
    }
    if (blockIdx.x == 0) {
        for (int64_t i = groups * 16 + threadIdx.x; i < n; i += 256) {
            const float f = elem_f32<T>(x, i);
            m = fmaxf(m, fabsf(f));
            q[i] = (uint8_t)e4m3_code(f * inv);
        }
    }
    if (amax_bits) block_amax(m, amax_bits);
}

// Gated activation of the expert MLP, quantised for the E4M3 down projection:
// for the rows r < offsets[E] (clamped to R_phys) of gu = [g | u] (2H wide),
//   h = silu(g) * u in float32,  hq[r, c] = E4M3(h * inv),  amax = max |h|.
// One thread per 16 consecutive columns of a row: two 32- or 64-byte loads (the
// gate and the up half), one 16-byte store.  rows * H / 16 < 2^31 (host-checked).
template <typename T>
__global__ __launch_bounds__(256) void swiglu_quantize_kernel(const T* gu, const int32_t* offsets,
                                                              int E, int64_t R_phys, int H16,
                                                              const float* scale, uint8_t* hq,
                                                              uint32_t* amax_bits) {
    constexpr int kIn = 16 * (int)sizeof(T) / 16;
    const float inv = inv_of(scale);
    int64_t rows = offsets[E];
    rows = rows < 0 ? 0 : rows > R_phys ? R_phys : rows;
    const uint32_t groups = (uint32_t)rows * (uint32_t)H16;
    const int64_t H = (int64_t)H16 * 16;
    const uint32_t stride = gridDim.x * 256u;
    float m = 0.0f;
    // two groups per pass, all four loads issued before either is converted
    for (uint32_t g = blockIdx.x * 256u + threadIdx.x; g < groups; g += 2 * stride) {
        const bool two = g + stride < groups;
        int64_t at[2];
        u32x4 gv[2][kIn], uv[2][kIn];
#pragma unroll
        for (int t = 0; t < 2; t++) {
            const uint32_t gg = g + t * stride;
            const uint32_t r = gg / (uint32_t)H16;
            const int64_t c = (int64_t)(gg - r * (uint32_t)H16) * 16;
            at[t] = (int64_t)r * H + c;
            if (t == 1 && !two) break;
            const T* gate = gu + (int64_t)r * 2 * H + c;
#pragma unroll
            for (int j = 0; j < kIn; j++) {
                gv[t][j] = __builtin_nontemporal_load((const u32x4*)gate + j);
                uv[t][j] = __builtin_nontemporal_load((const u32x4*)(gate + H) + j);
            }
        }
#pragma unroll
        for (int t = 0; t < 2; t++) {
            if (t == 1 && !two) break;
            float p[16];
#pragma unroll
            for (int e = 0; e < 16; e++) {
                const float h = silu_f(group_elem<T>(gv[t], e)) * group_elem<T>(uv[t], e);
                m = fmaxf(m, fabsf(h));
                p[e] = h * inv;
            }
            u32x4 out;
#pragma unroll
            for (int j = 0; j < 4; j++)
                out[j] = e4m3_pack4(p[4 * j], p[4 * j + 1], p[4 * j + 2], p[4 * j + 3]);
            *(u32x4*)(hq + at[t]) = out;
        }
    }
    if (amax_bits) block_amax(m, amax_bits);
}

// Delayed scaling's state update for one tensor: history (newest first) shifted
// by one with this step's amax in front, then scale[0] = m / 448 for m the largest
// finite entry (the value that maps to E4M3's largest code), or 1 when m is 0.
// One block of 1024 threads, len <= 1024: every entry is read before any is written.
__global__ __launch_bounds__(1024) void fp8_scale_update_kernel(float* history, int len,
                                                                const float* amax,
                                                                float* scale) {
    __shared__ float red[16];
    const int t = threadIdx.x;
    float v = 0.0f;
    if (t < len) v = t == 0 ? amax[0] : history[t - 1];
    __syncthreads();
    if (t < len) history[t] = v;
    float m = (t < len && isfinite(v) && v > 0.0f) ? v : 0.0f;
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) m = fmaxf(m, __shfl_xor(m, off, 64));
    if ((t & 63) == 0) red[t >> 6] = m;
    __syncthreads();
    if (t == 0) {
        float mm = 0.0f;
        for (int w = 0; w < 16; w++) mm = fmaxf(mm, red[w]);
        scale[0] = mm > 0.0f ? mm / 448.0f : 1.0f;
    }
}

}  // namespace

hipError_t launch_zero_u32(uint32_t* p, hipStream_t s) {
    hipLaunchKernelGGL(zero_u32_kernel, dim3(1), dim3(1), 0, s, p);
    return hipGetLastError();
}

hipError_t launch_fp8_scale_update(float* history, int len, const float* amax, float* scale,
                                   hipStream_t s) {
    hipLaunchKernelGGL(fp8_scale_update_kernel, dim3(1), dim3(1024), 0, s, history, len, amax,
                       scale);
    return hipGetLastError();
}

hipError_t launch_swiglu_quantize_e4m3(const void* gu, moe_dtype dt, const int32_t* offsets,
                                       int E, int64_t R_phys, int64_t H, const float* scale,
                                       uint8_t* hq, float* amax, hipStream_t s) {
    uint32_t* ab = (uint32_t*)amax;
    if (ab) hipLaunchKernelGGL(zero_u32_kernel, dim3(1), dim3(1), 0, s, ab);
    if (R_phys <= 0) return hipGetLastError();
    const int H16 = (int)(H / 16);
    int64_t grid = (R_phys * H16 + 255) / 256;
    if (grid > kQuantBlocks) grid = kQuantBlocks;
    if (dt == MOE_BF16)
        hipLaunchKernelGGL(swiglu_quantize_kernel<bf16_t>, dim3((unsigned)grid), dim3(256), 0, s,
                           (const bf16_t*)gu, offsets, E, R_phys, H16, scale, hq, ab);
    else
        hipLaunchKernelGGL(swiglu_quantize_kernel<float>, dim3((unsigned)grid), dim3(256), 0, s,
                           (const float*)gu, offsets, E, R_phys, H16, scale, hq, ab);
    return hipGetLastError();
}

hipError_t launch_quantize_e4m3(const void* x, moe_dtype dt, int64_t n, const float* scale,
                                uint8_t* q, float* amax, hipStream_t s) {
    uint32_t* ab = (uint32_t*)amax;
    if (ab) hipLaunchKernelGGL(zero_u32_kernel, dim3(1), dim3(1), 0, s, ab);
    if (n <= 0) return hipGetLastError();
    const int64_t groups = n / 16;
    int64_t grid = (groups + 255) / 256;
    if (grid < 1) grid = 1;
    if (grid > kQuantBlocks) grid = kQuantBlocks;
    if (dt == MOE_BF16)
        hipLaunchKernelGGL(quantize_kernel<bf16_t>, dim3((unsigned)grid), dim3(256), 0, s,
                           (const bf16_t*)x, n, scale, q, ab);
    else
        hipLaunchKernelGGL(quantize_kernel<float>, dim3((unsigned)grid), dim3(256), 0, s,
                           (const float*)x, n, scale, q, ab);
    return hipGetLastError();
}

}  // namespace moe
