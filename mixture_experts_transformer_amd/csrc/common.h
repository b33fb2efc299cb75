// Shared device helpers for the gfx950 kernels: element types, MFMA fragment
// traits, wave reductions.  Internal to libmoe; not part of the C ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/moe.h"

namespace moe {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float floatx16 __attribute__((ext_vector_type(16)));
typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef uint16_t u16;

struct bf16_t { u16 bits; };   // storage tag for bfloat16 arrays
struct fp8_t { uint8_t bits; }; // storage tag for OCP E4M3 arrays
typedef int intx8 __attribute__((ext_vector_type(8)));
typedef int intx4 __attribute__((ext_vector_type(4)));

constexpr int kWave = 64;
constexpr int kNumXcd = 8;     // MI355X: 8 XCDs, workgroups dealt round-robin

// ---------------------------------------------------------------- bf16 -----
__device__ __forceinline__ float bf16_to_f32(u16 b) {
    return __uint_as_float((uint32_t)b << 16);
}
// float32 -> bfloat16, round to nearest even (NaN kept quiet).
__device__ __forceinline__ u16 f32_to_bf16(float f) {
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7fffffffu) > 0x7f800000u) return (u16)((u >> 16) | 0x40);
    u += 0x7fffu + ((u >> 16) & 1u);
    return (u16)(u >> 16);
}

template <typename T> struct Elem;
template <> struct Elem<float> {
    typedef float store_t;
    static constexpr int kBytes = 4;
    __device__ static float load(const float* p, int64_t i) { return p[i]; }
    __device__ static void store(float* p, int64_t i, float v) { p[i] = v; }
};
template <> struct Elem<fp8_t> {
    typedef uint8_t store_t;
    static constexpr int kBytes = 1;
};
template <> struct Elem<bf16_t> {
    typedef u16 store_t;
    static constexpr int kBytes = 2;
    __device__ static float load(const bf16_t* p, int64_t i) { return bf16_to_f32(p[i].bits); }
    __device__ static void store(bf16_t* p, int64_t i, float v) { p[i].bits = f32_to_bf16(v); }
};

// ---------------------------------------------------------------- MFMA -----
// 32x32 output tiles.  bf16: v_mfma_f32_32x32x16_bf16, K = 16 per instruction,
// each lane holds 8 consecutive k of one row (lane%32) starting at 8*(lane/32).
// f32: v_mfma_f32_32x32x2_f32, K = 2, each lane holds k = lane/32 of row lane%32.
// Output (both): lane holds column lane%32, rows 8*(i/4) + 4*(lane/32) + i%4 for
// accumulator register i = 0..15.
template <typename T> struct Mfma;
template <> struct Mfma<bf16_t> {
    static constexpr int kK = 16;          // k per instruction
    static constexpr int kLaneK = 8;       // consecutive k per lane
    typedef bf16x8 frag;
    __device__ static frag lds_frag(const char* row_base, int kbyte) {
        return *reinterpret_cast<const frag*>(row_base + kbyte);
    }
    __device__ static floatx16 mma(frag a, frag b, floatx16 c) {
        return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
    }
};
template <> struct Mfma<float> {
    static constexpr int kK = 2;
    static constexpr int kLaneK = 1;
    typedef float frag;
    __device__ static frag lds_frag(const char* row_base, int kbyte) {
        return *reinterpret_cast<const float*>(row_base + kbyte);
    }
    __device__ static floatx16 mma(frag a, frag b, floatx16 c) {
        return __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, c, 0, 0, 0);
    }
};

// fp8 (OCP E4M3 operands): v_mfma_f32_32x32x64_f8f6f4 with format 0 for both
// operands and no block scales, K = 64, each lane holds 32 consecutive k of row
// lane%32 starting at 32*(lane/32) (checked on the hardware); output as above.
template <> struct Mfma<fp8_t> {
    static constexpr int kK = 64;
    static constexpr int kLaneK = 32;
    typedef intx8 frag;
    __device__ static floatx16 mma(frag a, frag b, floatx16 c) {
        return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 0, 0, 0);
    }
};

__device__ __forceinline__ int acc_row(int i, int lane) {
    return 8 * (i >> 2) + 4 * (lane >> 5) + (i & 3);
}

// ------------------------------------------------------------- activation --
// silu(v) = v / (1 + exp(-v)) with the accurate expf and IEEE division.
__device__ __forceinline__ float silu_f(float v) { return v / (1.0f + expf(-v)); }

// silu(v) in float32 to within a few units in the last place, in about half the
// instructions of silu_f (for the GEMM epilogues, which apply it to every
// hidden value).  exp(-v) = 2^t, t = -v log2(e): t is rounded once (t_hi) and
// its rounding error plus the error of the float log2(e) form t_lo exactly
// enough (a fused multiply-add and a second constant), so 2^t = 2^t_hi (the
// hardware exp2, within 1 ulp) times 1 + t_lo ln 2.  The quotient v / d comes
// from the hardware reciprocal of d = 1 + exp(-v) and one Newton correction
// of the quotient itself, q + (v - d q) / d.  The exponent is capped at 80 (for
// v < -80, |silu(v)| < 1e-33 either way) so that d stays finite, and v > 80
// returns v (exp(-v) is then below half an ulp of 1).
__device__ __forceinline__ float silu_fast(float v) {
    const float x = fminf(-v, 80.0f);
    const float th = x * 1.44269502162933349609375f;                  // log2(e) rounded
    const float tl = fmaf(x, 1.44269502162933349609375f, -th) + x * 1.925963033500011e-08f;
    float e = __builtin_amdgcn_exp2f(th);
    e = fmaf(e, tl * 0.693147180559945309f, e);
    const float d = 1.0f + e;
    const float r = __builtin_amdgcn_rcpf(d);
    const float q = v * r;
    const float qc = fmaf(fmaf(-d, q, v), r, q);
    return v > 80.0f ? v : qc;
}

// Two floats to two bfloat16 (round to nearest even), packed low then high: the
// gfx950 conversion instruction.
typedef __bf16 bf16x2_hw __attribute__((ext_vector_type(2)));
typedef float floatx2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    const floatx2_t x = {lo, hi};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(x, bf16x2_hw));
}

// ------------------------------------------------------------------- misc --
__device__ __forceinline__ int64_t ceil_div64(int64_t a, int64_t b) { return (a + b - 1) / b; }

}  // namespace moe

namespace moe {
// Exclusive prefix sum across a block of up to 1024 threads (blockDim.x a
// multiple of 64).  `red` holds 16 ints of LDS.  Returns this thread's exclusive
// prefix; `total` receives the block sum.
__device__ __forceinline__ int block_exclusive_scan_1024(int v, int* red, int& total) {
    const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
    const int nw = blockDim.x >> 6;
    int x = v;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        int y = __shfl_up(x, off, 64);
        if (lane >= off) x += y;
    }
    if (lane == 63) red[wid] = x;
    __syncthreads();
    if (wid == 0) {
        int w = lane < nw ? red[lane] : 0;
#pragma unroll
        for (int off = 1; off < 16; off <<= 1) {
            int y = __shfl_up(w, off, 64);
            if (lane >= off) w += y;
        }
        if (lane < nw) red[lane] = w;
    }
    __syncthreads();
    total = red[nw - 1];
    const int before = wid > 0 ? red[wid - 1] : 0;
    __syncthreads();
    return before + x - v;
}
}  // namespace moe
