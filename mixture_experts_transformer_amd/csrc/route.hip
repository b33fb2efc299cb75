// Router: optional RMSNorm, float32 logits on the matrix cores, top-k and
// routing weights, in one kernel.
//
// Each workgroup owns 32 tokens and every expert.  Phase 1 computes the
// tokens' inverse RMS (one wave per 8 tokens, float32 sums).  Phase 2 is the
// logits GEMM l = r W_r^T on v_mfma_f32_32x32x2_f32: 16-wide K steps of the
// normalised rows r (written once to the optional r_out as they are formed) and
// of W_r staged in LDS, the 32-column expert blocks dealt round-robin to the 4
// waves.  Phase 3 puts the 32 x E logits (plus bias) in LDS and each wave picks
// the top-k of 8 tokens with wavefront argmax reductions over packed
// (value, id) keys, then forms the weights exp(l_j - l_max) / sum_sel exp(l_i - l_max),
// which equals softmax over all experts renormalised over the selected ones.
//
// Sources: the latent is normalised before routing (Marin 535B-A23B article,
// section "What is actually being trained"); router weight and bias (section
// "The one knob nobody pinned"); router precision matters for which experts are
// chosen (section "What I'd take from it").
#include "common.h"
#include "kernels.h"

namespace moe {

namespace {

constexpr int kTok = 32;          // tokens per workgroup
constexpr int kThreads = 256;
constexpr int kKStep = 16;        // float32 K per LDS stage (64 bytes per row)
constexpr int kLd = 20;           // padded LDS row (floats)
constexpr int kMaxE = 512;

template <typename T>
__device__ __forceinline__ float load_el(const void* p, int64_t i) {
    return Elem<T>::load((const T*)p, i);
}

// Orderable 32-bit key of a float: larger float -> larger key; -0 == +0;
// NaN below everything.
__device__ __forceinline__ uint32_t order_key(float v) {
    if (v != v) return 0u;
    if (v == 0.0f) v = 0.0f;
    uint32_t u = __float_as_uint(v);
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ uint64_t wave_max_u64(uint64_t x) {
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) {
        uint32_t lo = __shfl_xor((uint32_t)x, off, 64);
        uint32_t hi = __shfl_xor((uint32_t)(x >> 32), off, 64);
        uint64_t y = ((uint64_t)hi << 32) | lo;
        x = y > x ? y : x;
    }
    return x;
}

template <typename Tin, typename Tr>
__global__ __launch_bounds__(kThreads) void route_kernel(
    const void* h, int64_t T, int d, const float* g, float eps, int apply_norm, const float* W_r,
    const float* b_r, int E, int k, void* r_out, float* logits_out, int32_t* ids, float* w) {
    __shared__ float inv_rms[kTok];
    __shared__ __attribute__((aligned(16))) float smem[2 * (kTok + kMaxE) * kLd];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int64_t t0 = (int64_t)blockIdx.x * kTok;
    const int ntok = (int)min((int64_t)kTok, T - t0);
    const int ncb = (E + 31) / 32;               // 32-column expert blocks
    const int Epad = ncb * 32;

    // ---- phase 1: inverse RMS per token
    if (apply_norm) {
        for (int tt = wave; tt < kTok; tt += 4) {
            float ss = 0.0f;
            if (tt < ntok) {
                for (int c = lane; c < d; c += 64) {
                    float v = load_el<Tin>(h, (t0 + tt) * d + c);
                    ss += v * v;
                }
            }
#pragma unroll
            for (int off = 32; off >= 1; off >>= 1) ss += __shfl_xor(ss, off, 64);
            if (lane == 0) inv_rms[tt] = 1.0f / sqrtf(ss / (float)d + eps);
        }
    } else if (tid < kTok) {
        inv_rms[tid] = 1.0f;
    }
    __syncthreads();

    // ---- phase 2: logits GEMM on the matrix cores
    floatx16 acc[kMaxE / 32 / 4];
#pragma unroll
    for (int i = 0; i < kMaxE / 32 / 4; i++)
#pragma unroll
        for (int v = 0; v < 16; v++) acc[i][v] = 0.0f;

    const int nk = d / kKStep;
    // stage loader: A = 32 rows x 16, one float per thread for 2 threads per
    // element pair... each of the 256 threads writes 2 A elements; B = E rows x 16.
    auto stage = [&](int kt, int buf) {
        float* As = smem + buf * (kTok + kMaxE) * kLd;
        float* Bs = As + kTok * kLd;
        const int kb = kt * kKStep;
        for (int q = tid; q < kTok * kKStep; q += kThreads) {
            const int tt = q / kKStep, c = q % kKStep;
            float v = 0.0f;
            if (tt < ntok) {
                v = load_el<Tin>(h, (t0 + tt) * d + kb + c);
                if (apply_norm) v = v * inv_rms[tt] * (g ? g[kb + c] : 1.0f);
                if (r_out) Elem<Tr>::store((Tr*)r_out, (t0 + tt) * d + kb + c, v);
            }
            As[tt * kLd + c] = v;
        }
        for (int q = tid; q < Epad * (kKStep / 4); q += kThreads) {
            const int e = q / (kKStep / 4), c4 = (q % (kKStep / 4)) * 4;
            float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
            if (e < E) v = *(const float4*)(W_r + (int64_t)e * d + kb + c4);
            *(float4*)(Bs + e * kLd + c4) = v;
        }
    };

    stage(0, 0);
    __syncthreads();
    for (int kt = 0; kt < nk; kt++) {
        const int buf = kt & 1;
        if (kt + 1 < nk) stage(kt + 1, buf ^ 1);
        const float* As = smem + buf * (kTok + kMaxE) * kLd;
        const float* Bs = As + kTok * kLd;
#pragma unroll
        for (int ks = 0; ks < kKStep / 2; ks++) {
            const int kk = ks * 2 + (lane >> 5);
            const float a = As[(lane & 31) * kLd + kk];
#pragma unroll
            for (int i = 0; i < kMaxE / 32 / 4; i++) {
                const int cb = wave + 4 * i;
                if (cb < ncb) {
                    const float b = Bs[(cb * 32 + (lane & 31)) * kLd + kk];
                    acc[i] = __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, acc[i], 0, 0, 0);
                }
            }
        }
        __syncthreads();
    }

    // ---- phase 3: logits tile in LDS, then top-k per token
    float* lt = smem;                                // [kTok][Epad + 1]
    const int ldl = Epad + 1;
#pragma unroll
    for (int i = 0; i < kMaxE / 32 / 4; i++) {
        const int cb = wave + 4 * i;
        if (cb < ncb) {
            const int e = cb * 32 + (lane & 31);
            const float bias = (b_r && e < E) ? b_r[e] : 0.0f;
#pragma unroll
            for (int v = 0; v < 16; v++) lt[acc_row(v, lane) * ldl + e] = acc[i][v] + bias;
        }
    }
    __syncthreads();
    if (logits_out) {
        for (int q = tid; q < ntok * E; q += kThreads) {
            const int tt = q / E, e = q % E;
            logits_out[(t0 + tt) * E + e] = lt[tt * ldl + e];
        }
    }
    for (int tt = wave; tt < ntok; tt += 4) {
        // each lane holds experts lane, lane + 64, ... ; taken ones are cleared
        constexpr int kPer = kMaxE / 64;
        uint64_t key[kPer];
#pragma unroll
        for (int q = 0; q < kPer; q++) {
            const int e = lane + 64 * q;
            key[q] = (e < E) ? (((uint64_t)order_key(lt[tt * ldl + e]) << 32) |
                                (uint64_t)(0xFFFFFFFFu - (uint32_t)e))
                             : 0ull;
        }
        float lmax = 0.0f, sel_l = 0.0f;
        int sel_e = 0;
        float sum = 0.0f;
        float my_val = 0.0f;
        int my_id = 0;
        for (int j = 0; j < k; j++) {
            uint64_t best = 0ull;
#pragma unroll
            for (int q = 0; q < kPer; q++) best = key[q] > best ? key[q] : best;
            best = wave_max_u64(best);
            sel_e = (int)(0xFFFFFFFFu - (uint32_t)best);
            sel_l = lt[tt * ldl + sel_e];
#pragma unroll
            for (int q = 0; q < kPer; q++)
                if (lane + 64 * q == sel_e) key[q] = 0ull;
            if (j == 0) lmax = sel_l;
            const float ex = expf(sel_l - lmax);
            sum += ex;
            if (lane == j) {
                my_val = ex;
                my_id = sel_e;
            }
        }
        if (lane < k) {
            ids[(t0 + tt) * k + lane] = my_id;
            w[(t0 + tt) * k + lane] = my_val / sum;
        }
    }
}

template <typename Tin, typename Tr>
hipError_t launch_rt(const void* h, int64_t T, int64_t d, const float* g, float eps,
                     int apply_norm, const float* W_r, const float* b_r, int E, int k,
                     void* r_out, float* logits, int32_t* ids, float* w, hipStream_t s) {
    const int64_t blocks = (T + kTok - 1) / kTok;
    if (blocks == 0) return hipSuccess;
    hipLaunchKernelGGL((route_kernel<Tin, Tr>), dim3((unsigned)blocks), dim3(kThreads), 0, s, h,
                       T, (int)d, g, eps, apply_norm, W_r, b_r, E, k, r_out, logits, ids, w);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_route(const void* h, moe_dtype h_dt, int64_t T, int64_t d, const float* g,
                        float eps, int apply_norm, const float* W_r, const float* b_r, int E,
                        int k, void* r_out, moe_dtype r_dt, float* logits, int32_t* ids, float* w,
                        hipStream_t s) {
    if (h_dt == MOE_F32) {
        if (r_dt == MOE_F32)
            return launch_rt<float, float>(h, T, d, g, eps, apply_norm, W_r, b_r, E, k, r_out,
                                           logits, ids, w, s);
        return launch_rt<float, bf16_t>(h, T, d, g, eps, apply_norm, W_r, b_r, E, k, r_out,
                                        logits, ids, w, s);
    }
    if (r_dt == MOE_F32)
        return launch_rt<bf16_t, float>(h, T, d, g, eps, apply_norm, W_r, b_r, E, k, r_out,
                                        logits, ids, w, s);
    return launch_rt<bf16_t, bf16_t>(h, T, d, g, eps, apply_norm, W_r, b_r, E, k, r_out, logits,
                                     ids, w, s);
}

}  // namespace moe
