// Router: RMSNorm scale, float32 logits on the matrix cores, top-k and routing
// weights, in one kernel.
//
// Each workgroup owns 32 tokens and every expert.  With r = h * inv_rms * g the
// logits are l = inv_rms * ((h * g) W_r^T) + b, so the row scale is applied once
// to the accumulators and the K loop reads h as stored:
//   1. inverse RMS of the 32 rows (one wave per 8 rows, float32 sums);
//   2. the logits GEMM on v_mfma_f32_32x32x2_f32.  h and W_r stream into a ring
//      of four LDS stages with global_load_lds_dwordx4 (16 values of K per
//      stage), as in the grouped GEMM.  Within a stage, lane half q of an MFMA
//      takes K values 8q..8q+7 in turn (any fixed assignment of K to MFMA steps
//      gives the same sum), so each lane fetches its values of a row with
//      16-byte (8-byte) reads of a chunk-swizzled row; g multiplies the h
//      operand.  Eight waves, two per SIMD: waves 0-3 take the first four MFMA
//      steps of every stage and waves 4-7 the last four, each for a quarter of
//      the expert columns; the two partial sums are added in a fixed order at
//      the end.  While a stage sits in LDS, the workgroup also writes that slice
//      of the normalised rows r (the experts' input) when asked;
//   3. logits (scaled, plus bias) go to LDS; each wave picks the top-k of 8
//      tokens with wavefront argmax reductions over packed (value, id) keys and
//      forms the weights exp(l_j - l_max) / sum_sel exp(l_i - l_max), which equal
//      softmax over all experts renormalised over the selected ones.
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
constexpr int kThreads = 512;
constexpr int kWaves = kThreads / 64;
constexpr int kKS = 16;           // K values per stage
constexpr int kStages = 4;
constexpr int kMaxE = 512;

// s_waitcnt vmcnt(N); see the grouped GEMM for the encoding.
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}
__device__ __forceinline__ void bare_barrier() {
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}
__device__ __forceinline__ void dma16(const void* g, void* l) {
    __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void*)g,
                                     (__attribute__((address_space(3))) void*)l, 16, 0, 0);
}

// Chunk swizzles (16-byte chunk c of row r stored at c ^ swz): conflict-free
// 16-byte reads of 32 consecutive rows for 64-byte rows (float32 W_r, float32
// h) and for 32-byte rows (bfloat16 h).
__device__ __forceinline__ int swz64(int r) { return ((r >> 1) & 3) ^ ((r >> 3) & 1); }
__device__ __forceinline__ int swz32(int r) { return ((r >> 2) ^ (r >> 3)) & 1; }

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

struct RouteParams {
    const void* h;
    int64_t T;
    int d;
    const float* g;
    float eps;
    int apply_norm;
    const float* W_r;
    const float* b_r;
    int E;
    int k;
    void* r_out;
    float* logits;
    int32_t* ids;
    float* w;
};

// NB = experts padded to a multiple of 128, over 128: each wave moves NB 1-KB
// slices of W_r per stage (16 rows each), plus one slice of h (or a dummy).
template <typename Tin, typename Tr, int NB>
__global__ __launch_bounds__(kThreads, 1) void route_kernel(RouteParams rp) {
    constexpr int kInB = (int)sizeof(typename Elem<Tin>::store_t);
    constexpr int kARow = kKS * kInB;                 // bytes of an h row per stage
    constexpr int kAInstr = kTok * kARow / 1024;      // real 1-KB h slices per stage
    constexpr int kEPad = NB * 16 * kWaves;
    constexpr int kNCB = kEPad / 32;                  // 32-expert MFMA column blocks
    constexpr int kCBW = (kNCB + 3) / 4;              // per wave (dealt round-robin to
                                                      // the four waves of a K half)
    constexpr int kBBytes = kEPad * 64;
    constexpr int kStageBytes = kTok * kARow + kBBytes;
    constexpr int kDma = NB + 1;                      // DMAs per wave per stage

    extern __shared__ __attribute__((aligned(16))) char lds[];
    __shared__ float inv_rms[kTok];
    char* const dummy = lds + kStages * kStageBytes;  // sink of the padding DMAs

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int kh = wave >> 2;                         // which half of each stage's MFMA steps
    const int wc = wave & 3;                          // which quarter of the expert columns
    const int64_t t0 = (int64_t)blockIdx.x * kTok;
    const int ntok = (int)min((int64_t)kTok, rp.T - t0);
    const int d = rp.d;

    // ---- 1. inverse RMS per row
    if (rp.apply_norm) {
        for (int tt = wave; tt < kTok; tt += kWaves) {
            float ss = 0.0f;
            if (tt < ntok) {
                const char* row = (const char*)rp.h + (t0 + tt) * (int64_t)d * kInB;
                for (int c = lane * (16 / kInB); c < d; c += 64 * (16 / kInB)) {
                    const uint4 u = *(const uint4*)(row + (int64_t)c * kInB);
                    if (kInB == 4) {
                        const float v[4] = {__uint_as_float(u.x), __uint_as_float(u.y),
                                            __uint_as_float(u.z), __uint_as_float(u.w)};
#pragma unroll
                        for (int e = 0; e < 4; e++) ss += v[e] * v[e];
                    } else {
                        const uint32_t ww[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
                        for (int e = 0; e < 4; e++) {
                            const float lo = __uint_as_float(ww[e] << 16);
                            const float hi = __uint_as_float(ww[e] & 0xffff0000u);
                            ss += lo * lo + hi * hi;
                        }
                    }
                }
            }
#pragma unroll
            for (int off = 32; off >= 1; off >>= 1) ss += __shfl_xor(ss, off, 64);
            if (lane == 0) inv_rms[tt] = 1.0f / sqrtf(ss / (float)d + rp.eps);
        }
    } else if (tid < kTok) {
        inv_rms[tid] = 1.0f;
    }

    // ---- 2. DMA sources (per lane, per stage offset kt * kKS elements)
    // h: slice i holds rows (1024 / kARow) * i + lane / (kARow / 16)
    const char* a_src;
    char* a_dst;
    {
        constexpr int kChunks = kARow / 16;
        const int slice = wave < kAInstr ? wave : 0;
        const int r = slice * (1024 / kARow) + lane / kChunks;
        const int c = lane % kChunks;
        const int pc = kChunks == 4 ? (c ^ swz64(r)) : (c ^ swz32(r));
        const int rr = r < ntok ? r : 0;
        a_src = (const char*)rp.h + ((t0 + rr) * (int64_t)d) * kInB + pc * 16;
        a_dst = wave < kAInstr ? lds + slice * 1024 : dummy;
    }
    const char* b_src[NB];
#pragma unroll
    for (int i = 0; i < NB; i++) {
        const int r = (wave * NB + i) * 16 + (lane >> 2);
        const int pc = (lane & 3) ^ swz64(r & 31);
        const int e = r < rp.E ? r : 0;
        b_src[i] = (const char*)(rp.W_r + (int64_t)e * d) + pc * 16;
    }
    auto issue = [&](int kt, int buf) __attribute__((always_inline)) {
        char* st = lds + buf * kStageBytes;
        dma16(a_src + (int64_t)kt * kARow, a_dst == dummy ? dummy : st + (a_dst - lds));
#pragma unroll
        for (int i = 0; i < NB; i++)
            dma16(b_src[i] + (int64_t)kt * 64, st + kTok * kARow + (wave * NB + i) * 1024);
    };

    floatx16 acc[kCBW];
#pragma unroll
    for (int i = 0; i < kCBW; i++)
#pragma unroll
        for (int v = 0; v < 16; v++) acc[i][v] = 0.0f;

    const int nk = d / kKS;
    const int q = lane >> 5;                // which half of the stage's K this lane takes
    const int row = lane & 31;
    __syncthreads();                        // inv_rms visible
#pragma unroll
    for (int s0 = 0; s0 < kStages - 1; s0++)
        if (s0 < nk) issue(s0, s0);

    for (int kt = 0; kt < nk; kt++) {
        if (kt + 2 < nk) wait_vmcnt<2 * kDma>();
        else if (kt + 1 < nk) wait_vmcnt<kDma>();
        else wait_vmcnt<0>();
        bare_barrier();
        if (kt + kStages - 1 < nk) issue(kt + kStages - 1, (kt + kStages - 1) % kStages);
        const char* st = lds + (kt % kStages) * kStageBytes;
        const int kb = kt * kKS;

        // this wave's four MFMA steps s = 4 kh .. 4 kh + 3 use K values
        // kb + 8q + s; g for them (scalar loads of the stage's 16 values)
        float gs[4];
#pragma unroll
        for (int s = 0; s < 4; s++) {
            const float g0 = rp.g ? rp.g[kb + 4 * kh + s] : 1.0f;
            const float g1 = rp.g ? rp.g[kb + 8 + 4 * kh + s] : 1.0f;
            gs[s] = q ? g1 : g0;
        }
        // this lane's 4 values of its h row
        float a[4];
        if (kInB == 4) {
            const float4 v0 = *(const float4*)(st + row * 64 + ((2 * q + kh) ^ swz64(row)) * 16);
            a[0] = v0.x; a[1] = v0.y; a[2] = v0.z; a[3] = v0.w;
        } else {
            const uint2 u = *(const uint2*)(st + row * 32 + (q ^ swz32(row)) * 16 + kh * 8);
            a[0] = __uint_as_float(u.x << 16);
            a[1] = __uint_as_float(u.x & 0xffff0000u);
            a[2] = __uint_as_float(u.y << 16);
            a[3] = __uint_as_float(u.y & 0xffff0000u);
        }
#pragma unroll
        for (int s = 0; s < 4; s++) a[s] *= gs[s];
#pragma unroll
        for (int i = 0; i < kCBW; i++) {
            const int cb = wc + 4 * i;
            if (cb < kNCB) {
                const char* brow = st + kTok * kARow + (cb * 32 + row) * 64;
                const float4 b0 = *(const float4*)(brow + ((2 * q + kh) ^ swz64(row)) * 16);
                const float b[4] = {b0.x, b0.y, b0.z, b0.w};
#pragma unroll
                for (int s = 0; s < 4; s++)
                    acc[i] = __builtin_amdgcn_mfma_f32_32x32x2f32(a[s], b[s], acc[i], 0, 0, 0);
            }
        }
        // the normalised rows of this K slice, for the experts
        if (rp.r_out) {
            for (int idx = tid; idx < kTok * kKS; idx += kThreads) {
                const int rr = idx / kKS, kk = idx % kKS;
                if (rr < ntok) {
                    const int off = kk * kInB;
                    const int pc = (kARow == 64) ? ((off >> 4) ^ swz64(rr)) : ((off >> 4) ^ swz32(rr));
                    const char* src = st + rr * kARow + pc * 16 + (off & 15);
                    const float hv = kInB == 4 ? *(const float*)src
                                               : bf16_to_f32(*(const u16*)src);
                    const float gk = rp.g ? rp.g[kb + kk] : 1.0f;
                    Elem<Tr>::store((Tr*)rp.r_out, (t0 + rr) * (int64_t)d + kb + kk,
                                    hv * inv_rms[rr] * gk);
                }
            }
        }
    }
    __syncthreads();

    // ---- 3. logits tile in LDS (first K half, then the second added in a
    // fixed order, scaled, plus bias), then top-k per token
    float* lt = (float*)lds;                 // [kTok][kEPad + 1]
    constexpr int ldl = kEPad + 1;
    for (int half = 0; half < 2; half++) {
        if (kh == half) {
#pragma unroll
            for (int i = 0; i < kCBW; i++) {
                const int cb = wc + 4 * i;
                if (cb < kNCB) {
                    const int e = cb * 32 + row;
                    const float bias = (rp.b_r && e < rp.E) ? rp.b_r[e] : 0.0f;
#pragma unroll
                    for (int v = 0; v < 16; v++) {
                        const int tr = acc_row(v, lane);
                        if (half == 0)
                            lt[tr * ldl + e] = acc[i][v];
                        else
                            lt[tr * ldl + e] = (lt[tr * ldl + e] + acc[i][v]) * inv_rms[tr] + bias;
                    }
                }
            }
        }
        __syncthreads();
    }
    const int E = rp.E, k = rp.k;
    if (rp.logits) {
        for (int idx = tid; idx < ntok * E; idx += kThreads) {
            const int tt = idx / E, e = idx % E;
            rp.logits[(t0 + tt) * E + e] = lt[tt * ldl + e];
        }
    }
    for (int tt = wave; tt < ntok; tt += kWaves) {
        // each lane holds experts lane, lane + 64, ... ; taken ones are cleared
        constexpr int kPer = kEPad / 64;
        uint64_t key[kPer];
#pragma unroll
        for (int qq = 0; qq < kPer; qq++) {
            const int e = lane + 64 * qq;
            key[qq] = (e < E) ? (((uint64_t)order_key(lt[tt * ldl + e]) << 32) |
                                 (uint64_t)(0xFFFFFFFFu - (uint32_t)e))
                              : 0ull;
        }
        float lmax = 0.0f, sum = 0.0f, my_val = 0.0f;
        int my_id = 0;
        for (int j = 0; j < k; j++) {
            uint64_t best = 0ull;
#pragma unroll
            for (int qq = 0; qq < kPer; qq++) best = key[qq] > best ? key[qq] : best;
            best = wave_max_u64(best);
            const int sel_e = (int)(0xFFFFFFFFu - (uint32_t)best);
            const float sel_l = lt[tt * ldl + sel_e];
#pragma unroll
            for (int qq = 0; qq < kPer; qq++)
                if (lane + 64 * qq == sel_e) key[qq] = 0ull;
            if (j == 0) lmax = sel_l;
            const float ex = expf(sel_l - lmax);
            sum += ex;
            if (lane == j) {
                my_val = ex;
                my_id = sel_e;
            }
        }
        if (lane < k) {
            rp.ids[(t0 + tt) * k + lane] = my_id;
            rp.w[(t0 + tt) * k + lane] = my_val / sum;
        }
    }
}

template <typename Tin, typename Tr, int NB>
hipError_t launch_nb(const RouteParams& rp, hipStream_t s) {
    constexpr int kInB = (int)sizeof(typename Elem<Tin>::store_t);
    constexpr size_t kStage = kTok * kKS * kInB + NB * 16 * kWaves * 64;
    constexpr size_t kTile = (size_t)kTok * (NB * 16 * kWaves + 1) * 4;
    const size_t lds = (kStages * kStage + 1024) > kTile ? (kStages * kStage + 1024) : kTile;
    hipError_t e = hipFuncSetAttribute((const void*)route_kernel<Tin, Tr, NB>,
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
    const int64_t blocks = (rp.T + kTok - 1) / kTok;
    hipLaunchKernelGGL((route_kernel<Tin, Tr, NB>), dim3((unsigned)blocks), dim3(kThreads), lds, s,
                       rp);
    return hipGetLastError();
}

template <typename Tin, typename Tr>
hipError_t launch_rt(const RouteParams& rp, hipStream_t s) {
    switch ((rp.E + 16 * kWaves - 1) / (16 * kWaves)) {
        case 1: return launch_nb<Tin, Tr, 1>(rp, s);
        case 2: return launch_nb<Tin, Tr, 2>(rp, s);
        case 3: return launch_nb<Tin, Tr, 3>(rp, s);
        default: return launch_nb<Tin, Tr, 4>(rp, s);
    }
}

}  // namespace

hipError_t launch_route(const void* h, moe_dtype h_dt, int64_t T, int64_t d, const float* g,
                        float eps, int apply_norm, const float* W_r, const float* b_r, int E,
                        int k, void* r_out, moe_dtype r_dt, float* logits, int32_t* ids, float* w,
                        hipStream_t s) {
    if (T == 0) return hipSuccess;
    RouteParams rp{h, T, (int)d, apply_norm ? g : nullptr, eps, apply_norm, W_r, b_r, E, k,
                   r_out, logits, ids, w};
    if (h_dt == MOE_F32)
        return r_dt == MOE_F32 ? launch_rt<float, float>(rp, s) : launch_rt<float, bf16_t>(rp, s);
    return r_dt == MOE_F32 ? launch_rt<bf16_t, float>(rp, s) : launch_rt<bf16_t, bf16_t>(rp, s);
}

}  // namespace moe
