// Router: RMSNorm scale, float32 logits on the matrix cores, top-k and routing
// weights, in one kernel (route_kernel), or in two for wide routers (the
// expert-split form further down).
//
// Each workgroup owns 32 tokens and every expert.  With r = h * inv_rms * g the
// logits are l = inv_rms * ((h * g) W_r^T) + b, so the row scale is applied once
// to the accumulators and the K loop reads h as stored:
//   1. inverse RMS of the 32 rows (one wave per 4 rows, float32 sums); the same
//      pass writes the normalised rows r (the experts' input) when asked, from
//      the row values it holds in registers;
//   2. the logits GEMM on v_mfma_f32_32x32x2_f32.  h and W_r stream into a ring
//      of LDS stages with global_load_lds_dwordx4, 32 values of K per stage so
//      that a float32 row piece is a whole 128-byte cache line.  Within a
//      stage, lane half q of an MFMA takes K values 16q..16q+15 in turn (any
//      fixed assignment of K to MFMA steps gives the same sum), so each lane
//      fetches its values of a row with 16-byte reads of a chunk-swizzled row;
//      g multiplies the h operand (scalar loads).  Eight waves, two per SIMD:
//      waves 0-3 take the first eight MFMA steps of every stage and waves 4-7
//      the last eight, each for a quarter of the expert columns; the two
//      partial sums are added in a fixed order at the end.  The K loop issues
//      no vector memory access besides the DMAs, so each wait only covers the
//      stage it needs;
//   3. logits (scaled, plus bias) go to LDS; each wave picks the top-k of 4
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
constexpr int kKS = 32;           // K values per stage
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

// a pointer every lane holds the same value of, moved to scalar registers (so a
// DMA takes it as its scalar base)
__device__ __forceinline__ const void* uniform_ptr(const void* p) {
    const uint64_t x = (uint64_t)p;
    const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)x);
    const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(x >> 32));
    return (const void*)(((uint64_t)hi << 32) | lo);
}

// One 1-KB DMA (64 lanes x 16 bytes) from a wave-uniform base plus a 32-bit
// per-lane offset into LDS at byte address lds_addr, written out so that the
// compiler neither rebuilds 64-bit addresses per stage nor inserts waits of its
// own for it: every wait for these loads is the explicit vmcnt wait before the
// stage's barrier.  (M0 needs one wait state before the load reads it.)
__device__ __forceinline__ void dma16_off(const void* sbase, uint32_t voff, uint32_t lds_addr) {
    asm volatile(
        "s_mov_b32 m0, %2\n\t"
        "s_nop 0\n\t"
        "global_load_lds_dwordx4 %0, %1"
        :
        : "v"(voff), "s"(sbase), "s"(lds_addr)
        : "memory", "m0");
}
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
    return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) char*)p;
}

// Chunk swizzles (16-byte chunk c of row r stored at c ^ swz): conflict-free
// 16-byte reads of 8 (16) consecutive rows for 128-byte rows (float32 W_r,
// float32 h) and for 64-byte rows (bfloat16 h).
__device__ __forceinline__ int swz128(int r) { return (r & 7) ^ ((r >> 3) & 1); }
__device__ __forceinline__ int swz64(int r) { return ((r >> 1) & 3) ^ ((r >> 3) & 1); }

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

// Top-k of one token's E logits by one wave, and its routing weights
// exp(l_j - l_max) / sum over the selected exp(l_i - l_max), which equal softmax
// over all experts renormalised over the selected ones.  Each lane holds experts
// lane, lane + 64, ... as packed (value, id) keys: a wavefront argmax per pick,
// taken keys cleared.  logit(e) returns expert e's logit.
template <int kPer, typename Get>
__device__ __forceinline__ void select_topk(int lane, int E, int k, Get logit, int32_t* ids,
                                            float* w) {
    uint64_t key[kPer];
#pragma unroll
    for (int qq = 0; qq < kPer; qq++) {
        const int e = lane + 64 * qq;
        key[qq] = (e < E) ? (((uint64_t)order_key(logit(e)) << 32) |
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
        const float sel_l = logit(sel_e);
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
        ids[lane] = my_id;
        w[lane] = my_val / sum;
    }
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

// NH = experts padded to a multiple of 128, over 128.  A stage holds 32 K values
// of the 32 h rows and of the 128 NH W_r rows; each wave moves 2 NH 1-KB slices
// of W_r (8 rows each) per stage, plus one slice of h (or a dummy).
template <int NH>
constexpr int route_stages() { return NH <= 3 ? 3 : 2; }

template <typename Tin, typename Tr, int NH>
__global__ __launch_bounds__(kThreads, 1) void route_kernel(RouteParams rp) {
    constexpr int kInB = (int)sizeof(typename Elem<Tin>::store_t);
    constexpr int kARow = kKS * kInB;                 // bytes of an h row per stage
    constexpr int kAChunks = kARow / 16;
    constexpr int kAInstr = kTok * kARow / 1024;      // real 1-KB h slices per stage
    constexpr int NB = 2 * NH;                        // W_r slices per wave per stage
    constexpr int kEPad = 128 * NH;
    constexpr int kNCB = kEPad / 32;                  // 32-expert MFMA column blocks
    constexpr int kCBW = NH;                          // per wave (dealt round-robin to
                                                      // the four waves of a K half)
    constexpr int kStages = route_stages<NH>();
    constexpr int kStageBytes = kTok * kARow + kEPad * 128;
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

    // ---- 1. inverse RMS per row (1 without the norm); then, if asked, the
    // normalised rows
    for (int tt = wave; tt < kTok; tt += kWaves) {
        const char* row = (const char*)rp.h + (t0 + tt) * (int64_t)d * kInB;
        float ir = 1.0f;
        if (rp.apply_norm) {
            float ss = 0.0f;
            if (tt < ntok) {
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
            ir = 1.0f / sqrtf(ss / (float)d + rp.eps);
        }
        if (lane == 0) inv_rms[tt] = ir;
        if (rp.r_out && tt < ntok) {
            // the row again (from L2), 4 values per lane per step
            for (int c = lane * 4; c < d; c += 256) {
                float v[4];
                if (kInB == 4) {
                    const float4 f = *(const float4*)(row + (int64_t)c * 4);
                    v[0] = f.x; v[1] = f.y; v[2] = f.z; v[3] = f.w;
                } else {
                    const uint2 u = *(const uint2*)(row + (int64_t)c * 2);
                    v[0] = __uint_as_float(u.x << 16);
                    v[1] = __uint_as_float(u.x & 0xffff0000u);
                    v[2] = __uint_as_float(u.y << 16);
                    v[3] = __uint_as_float(u.y & 0xffff0000u);
                }
                const float4 gg = rp.g ? *(const float4*)(rp.g + c) : make_float4(1, 1, 1, 1);
                v[0] *= ir * gg.x;
                v[1] *= ir * gg.y;
                v[2] *= ir * gg.z;
                v[3] *= ir * gg.w;
                const int64_t o = (t0 + tt) * (int64_t)d + c;
                if (sizeof(typename Elem<Tr>::store_t) == 4) {
                    *(float4*)((float*)rp.r_out + o) = make_float4(v[0], v[1], v[2], v[3]);
                } else {
                    uint2 u;
                    u.x = (uint32_t)f32_to_bf16(v[0]) | ((uint32_t)f32_to_bf16(v[1]) << 16);
                    u.y = (uint32_t)f32_to_bf16(v[2]) | ((uint32_t)f32_to_bf16(v[3]) << 16);
                    *(uint2*)((u16*)rp.r_out + o) = u;
                }
            }
        }
    }

    // ---- 2. DMA sources (per lane, per stage offset kt * kKS elements)
    const int nk = (d + kKS - 1) / kKS;
    const bool tail16 = (d % kKS) != 0;
    // Each DMA source is a wave-uniform base (advanced per stage in scalar
    // registers) plus a fixed 32-bit per-lane offset, so no address register is
    // rewritten while its DMA may still be in flight.  When d is an odd multiple
    // of 16 the last stage takes the row's last 32 values (its base moved back
    // by 16): its first half was already summed in the previous stage and is
    // zeroed, its second half is the 16-value tail (d >= 48 then).
    const char* const a_base = (const char*)rp.h + t0 * (int64_t)d * kInB;
    uint32_t a_off;
    char* a_dst;
    {
        const int slice = wave < kAInstr ? wave : 0;
        const int r = slice * (1024 / kARow) + lane / kAChunks;
        const int c = lane % kAChunks;
        const int pc = kAChunks == 8 ? (c ^ swz128(r)) : (c ^ swz64(r));
        const int rr = r < ntok ? r : 0;
        a_off = (uint32_t)(rr * d * kInB + pc * 16);
        a_dst = wave < kAInstr ? lds + slice * 1024 : dummy;
    }
    uint32_t b_off[NB];
#pragma unroll
    for (int i = 0; i < NB; i++) {
        const int r = (wave * NB + i) * 8 + (lane >> 3);
        const int pc = (lane & 7) ^ swz128(r & 31);
        const int e = r < rp.E ? r : 0;
        b_off[i] = (uint32_t)(e * d * 4 + pc * 16);
    }
    auto issue = [&](int kt, int buf) __attribute__((always_inline)) {
        char* st = lds + buf * kStageBytes;
        char* const ad = a_dst == dummy ? dummy : st + (a_dst - lds);
        const int64_t k0 = (int64_t)kt * kKS - (tail16 && kt == nk - 1 ? kKS / 2 : 0);
        const void* const Ak = uniform_ptr(a_base + k0 * kInB);
        const void* const Bk = uniform_ptr((const char*)rp.W_r + k0 * 4);
        const uint32_t st_addr = lds_addr(st);
        dma16_off(Ak, a_off, lds_addr(ad));
#pragma unroll
        for (int i = 0; i < NB; i++)
            dma16_off(Bk, b_off[i], st_addr + kTok * kARow + (wave * NB + i) * 1024);
    };

    floatx16 acc[kCBW];
#pragma unroll
    for (int i = 0; i < kCBW; i++)
#pragma unroll
        for (int v = 0; v < 16; v++) acc[i][v] = 0.0f;

    const int q = lane >> 5;                // which half of the stage's K this lane takes
    const int row = lane & 31;
    // This lane's eight MFMA steps of stage kt use K values kt*32 + 16 q + 8 kh
    // + 0..7 (in the tail stage, values 16 lower; its q = 0 lanes are zeroed).
    // The gains of both halves are scalar loads issued at the end of the stage
    // before, after its MFMAs.
    // (read through the constant address space: the gains are never written
    // here, and the loads then go through the scalar unit)
    typedef const __attribute__((address_space(4))) float* cgp;
    typedef float f32x8 __attribute__((ext_vector_type(8)));
    f32x8 g0n, g1n;
    auto load_g = [&](int kt) __attribute__((always_inline)) {
        const int kb = kt * kKS;
        const bool tl = tail16 && kt == nk - 1;
        if (rp.g) {
            // in the tail stage the q = 1 lanes take the first 16 gains
            const cgp g = (cgp)rp.g + kb + 8 * kh;
            g0n = *(const __attribute__((address_space(4))) f32x8*)g;
            g1n = *(const __attribute__((address_space(4))) f32x8*)(g + (tl ? 0 : 16));
        } else {
            g0n = 1.0f;
            g1n = 1.0f;
        }
    };
    __syncthreads();                        // inv_rms visible
    load_g(0);
#pragma unroll
    for (int s0 = 0; s0 < kStages - 1; s0++)
        if (s0 < nk) issue(s0, s0);

    int buf = 0;
    for (int kt = 0; kt < nk; kt++) {
        // stage kt has landed once at most the later issued stages are in flight
        if (kStages == 3 && kt + 1 < nk) wait_vmcnt<kDma>();
        else wait_vmcnt<0>();
        bare_barrier();
        const bool dead = tail16 && kt == nk - 1 && q == 0;
        const f32x8 gq = q ? g1n : g0n;
        float gs[8];
#pragma unroll
        for (int s2 = 0; s2 < 8; s2++) gs[s2] = dead ? 0.0f : gq[s2];
        {
            // into the slot of stage kt-1; past the last stage the DMAs re-read
            // it into a slot nothing reads any more
            const int nb = buf == 0 ? kStages - 1 : buf - 1;
            issue(min(kt + kStages - 1, nk - 1), nb);
        }
        const char* st = lds + buf * kStageBytes;
        buf = buf + 1 == kStages ? 0 : buf + 1;
        // this lane's 8 values of its h row
        float a[8];
        if (kInB == 4) {
            const int c0 = 4 * q + 2 * kh;
            const float4 v0 = *(const float4*)(st + row * 128 + ((c0) ^ swz128(row)) * 16);
            const float4 v1 = *(const float4*)(st + row * 128 + ((c0 + 1) ^ swz128(row)) * 16);
            a[0] = v0.x; a[1] = v0.y; a[2] = v0.z; a[3] = v0.w;
            a[4] = v1.x; a[5] = v1.y; a[6] = v1.z; a[7] = v1.w;
        } else {
            const uint4 u = *(const uint4*)(st + row * 64 + ((2 * q + kh) ^ swz64(row)) * 16);
            const uint32_t ww[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
            for (int e = 0; e < 4; e++) {
                a[2 * e] = __uint_as_float(ww[e] << 16);
                a[2 * e + 1] = __uint_as_float(ww[e] & 0xffff0000u);
            }
        }
#pragma unroll
        for (int s2 = 0; s2 < 8; s2++) a[s2] *= gs[s2];
#pragma unroll
        for (int i = 0; i < kCBW; i++) {
            const int cb = wc + 4 * i;
            if (cb < kNCB) {
                const char* brow = st + kTok * kARow + (cb * 32 + row) * 128;
                const int c0 = 4 * q + 2 * kh;
                const float4 b0 = *(const float4*)(brow + ((c0) ^ swz128(row)) * 16);
                const float4 b1 = *(const float4*)(brow + ((c0 + 1) ^ swz128(row)) * 16);
                const float b[8] = {b0.x, b0.y, b0.z, b0.w, b1.x, b1.y, b1.z, b1.w};
#pragma unroll
                for (int s2 = 0; s2 < 8; s2++)
                    acc[i] = __builtin_amdgcn_mfma_f32_32x32x2f32(a[s2], b[s2], acc[i], 0, 0, 0);
            }
        }
        // the next stage's gains, once this stage's MFMAs are issued
        load_g(min(kt + 1, nk - 1));
    }
    // The last stage's re-read may still be landing in a ring slot the logits
    // tile below overlaps; the compiler does not see the DMAs, so the wait is
    // explicit.
    wait_vmcnt<0>();
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
    for (int tt = wave; tt < ntok; tt += kWaves)
        select_topk<kEPad / 64>(
            lane, E, k, [&](int e) { return lt[tt * ldl + e]; }, rp.ids + (t0 + tt) * k,
            rp.w + (t0 + tt) * k);
}

// ---- Expert-split form, for wide routers (E > 256) with a logits output.  The
// float32 W_r of 384 experts (384 x 3,072 x 4 bytes = 4.7 MB) does not fit one
// XCD's 4 MB L2, and every workgroup of route_kernel streams all of it for its
// 32 tokens.  Here a workgroup owns 64 tokens and one half of the experts, and
// the halves are dealt by XCD: workgroup b runs on XCD b % 8, and XCDs 0-3 take
// the first half, 4-7 the second, so each XCD's L2 serves one 2.4 MB half to its
// 32 CUs.  The row pass of route_kernel (the inverse RMS and the normalised
// rows, computed by each workgroup for its 32 rows before its logits loop) is
// replaced:
// the inverse RMS is summed from the h values the K loop already reads, and the
// normalised rows are written by a second kernel with one wave per token.  Two
// kernels:
//   route_logits_kernel: the logits of its 64 tokens x E/2 experts, as in
//     route_kernel (float32 MFMAs on g-scaled h, K halves summed in a fixed
//     order, then scaled by the inverse RMS, plus bias), written to the logits
//     output; the first half's workgroups leave the inverse RMS in
//     topk_w[t * k] for the second kernel;
//   route_select_kernel: one wave per token: the normalised row r (when asked),
//     then top-k and the weights from the logits.
constexpr int kTokS = 64;   // tokens per workgroup in the expert-split form

// CB: 32-expert MFMA column blocks per wave; a half holds up to 64 CB experts
template <typename Tin, int CB>
__global__ __launch_bounds__(kThreads, 1) void route_logits_kernel(RouteParams rp, int EH) {
    constexpr int kInB = (int)sizeof(typename Elem<Tin>::store_t);
    constexpr int kARow = kKS * kInB;                 // bytes of an h row per stage
    constexpr int kAChunks = kARow / 16;
    constexpr int kASlices = kTokS * kARow / 1024;    // 1-KB h slices per stage (8 or 4)
    constexpr int kEP = 64 * CB;                      // experts of a half, padded
    constexpr int kStageBytes = kTokS * kARow + kEP * 128;
    constexpr int kStages = kStageBytes <= 32768 ? 4 : 3;
    constexpr int kDma = CB + 1;                      // DMAs per wave per stage
    static_assert(kASlices <= kWaves, "one h slice per wave at most");

    extern __shared__ __attribute__((aligned(16))) char lds[];
    __shared__ float inv_rms[kTokS];
    __shared__ float ss_half[2][kTokS];
    char* const dummy = lds + kStages * kStageBytes;  // sink of the padding DMAs

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int kh = wave >> 2;                         // which half of each stage's MFMA steps
    const int wr = (wave >> 1) & 1;                   // which 32 of the 64 rows
    const int wc = wave & 1;                          // which CB column blocks of the half
    const int xcd = blockIdx.x & 7;
    const int hf = xcd >> 2;                          // expert half
    const int64_t t0 = ((int64_t)(xcd & 3) + 4 * (int64_t)(blockIdx.x >> 3)) * kTokS;
    if (t0 >= rp.T) return;
    const int ntok = (int)min((int64_t)kTokS, rp.T - t0);
    const int e0 = hf * EH;                           // first expert of the half
    const int ne = min(EH, rp.E - e0);                // experts of the half
    const int d = rp.d;
    const int nk = (d + kKS - 1) / kKS;
    const bool tail16 = (d % kKS) != 0;

    // DMA sources: wave-uniform bases advanced per stage plus fixed 32-bit lane
    // offsets, as in route_kernel (the tail stage is moved back by 16 values)
    const char* const a_base = (const char*)rp.h + t0 * (int64_t)d * kInB;
    const char* const b_base = (const char*)rp.W_r + (int64_t)e0 * d * 4;
    uint32_t a_off;
    {
        const int slice = wave < kASlices ? wave : 0;
        const int r = slice * (1024 / kARow) + lane / kAChunks;
        const int c = lane % kAChunks;
        const int pc = kAChunks == 8 ? (c ^ swz128(r)) : (c ^ swz64(r));
        const int rr = r < ntok ? r : 0;
        a_off = (uint32_t)(rr * d * kInB + pc * 16);
    }
    uint32_t b_off[CB];
#pragma unroll
    for (int i = 0; i < CB; i++) {
        const int r = (wave * CB + i) * 8 + (lane >> 3);
        const int pc = (lane & 7) ^ swz128(r & 31);
        const int e = r < ne ? r : 0;
        b_off[i] = (uint32_t)(e * d * 4 + pc * 16);
    }
    auto issue = [&](int kt, int buf) __attribute__((always_inline)) {
        char* st = lds + buf * kStageBytes;
        const int64_t k0 = (int64_t)kt * kKS - (tail16 && kt == nk - 1 ? kKS / 2 : 0);
        const void* const Ak = uniform_ptr(a_base + k0 * kInB);
        const void* const Bk = uniform_ptr(b_base + k0 * 4);
        const uint32_t st_addr = lds_addr(st);
        dma16_off(Ak, a_off, wave < kASlices ? st_addr + wave * 1024 : lds_addr(dummy));
#pragma unroll
        for (int i = 0; i < CB; i++)
            dma16_off(Bk, b_off[i], st_addr + kTokS * kARow + (wave * CB + i) * 1024);
    };

    floatx16 acc[CB];
#pragma unroll
    for (int i = 0; i < CB; i++)
#pragma unroll
        for (int v = 0; v < 16; v++) acc[i][v] = 0.0f;

    const int q = lane >> 5;                // which half of the stage's K this lane takes
    const int row = lane & 31;
    const int arow = wr * 32 + row;         // this lane's h row within the 64
    typedef const __attribute__((address_space(4))) float* cgp;
    typedef float f32x8 __attribute__((ext_vector_type(8)));
    f32x8 g0n, g1n;
    auto load_g = [&](int kt) __attribute__((always_inline)) {
        const int kb = kt * kKS;
        const bool tl = tail16 && kt == nk - 1;
        if (rp.g) {
            const cgp g = (cgp)rp.g + kb + 8 * kh;
            g0n = *(const __attribute__((address_space(4))) f32x8*)g;
            g1n = *(const __attribute__((address_space(4))) f32x8*)(g + (tl ? 0 : 16));
        } else {
            g0n = 1.0f;
            g1n = 1.0f;
        }
    };
    load_g(0);
#pragma unroll
    for (int s0 = 0; s0 < kStages - 1; s0++)
        if (s0 < nk) issue(s0, s0);

    // sum of squares of this lane's h values (waves of the first column half
    // only: the other half reads the same values)
    float ss = 0.0f;
    int buf = 0;
    for (int kt = 0; kt < nk; kt++) {
        // stage kt has landed once at most the kStages - 2 later stages are in
        // flight (every iteration issues one, re-reads past the end included)
        if (nk >= kStages - 1) wait_vmcnt<(kStages - 2) * kDma>();
        else wait_vmcnt<0>();
        bare_barrier();
        const bool dead = tail16 && kt == nk - 1 && q == 0;
        const f32x8 gq = q ? g1n : g0n;
        float gs[8];
#pragma unroll
        for (int s2 = 0; s2 < 8; s2++) gs[s2] = dead ? 0.0f : gq[s2];
        {
            // into the slot of stage kt-1; past the last stage the DMAs re-read
            // it into a slot nothing reads any more
            const int nb = buf == 0 ? kStages - 1 : buf - 1;
            issue(min(kt + kStages - 1, nk - 1), nb);
        }
        const char* st = lds + buf * kStageBytes;
        buf = buf + 1 == kStages ? 0 : buf + 1;
        float a[8];
        if (kInB == 4) {
            const int c0 = 4 * q + 2 * kh;
            const float4 v0 = *(const float4*)(st + arow * 128 + ((c0) ^ swz128(arow)) * 16);
            const float4 v1 = *(const float4*)(st + arow * 128 + ((c0 + 1) ^ swz128(arow)) * 16);
            a[0] = v0.x; a[1] = v0.y; a[2] = v0.z; a[3] = v0.w;
            a[4] = v1.x; a[5] = v1.y; a[6] = v1.z; a[7] = v1.w;
        } else {
            const uint4 u = *(const uint4*)(st + arow * 64 + ((2 * q + kh) ^ swz64(arow)) * 16);
            const uint32_t ww[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
            for (int e = 0; e < 4; e++) {
                a[2 * e] = __uint_as_float(ww[e] << 16);
                a[2 * e + 1] = __uint_as_float(ww[e] & 0xffff0000u);
            }
        }
        if (wc == 0 && !dead) {
#pragma unroll
            for (int s2 = 0; s2 < 8; s2++) ss += a[s2] * a[s2];
        }
#pragma unroll
        for (int s2 = 0; s2 < 8; s2++) a[s2] *= gs[s2];
        // the column blocks' MFMAs interleaved step by step (CB independent
        // accumulations in flight)
        float b[CB][8];
#pragma unroll
        for (int i = 0; i < CB; i++) {
            const char* brow = st + kTokS * kARow + ((wc * CB + i) * 32 + row) * 128;
            const int c0 = 4 * q + 2 * kh;
            const float4 b0 = *(const float4*)(brow + ((c0) ^ swz128(row)) * 16);
            const float4 b1 = *(const float4*)(brow + ((c0 + 1) ^ swz128(row)) * 16);
            b[i][0] = b0.x; b[i][1] = b0.y; b[i][2] = b0.z; b[i][3] = b0.w;
            b[i][4] = b1.x; b[i][5] = b1.y; b[i][6] = b1.z; b[i][7] = b1.w;
        }
#pragma unroll
        for (int s2 = 0; s2 < 8; s2++)
#pragma unroll
            for (int i = 0; i < CB; i++)
                acc[i] = __builtin_amdgcn_mfma_f32_32x32x2f32(a[s2], b[i][s2], acc[i], 0, 0, 0);
        load_g(min(kt + 1, nk - 1));
    }
    // the last re-read may still be landing in a slot the logits tile overlaps
    wait_vmcnt<0>();

    // ---- inverse RMS of the 64 rows: lanes row and row + 32 hold the two K
    // quarters of a stage, the kh waves its two halves (summed in that order)
    ss += __shfl_xor(ss, 32, 64);
    if (wc == 0 && lane < 32) ss_half[kh][arow] = ss;
    __syncthreads();
    if (tid < kTokS) {
        const float t2 = ss_half[0][tid] + ss_half[1][tid];
        inv_rms[tid] = rp.apply_norm ? 1.0f / sqrtf(t2 / (float)d + rp.eps) : 1.0f;
    }
    __syncthreads();

    // ---- logits tile in LDS (first K half, then the second added, scaled,
    // plus bias), written out
    float* lt = (float*)lds;                 // [kTokS][kEP + 1]
    constexpr int ldl = kEP + 1;
    for (int half = 0; half < 2; half++) {
        if (kh == half) {
#pragma unroll
            for (int i = 0; i < CB; i++) {
                const int el = (wc * CB + i) * 32 + row;
                const float bias = (rp.b_r && el < ne) ? rp.b_r[e0 + el] : 0.0f;
#pragma unroll
                for (int v = 0; v < 16; v++) {
                    const int tr = wr * 32 + acc_row(v, lane);
                    if (half == 0)
                        lt[tr * ldl + el] = acc[i][v];
                    else
                        lt[tr * ldl + el] = (lt[tr * ldl + el] + acc[i][v]) * inv_rms[tr] + bias;
                }
            }
        }
        __syncthreads();
    }
    const int E = rp.E;
    for (int idx = tid; idx < ntok * ne; idx += kThreads) {
        const int tt = idx / ne, j = idx % ne;
        rp.logits[(t0 + tt) * E + e0 + j] = lt[tt * ldl + j];
    }
    if (hf == 0 && rp.r_out)
        for (int tt = tid; tt < ntok; tt += kThreads) rp.w[(t0 + tt) * rp.k] = inv_rms[tt];
}

// One wave per token: the normalised row r = h * inv_rms * g (when asked), then
// top-k over the token's logits.  KPER = experts per lane (E padded to 64 KPER).
template <typename Tin, typename Tr, int KPER>
__global__ __launch_bounds__(256) void route_select_kernel(RouteParams rp) {
    constexpr int kInB = (int)sizeof(typename Elem<Tin>::store_t);
    const int lane = threadIdx.x & 63;
    const int64_t t = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    if (t >= rp.T) return;
    const int E = rp.E, k = rp.k, d = rp.d;
    if (rp.r_out) {
        // the inverse RMS the logits kernel left in this token's first weight
        const float ir = rp.w[t * k];
        const char* row = (const char*)rp.h + t * (int64_t)d * kInB;
        // U chunks of 4 values per lane per pass, all loaded before any is stored
        // (one pass per 6 KB of float32 row: the wave's loads are in flight together)
        constexpr int U = 6;
        for (int c0 = lane * 4; c0 < d; c0 += 256 * U) {
            float v[U][4];
            float4 gg[U];
#pragma unroll
            for (int u = 0; u < U; u++) {
                const int c = c0 + 256 * u;
                if (c < d) {
                    if (kInB == 4) {
                        const float4 f = *(const float4*)(row + (int64_t)c * 4);
                        v[u][0] = f.x; v[u][1] = f.y; v[u][2] = f.z; v[u][3] = f.w;
                    } else {
                        const uint2 x = *(const uint2*)(row + (int64_t)c * 2);
                        v[u][0] = __uint_as_float(x.x << 16);
                        v[u][1] = __uint_as_float(x.x & 0xffff0000u);
                        v[u][2] = __uint_as_float(x.y << 16);
                        v[u][3] = __uint_as_float(x.y & 0xffff0000u);
                    }
                    gg[u] = rp.g ? *(const float4*)(rp.g + c) : make_float4(1, 1, 1, 1);
                }
            }
#pragma unroll
            for (int u = 0; u < U; u++) {
                const int c = c0 + 256 * u;
                if (c < d) {
                    v[u][0] *= ir * gg[u].x;
                    v[u][1] *= ir * gg[u].y;
                    v[u][2] *= ir * gg[u].z;
                    v[u][3] *= ir * gg[u].w;
                    const int64_t o = t * (int64_t)d + c;
                    if (sizeof(typename Elem<Tr>::store_t) == 4) {
                        *(float4*)((float*)rp.r_out + o) =
                            make_float4(v[u][0], v[u][1], v[u][2], v[u][3]);
                    } else {
                        uint2 x;
                        x.x = (uint32_t)f32_to_bf16(v[u][0]) | ((uint32_t)f32_to_bf16(v[u][1]) << 16);
                        x.y = (uint32_t)f32_to_bf16(v[u][2]) | ((uint32_t)f32_to_bf16(v[u][3]) << 16);
                        *(uint2*)((u16*)rp.r_out + o) = x;
                    }
                }
            }
        }
    }
    const float* lrow = rp.logits + t * E;
    select_topk<KPER>(lane, E, k, [&](int e) { return lrow[e]; }, rp.ids + t * k, rp.w + t * k);
}

template <typename Tin, typename Tr, int CB>
hipError_t launch_split(const RouteParams& rp, hipStream_t s) {
    constexpr int kInB = (int)sizeof(typename Elem<Tin>::store_t);
    constexpr size_t kStage = (size_t)kTokS * kKS * kInB + (size_t)64 * CB * 128;
    constexpr size_t kRing = (kStage <= 32768 ? 4 : 3) * kStage + 1024;
    constexpr size_t kTile = (size_t)kTokS * (64 * CB + 1) * 4;
    const size_t lds = kRing > kTile ? kRing : kTile;
    hipError_t e = hipFuncSetAttribute((const void*)route_logits_kernel<Tin, CB>,
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
    const int EH = (rp.E + 1) / 2;
    const int64_t ntb = (rp.T + kTokS - 1) / kTokS;      // token blocks
    const int64_t blocks = 8 * ((ntb + 3) / 4);          // 4 token blocks per XCD row
    hipLaunchKernelGGL((route_logits_kernel<Tin, CB>), dim3((unsigned)blocks), dim3(kThreads), lds,
                       s, rp, EH);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((route_select_kernel<Tin, Tr, 2 * CB>), dim3((unsigned)((rp.T + 3) / 4)),
                       dim3(256), 0, s, rp);
    return hipGetLastError();
}

template <typename Tin, typename Tr, int NH>
hipError_t launch_nh(const RouteParams& rp, hipStream_t s) {
    constexpr int kInB = (int)sizeof(typename Elem<Tin>::store_t);
    constexpr size_t kStage = (size_t)kTok * kKS * kInB + (size_t)128 * NH * 128;
    constexpr size_t kTile = (size_t)kTok * (128 * NH + 1) * 4;
    constexpr size_t kRing = route_stages<NH>() * kStage + 1024;
    const size_t lds = kRing > kTile ? kRing : kTile;
    hipError_t e = hipFuncSetAttribute((const void*)route_kernel<Tin, Tr, NH>,
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
    const int64_t blocks = (rp.T + kTok - 1) / kTok;
    hipLaunchKernelGGL((route_kernel<Tin, Tr, NH>), dim3((unsigned)blocks), dim3(kThreads), lds, s,
                       rp);
    return hipGetLastError();
}

template <typename Tin, typename Tr>
hipError_t launch_rt(const RouteParams& rp, hipStream_t s) {
    // wide routers whose logits have somewhere to go take the expert-split form
    if (rp.E > 256 && rp.logits)
        return rp.E > 384 ? launch_split<Tin, Tr, 4>(rp, s) : launch_split<Tin, Tr, 3>(rp, s);
    switch ((rp.E + 127) / 128) {
        case 1: return launch_nh<Tin, Tr, 1>(rp, s);
        case 2: return launch_nh<Tin, Tr, 2>(rp, s);
        case 3: return launch_nh<Tin, Tr, 3>(rp, s);
        default: return launch_nh<Tin, Tr, 4>(rp, s);
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
