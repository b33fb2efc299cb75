// Grouped / dense MFMA GEMM for gfx950, with the epilogues the layer needs.
//
//   C[r, n] = epi( sum_s sum_k A_s[arow(r), k] * B_s[brow(g, n), k] )
//
// Both operands are contiguous along k ("[out, in]" weights).  Rows may be
// grouped by expert (the pages' ragged_dot with group sizes / cu_seqlens:
// Marin: Week of April 26th summary; Marin 535B-A23B article, section "21% to
// 27% MFU without stopping the run"): rows [offsets[g], offsets[g+1]) use expert
// g's weights.  Only active rows are computed: a 32-row MFMA block that lies
// wholly past its group's end issues no loads and no MFMAs (the "mask-free"
// ragged expert MLP of the same article section).  A rows may be gathered
// through a row map (the layer reads its routed rows straight from the token
// matrix instead of a permuted copy).
//
// Tiling: 256 threads = 4 waves as 2 x 2.  A block tile is BM rows x 128 LDS
// columns of B; a K step is 64 bytes of every row (32 bf16 / 16 f32), staged in
// LDS with 80-byte rows (16 bytes of padding keep the 16-byte fragment reads of
// 16 consecutive rows on distinct banks) and double-buffered through registers.
// Wave (wm, wn) owns the 32-row blocks wm, wm+2, ... (interleaved so both row
// waves stay busy on a partial tile) and LDS columns [64 wn, 64 wn + 64) as two
// 32-column MFMA blocks.  For the SwiGLU epilogue those two blocks are the gate
// and the up rows of the same 32 hidden columns, so the activation is formed in
// registers and neither G nor U is ever stored.
//
// Scheduling: a persistent grid (a multiple of 8 workgroups).  Workgroups are
// dealt to the 8 XCDs round-robin, so workgroup b runs on XCD b % 8; each XCD
// takes a contiguous eighth of the tile sequence, which keeps an expert's
// activation panel and weight tiles in that XCD's L2 while it is in use.  The
// number of row tiles of a grouped GEMM is read from the device-side tile prefix
// written by the kernel before it on the same stream (stream order is the fence;
// nothing reads the boundaries before that kernel has finished).
#include "common.h"
#include "kernels.h"

namespace moe {

namespace {

constexpr int kThreads = 256;
constexpr int kBN = 128;          // LDS rows of B per tile
constexpr int kRowBytes = 64;     // bytes of each row per K step
constexpr int kLdsRow = 80;       // padded LDS row stride
constexpr int kStageLd = 68;      // epilogue staging row stride (floats)

template <typename OutT, int kVec>
__device__ __forceinline__ void store_vec(OutT* C, int64_t off, const float* v);
template <>
__device__ __forceinline__ void store_vec<float, 4>(float* C, int64_t off, const float* v) {
    *(float4*)(C + off) = make_float4(v[0], v[1], v[2], v[3]);
}
template <>
__device__ __forceinline__ void store_vec<bf16_t, 8>(bf16_t* C, int64_t off, const float* v) {
    uint4 u;
    u.x = (uint32_t)f32_to_bf16(v[0]) | ((uint32_t)f32_to_bf16(v[1]) << 16);
    u.y = (uint32_t)f32_to_bf16(v[2]) | ((uint32_t)f32_to_bf16(v[3]) << 16);
    u.z = (uint32_t)f32_to_bf16(v[4]) | ((uint32_t)f32_to_bf16(v[5]) << 16);
    u.w = (uint32_t)f32_to_bf16(v[6]) | ((uint32_t)f32_to_bf16(v[7]) << 16);
    *(uint4*)(C + off) = u;
}

__device__ __forceinline__ int find_group(const int32_t* tp, int G, int m) {
    // largest g in [0, G) with tp[g] <= m  (tp non-decreasing, tp[0] = 0)
    int lo = 0, hi = G;           // invariant: tp[lo] <= m < tp[hi]
    while (hi - lo > 1) {
        int mid = (lo + hi) >> 1;
        if (tp[mid] <= m) lo = mid; else hi = mid;
    }
    return lo;
}

template <typename T, typename OutT, int EPI, int BM>
__global__ __launch_bounds__(kThreads, 1) void gemm_kernel(GemmParams p) {
    constexpr int kElem = Elem<T>::kBytes;
    constexpr int kRB = BM / 64;                 // row blocks per wave
    constexpr int kAChunks = BM * 4 / kThreads;  // 16-byte chunks per thread (A)
    constexpr int kBChunks = kBN * 4 / kThreads; // (B)
    constexpr int kSteps = kRowBytes / (Mfma<T>::kK * kElem);
    constexpr int kColsOut = (EPI == EPI_SWIGLU) ? kBN / 2 : kBN;

    __shared__ __attribute__((aligned(16))) char lds[2][(BM + kBN) * kLdsRow];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int wm = wave >> 1, wn = wave & 1;

    // ---- tile space
    const int64_t n_tiles_n = (p.N + kColsOut - 1) / kColsOut;
    int64_t n_tiles_m;
    if (p.offsets) n_tiles_m = p.tile_prefix[p.G];
    else n_tiles_m = (p.M + BM - 1) / BM;
    const int64_t total = n_tiles_m * n_tiles_n;
    const int xcd = blockIdx.x % kNumXcd;
    const int slot = blockIdx.x / kNumXcd;
    const int nslots = gridDim.x / kNumXcd;
    const int64_t lo = total * xcd / kNumXcd;
    const int64_t hi = total * (xcd + 1) / kNumXcd;

    for (int64_t t = lo + slot; t < hi; t += nslots) {
        // ---- tile coordinates (grouped swizzle along m)
        const int64_t gsz = (int64_t)p.group_m * n_tiles_n;
        const int64_t super = t / gsz;
        const int64_t within = t - super * gsz;
        const int64_t m_first = super * p.group_m;
        const int64_t gm = min((int64_t)p.group_m, n_tiles_m - m_first);
        const int64_t tm = m_first + within % gm;
        const int64_t tn = within / gm;

        int g = 0;
        int64_t row0, rows_valid;
        if (p.offsets) {
            g = find_group(p.tile_prefix, p.G, (int)tm);
            const int64_t mloc = tm - p.tile_prefix[g];
            row0 = p.offsets[g] + mloc * BM;
            rows_valid = min((int64_t)BM, (int64_t)p.offsets[g + 1] - row0);
        } else {
            row0 = tm * BM;
            rows_valid = min((int64_t)BM, p.M - row0);
        }
        const int nrb_active = (int)((rows_valid + 31) >> 5);       // active 32-row blocks
        const int n_act = (nrb_active - wm + 1) >> 1;              // this wave's active blocks
        const int64_t n0 = tn * kColsOut;

        // ---- per-thread source rows
        int64_t a_row[kAChunks];
        bool a_ok[kAChunks];
#pragma unroll
        for (int i = 0; i < kAChunks; i++) {
            // rows of a 32-row block past the group's end are never loaded
            // (wave-uniform: a wave's 16 rows of chunk i share one block);
            // rows past the end inside a partial block read the first row
            // instead, and their results are never stored.
            const int r = (tid >> 2) + 64 * i;
            a_ok[i] = (r >> 5) < nrb_active;
            int64_t src = row0 + (r < rows_valid ? r : 0);
            if (p.a_rows) src = p.a_rows[src] / p.a_div;
            a_row[i] = src;
        }
        int64_t b_row[kBChunks];
#pragma unroll
        for (int i = 0; i < kBChunks; i++) {
            const int j = (tid >> 2) + 64 * i;       // LDS row of B
            int64_t col, brow;
            if (EPI == EPI_SWIGLU) {
                const int half = (j >> 5) & 1;
                col = n0 + (j >> 6) * 32 + (j & 31);
                const int64_t zi = col / p.n_per, cc = col - zi * p.n_per;
                brow = zi * 2 * p.n_per + cc + half * p.n_per;
            } else {
                col = n0 + j;
                brow = col;
            }
            b_row[i] = (col < p.N ? brow : 0) + (int64_t)g * p.b_group_rows;
        }
        const int c16 = (tid & 3) * 16;

        floatx16 acc[kRB][2];
#pragma unroll
        for (int i = 0; i < kRB; i++)
#pragma unroll
            for (int j = 0; j < 2; j++)
#pragma unroll
                for (int v = 0; v < 16; v++) acc[i][j][v] = 0.0f;

        // K segments run one after the other, each with its own prologue, so
        // only the current segment's row addresses are live.
#pragma unroll 1
        for (int sidx = 0; sidx < p.nseg; sidx++) {
            const char* A = (const char*)p.seg[0].A;
            const char* B = (const char*)p.seg[0].B;
            int64_t lda = p.seg[0].lda, ldb = p.seg[0].ldb;
            int K = p.seg[0].K;
#pragma unroll
            for (int q = 1; q < kMaxSeg; q++) {
                if (sidx == q) {
                    A = (const char*)p.seg[q].A;
                    B = (const char*)p.seg[q].B;
                    lda = p.seg[q].lda;
                    ldb = p.seg[q].ldb;
                    K = p.seg[q].K;
                }
            }
            const int nk = K * kElem / kRowBytes;
            const char* a_ptr[kAChunks];
            const char* b_ptr[kBChunks];
#pragma unroll
            for (int i = 0; i < kAChunks; i++) a_ptr[i] = A + a_row[i] * lda * kElem + c16;
#pragma unroll
            for (int i = 0; i < kBChunks; i++) b_ptr[i] = B + b_row[i] * ldb * kElem + c16;

            uint4 ra[kAChunks], rb[kBChunks];
            auto load_regs = [&](int kt) {
                const int64_t koff = (int64_t)kt * kRowBytes;
#pragma unroll
                for (int i = 0; i < kAChunks; i++)
                    if (a_ok[i]) ra[i] = *(const uint4*)(a_ptr[i] + koff);
#pragma unroll
                for (int i = 0; i < kBChunks; i++) rb[i] = *(const uint4*)(b_ptr[i] + koff);
            };
            auto store_lds = [&](int buf) {
                char* As = lds[buf];
                char* Bs = lds[buf] + BM * kLdsRow;
#pragma unroll
                for (int i = 0; i < kAChunks; i++) {
                    const int r = (tid >> 2) + 64 * i;
                    if (a_ok[i]) *(uint4*)(As + r * kLdsRow + c16) = ra[i];
                }
#pragma unroll
                for (int i = 0; i < kBChunks; i++) {
                    const int j = (tid >> 2) + 64 * i;
                    *(uint4*)(Bs + j * kLdsRow + c16) = rb[i];
                }
            };

            __syncthreads();      // earlier readers of LDS are done
            load_regs(0);
            store_lds(0);
            __syncthreads();

#pragma unroll 1
            for (int kt = 0; kt < nk; kt++) {
                const int buf = kt & 1;
                if (kt + 1 < nk) load_regs(kt + 1);
                const char* As = lds[buf];
                const char* Bs = lds[buf] + BM * kLdsRow;
#pragma unroll
                for (int ks = 0; ks < kSteps; ks++) {
                    const int kbyte =
                        ks * Mfma<T>::kK * kElem + (lane >> 5) * Mfma<T>::kLaneK * kElem;
                    typename Mfma<T>::frag bfr[2];
#pragma unroll
                    for (int j = 0; j < 2; j++)
                        bfr[j] = Mfma<T>::lds_frag(Bs + (wn * 64 + j * 32 + (lane & 31)) * kLdsRow,
                                                   kbyte);
#pragma unroll
                    for (int i = 0; i < kRB; i++) {
                        if (i < n_act) {
                            typename Mfma<T>::frag afr = Mfma<T>::lds_frag(
                                As + ((wm + 2 * i) * 32 + (lane & 31)) * kLdsRow, kbyte);
                            acc[i][0] = Mfma<T>::mma(afr, bfr[0], acc[i][0]);
                            acc[i][1] = Mfma<T>::mma(afr, bfr[1], acc[i][1]);
                        }
                    }
                }
                if (kt + 1 < nk) store_lds(buf ^ 1);
                __syncthreads();
            }
        }

        OutT* C = (OutT*)p.C;
        // ---- epilogue, staged through LDS so that every global store is a
        // 16-byte chunk of a row.  All waves walk the same number of steps (the
        // barriers are block-wide); a wave with no active row block idles.
        float* stage = (float*)lds[0] + wave * (32 * kStageLd);
#pragma unroll
        for (int i = 0; i < kRB; i++) {
            const bool act = i < n_act;
            const int rbase = (wm + 2 * i) * 32;
            if (act) {
#pragma unroll
                for (int v = 0; v < 16; v++) {
                    const int r = acc_row(v, lane);
                    if (EPI == EPI_SWIGLU) {
                        stage[r * kStageLd + (lane & 31)] = silu_f(acc[i][0][v]) * acc[i][1][v];
                    } else {
                        stage[r * kStageLd + (lane & 31)] = acc[i][0][v];
                        stage[r * kStageLd + 32 + (lane & 31)] = acc[i][1][v];
                    }
                }
            }
            __syncthreads();
            if (act) {
                // the wave's 32 x W block (W = 32 hidden columns for SwiGLU, else
                // 64 columns) leaves in chunks of kVec output elements
                constexpr int W = (EPI == EPI_SWIGLU) ? 32 : 64;
                constexpr int kVec = 16 / sizeof(typename Elem<OutT>::store_t);
                constexpr int kChunksPerRow = W / kVec;
                const int64_t cbase = (EPI == EPI_SWIGLU) ? n0 + wn * 32 : n0 + wn * 64;
#pragma unroll
                for (int q = lane; q < 32 * kChunksPerRow; q += 64) {
                    const int r = q / kChunksPerRow;
                    const int cc = (q % kChunksPerRow) * kVec;
                    const int64_t grow = rbase + r;
                    const int64_t col = cbase + cc;
                    if (grow < rows_valid && col < p.N) {
                        float vals[kVec];
#pragma unroll
                        for (int e = 0; e < kVec; e++) vals[e] = stage[r * kStageLd + cc + e];
                        const int64_t off = (row0 + grow) * p.ldc + col;
                        if (EPI == EPI_ADD) {
                            const int64_t aoff = (row0 + grow) * p.ld_add + col;
#pragma unroll
                            for (int e = 0; e < kVec; e++)
                                vals[e] += Elem<OutT>::load((const OutT*)p.addend, aoff + e);
                        }
                        store_vec<OutT, kVec>(C, off, vals);
                    }
                }
            }
            __syncthreads();
        }
    }
}

// Exclusive prefix over groups of ceil(rows_g / BM): the row-tile index each
// group starts at.  One block, G <= 1024.
__global__ __launch_bounds__(1024) void tile_prefix_kernel(const int32_t* offsets, int G, int BM,
                                                           int32_t* tp) {
    __shared__ int red[16];
    const int tid = threadIdx.x;
    int v = 0;
    if (tid < G) v = (offsets[tid + 1] - offsets[tid] + BM - 1) / BM;
    int total;
    const int ex = block_exclusive_scan_1024(v, red, total);
    if (tid < G) tp[tid] = ex;
    if (tid == 0) tp[G] = total;
}

template <typename T, typename OutT, int EPI, int BM>
hipError_t launch_t(const GemmParams& p, int grid, hipStream_t s) {
    hipLaunchKernelGGL((gemm_kernel<T, OutT, EPI, BM>), dim3(grid), dim3(kThreads), 0, s, p);
    return hipGetLastError();
}

}  // namespace

int gemm_block_m() { return 256; }

int gemm_cols_per_tile(int epi) { return epi == EPI_SWIGLU ? kBN / 2 : kBN; }

hipError_t launch_tile_prefix(const int32_t* offsets, int G, int BM, int32_t* tp, hipStream_t s) {
    hipLaunchKernelGGL(tile_prefix_kernel, dim3(1), dim3(1024), 0, s, offsets, G, BM, tp);
    return hipGetLastError();
}

hipError_t launch_gemm(const GemmParams& p, moe_dtype in_dt, bool out_f32, int epi,
                       int64_t max_tiles, hipStream_t s) {
    int dev = 0, cus = 256;
    hipGetDevice(&dev);
    hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
    int64_t grid = (int64_t)cus * 2;
    if (max_tiles < grid) grid = max_tiles;
    grid = ((grid + kNumXcd - 1) / kNumXcd) * kNumXcd;
    if (grid < kNumXcd) grid = kNumXcd;
    constexpr int BM = 256;
    if (in_dt == MOE_BF16) {
        if (epi == EPI_STORE)
            return out_f32 ? launch_t<bf16_t, float, EPI_STORE, BM>(p, (int)grid, s)
                           : launch_t<bf16_t, bf16_t, EPI_STORE, BM>(p, (int)grid, s);
        if (epi == EPI_SWIGLU) return launch_t<bf16_t, bf16_t, EPI_SWIGLU, BM>(p, (int)grid, s);
        return launch_t<bf16_t, bf16_t, EPI_ADD, BM>(p, (int)grid, s);
    }
    if (epi == EPI_STORE) return launch_t<float, float, EPI_STORE, BM>(p, (int)grid, s);
    if (epi == EPI_SWIGLU) return launch_t<float, float, EPI_SWIGLU, BM>(p, (int)grid, s);
    return launch_t<float, float, EPI_ADD, BM>(p, (int)grid, s);
}

}  // namespace moe
