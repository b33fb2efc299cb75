// Grouping of assignments by expert: histogram, scan, stable rank, scatter.
//
// The pages' grouped GEMM reads each expert's row range from a cu_seqlens
// array, and their hang came from a consumer reading those boundaries before
// the producer's writes were visible (Marin 535B-A23B article, section "21% to
// 27% MFU without stopping the run").  Here the boundaries are produced by
// kernels on the caller's stream and consumed only by kernels enqueued after
// them on that stream, so every read follows the producer's completion.
//
// Determinism: ranks come from the arrival order of assignments, never from
// the order atomics happen to land, so every integer output is a pure function
// of the ids (required bit-exact).
//   pass 1  one wave per segment of 256 or more assignments (at most 4,096
//           segments): a lane's rank among equal
//           ids of its 64-lane step comes from ballots (a match-any built bit by
//           bit), plus the segment's running count in LDS; writes per-assignment
//           local ranks and per-segment counts.
//   pass 2  one workgroup per expert: exclusive scan of that expert's segment
//           counts (each segment's base) and the expert's total.
//   pass 3  one workgroup: the capacity cut, the exclusive scan of kept rows
//           (offsets), the drop count and optionally the GEMM's row-tile prefix.
//   pass 4  one thread per assignment: row = offsets[e] + base + local rank,
//           dropped if that rank reaches the capacity; writes slot_row/row_src,
//           and marks the rows past the last kept one empty.
//   pass 5  (only with a source) one wave per destination row copies the row.
#include "common.h"
#include "e4m3.h"
#include "kernels.h"

namespace moe {

namespace {

constexpr int kStepIds = 256;     // ids a pass-1 wave loads at a time
constexpr int kMaxSeg = 4096;     // segments at most (bounds the workspace)
constexpr int kMaxE = 1024;

// Assignments per pass-1 segment: 256, or more so that there are at most
// kMaxSeg segments (a multiple of 256).
inline int64_t seg_len(int64_t n) {
    const int64_t per = (n + kMaxSeg - 1) / kMaxSeg;
    return per <= kStepIds ? kStepIds : (per + kStepIds - 1) / kStepIds * kStepIds;
}

__global__ __launch_bounds__(256) void rank_kernel(const int32_t* ids, int64_t n, int64_t seg_n,
                                                   int E, int32_t* local_rank, int32_t* seg_count) {
    __shared__ int32_t hist[4][kMaxE];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int64_t seg = (int64_t)blockIdx.x * 4 + wave;
    const int64_t nseg = (n + seg_n - 1) / seg_n;
    int32_t* H = hist[wave];
    for (int e = lane; e < E; e += 64) H[e] = 0;
    __builtin_amdgcn_wave_barrier();
    if (seg < nseg) {
        const int64_t a0 = seg * seg_n;
        const int64_t a1 = min(n, a0 + seg_n);
        const uint64_t lt_mask = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
        for (int64_t b0 = a0; b0 < a1; b0 += kStepIds) {
        // the next kStepIds ids, loaded up front
        int idv[kStepIds / 64];
#pragma unroll
        for (int q = 0; q < kStepIds / 64; q++) {
            const int64_t a = b0 + 64 * q + lane;
            idv[q] = a < a1 ? ids[a] : -1;
        }
#pragma unroll
        for (int q = 0; q < kStepIds / 64; q++) {
            const int64_t a = b0 + 64 * q + lane;
            const bool in = a < a1;
            const int id = idv[q];
            const bool valid = in && id >= 0 && id < E;
            // lanes with the same (valid, id)
            uint64_t match = __ballot(valid);
            if (!valid) match = ~match;
#pragma unroll
            for (int b = 0; b < 10; b++) {
                const bool bit = (id >> b) & 1;
                const uint64_t bal = __ballot(bit);
                match &= bit ? bal : ~bal;
            }
            const int before = __popcll(match & lt_mask);
            const int cnt = __popcll(match);
            int prev = 0;
            if (valid) prev = H[id];
            __builtin_amdgcn_wave_barrier();
            // the last lane of each id group advances that id's running count
            const bool last = valid && before == cnt - 1;
            if (last) H[id] = prev + cnt;
            __builtin_amdgcn_wave_barrier();
            if (in) local_rank[a] = valid ? prev + before : -1;
        }
        }
        for (int e = lane; e < E; e += 64) seg_count[seg * E + e] = H[e];
    }
}

// One workgroup per expert e: seg_count[s][e] becomes the number of e's
// assignments in segments before s; counts[e] the total.
__global__ __launch_bounds__(256) void colscan_kernel(int64_t nseg, int E, int32_t* seg_count,
                                                      int32_t* counts) {
    __shared__ int red[16];
    const int e = blockIdx.x, tid = threadIdx.x;
    const int64_t per = (nseg + 255) / 256;           // consecutive segments per thread
    const int64_t s0 = tid * per;
    int sum = 0;
    for (int64_t s = s0; s < min(nseg, s0 + per); s++) sum += seg_count[s * E + e];
    int total;
    int run = block_exclusive_scan_1024(sum, red, total);
    for (int64_t s = s0; s < min(nseg, s0 + per); s++) {
        const int c = seg_count[s * E + e];
        seg_count[s * E + e] = run;
        run += c;
    }
    if (tid == 0) counts[e] = total;
}

__global__ __launch_bounds__(1024) void scan_kernel(int E, int64_t capacity, const int32_t* counts,
                                                    int32_t* offsets, int64_t* n_dropped,
                                                    int32_t* tile_prefix, int tile_bm) {
    __shared__ int red[16];
    __shared__ long long dred[16];
    const int tid = threadIdx.x;
    int kept = 0, tiles = 0;
    long long dropped = 0;
    if (tid < E) {
        const int run = counts[tid];
        kept = (capacity >= 0 && run > capacity) ? (int)capacity : run;
        dropped = run - kept;
        if (tile_prefix) tiles = (kept + tile_bm - 1) / tile_bm;
    }
    int total;
    const int ex = block_exclusive_scan_1024(kept, red, total);
    if (tid < E) offsets[tid] = ex;
    if (tid == 0) offsets[E] = total;
    if (tile_prefix) {
        int ttot;
        const int tex = block_exclusive_scan_1024(tiles, red, ttot);
        if (tid < E) tile_prefix[tid] = tex;
        if (tid == 0) tile_prefix[E] = ttot;
    }
    // drop count: wave sums, then one wave over the partials
    long long d = dropped;
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) d += __shfl_xor(d, off, 64);
    if ((tid & 63) == 0) dred[tid >> 6] = d;
    __syncthreads();
    if (tid == 0) {
        long long s = 0;
        for (int i = 0; i < (int)(blockDim.x >> 6); i++) s += dred[i];
        *n_dropped = s;
    }
}

// One thread per index i < max(n, R_phys): places assignment i (if i < n) and
// marks row i empty if it lies past the last kept row (if i < R_phys).
__global__ __launch_bounds__(256) void place_kernel(const int32_t* ids, int64_t n, int64_t seg_n,
                                                    int E, int64_t capacity,
                                                    const int32_t* local_rank,
                                                    const int32_t* seg_base, const int32_t* offsets,
                                                    int64_t R_phys, int32_t* slot_row,
                                                    int32_t* row_src) {
    const int64_t a = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (a < R_phys && a >= offsets[E]) row_src[a] = -1;
    if (a >= n) return;
    const int lr = local_rank[a];
    if (lr < 0) {
        slot_row[a] = -1;
        return;
    }
    const int e = ids[a];
    const int rank = seg_base[(a / seg_n) * E + e] + lr;
    if (capacity >= 0 && rank >= capacity) {
        slot_row[a] = -1;
        return;
    }
    const int row = offsets[e] + rank;
    slot_row[a] = row;
    row_src[row] = (int32_t)a;
}

// Row copy when each source row feeds one assignment (src_div == 1): one wave
// per kept destination row.  Each pass issues the loads of 8 16-byte chunks per
// lane before any store, so a wave keeps 8 KB in flight; lanes past the row's
// end re-read its last chunk and store nothing.  Every row is read once and
// written once, so loads and stores are both non-temporal.
constexpr int kCopyChunks = 8;

__global__ __launch_bounds__(256) void copy_kernel(const int32_t* offsets, int E, int64_t R_phys,
                                                   const int32_t* row_src, const char* src,
                                                   char* dst, int64_t row_bytes) {
    const int lane = threadIdx.x & 63;
    const int64_t r = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    if (r >= R_phys || r >= offsets[E]) return;
    const char* s = src + (int64_t)row_src[r] * row_bytes;
    char* d = dst + r * row_bytes;
    const int64_t nchunk = row_bytes / 16;
    for (int64_t c0 = 0; c0 < nchunk; c0 += 64 * kCopyChunks) {
        u32x4 v[kCopyChunks];
#pragma unroll
        for (int q = 0; q < kCopyChunks; q++) {
            const int64_t c = min(c0 + lane + 64 * q, nchunk - 1);
            v[q] = __builtin_nontemporal_load((const u32x4*)(s + c * 16));
        }
#pragma unroll
        for (int q = 0; q < kCopyChunks; q++) {
            const int64_t c = c0 + lane + 64 * q;
            if (c < nchunk) __builtin_nontemporal_store(v[q], (u32x4*)(d + c * 16));
        }
    }
}

// One wave per source row, for source rows shared by several assignments
// (src_div > 1): the row is loaded once and stored to the destination row of
// each of its kept assignments, so each source byte crosses HBM once rather
// than once per assignment.  Lane j of a block of 64 assignments holds the
// row of assignment a0 + jb + j; a source row none of whose assignments was
// kept is not read.  Each kept row has exactly one assignment, so this writes
// the same rows as the gather above.
__global__ __launch_bounds__(256) void scatter_copy_kernel(const int32_t* slot_row, int64_t n,
                                                           int64_t n_src, const char* src,
                                                           char* dst, int64_t row_bytes,
                                                           int src_div) {
    const int lane = threadIdx.x & 63;
    const int64_t s = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    if (s >= n_src) return;
    const int64_t a0 = s * src_div;
    const int64_t na = min((int64_t)src_div, n - a0);
    const char* sp = src + s * row_bytes;
    const int64_t nchunk = row_bytes / 16;
    for (int64_t jb = 0; jb < na; jb += 64) {
        const int32_t my = jb + lane < na ? slot_row[a0 + jb + lane] : -1;
        const uint64_t kept = __ballot(my >= 0);
        if (!kept) continue;
        for (int64_t c0 = 0; c0 < nchunk; c0 += 64 * kCopyChunks) {
            u32x4 v[kCopyChunks];
#pragma unroll
            for (int q = 0; q < kCopyChunks; q++) {
                const int64_t c = min(c0 + lane + 64 * q, nchunk - 1);
                v[q] = __builtin_nontemporal_load((const u32x4*)(sp + c * 16));
            }
            for (uint64_t m = kept; m; m &= m - 1) {
                const int j = __builtin_ctzll(m);
                const int64_t r = __builtin_amdgcn_readlane(my, j);
                char* d = dst + r * row_bytes;
#pragma unroll
                for (int q = 0; q < kCopyChunks; q++) {
                    const int64_t c = c0 + lane + 64 * q;
                    if (c < nchunk) __builtin_nontemporal_store(v[q], (u32x4*)(d + c * 16));
                }
            }
        }
    }
}

// The same two copies writing E4M3 codes of the rows divided by the scale (the
// fp8 permutation leg: the rows leave the grouping step already quantised, as
// moe_quantize_e4m3 would quantise them).  A lane converts 16 elements (32 or 64
// bytes read, 16 bytes written) and keeps kCopyChunks 16-byte loads in flight.
// amax: max |x| over the source rows read, i.e. those with a kept assignment.
// Waves stride over the rows on a grid of at most kE4m3Blocks blocks, so the
// amax takes one atomic per block, not per four rows.
constexpr int kE4m3Blocks = 2048;
template <typename T>
__global__ __launch_bounds__(256) void copy_e4m3_kernel(const int32_t* offsets, int E,
                                                        int64_t R_phys, const int32_t* row_src,
                                                        const T* src, uint8_t* dst, int64_t width,
                                                        const float* scale, uint32_t* amax_bits) {
    constexpr int kIn = (int)sizeof(T);               // 16-byte loads per 16 codes
    constexpr int kOut = kCopyChunks / kIn;
    const float inv = inv_of(scale);
    const int lane = threadIdx.x & 63;
    const int64_t rows = min(R_phys, (int64_t)offsets[E]);
    float m = 0.0f;
    for (int64_t r = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6); r < rows;
         r += (int64_t)gridDim.x * 4) {
        const T* sp = src + (int64_t)row_src[r] * width;
        uint8_t* d = dst + r * width;
        const int64_t nout = width / 16;
        for (int64_t c0 = 0; c0 < nout; c0 += 64 * kOut) {
            u32x4 v[kOut][kIn];
#pragma unroll
            for (int q = 0; q < kOut; q++) {
                const int64_t c = min(c0 + lane + 64 * q, nout - 1);
#pragma unroll
                for (int j = 0; j < kIn; j++)
                    v[q][j] = __builtin_nontemporal_load((const u32x4*)(sp + c * 16) + j);
            }
#pragma unroll
            for (int q = 0; q < kOut; q++) {
                const int64_t c = c0 + lane + 64 * q;
                if (c >= nout) continue;
                float p[16];
#pragma unroll
                for (int e = 0; e < 16; e++) {
                    const float f = group_elem<T>(v[q], e);
                    m = fmaxf(m, fabsf(f));
                    p[e] = f * inv;
                }
                u32x4 out;
#pragma unroll
                for (int j = 0; j < 4; j++)
                    out[j] = e4m3_pack4(p[4 * j], p[4 * j + 1], p[4 * j + 2], p[4 * j + 3]);
                __builtin_nontemporal_store(out, (u32x4*)(d + c * 16));
            }
        }
    }
    if (amax_bits) block_amax(m, amax_bits);
}

template <typename T>
__global__ __launch_bounds__(256) void scatter_copy_e4m3_kernel(
    const int32_t* slot_row, int64_t n, int64_t n_src, const T* src, uint8_t* dst, int64_t width,
    int src_div, const float* scale, uint32_t* amax_bits) {
    constexpr int kIn = (int)sizeof(T);
    constexpr int kOut = kCopyChunks / kIn;
    const float inv = inv_of(scale);
    const int lane = threadIdx.x & 63;
    float m = 0.0f;
    for (int64_t s = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6); s < n_src;
         s += (int64_t)gridDim.x * 4) {
        const int64_t a0 = s * src_div;
        const int64_t na = min((int64_t)src_div, n - a0);
        const T* sp = src + s * width;
        const int64_t nout = width / 16;
        for (int64_t jb = 0; jb < na; jb += 64) {
            const int32_t my = jb + lane < na ? slot_row[a0 + jb + lane] : -1;
            const uint64_t kept = __ballot(my >= 0);
            if (!kept) continue;
            for (int64_t c0 = 0; c0 < nout; c0 += 64 * kOut) {
                u32x4 v[kOut][kIn];
#pragma unroll
                for (int q = 0; q < kOut; q++) {
                    const int64_t c = min(c0 + lane + 64 * q, nout - 1);
#pragma unroll
                    for (int j = 0; j < kIn; j++)
                        v[q][j] = __builtin_nontemporal_load((const u32x4*)(sp + c * 16) + j);
                }
                u32x4 out[kOut];
#pragma unroll
                for (int q = 0; q < kOut; q++) {
                    float p[16];
                    const bool valid = c0 + lane + 64 * q < nout;
#pragma unroll
                    for (int e = 0; e < 16; e++) {
                        const float f = group_elem<T>(v[q], e);
                        if (valid) m = fmaxf(m, fabsf(f));
                        p[e] = f * inv;
                    }
#pragma unroll
                    for (int j = 0; j < 4; j++)
                        out[q][j] = e4m3_pack4(p[4 * j], p[4 * j + 1], p[4 * j + 2], p[4 * j + 3]);
                }
                for (uint64_t mk = kept; mk; mk &= mk - 1) {
                    const int j = __builtin_ctzll(mk);
                    const int64_t r = __builtin_amdgcn_readlane(my, j);
                    uint8_t* d = dst + r * width;
#pragma unroll
                    for (int q = 0; q < kOut; q++) {
                        const int64_t c = c0 + lane + 64 * q;
                        if (c < nout) __builtin_nontemporal_store(out[q], (u32x4*)(d + c * 16));
                    }
                }
            }
        }
    }
    if (amax_bits) block_amax(m, amax_bits);
}

// Expert-parallel dispatch, sender side: the destination peer of each assignment
// (experts are dealt to peers in contiguous blocks of epp) ...
__global__ __launch_bounds__(256) void peer_of_kernel(const int32_t* ids, int64_t n, int epp,
                                                      int32_t* peer) {
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i < n) peer[i] = ids[i] < 0 ? -1 : ids[i] / epp;
}

// ... and, once the rows are grouped by peer, the local expert id each sent row
// carries with it (-1 for the rows past the kept total).
__global__ __launch_bounds__(256) void payload_ids_kernel(const int32_t* ids,
                                                          const int32_t* row_src,
                                                          const int32_t* offsets, int P,
                                                          int64_t R_phys, int epp,
                                                          int32_t* payload) {
    const int64_t r = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (r < R_phys) payload[r] = r < offsets[P] ? ids[row_src[r]] % epp : -1;
}

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

}  // namespace

size_t permute_ws_bytes(int64_t n, int E) {
    const int64_t nseg = (n + seg_len(n) - 1) / seg_len(n);
    return align256((size_t)(n > 0 ? n : 1) * 4) + align256((size_t)(nseg > 0 ? nseg : 1) * E * 4);
}

hipError_t launch_permute(const int32_t* ids, int64_t n, int E, int64_t capacity, const void* src,
                          int elem_bytes, int64_t width, int src_div, void* dst, int64_t R_phys,
                          int32_t* slot_row, int32_t* row_src, int32_t* counts, int32_t* offsets,
                          int64_t* n_dropped, int32_t* tile_prefix, int tile_bm, void* ws,
                          hipStream_t s, bool out_e4m3, const float* scale, float* amax) {
    const int64_t seg_n = seg_len(n);
    const int64_t nseg = (n + seg_n - 1) / seg_n;
    int32_t* local_rank = (int32_t*)ws;
    int32_t* seg_count = (int32_t*)((char*)ws + align256((size_t)(n > 0 ? n : 1) * 4));
    if (nseg > 0)
        hipLaunchKernelGGL(rank_kernel, dim3((unsigned)((nseg + 3) / 4)), dim3(256), 0, s, ids, n,
                           seg_n, E, local_rank, seg_count);
    // with no segments this writes zero counts
    hipLaunchKernelGGL(colscan_kernel, dim3((unsigned)E), dim3(256), 0, s, nseg, E, seg_count,
                       counts);
    hipLaunchKernelGGL(scan_kernel, dim3(1), dim3(1024), 0, s, E, capacity, counts, offsets,
                       n_dropped, tile_prefix, tile_bm);
    const int64_t m = n > R_phys ? n : R_phys;
    if (m > 0) {
        hipLaunchKernelGGL(place_kernel, dim3((unsigned)((m + 255) / 256)), dim3(256), 0, s, ids,
                           n, seg_n, E, capacity, local_rank, seg_count, offsets, R_phys, slot_row,
                           row_src);
    }
    if (out_e4m3) {
        // dst holds E4M3 codes of width bytes a row; elem_bytes is the source's
        uint32_t* ab = (uint32_t*)amax;
        if (ab) {
            hipError_t e = launch_zero_u32(ab, s);
            if (e != hipSuccess) return e;
        }
        if (!src || R_phys <= 0 || n <= 0) return hipGetLastError();
        const bool bf = elem_bytes == 2;
        if (src_div == 1) {
            const dim3 g((unsigned)std::min<int64_t>((R_phys + 3) / 4, kE4m3Blocks));
            if (bf)
                hipLaunchKernelGGL(copy_e4m3_kernel<bf16_t>, g, dim3(256), 0, s, offsets, E,
                                   R_phys, row_src, (const bf16_t*)src, (uint8_t*)dst, width,
                                   scale, ab);
            else
                hipLaunchKernelGGL(copy_e4m3_kernel<float>, g, dim3(256), 0, s, offsets, E,
                                   R_phys, row_src, (const float*)src, (uint8_t*)dst, width,
                                   scale, ab);
        } else {
            const int64_t n_src = (n + src_div - 1) / src_div;
            const dim3 g((unsigned)std::min<int64_t>((n_src + 3) / 4, kE4m3Blocks));
            if (bf)
                hipLaunchKernelGGL(scatter_copy_e4m3_kernel<bf16_t>, g, dim3(256), 0, s, slot_row,
                                   n, n_src, (const bf16_t*)src, (uint8_t*)dst, width, src_div,
                                   scale, ab);
            else
                hipLaunchKernelGGL(scatter_copy_e4m3_kernel<float>, g, dim3(256), 0, s, slot_row,
                                   n, n_src, (const float*)src, (uint8_t*)dst, width, src_div,
                                   scale, ab);
        }
        return hipGetLastError();
    }
    if (src && R_phys > 0) {
        if (src_div == 1) {
            hipLaunchKernelGGL(copy_kernel, dim3((unsigned)((R_phys + 3) / 4)), dim3(256),
                               0, s, offsets, E, R_phys, row_src, (const char*)src, (char*)dst,
                               width * elem_bytes);
        } else if (n > 0) {
            const int64_t n_src = (n + src_div - 1) / src_div;
            hipLaunchKernelGGL(scatter_copy_kernel, dim3((unsigned)((n_src + 3) / 4)), dim3(256),
                               0, s, slot_row, n, n_src, (const char*)src, (char*)dst,
                               width * elem_bytes, src_div);
        }
    }
    return hipGetLastError();
}

hipError_t launch_peer_of(const int32_t* ids, int64_t n, int epp, int32_t* peer, hipStream_t s) {
    if (n > 0)
        hipLaunchKernelGGL(peer_of_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, ids,
                           n, epp, peer);
    return hipGetLastError();
}

hipError_t launch_payload_ids(const int32_t* ids, const int32_t* row_src, const int32_t* offsets,
                              int P, int64_t R_phys, int epp, int32_t* payload, hipStream_t s) {
    if (R_phys > 0)
        hipLaunchKernelGGL(payload_ids_kernel, dim3((unsigned)((R_phys + 255) / 256)), dim3(256), 0,
                           s, ids, row_src, offsets, P, R_phys, epp, payload);
    return hipGetLastError();
}

}  // namespace moe
