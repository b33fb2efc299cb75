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
//   pass 3  every workgroup first recomputes, into LDS, the capacity cut and the
//           exclusive scan of kept rows over all experts (E <= 1024 counts, a
//           few hundred cycles), so no workgroup waits on another and no pass
//           of its own is launched for it; workgroup 0 also writes the offsets,
//           the drop count and optionally the GEMM's row-tile prefix.  Then
//           row = offsets[e] + base + local rank, dropped if that rank reaches
//           the capacity; writes slot_row/row_src and marks the rows past the
//           last kept one empty.  With a source row shared by several
//           assignments, the same kernel copies each source row (one wave per
//           source row) to the rows of its kept assignments; otherwise one thread
//           per assignment places, and with one source row per assignment a
//           fourth pass gathers the rows in destination order.
#include <algorithm>

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

// Start of every placement workgroup (256 threads): kept = min(count, capacity)
// per expert and offs[x] = the exclusive prefix of kept (offs[E] the total), into
// the workgroup's LDS.  Workgroup 0 also writes offsets[0..E], n_dropped and,
// if tile_prefix is given, the exclusive prefix of each expert's row tiles of
// tile_bm rows (tile_prefix[E] the total).  Returns the kept total.
__device__ int expert_offsets(const int32_t* counts, int E, int64_t capacity, int32_t* offs,
                              int* red, int32_t* offsets, int64_t* n_dropped,
                              int32_t* tile_prefix, int tile_bm) {
    __shared__ long long dred[4];
    constexpr int kPer = kMaxE / 256;                 // experts per thread
    const int tid = threadIdx.x;
    int kept[kPer];
    int ksum = 0;
#pragma unroll
    for (int q = 0; q < kPer; q++) {
        const int x = tid * kPer + q;
        const int c = x < E ? counts[x] : 0;
        kept[q] = (capacity >= 0 && c > capacity) ? (int)capacity : c;
        ksum += kept[q];
    }
    int ktot;
    const int kex = block_exclusive_scan_1024(ksum, red, ktot);
    int run = kex;
#pragma unroll
    for (int q = 0; q < kPer; q++) {
        const int x = tid * kPer + q;
        if (x < E) offs[x] = run;
        run += kept[q];
    }
    if (tid == 0) offs[E] = ktot;
    if (blockIdx.x == 0) {                            // uniform over the workgroup
        run = kex;
        int tsum = 0;
        long long dsum = 0;
#pragma unroll
        for (int q = 0; q < kPer; q++) {
            const int x = tid * kPer + q;
            if (x < E) {
                offsets[x] = run;
                dsum += counts[x] - kept[q];
            }
            run += kept[q];
            if (tile_prefix) tsum += (kept[q] + tile_bm - 1) / tile_bm;
        }
        if (tid == 0) offsets[E] = ktot;
        if (tile_prefix) {
            int ttot;
            int tex = block_exclusive_scan_1024(tsum, red, ttot);
#pragma unroll
            for (int q = 0; q < kPer; q++) {
                const int x = tid * kPer + q;
                if (x < E) tile_prefix[x] = tex;
                tex += (kept[q] + tile_bm - 1) / tile_bm;
            }
            if (tid == 0) tile_prefix[E] = ttot;
        }
#pragma unroll
        for (int off = 32; off >= 1; off >>= 1) dsum += __shfl_xor(dsum, off, 64);
        if ((tid & 63) == 0) dred[tid >> 6] = dsum;
        __syncthreads();
        if (tid == 0) *n_dropped = dred[0] + dred[1] + dred[2] + dred[3];
    }
    __syncthreads();
    return ktot;
}

// One thread per index i < max(n, R_phys): places assignment i (if i < n) and
// marks row i empty if it lies past the last kept row (if i < R_phys).
__global__ __launch_bounds__(256) void place_kernel(const int32_t* ids, int64_t n, int64_t seg_n,
                                                    int E, int64_t capacity, const int32_t* counts,
                                                    const int32_t* local_rank,
                                                    const int32_t* seg_base, int32_t* offsets,
                                                    int64_t* n_dropped, int32_t* tile_prefix,
                                                    int tile_bm, int64_t R_phys, int32_t* slot_row,
                                                    int32_t* row_src) {
    __shared__ int32_t offs[kMaxE + 1];
    __shared__ int red[16];
    const int kept_total = expert_offsets(counts, E, capacity, offs, red, offsets, n_dropped,
                                          tile_prefix, tile_bm);
    const int64_t a = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (a < R_phys && a >= kept_total) row_src[a] = -1;
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
    const int row = offs[e] + rank;
    slot_row[a] = row;
    row_src[row] = (int32_t)a;
}

constexpr int kCopyChunks = 8;   // 16-byte loads in flight per lane (E4M3 copies)

// Placement fused with the row copy: one wave per source row s, whose
// assignments are a = s * src_div + j (j < src_div).  Lane j places assignment
// a as place_kernel does (slot_row, row_src); the wave then reads the row once
// (C 16-byte chunks per lane per pass, sized to the row width so that no lane
// re-reads a chunk) and stores it to the row of each kept assignment.  A source
// row none of whose assignments was kept is not read.  The rows of row_src past
// the kept total are cleared by all waves in a grid-stride pass.  Loads and
// stores are non-temporal: every byte is read once and written once.
template <int C>
__global__ __launch_bounds__(256) void place_copy_kernel(
    const int32_t* ids, int64_t n, int64_t seg_n, int E, int64_t capacity, const int32_t* counts,
    const int32_t* local_rank, const int32_t* seg_base, int32_t* offsets, int64_t* n_dropped,
    int32_t* tile_prefix, int tile_bm, int64_t R_phys, int32_t* slot_row, int32_t* row_src,
    int64_t n_src, const char* src, char* dst, int64_t row_bytes, int src_div) {
    __shared__ int32_t offs[kMaxE + 1];
    __shared__ int red[16];
    const int64_t kept_total = expert_offsets(counts, E, capacity, offs, red, offsets, n_dropped,
                                              tile_prefix, tile_bm);
    const int lane = threadIdx.x & 63;
    const int64_t wave = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    const int64_t nwaves = (int64_t)gridDim.x * 4;
    for (int64_t r = kept_total + wave * 64 + lane; r < R_phys; r += nwaves * 64) row_src[r] = -1;
    if (wave >= n_src) return;
    const int64_t a0 = wave * src_div;
    const int64_t na = min((int64_t)src_div, n - a0);
    const char* sp = src + wave * row_bytes;
    const int64_t nchunk = row_bytes / 16;
    for (int64_t jb = 0; jb < na; jb += 64) {
        int32_t my = -1;
        if (jb + lane < na) {
            const int64_t a = a0 + jb + lane;
            const int lr = local_rank[a];
            if (lr >= 0) {
                const int e = ids[a];
                const int rank = seg_base[(a / seg_n) * E + e] + lr;
                if (capacity < 0 || rank < capacity) my = offs[e] + rank;
            }
            slot_row[a] = my;
            if (my >= 0) row_src[my] = (int32_t)a;
        }
        const uint64_t kept = __ballot(my >= 0);
        if (!kept) continue;
        for (int64_t c0 = 0; c0 < nchunk; c0 += 64 * C) {
            u32x4 v[C];
#pragma unroll
            for (int q = 0; q < C; q++) {
                const int64_t c = min(c0 + lane + 64 * q, nchunk - 1);
                v[q] = __builtin_nontemporal_load((const u32x4*)(sp + c * 16));
            }
            for (uint64_t m = kept; m; m &= m - 1) {
                const int j = __builtin_ctzll(m);
                const int64_t r = __builtin_amdgcn_readlane(my, j);
                char* d = dst + r * row_bytes;
#pragma unroll
                for (int q = 0; q < C; q++) {
                    const int64_t c = c0 + lane + 64 * q;
                    if (c < nchunk) __builtin_nontemporal_store(v[q], (u32x4*)(d + c * 16));
                }
            }
        }
    }
}

// Row copy when each source row feeds one assignment (src_div == 1), after the
// placement: one wave per kept destination row, in row order, gathers its source
// row through row_src, so the stores run through the destination in sequence.
// C 16-byte chunks per lane per pass; loads and stores are non-temporal.
template <int C>
__global__ __launch_bounds__(256) void gather_copy_kernel(const int32_t* offsets, int E,
                                                          int64_t R_phys, const int32_t* row_src,
                                                          const char* src, char* dst,
                                                          int64_t row_bytes) {
    const int lane = threadIdx.x & 63;
    const int64_t r = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    if (r >= R_phys || r >= offsets[E]) return;
    const char* sp = src + (int64_t)row_src[r] * row_bytes;
    char* d = dst + r * row_bytes;
    const int64_t nchunk = row_bytes / 16;
    for (int64_t c0 = 0; c0 < nchunk; c0 += 64 * C) {
        u32x4 v[C];
#pragma unroll
        for (int q = 0; q < C; q++) {
            const int64_t c = min(c0 + lane + 64 * q, nchunk - 1);
            v[q] = __builtin_nontemporal_load((const u32x4*)(sp + c * 16));
        }
#pragma unroll
        for (int q = 0; q < C; q++) {
            const int64_t c = c0 + lane + 64 * q;
            if (c < nchunk) __builtin_nontemporal_store(v[q], (u32x4*)(d + c * 16));
        }
    }
}

// 16-byte chunks per lane per pass for rows of nchunk chunks: the choice among
// 4, 6 and 8 that leaves the fewest idle lane slots (the larger on a tie).
int copy_chunks_for(int64_t nchunk) {
    int best = 8;
    int64_t waste = -1;
    for (int c : {8, 6, 4}) {
        const int64_t per = 64 * (int64_t)c;
        const int64_t w = (nchunk + per - 1) / per * per - nchunk;
        if (waste < 0 || w < waste) {
            waste = w;
            best = c;
        }
    }
    return best;
}

// The row copies writing E4M3 codes of the rows divided by the scale (the fp8
// permutation leg: the rows leave the grouping step already quantised, as
// moe_quantize_e4m3 would quantise them), after the placement kernel: with one
// source row per assignment (src_div == 1) one wave per kept destination row
// gathers its source row through row_src; otherwise one wave per source row
// stores it to each kept assignment's row, found in slot_row.  A lane converts
// 16 elements (32 or 64 bytes read, 16 bytes written) and keeps kCopyChunks
// 16-byte loads in flight.
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
    // the placement always runs, at least one workgroup: workgroup 0 writes the
    // offsets, the drop count and the tile prefix
    const int64_t row_bytes = width * elem_bytes;
    if (src && R_phys > 0 && !out_e4m3 && src_div > 1) {
        // placement and the row copy in one kernel, one wave per source row
        const int64_t n_src = (n + src_div - 1) / src_div;
        const int64_t waves = std::max<int64_t>(n_src, (R_phys + 63) / 64);
        const dim3 g((unsigned)std::max<int64_t>(1, (waves + 3) / 4));
#define MOE_PLACE_COPY(C)                                                                       \
    hipLaunchKernelGGL(place_copy_kernel<C>, g, dim3(256), 0, s, ids, n, seg_n, E, capacity,    \
                       counts, local_rank, seg_count, offsets, n_dropped, tile_prefix, tile_bm, \
                       R_phys, slot_row, row_src, n_src, (const char*)src, (char*)dst,          \
                       row_bytes, src_div)
        switch (copy_chunks_for(row_bytes / 16)) {
            case 4: MOE_PLACE_COPY(4); break;
            case 6: MOE_PLACE_COPY(6); break;
            default: MOE_PLACE_COPY(8);
        }
#undef MOE_PLACE_COPY
        return hipGetLastError();
    }
    const int64_t m = std::max<int64_t>(1, n > R_phys ? n : R_phys);
    hipLaunchKernelGGL(place_kernel, dim3((unsigned)((m + 255) / 256)), dim3(256), 0, s, ids, n,
                       seg_n, E, capacity, counts, local_rank, seg_count, offsets, n_dropped,
                       tile_prefix, tile_bm, R_phys, slot_row, row_src);
    if (src && R_phys > 0 && !out_e4m3) {
        // one source row per assignment: gather in destination order
        const dim3 g((unsigned)((R_phys + 3) / 4));
#define MOE_GATHER_COPY(C)                                                                       \
    hipLaunchKernelGGL(gather_copy_kernel<C>, g, dim3(256), 0, s, offsets, E, R_phys, row_src,   \
                       (const char*)src, (char*)dst, row_bytes)
        switch (copy_chunks_for(row_bytes / 16)) {
            case 4: MOE_GATHER_COPY(4); break;
            case 6: MOE_GATHER_COPY(6); break;
            default: MOE_GATHER_COPY(8);
        }
#undef MOE_GATHER_COPY
        return hipGetLastError();
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
