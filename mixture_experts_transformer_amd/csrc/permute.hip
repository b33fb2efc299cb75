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
//   pass 1  one wave per segment of kSeg assignments, in order: a lane's rank
//           among equal ids of its 64-lane step comes from ballots (a match-any
//           built bit by bit), plus the segment's running count in LDS; writes
//           per-assignment local ranks and per-segment counts.
//   pass 2  one workgroup: per expert, exclusive scan of segment counts (the
//           segment's base), the capacity cut, the exclusive scan of kept rows
//           (offsets), the drop count and optionally the GEMM's row-tile prefix.
//   pass 3  one thread per assignment: row = offsets[e] + base + local rank,
//           dropped if that rank reaches the capacity; writes slot_row/row_src.
//   pass 4  one wave per destination row: copies the source row (optional) and
//           clears row_src past the last kept row.
#include "common.h"
#include "kernels.h"

namespace moe {

namespace {

constexpr int kSeg = 4096;        // assignments per pass-1 wave
constexpr int kMaxE = 1024;

struct PermWs {
    int32_t* local_rank;          // [n]
    int32_t* seg_count;           // [nseg][E] (counts, then bases in place)
};

__global__ __launch_bounds__(256) void rank_kernel(const int32_t* ids, int64_t n, int E,
                                                   int32_t* local_rank, int32_t* seg_count) {
    __shared__ int32_t hist[4][kMaxE];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int64_t seg = (int64_t)blockIdx.x * 4 + wave;
    const int64_t nseg = (n + kSeg - 1) / kSeg;
    int32_t* H = hist[wave];
    for (int e = lane; e < E; e += 64) H[e] = 0;
    __builtin_amdgcn_wave_barrier();
    if (seg < nseg) {
        const int64_t a0 = seg * kSeg;
        const int64_t a1 = min(n, a0 + kSeg);
        const uint64_t lt_mask = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
        for (int64_t base = a0; base < a1; base += 64) {
            const int64_t a = base + lane;
            const bool in = a < a1;
            int id = in ? ids[a] : -1;
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
        for (int e = lane; e < E; e += 64) seg_count[seg * E + e] = H[e];
    }
}

__global__ __launch_bounds__(1024) void scan_kernel(int64_t nseg, int E, int64_t capacity,
                                                    int32_t* seg_count, int32_t* counts,
                                                    int32_t* offsets, int64_t* n_dropped,
                                                    int32_t* tile_prefix, int tile_bm) {
    __shared__ int red[16];
    __shared__ long long dred[16];
    const int tid = threadIdx.x;
    int kept = 0, tiles = 0;
    long long dropped = 0;
    if (tid < E) {
        int run = 0;
        for (int64_t s = 0; s < nseg; s++) {
            const int c = seg_count[s * E + tid];
            seg_count[s * E + tid] = run;
            run += c;
        }
        counts[tid] = run;
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

__global__ __launch_bounds__(256) void place_kernel(const int32_t* ids, int64_t n, int E,
                                                    int64_t capacity, const int32_t* local_rank,
                                                    const int32_t* seg_base, const int32_t* offsets,
                                                    int32_t* slot_row, int32_t* row_src) {
    const int64_t a = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (a >= n) return;
    const int lr = local_rank[a];
    if (lr < 0) {
        slot_row[a] = -1;
        return;
    }
    const int e = ids[a];
    const int rank = seg_base[(a / kSeg) * E + e] + lr;
    if (capacity >= 0 && rank >= capacity) {
        slot_row[a] = -1;
        return;
    }
    const int row = offsets[e] + rank;
    slot_row[a] = row;
    row_src[row] = (int32_t)a;
}

// One wave per destination row: copy the source row in 16-byte chunks, or mark
// the row empty when it lies past the last kept row.
__global__ __launch_bounds__(256) void copy_kernel(const int32_t* offsets, int E, int64_t R_phys,
                                                   int32_t* row_src, const char* src, char* dst,
                                                   int64_t row_bytes, int src_div) {
    const int lane = threadIdx.x & 63;
    const int64_t r = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    if (r >= R_phys) return;
    const int total = offsets[E];
    if (r >= total) {
        if (lane == 0) row_src[r] = -1;
        return;
    }
    if (!src) return;
    const int64_t a = row_src[r];
    const char* s = src + (a / src_div) * row_bytes;
    char* d = dst + r * row_bytes;
    for (int64_t c = (int64_t)lane * 16; c < row_bytes; c += 64 * 16)
        *(uint4*)(d + c) = *(const uint4*)(s + c);
}

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

}  // namespace

size_t permute_ws_bytes(int64_t n, int E) {
    const int64_t nseg = (n + kSeg - 1) / kSeg;
    return align256((size_t)(n > 0 ? n : 1) * 4) + align256((size_t)(nseg > 0 ? nseg : 1) * E * 4);
}

hipError_t launch_permute(const int32_t* ids, int64_t n, int E, int64_t capacity, const void* src,
                          int elem_bytes, int64_t width, int src_div, void* dst, int64_t R_phys,
                          int32_t* slot_row, int32_t* row_src, int32_t* counts, int32_t* offsets,
                          int64_t* n_dropped, int32_t* tile_prefix, int tile_bm, void* ws,
                          hipStream_t s) {
    const int64_t nseg = (n + kSeg - 1) / kSeg;
    int32_t* local_rank = (int32_t*)ws;
    int32_t* seg_count = (int32_t*)((char*)ws + align256((size_t)(n > 0 ? n : 1) * 4));
    if (nseg > 0) {
        hipLaunchKernelGGL(rank_kernel, dim3((unsigned)((nseg + 3) / 4)), dim3(256), 0, s, ids, n,
                           E, local_rank, seg_count);
    }
    hipLaunchKernelGGL(scan_kernel, dim3(1), dim3(1024), 0, s, nseg, E, capacity, seg_count,
                       counts, offsets, n_dropped, tile_prefix, tile_bm);
    if (n > 0) {
        hipLaunchKernelGGL(place_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, ids,
                           n, E, capacity, local_rank, seg_count, offsets, slot_row, row_src);
    }
    if (R_phys > 0) {
        hipLaunchKernelGGL(copy_kernel, dim3((unsigned)((R_phys + 3) / 4)), dim3(256), 0, s,
                           offsets, E, R_phys, row_src, (const char*)src, (char*)dst,
                           width * elem_bytes, src_div);
    }
    return hipGetLastError();
}

}  // namespace moe
