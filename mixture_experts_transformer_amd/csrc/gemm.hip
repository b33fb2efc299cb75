// Grouped / dense MFMA GEMM for gfx950, with the epilogues the layer needs.
//
//   C[r, n] = epi( sum_s sum_k A_s[arow(r), k] * B_s[brow(g, n), k] )
//
// Both operands are contiguous along k ("[out, in]" weights).  Rows may be
// grouped by expert (the pages' ragged_dot with group sizes / cu_seqlens:
// Marin: Week of April 26th summary; Marin 535B-A23B article, section "21% to
// 27% MFU without stopping the run"): rows [offsets[g], offsets[g+1]) use expert
// g's weights.  Only active rows are computed: a 32-row MFMA block that lies
// wholly past its group's end issues no MFMAs (the "mask-free" ragged expert MLP
// of the same article section).  A rows may be gathered through a row map (the
// layer reads its routed rows straight from the token matrix instead of a
// permuted copy).
//
// Tiling (one workgroup per CU): 512 threads = 8 waves (two per SIMD) as 2 x 4
// over a 256 x 256 output tile.  Operands go straight from global memory into
// LDS with global_load_lds_dwordx4 (no staging registers, no LDS write
// instructions).  A K step is 128 bytes -- one whole cache line -- of each of the
// 256 A rows and 256 B rows (64 KB): with 64-byte row pieces every DMA
// instruction would touch half of each of 16 lines and the L2-to-LDS rate
// halves.  One operand's steps rotate through three LDS slots and run two steps
// ahead, the other's alternate in two: all 160 KB of LDS.  The host picks the
// operand per launch -- the one whose slices come from farthest away: B (the
// weights) where a grouped GEMM streams each expert's weights once, A otherwise.
// The fragments of a K step are read in four quarters, each while the MFMAs of
// the previous quarter run, so the barrier at the end of a step finds its slots
// fully read and they are refilled at once.  Within a row the eight 16-byte
// chunks are XOR-swizzled by a function of the row, chosen so that the fragment
// reads of 8 (or 16) consecutive rows hit distinct banks; the swizzle is applied
// on the global side, since each DMA instruction fills 1 KB of LDS contiguously.
// Each DMA source is a wave-uniform base plus a 32-bit per-lane offset.  Waits
// are explicit (vmcnt) followed by a bare s_barrier.  The grouped GEMMs' outputs
// can be stored non-temporally (they are re-read from HBM by the next kernel).
//
// Each wave owns up to 4 x 2 blocks of v_mfma_f32_32x32x16_bf16 (a 128 x 64
// sub-tile, 128 accumulators).  The wave's 32-row blocks are interleaved (wm,
// wm+2, ...) so both row waves stay busy on a partial tile, and the tile body is
// specialised on how many of them are active, so each case is straight-line
// MFMA code.  The MFMAs take the B fragment as their first operand, so each
// lane ends up holding one output row and four consecutive columns per group
// of accumulator registers.  For the SwiGLU epilogue a wave's two column blocks
// are the gate and the up rows of the same 32 hidden columns, so the activation
// is formed on the way out and neither G nor U is ever stored.  Results are
// rounded to bf16 two at a time by the hardware conversion and leave through a
// per-wave LDS piece (written four values per lane at a time, read back in
// 16-byte row chunks), with no block-wide barrier.
//
// Scheduling: a persistent grid (a multiple of 8 workgroups).  Workgroups are
// dealt to the 8 XCDs round-robin, so workgroup b runs on XCD b % 8; each XCD
// takes a contiguous eighth of the tile sequence, which keeps an expert's
// activation panel and weight tiles in that XCD's L2 while it is in use.  The
// number of row tiles of a grouped GEMM is read from the device-side tile prefix
// written by the kernel before it on the same stream (stream order is the fence;
// nothing reads the boundaries before that kernel has finished).
#include <stddef.h>

#include <type_traits>

#include "common.h"
#include "kernels.h"

namespace moe {

namespace {

constexpr int kThreads = 512;
constexpr int kWaves = kThreads / 64;
constexpr int kBM = 256;          // rows per tile
constexpr int kBN = 256;          // B rows (LDS columns) per tile
constexpr int kRowBytes = 128;    // bytes of each row per K step: whole cache lines
constexpr int kOpBytes = kBM * kRowBytes;              // one operand's K step: 32 KB
constexpr int kSlotsFar = 3;      // LDS ring of the operand that runs two steps ahead
constexpr int kSlotsNear = 2;     // LDS ring of the other operand
constexpr int kDmaPerOperand = kBM * kRowBytes / 1024 / kWaves;   // 1-KB DMAs per wave

static_assert(kBM == kBN, "the DMA split assumes equal operand tiles");

// Chunk swizzle of LDS row r (128-byte rows, eight 16-byte chunks): chunk c is
// stored at c ^ swz(r).  Fragment reads of rows r..r+7 (r..r+15) then hit
// distinct banks whether the LDS serves 8 or 16 lanes of a 16-byte read per cycle.
__device__ __forceinline__ int swz(int r) { return (r & 7) ^ ((r >> 3) & 1); }

// Operands stored [reduction][column] (LAY_BT's B, both of LAY_DW's): a slot
// holds 256 / kSubW sub-blocks of kSubW columns (128 bytes), and LDS row kk of
// sub-block b is columns [b kSubW, (b + 1) kSubW) at reduction index kk of the
// step.  Chunk c of that row is stored at c ^ swzT(kk): the four rows that one
// 16-lane transpose read touches then fall on distinct banks.
__device__ __forceinline__ int swzT(int kk) { return ((kk >> 1) & 1) << 2; }

// bf16 fragment of a [reduction][column] slot: ds_read_b64_tr_b16 gives lane j
// of each 16-lane group element j % 4 of the 8 bytes that lane 4 i + j / 4 of
// the group points at (i = 0..3).  With the group's lanes on 4 consecutive rows
// (4 lanes of 4 columns each per row), every lane receives 4 consecutive
// reduction indices of one column; two reads 4 rows apart make the 8 the MFMA
// operand holds.
//
// In the kernels with such operands every fragment read is written out in
// inline asm: for an LDS transpose read it emits itself, the compiler first
// waits for every LDS DMA in flight (vmcnt(0)), which would make each K step
// wait for the loads issued two steps ahead.  A written-out read's result is
// undefined until lds_fence (s_waitcnt lgkmcnt(0), then an empty asm that
// "redefines" each fragment register, so no use can move above the wait), and
// the two halves of a transposed fragment stay apart until then, so nothing
// copies them early.
typedef short v4i16 __attribute__((ext_vector_type(4)));
struct TrPair { v4i16 lo, hi; };
__device__ __forceinline__ uint32_t lds_u32(const void* p) {
    return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) char*)p;
}
__device__ __forceinline__ void asm_read(TrPair& f, const char* p) {
    const uint32_t a = lds_u32(p);
    asm volatile("ds_read_b64_tr_b16 %0, %1" : "=v"(f.lo) : "v"(a));
    asm volatile("ds_read_b64_tr_b16 %0, %1 offset:512" : "=v"(f.hi) : "v"(a));
    static_assert(4 * kRowBytes == 512, "the second half is four rows down");
}
__device__ __forceinline__ void asm_read(bf16x8& f, const char* p) {
    asm volatile("ds_read_b128 %0, %1" : "=v"(f) : "v"(lds_u32(p)));
}
__device__ __forceinline__ void asm_read(float& f, const char* p) {
    asm volatile("ds_read_b32 %0, %1" : "=v"(f) : "v"(lds_u32(p)));
}
// an fp8 fragment: two 16-byte chunks of a row, placed apart by the swizzle (the
// compiler likewise waits for every LDS DMA before its own reads of them)
struct I4Pair { intx4 lo, hi; };
__device__ __forceinline__ void asm_read2(I4Pair& f, const char* p0, const char* p1) {
    asm volatile("ds_read_b128 %0, %1" : "=v"(f.lo) : "v"(lds_u32(p0)));
    asm volatile("ds_read_b128 %0, %1" : "=v"(f.hi) : "v"(lds_u32(p1)));
}
__device__ __forceinline__ void tie(I4Pair& f) { asm volatile("" : "+v"(f.lo), "+v"(f.hi)); }
__device__ __forceinline__ intx8 as_frag(const I4Pair& f) {
    return __builtin_shufflevector(f.lo, f.hi, 0, 1, 2, 3, 4, 5, 6, 7);
}
__device__ __forceinline__ void tie(TrPair& f) { asm volatile("" : "+v"(f.lo), "+v"(f.hi)); }
__device__ __forceinline__ void tie(bf16x8& f) { asm volatile("" : "+v"(f)); }
__device__ __forceinline__ void tie(float& f) { asm volatile("" : "+v"(f)); }
__device__ __forceinline__ bf16x8 as_frag(const TrPair& f) {
    return __builtin_bit_cast(bf16x8, __builtin_shufflevector(f.lo, f.hi, 0, 1, 2, 3, 4, 5, 6, 7));
}
__device__ __forceinline__ bf16x8 as_frag(const bf16x8& f) { return f; }
__device__ __forceinline__ float as_frag(const float& f) { return f; }
__device__ __forceinline__ void zero_elem(TrPair& f, int e) {
    if (e < 4) f.lo[e] = 0;
    else f.hi[e - 4] = 0;
}
__device__ __forceinline__ void zero_elem(float& f, int) { f = 0.0f; }

// s_waitcnt vmcnt(N) (gfx9 encoding: vmcnt split over bits 3:0 and 15:14;
// expcnt and lgkmcnt left at "no wait").
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}
// Workgroup barrier without a global-memory fence: the only cross-wave data
// here is LDS written by the DMA loads, whose completion each wave has already
// waited for (vmcnt), and the wave's own LDS reads are drained (lgkmcnt) so no
// read can still be pending when another wave refills the buffer.  The memory
// clobber keeps the compiler from moving LDS accesses across.
__device__ __forceinline__ void bare_barrier() {
    // lgkmcnt(0) through the builtin, so the compiler's own wait insertion knows
    // every earlier LDS read has completed and adds no wait for them later
    __builtin_amdgcn_s_waitcnt(0xC07F);
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

// One 1-KB DMA (64 lanes x 16 bytes) from a wave-uniform base plus a 32-bit per-lane
// offset into LDS at wave-uniform byte address lds_addr.  Written out so that the
// address is the scalar base plus the lane's 32-bit offset: through the builtin the
// compiler built a 64-bit address per lane and DMA (one 64-bit add each) and kept
// the offsets as 64-bit values; this form measured 1.5-3.5% faster on the grouped
// and dense GEMMs.  The compiler does not see these loads, so it adds no waits of
// its own for them; every wait for them is the kernel's explicit vmcnt wait.  M0
// needs one wait state before the load reads it.
__device__ __forceinline__ void dma16_off(const char* sbase, uint32_t voff, uint32_t lds_addr) {
    asm volatile(
        "s_mov_b32 m0, %2\n\t"
        "s_nop 0\n\t"
        "global_load_lds_dwordx4 %0, %1"
        :
        : "v"(voff), "s"(sbase), "s"(lds_addr)
        : "memory", "m0");
}

__device__ __forceinline__ int64_t uniform64(int64_t x) {
    const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)x);
    const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)((uint64_t)x >> 32));
    return (int64_t)(((uint64_t)hi << 32) | lo);
}

// Wave-uniform reads of the launch's read-only tables (group offsets, tile
// prefix, XCD ranges: written by kernels before this one on the stream, never
// during it), through the constant address space, so they are scalar loads.
// A vector load would wait with vmcnt, which on gfx950 also counts stores: the
// next tile's group lookup after an epilogue would wait for that tile's output
// stores to be acknowledged, once per step of the binary search.
typedef const __attribute__((address_space(4))) int32_t* const_i32_p;
typedef const __attribute__((address_space(4))) int64_t* const_i64_p;
__device__ __forceinline__ int32_t ld_uniform(const int32_t* t, int64_t i) {
    return ((const_i32_p)t)[i];
}
__device__ __forceinline__ int64_t ld_uniform(const int64_t* t, int64_t i) {
    return ((const_i64_p)t)[i];
}

__device__ __forceinline__ int find_group(const int32_t* tp, int G, int m) {
    // largest g in [0, G) with tp[g] <= m  (tp non-decreasing, tp[0] = 0)
    int lo = 0, hi = G;           // invariant: tp[lo] <= m < tp[hi]
    while (hi - lo > 1) {
        int mid = (lo + hi) >> 1;
        if (ld_uniform(tp, mid) <= m) lo = mid; else hi = mid;
    }
    return lo;
}

// 16-byte output store; nt: non-temporal (the output is re-read from HBM anyway).
// Outputs are global memory: the pointer is cast to the global address space, so
// the store is a global store even where the address came through an integer
// (a flat store would also count in lgkmcnt, and every later LDS wait of the
// epilogue would then wait for it to complete).
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(1))) u32x4 g_u32x4;
__device__ __forceinline__ void store16(void* dst, u32x4 x, bool nt) {
    g_u32x4* const g = (g_u32x4*)dst;
    if (nt) __builtin_nontemporal_store(x, g);
    else *g = x;
}
// an element of a global array (the epilogue's addends)
template <typename E>
__device__ __forceinline__ E ld_global(const E* p, int i) {
    return ((const __attribute__((address_space(1))) E*)p)[i];
}
// 16-byte store at system scope, non-temporal (sc0 sc1 nt).  The float32 weight
// gradients (29 GB at the 535B expert shape) are written once and never re-read by
// the kernel; as default stores they evict the operand strips the next tiles
// re-read from L2.  Measured on dW_gu at that shape: fetched bytes about halved
// (8.3 -> 4.6 GB raw FETCH_SIZE) and the kernel 1-3% faster; without any stores the
// same kernel fetches its inputs once (0.59 GB).  A plain vector store, written out
// because the builtins offer no way to set both scope bits.  A store of more than 8
// bytes reads its data registers after issue, so an instruction that overwrites them
// right after the store needs one wait state; the compiler inserts it only for
// stores it can see, so the written-out store carries its own s_nop.
__device__ __forceinline__ void store16_stream(void* dst, u32x4 x) {
    asm volatile("global_store_dwordx4 %0, %1, off sc0 sc1 nt\n\ts_nop 0" ::"v"(dst), "v"(x)
                 : "memory");
}
template <typename OutT, int kVec>
__device__ __forceinline__ void store_vec(OutT* C, int64_t off, const float* v, bool nt);
template <>
__device__ __forceinline__ void store_vec<float, 4>(float* C, int64_t off, const float* v,
                                                    bool nt) {
    const u32x4 x = {__float_as_uint(v[0]), __float_as_uint(v[1]), __float_as_uint(v[2]),
                     __float_as_uint(v[3])};
    store16(C + off, x, nt);
}
template <>
__device__ __forceinline__ void store_vec<bf16_t, 8>(bf16_t* C, int64_t off, const float* v,
                                                     bool nt) {
    u32x4 x;
    x[0] = pack_bf16x2(v[0], v[1]);
    x[1] = pack_bf16x2(v[2], v[3]);
    x[2] = pack_bf16x2(v[4], v[5]);
    x[3] = pack_bf16x2(v[6], v[7]);
    store16(C + off, x, nt);
}

// AA: A's steps run two ahead in the three-slot ring (dense GEMMs, and grouped
// ones whose weights serve several row tiles); otherwise B's do (grouped GEMMs
// that stream each expert's weights once).
template <typename T, typename OutT, int EPI, bool AA, int LAY, bool SPLIT = false>
__global__ __launch_bounds__(kThreads, 1) void gemm_kernel(GemmParams p) {
    constexpr bool kAT = (LAY & 1) != 0;      // A stored [reduction][row]
    constexpr bool kBT = (LAY & 2) != 0;      // B stored [reduction][column]
    constexpr bool kRK = (LAY & 4) != 0;      // reduction over each group's rows
    constexpr int kSlotsA = AA ? kSlotsFar : kSlotsNear;
    constexpr int kBBase = kSlotsA * kOpBytes;             // B ring offset in LDS
    constexpr int kElem = Elem<T>::kBytes;
    constexpr bool kFp8 = std::is_same<T, fp8_t>::value;
    constexpr int kSteps = kRowBytes / (Mfma<T>::kK * kElem);   // MFMA k-steps per K step
    // k-steps per quarter step.  fp8 has two 64-wide k-steps per K step, so its
    // quarter q is k-step q / 2 against column block q % 2 (A's fragments are read
    // in both quarters of a k-step).
    constexpr int kSub = kFp8 ? 1 : kSteps / 4;
    static_assert(kFp8 ? kSteps == 2 : kSteps % 4 == 0, "a K step splits into four quarters");
    static_assert(!kFp8 || LAY == LAY_NN, "fp8 operands are row-major");
    constexpr int kColsOut = (EPI == EPI_SWIGLU) ? kBN / 2 : kBN;
    constexpr int kKStep = kRowBytes / kElem;          // reduction indices per K step
    constexpr int kSubW = kRowBytes / kElem;           // columns per [reduction][column] sub-block
    constexpr int kSubBytes = kKStep * kRowBytes;      // bytes of one such sub-block
    static_assert(!kRK || (kAT && kBT), "a row-group reduction reads both operands transposed");

    extern __shared__ __attribute__((aligned(16))) char lds[];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform
    const int wm = wave >> 2, wn = wave & 3;

    // ---- tile space
    const int64_t n_tiles_n = (p.N + kColsOut - 1) / kColsOut;
    int64_t n_tiles_m;
    if constexpr (kRK) n_tiles_m = (int64_t)p.G * ((p.M + kBM - 1) / kBM);
    else n_tiles_m = p.offsets ? (int64_t)ld_uniform(p.tile_prefix, p.G) : (p.M + kBM - 1) / kBM;
    const int64_t total = n_tiles_m * n_tiles_n;
    const int xcd = blockIdx.x % kNumXcd;
    const int slot = blockIdx.x / kNumXcd;
    const int nslots = gridDim.x / kNumXcd;
    int64_t lo = total * xcd / kNumXcd;
    int64_t hi = total * (xcd + 1) / kNumXcd;
    if constexpr (kRK) {
        // reduction over each group's rows: the XCD ranges come balanced by cost
        // (launch_dw_split); without them, equal tile counts
        if (p.xcd_split) {
            lo = uniform64(ld_uniform(p.xcd_split, xcd));
            hi = uniform64(ld_uniform(p.xcd_split, xcd + 1));
        }
    }
    // SPLIT (dense GEMMs whose last round of tiles is at most half full): each
    // XCD's workgroups take its tiles in rounds of nslots, and the tiles of the
    // last round are split by rows into `pieces` (2 or 4) parts, so that it keeps
    // as many CUs busy as it can (384 tiles on 256 CUs: the 16 tiles per XCD of
    // the second round become 32 half tiles).  A row's result is computed the
    // same way whichever piece it is in.  A separate instantiation: adding this
    // to every GEMM made the grouped ones 4-7% slower.
    static_assert(!SPLIT || !kRK, "no row split of a weight-gradient tile");
    int64_t full = hi - lo, rem = 0;
    int pieces = 1;
    if constexpr (SPLIT) {
        full = ((hi - lo) / nslots) * nslots;
        rem = (hi - lo) - full;
        if (rem * 4 <= nslots) pieces = 4;
        else if (rem * 2 <= nslots) pieces = 2;
    }
    const int64_t n_units = full + rem * pieces;

    // fragment read offsets (the swizzle depends only on row % 32)
    const int fl = swz(lane & 31);
    const int rd_row = (lane & 31) * kRowBytes;
    // Fragment offsets in a [reduction][column] slot.  bf16: the lane's offset
    // for a 32-column block at column 0 (tro0) or 32 (tro1) of its sub-block
    // (lanes of a 16-lane group on rows kr..kr+3, columns cp..cp+3; see
    // tr_frag_bf16).  f32: row lane / 32 and column lane % 32 of the MFMA
    // k-step, whose chunk swizzle alternates with the k-step's parity.
    int tro0 = 0, tro1 = 0;
    if constexpr (kAT || kBT) {
        if constexpr (kElem == 2) {
            const int j = lane & 15;
            const int kr = 8 * (lane >> 5) + (j >> 2);
            const int cp = 16 * ((lane >> 4) & 1) + 4 * (j & 3);
            const int c1 = 32 + cp;
            tro0 = kr * kRowBytes + (((cp >> 3) ^ swzT(kr)) << 4) + ((cp & 7) << 1);
            tro1 = kr * kRowBytes + (((c1 >> 3) ^ swzT(kr)) << 4) + ((c1 & 7) << 1);
        } else {
            const int c = lane & 31;
            tro0 = (lane >> 5) * kRowBytes + ((c >> 2) << 4) + ((c & 3) << 2);
            tro1 = (lane >> 5) * kRowBytes + (((c >> 2) ^ 4) << 4) + ((c & 3) << 2);
        }
    }
    // LDS address of the lane's fragment of the 32-column block at m_base for
    // MFMA k-step ks, in a [reduction][column] slot
    auto t_addr = [&](const char* slot, int m_base, int ks) __attribute__((always_inline)) {
        const char* q = slot + (m_base / kSubW) * kSubBytes + ks * (Mfma<T>::kK * kRowBytes);
        if constexpr (kElem == 2) return q + ((m_base & 32) ? tro1 : tro0);
        else return q + ((ks & 1) ? tro1 : tro0);
    };

    // ---- a tile: its rows, columns and expert
    struct Tile {
        int64_t row0, rows_valid, n0;
        int g, nrb;
        int64_t kbeg, mc0;     // LAY_DW: first row of the group, first A column
        int klen;              // LAY_DW: rows of the group
    };
    auto tile_at = [&](int64_t t) __attribute__((always_inline)) {
        // grouped swizzle along m
        const int64_t gsz = (int64_t)p.group_m * n_tiles_n;
        const int64_t super = t / gsz;
        const int64_t within = t - super * gsz;
        const int64_t m_first = super * p.group_m;
        const int64_t gm = min((int64_t)p.group_m, n_tiles_m - m_first);
        const int64_t tm = m_first + within % gm;
        const int64_t tn = within / gm;
        Tile tl;
        tl.g = 0;
        tl.kbeg = 0;
        tl.mc0 = 0;
        tl.klen = 0;
        if constexpr (kRK) {
            // output rows: group g's [M, N] block of C, row tile tm % ntm
            const int64_t ntm = (p.M + kBM - 1) / kBM;
            tl.g = (int)(tm / ntm);
            tl.mc0 = (tm - (int64_t)tl.g * ntm) * kBM;
            tl.row0 = (int64_t)tl.g * p.M + tl.mc0;
            tl.rows_valid = min((int64_t)kBM, p.M - tl.mc0);
            tl.kbeg = ld_uniform(p.offsets, tl.g);
            tl.klen = ld_uniform(p.offsets, tl.g + 1) - (int)tl.kbeg;
        } else if (p.offsets) {
            tl.g = find_group(p.tile_prefix, p.G, (int)tm);
            const int64_t mloc = tm - ld_uniform(p.tile_prefix, tl.g);
            tl.row0 = ld_uniform(p.offsets, tl.g) + mloc * kBM;
            tl.rows_valid = min((int64_t)kBM, (int64_t)ld_uniform(p.offsets, tl.g + 1) - tl.row0);
        } else {
            tl.row0 = tm * kBM;
            tl.rows_valid = min((int64_t)kBM, p.M - tl.row0);
        }
        tl.nrb = (int)((tl.rows_valid + 31) >> 5);       // active 32-row blocks
        tl.n0 = tn * kColsOut;
        return tl;
    };
    // the tile (or the rows of a tile) that unit u of this XCD computes
    auto unit_at = [&](int64_t u) __attribute__((always_inline)) {
        int64_t ti = u, skip = 0;
        int sub = kBM;
        if (u >= full) {
            const int64_t v = u - full;
            ti = full + v / pieces;
            sub = kBM / pieces;
            skip = (v - (ti - full) * pieces) * sub;
        }
        Tile tl = tile_at(lo + ti);
        tl.row0 += skip;
        tl.rows_valid = max((int64_t)0, min((int64_t)sub, tl.rows_valid - skip));
        tl.nrb = (int)((tl.rows_valid + 31) >> 5);
        return tl;
    };

    // ---- DMA sources.  Wave w fills LDS rows 32 w + 8 i + lane / 8 (i < 4)
    // of each operand, chunk lane % 8, which holds logical chunk (lane % 8) ^
    // swz(row).  Each source is a wave-uniform base (A's tile or gather base,
    // B's group) plus a 32-bit per-lane byte offset; the host checks that every
    // offset fits.
    constexpr int kLanesPerRow = kRowBytes / 16;
    const int lrow = wave * ((64 / kLanesPerRow) * kDmaPerOperand) + lane / kLanesPerRow;
    int chunk[kDmaPerOperand];
#pragma unroll
    for (int i = 0; i < kDmaPerOperand; i++)
        chunk[i] = ((lane % kLanesPerRow) ^ swz((lrow + (64 / kLanesPerRow) * i) & 31)) * 16;
    int32_t a_src[kDmaPerOperand], b_src[kDmaPerOperand];
    auto set_sources = [&](const Tile& tl) __attribute__((always_inline)) {
#pragma unroll
        for (int i = 0; i < kDmaPerOperand; i++) {
            const int r = lrow + (64 / kLanesPerRow) * i;
            if constexpr (!kAT) {
                // rows past the group's end read the tile's first row; their
                // results are never stored
                const int rl = r < tl.rows_valid ? r : 0;
                // gathered: the source row itself; else the row within the tile
                a_src[i] = p.a_rows ? p.a_rows[tl.row0 + rl] / p.a_div : rl;
            }
            if constexpr (!kBT) {
                int64_t col, brow;
                if (EPI == EPI_SWIGLU) {
                    // each 64-row slice of B: [gate 32 | up 32] of 32 hidden columns
                    const int up = (r >> 5) & 1;
                    col = tl.n0 + (r >> 6) * 32 + (r & 31);
                    const int64_t zi = col / p.n_per, cc = col - zi * p.n_per;
                    brow = zi * 2 * p.n_per + cc + up * p.n_per;
                } else {
                    col = tl.n0 + r;
                    brow = col;
                }
                b_src[i] = (int32_t)(col < p.N ? brow : 0);     // row within the group
            }
        }
    };
    // one K segment's bases and offsets for a tile
    const char* A_t = nullptr;
    const char* B_t = nullptr;
    int nk = 0;
    uint32_t a_off[kDmaPerOperand], b_off[kDmaPerOperand];
    uint32_t a_off_t[kDmaPerOperand], b_off_t[kDmaPerOperand];   // LAY_DW: the last step's
    int64_t a_step = kRowBytes, b_step = kRowBytes;              // bytes per K step
    int kvalid = kKStep;          // LAY_DW: reduction rows of the last step
    // Per-lane byte offset of a [reduction][column] operand's DMA into LDS row
    // rho of a slot: sub-block rho / kKStep, reduction index rho % kKStep (read
    // from row min(that, kmax)).  Sub-blocks at or past `ext` columns read
    // sub-block 0; their results are never stored.
    auto t_off = [&](int rho, int64_t ld, int64_t ext, int kmax) __attribute__((always_inline)) {
        const int b = rho / kKStep, kk = rho % kKStep;
        const int bb = (int64_t)b * kSubW < ext ? b : 0;
        const int kr = kk < kmax ? kk : kmax;
        return (uint32_t)((int64_t)kr * ld * kElem) + (uint32_t)(bb * kRowBytes) +
               (uint32_t)((((lane % kLanesPerRow) ^ swzT(kk))) * 16);
    };
    auto set_segment = [&](const Tile& tl, int sidx) __attribute__((always_inline)) {
        // The kernel's only argument is p, laid out at the start of the
        // kernel-argument segment; reading the selected segment from there keeps
        // it in scalar loads (indexing p.seg directly would copy the argument to
        // private memory).
        const GemmSeg* segs = (const GemmSeg*)(
            (const char*)__builtin_amdgcn_kernarg_segment_ptr() + offsetof(GemmParams, seg));
        const char* A = (const char*)uniform64((int64_t)segs[sidx].A);
        const char* B = (const char*)uniform64((int64_t)segs[sidx].B);
        const int64_t lda = uniform64(segs[sidx].lda);
        const int64_t ldb = uniform64(segs[sidx].ldb);
        if constexpr (kRK) {
            nk = __builtin_amdgcn_readfirstlane((tl.klen + kKStep - 1) / kKStep);
            kvalid = __builtin_amdgcn_readfirstlane(tl.klen - (nk - 1) * kKStep);
        } else {
            const int K = __builtin_amdgcn_readfirstlane(segs[sidx].K);
            nk = __builtin_amdgcn_readfirstlane(K * kElem / kRowBytes);
        }
        if constexpr (kAT) {
            A_t = (const char*)uniform64((int64_t)(A + (tl.kbeg * lda + tl.mc0) * kElem));
            a_step = uniform64((int64_t)kKStep * lda * kElem);
        } else {
            const int64_t a_row_base = p.a_rows ? 0 : tl.row0;
            A_t = (const char*)uniform64((int64_t)(A + a_row_base * lda * kElem));
        }
        if constexpr (kBT) {
            const int64_t k0 = kRK ? tl.kbeg : (int64_t)tl.g * p.b_group_rows;
            B_t = (const char*)uniform64((int64_t)(B + (k0 * ldb + tl.n0) * kElem));
            b_step = uniform64((int64_t)kKStep * ldb * kElem);
        } else {
            const int64_t b_row_base = (int64_t)tl.g * p.b_group_rows;
            B_t = (const char*)uniform64((int64_t)(B + b_row_base * ldb * kElem));
        }
#pragma unroll
        for (int i = 0; i < kDmaPerOperand; i++) {
            const int rho = lrow + (64 / kLanesPerRow) * i;
            if constexpr (kAT) {
                a_off[i] = t_off(rho, lda, tl.rows_valid, kKStep - 1);
                if constexpr (kRK) a_off_t[i] = t_off(rho, lda, tl.rows_valid, kvalid - 1);
            } else {
                a_off[i] = (uint32_t)((int64_t)a_src[i] * lda * kElem) + chunk[i];
            }
            if constexpr (kBT) {
                b_off[i] = t_off(rho, ldb, p.N - tl.n0, kKStep - 1);
                if constexpr (kRK) b_off_t[i] = t_off(rho, ldb, p.N - tl.n0, kvalid - 1);
            } else {
                b_off[i] = (uint32_t)((int64_t)b_src[i] * ldb * kElem) + chunk[i];
            }
        }
    };
    char* const a_lds = lds + (wave * kDmaPerOperand) * 1024;
    char* const b_lds = lds + kBBase + (wave * kDmaPerOperand) * 1024;
    // A DMAs i0, i0+1, ... (n of them) of step kt
    // (LAY_DW: the last step's rows past the group's end re-read its last row)
    auto issue_a = [&](int kt, int slot, int i0, int n) __attribute__((always_inline)) {
        const char* const Ak = (const char*)uniform64(
            (int64_t)(A_t + (int64_t)kt * (kAT ? a_step : (int64_t)kRowBytes)));
#pragma unroll
        for (int i = 0; i < kDmaPerOperand; i++)
            if (i >= i0 && i < i0 + n) {
                uint32_t o = a_off[i];
                if constexpr (kRK) o = kt == nk - 1 ? a_off_t[i] : o;
                dma16_off(Ak, o, __builtin_amdgcn_readfirstlane(
                                     lds_u32(a_lds + slot * kOpBytes + i * 1024)));
            }
    };
    // B DMAs i0, i0+1, ... (n of them) of step kt
    auto issue_b = [&](int kt, int slot, int i0, int n) __attribute__((always_inline)) {
        const char* const Bk = (const char*)uniform64(
            (int64_t)(B_t + (int64_t)kt * (kBT ? b_step : (int64_t)kRowBytes)));
#pragma unroll
        for (int i = 0; i < kDmaPerOperand; i++)
            if (i >= i0 && i < i0 + n) {
                uint32_t o = b_off[i];
                if constexpr (kRK) o = kt == nk - 1 ? b_off_t[i] : o;
                dma16_off(Bk, o, __builtin_amdgcn_readfirstlane(
                                     lds_u32(b_lds + slot * kOpBytes + i * 1024)));
            }
    };
    // the operand in the three-slot ring ("far") and the other one ("near")
    auto issue_far = [&](int kt, int slot, int i0, int n) __attribute__((always_inline)) {
        if constexpr (AA) issue_a(kt, slot, i0, n);
        else issue_b(kt, slot, i0, n);
    };
    auto issue_near = [&](int kt, int slot) __attribute__((always_inline)) {
        if constexpr (AA) issue_b(kt, slot, 0, kDmaPerOperand);
        else issue_a(kt, slot, 0, kDmaPerOperand);
    };
    // Issue order, per wave: F0 N0 F1 N1 (this prologue; F = the far operand,
    // N = the near one), then during step kt's quarters 1-2 F(kt+2), and after
    // step kt's barrier N(kt+2).  When step kt+1 is needed, the only younger
    // loads are F(kt+2)'s, so the wait is a constant kDmaPerOperand while the far
    // operand runs two steps ahead.  Past the last step, the same DMAs re-read
    // the last step into slots nothing reads any more, which keeps the count
    // fixed.
    auto prologue = [&]() __attribute__((always_inline)) {
        if (kRK && nk == 0) return;          // an empty group: nothing to load
        issue_far(0, 0, 0, kDmaPerOperand);
        issue_near(0, 0);
        if (nk > 1) {
            issue_far(1, 1, 0, kDmaPerOperand);
            issue_near(1, 1);
        }
    };

    // Epilogue staging: each wave owns a 4 KB piece of the far ring's third
    // slot, which the next tile's first loads (slots 0 and 1 of both rings)
    // leave alone.
    float* const stage = (float*)(lds + (AA ? 0 : kBBase) + 2 * kOpBytes + wave * 4096);
    static_assert(kSlotsFar == 3 && kWaves * 4096 == kOpBytes, "staging layout");

    // this workgroup's unit (SPLIT) or tile
    int64_t t = SPLIT ? (int64_t)slot : lo + slot;
    if (t >= (SPLIT ? n_units : hi)) return;
    Tile cur = SPLIT ? unit_at(t) : tile_at(t);
    set_sources(cur);
    set_segment(cur, 0);
    __syncthreads();
    prologue();

    // The rest of a tile is specialised on the number of active row blocks of
    // this wave: each case is straight-line MFMA code with its own accumulator
    // set.  It ends by issuing the next tile's first loads and reports whether
    // there is a next tile.  (Issuing them before the epilogue measured slower.)
    auto tile_body = [&](auto nact_c) __attribute__((always_inline)) -> bool {
        constexpr int NACT = decltype(nact_c)::value;
        constexpr int NA = NACT > 0 ? NACT : 1;
        typedef typename Mfma<T>::frag Frag;
        // fragments as read: a transposed bf16 fragment and an fp8 fragment are two
        // halves until fenced; these kernels write every fragment read out
        constexpr bool kTK = kAT || kBT || kFp8;
        using FragA = std::conditional_t<kFp8, I4Pair,
                                         std::conditional_t<kAT && kElem == 2, TrPair, Frag>>;
        using FragB = std::conditional_t<kFp8, I4Pair,
                                         std::conditional_t<kBT && kElem == 2, TrPair, Frag>>;
        floatx16 acc[NA][2];
#pragma unroll
        for (int i = 0; i < NACT; i++)
#pragma unroll
            for (int j = 0; j < 2; j++)
#pragma unroll
                for (int v = 0; v < 16; v++) acc[i][j][v] = 0.0f;

        // Fragments of one quarter of a K step (kSub MFMA k-steps).
        auto load_sub = [&](int sa, int sb, int q, FragA (&fa)[kSub][NA], FragB (&fb)[kSub][2])
            __attribute__((always_inline)) {
            const char* As = lds + sa * kOpBytes + rd_row;
            const char* Bs = lds + kBBase + sb * kOpBytes + rd_row;
            if constexpr (kFp8) {
                // a lane's 32 bytes of k are two chunks of its row, which the
                // swizzle places apart
                const int c0 = (q >> 1) * 4 + (lane >> 5) * 2;
                const int o0 = (c0 ^ fl) << 4, o1 = ((c0 + 1) ^ fl) << 4;
                const char* rb = Bs + (wn * 64 + (q & 1) * 32) * kRowBytes;
                asm_read2(fb[0][0], rb + o0, rb + o1);
#pragma unroll
                for (int i = 0; i < NACT; i++) {
                    const char* ra = As + ((wm + 2 * i) * 32) * kRowBytes;
                    asm_read2(fa[0][i], ra + o0, ra + o1);
                }
            } else {
#pragma unroll
                for (int hs = 0; hs < kSub; hs++) {
                    const int ks = q * kSub + hs;
                    const int kb = ks * Mfma<T>::kK * kElem + (lane >> 5) * Mfma<T>::kLaneK * kElem;
                    const int kbyte = (((kb >> 4) ^ fl) << 4) | (kb & 15);
#pragma unroll
                    for (int j = 0; j < 2; j++) {
                        if constexpr (kBT)
                            asm_read(fb[hs][j], t_addr(lds + kBBase + sb * kOpBytes, wn * 64 + j * 32, ks));
                        else if constexpr (kTK)
                            asm_read(fb[hs][j], Bs + (wn * 64 + j * 32) * kRowBytes + kbyte);
                        else
                            fb[hs][j] = Mfma<T>::lds_frag(Bs + (wn * 64 + j * 32) * kRowBytes, kbyte);
                    }
#pragma unroll
                    for (int i = 0; i < NACT; i++) {
                        if constexpr (kAT)
                            asm_read(fa[hs][i], t_addr(lds + sa * kOpBytes, (wm + 2 * i) * 32, ks));
                        else if constexpr (kTK)
                            asm_read(fa[hs][i], As + ((wm + 2 * i) * 32) * kRowBytes + kbyte);
                        else
                            fa[hs][i] = Mfma<T>::lds_frag(As + ((wm + 2 * i) * 32) * kRowBytes, kbyte);
                    }
                }
            }
        };
        // LAY_DW, last step: zero the operand elements at reduction indices past
        // the group's end (their LDS rows hold copies of its last row)
        auto mask_sub = [&](int q, FragA (&fa)[kSub][NA], FragB (&fb)[kSub][2])
            __attribute__((always_inline)) {
            if constexpr (kRK)
#pragma unroll
            for (int hs = 0; hs < kSub; hs++) {
                const int kf = (q * kSub + hs) * Mfma<T>::kK + (lane >> 5) * Mfma<T>::kLaneK;
#pragma unroll
                for (int e = 0; e < Mfma<T>::kLaneK; e++) {
                    if (kf + e >= kvalid) {
#pragma unroll
                        for (int i = 0; i < NACT; i++) zero_elem(fa[hs][i], e);
#pragma unroll
                        for (int j = 0; j < 2; j++) zero_elem(fb[hs][j], e);
                    }
                }
            }
        };
        // written-out reads: wait for them and make their registers defined
        auto fence_sub = [&](FragA (&fa)[kSub][NA], FragB (&fb)[kSub][2])
            __attribute__((always_inline)) {
            if constexpr (kTK) {
                asm volatile("s_waitcnt lgkmcnt(0)");
#pragma unroll
                for (int hs = 0; hs < kSub; hs++) {
#pragma unroll
                    for (int i = 0; i < NACT; i++) tie(fa[hs][i]);
#pragma unroll
                    for (int j = 0; j < 2; j++) tie(fb[hs][j]);
                }
            }
        };
        // the MFMAs of quarter q (fp8: one column block, q % 2)
        auto mma_sub = [&](int q, FragA (&fa)[kSub][NA], FragB (&fb)[kSub][2])
            __attribute__((always_inline)) {
            if constexpr (kFp8) {
                if (q & 1) {
#pragma unroll
                    for (int i = 0; i < NACT; i++)
                        acc[i][1] = Mfma<T>::mma(as_frag(fb[0][0]), as_frag(fa[0][i]), acc[i][1]);
                } else {
#pragma unroll
                    for (int i = 0; i < NACT; i++)
                        acc[i][0] = Mfma<T>::mma(as_frag(fb[0][0]), as_frag(fa[0][i]), acc[i][0]);
                }
            } else {
#pragma unroll
                for (int hs = 0; hs < kSub; hs++)
#pragma unroll
                    for (int i = 0; i < NACT; i++)
#pragma unroll
                        for (int j = 0; j < 2; j++)
                            acc[i][j] = Mfma<T>::mma(as_frag(fb[hs][j]), as_frag(fa[hs][i]), acc[i][j]);
            }
        };
        // Instruction order within a quarter step: one MFMA, then the fragment
        // reads of the next quarter, then the remaining MFMAs with NV DMA
        // instructions interleaved, so the reads have the whole quarter step to
        // complete and the DMA issue never holds up the matrix cores for long.
        auto order_sub = [&](auto nv_c) __attribute__((always_inline)) {
            constexpr int NV = decltype(nv_c)::value;
            constexpr int kReads = kFp8 ? 2 * (NACT + 1) : kSub * (NACT + 2);
            constexpr int kMfmas = kFp8 ? NACT : kSub * NACT * 2;
            constexpr int kPair = NV < kMfmas - 1 ? NV : kMfmas - 1;
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
            __builtin_amdgcn_sched_group_barrier(0x100, kReads, 0);
#pragma unroll
            for (int v = 0; v < kPair; v++) {
                __builtin_amdgcn_sched_group_barrier(0x010, 1, 0);
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
            }
            if (NV > kPair) __builtin_amdgcn_sched_group_barrier(0x010, NV - kPair, 0);
            if (kMfmas - 1 - kPair > 0)
                __builtin_amdgcn_sched_group_barrier(0x008, kMfmas - 1 - kPair, 0);
        };
        using V0 = std::integral_constant<int, 0>;
        using V2 = std::integral_constant<int, 2>;
        using VA = std::integral_constant<int, kDmaPerOperand>;

        // K segments run one after the other, each with its own pipeline fill
        // (the first one's loads are already in flight).
#pragma unroll 1
        for (int sidx = 0; sidx < p.nseg; sidx++) {
            if (sidx > 0) {
                // every DMA of the last segment has landed (its last steps re-read
                // into slots the new segment's first loads reuse) and every wave is
                // done with the slots.  The DMAs are invisible to the compiler, so
                // the wait is explicit.
                wait_vmcnt<0>();
                __syncthreads();
                set_segment(cur, sidx);
                prologue();
            }
            if (kRK && nk == 0) continue;   // an empty group: its block of C is zero
            // step 0 landed once at most step 1's loads are outstanding (the
            // previous tile's stores are older still)
            if (nk > 1) wait_vmcnt<2 * kDmaPerOperand>();
            else wait_vmcnt<0>();
            bare_barrier();
            FragA f0a[kSub][NA], f1a[kSub][NA];
            FragB f0b[kSub][2], f1b[kSub][2];
            if (NACT > 0) load_sub(0, 0, 0, f0a, f0b);

            // Software pipeline over the quarters of the K steps: each quarter's
            // fragments are read while the MFMAs of the previous one run.  After
            // the third quarter's reads the wave waits for step kt+1 to land and
            // meets the others at the barrier; by then every read of step kt's
            // slots has completed, so the near ring's is refilled at once with
            // step kt+2 and the far ring's during the next step with step kt+3.
            int sf = 0, sn = 0;           // far and near ring slots of step kt
#pragma unroll 1
            for (int kt = 0; kt + 1 < nk; kt++) {
                const int kf2 = min(kt + 2, nk - 1);              // far step issued now
                const int sf2 = sf == 0 ? kSlotsFar - 1 : sf - 1;  // its slot, (kt + 2) % 3
                const int sa = AA ? sf : sn, sb = AA ? sn : sf;
                if (NACT > 0 && kTK) {
                    fence_sub(f0a, f0b);
                    load_sub(sa, sb, 1, f1a, f1b);
                    mma_sub(0, f0a, f0b);
                    issue_far(kf2, sf2, 0, kDmaPerOperand / 2);
                    fence_sub(f1a, f1b);
                    load_sub(sa, sb, 2, f0a, f0b);
                    mma_sub(1, f1a, f1b);
                    issue_far(kf2, sf2, kDmaPerOperand / 2, kDmaPerOperand / 2);
                    fence_sub(f0a, f0b);
                    load_sub(sa, sb, 3, f1a, f1b);
                    mma_sub(2, f0a, f0b);
                } else if (NACT > 0) {
                    load_sub(sa, sb, 1, f1a, f1b);
                    mma_sub(0, f0a, f0b);
                    issue_far(kf2, sf2, 0, kDmaPerOperand / 2);
                    order_sub(V2{});
                    load_sub(sa, sb, 2, f0a, f0b);
                    mma_sub(1, f1a, f1b);
                    issue_far(kf2, sf2, kDmaPerOperand / 2, kDmaPerOperand / 2);
                    order_sub(V2{});
                    load_sub(sa, sb, 3, f1a, f1b);
                    mma_sub(2, f0a, f0b);
                    order_sub(V0{});
                } else {
                    issue_far(kf2, sf2, 0, kDmaPerOperand);
                }
                // keep this step's MFMAs ahead of the wait, so they run while the
                // wave waits at the barrier
                __builtin_amdgcn_sched_barrier(0);
                wait_vmcnt<kDmaPerOperand>();   // A, B of kt+1 landed
                bare_barrier();
                sf = sf == kSlotsFar - 1 ? 0 : sf + 1;
                if (NACT > 0 && kTK) {
                    fence_sub(f1a, f1b);
                    load_sub(AA ? sf : sn ^ 1, AA ? sn ^ 1 : sf, 0, f0a, f0b);
                    mma_sub(3, f1a, f1b);
                    issue_near(min(kt + 2, nk - 1), sn);
                } else if (NACT > 0) {
                    load_sub(AA ? sf : sn ^ 1, AA ? sn ^ 1 : sf, 0, f0a, f0b);
                    mma_sub(3, f1a, f1b);
                    issue_near(min(kt + 2, nk - 1), sn);
                    order_sub(VA{});
                } else {
                    issue_near(min(kt + 2, nk - 1), sn);
                }
                sn ^= 1;
            }
            const int sa = AA ? sf : sn, sb = AA ? sn : sf;
            // last step (its first quarter is already in registers)
            const bool tail = kRK && kvalid < kKStep;
            if (NACT > 0 && kTK) {
                fence_sub(f0a, f0b);
                if (tail) mask_sub(0, f0a, f0b);
                load_sub(sa, sb, 1, f1a, f1b);
                mma_sub(0, f0a, f0b);
                fence_sub(f1a, f1b);
                if (tail) mask_sub(1, f1a, f1b);
                load_sub(sa, sb, 2, f0a, f0b);
                mma_sub(1, f1a, f1b);
                fence_sub(f0a, f0b);
                if (tail) mask_sub(2, f0a, f0b);
                load_sub(sa, sb, 3, f1a, f1b);
                mma_sub(2, f0a, f0b);
                fence_sub(f1a, f1b);
                if (tail) mask_sub(3, f1a, f1b);
                mma_sub(3, f1a, f1b);
            } else if (NACT > 0) {
                load_sub(sa, sb, 1, f1a, f1b);
                mma_sub(0, f0a, f0b);
                load_sub(sa, sb, 2, f0a, f0b);
                mma_sub(1, f1a, f1b);
                load_sub(sa, sb, 3, f1a, f1b);
                mma_sub(2, f0a, f0b);
                mma_sub(3, f1a, f1b);
            }
        }
        // every wave is done reading the slots and every DMA has landed (the last
        // steps' re-reads may still be in flight into the slot the epilogue stages
        // through; the compiler does not see the DMAs, so the wait is explicit)
        wait_vmcnt<0>();
        __syncthreads();

        const Tile done = cur;
        const bool more = t + nslots < (SPLIT ? n_units : hi);

        // ---- epilogue.  The MFMAs take the B fragment first, so in each 32 x 32
        // block a lane holds one row (lane % 32) and, in accumulator registers
        // 4 q .. 4 q + 3, the four consecutive columns 8 q + 4 (lane / 32) + 0..3.
        // A block goes through the wave's own 4 KB LDS piece (no block-wide
        // barrier: only the wave reads what it wrote), written four values at a
        // time and read back a row chunk at a time, so every global store is a
        // 16-byte chunk of a row.  Rows of the piece are 128 bytes; their 16-byte
        // chunks are XOR-swizzled by the row so that the writes of 8 consecutive
        // rows fall on distinct banks.
        OutT* const C = (OutT*)p.C;
        const bool nt_out = p.nt_store != 0;
        if constexpr (kFp8) {
            const float sc = (p.scale_a ? *p.scale_a : 1.0f) * (p.scale_b ? *p.scale_b : 1.0f);
#pragma unroll
            for (int i = 0; i < NACT; i++)
#pragma unroll
                for (int j = 0; j < 2; j++)
#pragma unroll
                    for (int v = 0; v < 16; v++) acc[i][j][v] *= sc;
        }
        const int er = lane & 31;          // the lane's row within a block
        const int eh = lane >> 5;          // which four of each eight columns
        const int esw = er & 7;            // chunk swizzle of that row
        char* const piece = (char*)stage;
        // float32 staging of one 32 x 32 block: four floats (one 16-byte chunk)
        // per write; chunk c of row r at chunk c ^ (r & 7)
        auto stage_f32 = [&](const float (&vals)[16]) __attribute__((always_inline)) {
#pragma unroll
            for (int q = 0; q < 4; q++) {
                const float4 x = {vals[4 * q], vals[4 * q + 1], vals[4 * q + 2], vals[4 * q + 3]};
                *(float4*)(piece + er * 128 + (((2 * q + eh) ^ esw) << 4)) = x;
            }
        };
        // value of row r, columns c .. c + 3 (c a multiple of 4) of a staged
        // float32 block
        auto staged_f32 = [&](int r, int c) __attribute__((always_inline)) {
            return *(const float4*)(piece + r * 128 + ((((c >> 2)) ^ (r & 7)) << 4));
        };
        constexpr int kVec = 16 / sizeof(typename Elem<OutT>::store_t);
        // write back a staged float32 block (32 rows of 32 columns starting at
        // tile row rbase, column cbase), with the epilogue's per-element work
        // A block's global addresses are a wave-uniform base (its first row and
        // column) plus a 32-bit lane offset: row r < 32 of rows ld elements apart
        // (every leading dimension here is far below 2^26).  The lane offsets are
        // formed from a copy of the lane index that an empty asm "redefines" inside
        // the helper, so they are recomputed at each block instead of being hoisted
        // out of the tile loop: hoisted (and, before, kept as 64-bit row and column
        // numbers) they were spilled and reloaded on every tile, and a reload after
        // the epilogue's stores waits for them to drain.
        auto blk_base = [&](const void* base, int64_t ld, int rbase, int64_t cbase)
            __attribute__((always_inline)) {
            return (const char*)uniform64(
                (int64_t)((const char*)base + ((done.row0 + rbase) * ld + cbase) * (int64_t)sizeof(OutT)));
        };
        // rows and columns of a block (32 rows at rbase, W columns at cbase) inside
        // the tile's valid rows and the output's columns
        auto blk_rows = [&](int rbase) __attribute__((always_inline)) {
            return (int)max((int64_t)0, min((int64_t)32, done.rows_valid - rbase));
        };
        auto blk_cols = [&](int64_t cbase, int W) __attribute__((always_inline)) {
            return (int)max((int64_t)0, min((int64_t)W, p.N - cbase));
        };
        // write back a staged float32 block (32 rows of 32 columns starting at
        // tile row rbase, column cbase), with the epilogue's per-element work
        auto store_f32_block = [&](int rbase, int64_t cbase) __attribute__((always_inline)) {
            constexpr int kChunks = 32 / kVec;
            const int rv = blk_rows(rbase), cv = blk_cols(cbase, 32);
            const int ldc = (int)p.ldc;
            OutT* const Cb = (OutT*)blk_base(p.C, p.ldc, rbase, cbase);
            int lane_v = lane;
            asm volatile("" : "+v"(lane_v));
#pragma unroll
            for (int q = lane_v; q < 32 * kChunks; q += 64) {
                const int r = q / kChunks;
                const int cc = (q % kChunks) * kVec;
                if (r < rv && cc < cv) {
                    float vals[kVec];
#pragma unroll
                    for (int e = 0; e < kVec; e += 4) {
                        const float4 x = staged_f32(r, cc + e);
                        vals[e] = x.x;
                        vals[e + 1] = x.y;
                        vals[e + 2] = x.z;
                        vals[e + 3] = x.w;
                    }
                    if (EPI == EPI_ADD) {
                        const OutT* const Ab = (const OutT*)blk_base(p.addend, p.ld_add, rbase, cbase);
                        const int aoff = r * (int)p.ld_add + cc;
#pragma unroll
                        for (int e = 0; e < kVec; e++) {
                            if constexpr (std::is_same<OutT, float>::value)
                                vals[e] += ld_global(Ab, aoff + e);
                            else
                                vals[e] += bf16_to_f32(ld_global((const u16*)Ab, aoff + e));
                        }
                    }
                    if constexpr (EPI == EPI_SWIGLU_BWD) {
                        // vals = dh.  With the forward's pre-activations g, u
                        // (float32): dG = dh u silu'(g), dU = dh silu(g), and
                        // h = silu(g) u, silu'(g) = s (1 + g (1 - s)), s = 1 / (1 + exp(-g))
                        const float* const gb = (const float*)uniform64((int64_t)(
                            (const float*)p.addend + (done.row0 + rbase) * p.ld_add + cbase));
                        const float* gu = gb + r * (int)p.ld_add + cc;
                        float dg[kVec], du[kVec], hv[kVec];
#pragma unroll
                        for (int e = 0; e < kVec; e++) {
                            const float g = ld_global(gu, e);
                            const float u = ld_global(gu, (int)p.n_per + e);
                            const float sg = 1.0f / (1.0f + expf(-g));
                            const float si = silu_f(g);
                            dg[e] = vals[e] * u * (sg * (1.0f + g * (1.0f - sg)));
                            du[e] = vals[e] * si;
                            hv[e] = si * u;
                        }
                        const int off = r * ldc + cc;
                        OutT* const C2b = (OutT*)blk_base(p.C2, p.ldc2, rbase, cbase);
                        store_vec<OutT, kVec>(Cb, off, dg, nt_out);
                        store_vec<OutT, kVec>(Cb, off + p.n_per, du, nt_out);
                        store_vec<OutT, kVec>(C2b, r * (int)p.ldc2 + cc, hv, nt_out);
                    } else {
                        if constexpr (kRK && std::is_same<OutT, float>::value) {
                            const u32x4 x = {__float_as_uint(vals[0]), __float_as_uint(vals[1]),
                                             __float_as_uint(vals[2]), __float_as_uint(vals[3])};
                            store16_stream(Cb + r * ldc + cc, x);
                        } else {
                            store_vec<OutT, kVec>(Cb, r * ldc + cc, vals, nt_out);
                        }
                    }
                }
            }
        };
        // bf16 staging of 32 rows x W columns (W = 32 or 64, rows of 2 W bytes):
        // four values (8 bytes) per write at columns cbase + 8 q + 4 (lane / 32);
        // 16-byte chunk c of row r at chunk c ^ (r & 7) (W = 64) or c ^ (r & 3)
        // (W = 32)
        auto stage_bf16 = [&](auto w_c, int cbase, const float (&vals)[16])
            __attribute__((always_inline)) {
            constexpr int W = decltype(w_c)::value;
            constexpr int kRow = 2 * W, kMask = W / 8 - 1;
#pragma unroll
            for (int q = 0; q < 4; q++) {
                const int c = cbase / 8 + q;
                uint2 x;
                x.x = pack_bf16x2(vals[4 * q], vals[4 * q + 1]);
                x.y = pack_bf16x2(vals[4 * q + 2], vals[4 * q + 3]);
                *(uint2*)(piece + er * kRow + ((c ^ (er & kMask)) << 4) + (eh << 3)) = x;
            }
        };
        // write back a staged bf16 block of 32 rows x W columns
        auto store_bf16_block = [&](auto w_c, int rbase, int64_t cbase) __attribute__((always_inline)) {
            constexpr int W = decltype(w_c)::value;
            constexpr int kRow = 2 * W, kMask = W / 8 - 1, kChunks = W / 8;
            const int rv = blk_rows(rbase), cv = blk_cols(cbase, W);
            const int ldc = (int)p.ldc;
            OutT* const Cb = (OutT*)blk_base(p.C, p.ldc, rbase, cbase);
            int lane_v = lane;
            asm volatile("" : "+v"(lane_v));
#pragma unroll
            for (int q = lane_v; q < 32 * kChunks; q += 64) {
                const int r = q / kChunks;
                const int cc = q % kChunks;
                if (r < rv && cc * 8 < cv) {
                    const u32x4 x = *(const u32x4*)(piece + r * kRow + ((cc ^ (r & kMask)) << 4));
                    store16(Cb + r * ldc + cc * 8, x, nt_out);
                }
            }
        };
        using I32 = std::integral_constant<int, 32>;
        using I64 = std::integral_constant<int, 64>;
        constexpr bool kBf16Out = std::is_same<OutT, bf16_t>::value;
#pragma unroll
        for (int i = 0; i < NACT; i++) {
            const int rbase = (wm + 2 * i) * 32;
            if (EPI == EPI_SWIGLU) {
                // a wave's two column blocks are the gate and the up rows of the
                // same 32 hidden columns: h = silu(G) * U in registers
                float hv[16];
#pragma unroll
                for (int v = 0; v < 16; v++) hv[v] = silu_fast(acc[i][0][v]) * acc[i][1][v];
                if constexpr (kBf16Out) {
                    stage_bf16(I32{}, 0, hv);
                    store_bf16_block(I32{}, rbase, done.n0 + wn * 32);
                } else {
                    stage_f32(hv);
                    store_f32_block(rbase, done.n0 + wn * 32);
                }
            } else if (EPI == EPI_STORE && kBf16Out) {
                // both column blocks at once: 64 columns of bf16, 128-byte rows
                float v0[16], v1[16];
#pragma unroll
                for (int v = 0; v < 16; v++) {
                    v0[v] = acc[i][0][v];
                    v1[v] = acc[i][1][v];
                }
                stage_bf16(I64{}, 0, v0);
                stage_bf16(I64{}, 32, v1);
                store_bf16_block(I64{}, rbase, done.n0 + wn * 64);
            } else {
#pragma unroll
                for (int j = 0; j < 2; j++) {
                    float vv[16];
#pragma unroll
                    for (int v = 0; v < 16; v++) vv[v] = acc[i][j][v];
                    stage_f32(vv);
                    store_f32_block(rbase, done.n0 + wn * 64 + j * 32);
                }
            }
        }
        // The next tile's first loads go out after the epilogue.  Issued before
        // it, they would overlap its work, but the epilogue reloads registers
        // the K loop spilled, and every scratch reload waits for all
        // outstanding loads (vmcnt(0)), the new tile's included: measured
        // slower (535B gate/up GEMM 3.10 -> 3.28 ms, pool FFN 2.84 -> 2.92 ms).
        if (more) {
            t += nslots;
            cur = SPLIT ? unit_at(t) : tile_at(t);
            set_sources(cur);
            set_segment(cur, 0);
            prologue();
        }
        return more;
    };

    bool more = true;
    while (more) {
        switch ((cur.nrb - wm + 1) >> 1) {       // this wave's active blocks
            case 4: more = tile_body(std::integral_constant<int, 4>{}); break;
            case 3: more = tile_body(std::integral_constant<int, 3>{}); break;
            case 2: more = tile_body(std::integral_constant<int, 2>{}); break;
            case 1: more = tile_body(std::integral_constant<int, 1>{}); break;
            default: more = tile_body(std::integral_constant<int, 0>{}); break;
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

// XCD ranges for a GEMM whose reduction runs over each group's rows (LAY_DW).
// A group's tiles cost in proportion to its reduction steps plus a fixed share
// for the pipeline fill and the epilogue's 256 x 256 stores (about eight steps'
// time for float32 output, five for bf16).  An equal split of the tile count
// is kept when no XCD gets over 5% more than its share of the cost (its ranges
// hold whole groups whenever the group count divides by 8); otherwise XCD x
// takes the contiguous tiles where the running cost passes x / 8 of the total,
// snapped to a group's start when every group is small next to an XCD's share.
// With skewed groups an equal count leaves one XCD with several times the work
// of another.  One wave; up to 16 groups per lane (G <= 1024); split[0..8].
__global__ __launch_bounds__(64) void dw_split_kernel(const int32_t* offsets, int G,
                                                      int64_t per_g, int k_step, int fixed,
                                                      int64_t* split) {
    constexpr int kPer = 16;
    __shared__ int64_t at_equal[kNumXcd + 1];   // running cost at the equal-count boundaries
    __shared__ int keep_equal;
    const int lane = threadIdx.x;
    const int64_t tiles = (int64_t)G * per_g;
    int64_t u[kPer];
    int64_t sum = 0;
#pragma unroll
    for (int j = 0; j < kPer; j++) {
        const int g = lane * kPer + j;
        u[j] = g < G ? fixed + (offsets[g + 1] - offsets[g] + k_step - 1) / k_step : 0;
        sum += per_g * u[j];
    }
    int64_t incl = sum;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        const int64_t y = __shfl_up(incl, off, 64);
        if (lane >= off) incl += y;
    }
    const int64_t total = __shfl(incl, 63, 64);
    const int64_t share = total / kNumXcd;
    for (int x = 0; x < kNumXcd; x++) {
        const int64_t t = tiles * x / kNumXcd;
        int64_t run = incl - sum;
        for (int j = 0; j < kPer; j++) {
            const int64_t g0 = (int64_t)(lane * kPer + j) * per_g;
            if (u[j] > 0 && g0 <= t && t < g0 + per_g) at_equal[x] = run + (t - g0) * u[j];
            run += per_g * u[j];
        }
    }
    if (lane == 0) at_equal[kNumXcd] = total;
    __syncthreads();
    if (lane == 0) {
        int64_t worst = 0;
        for (int x = 0; x < kNumXcd; x++) worst = max(worst, at_equal[x + 1] - at_equal[x]);
        keep_equal = worst * kNumXcd * 100 <= total * 105;
    }
    __syncthreads();
    if (keep_equal) {
        if (lane <= kNumXcd) split[lane] = tiles * lane / kNumXcd;
        return;
    }
    for (int x = 0; x < kNumXcd; x++) {
        const int64_t target = total * x / kNumXcd;
        int64_t run = incl - sum;
        for (int j = 0; j < kPer; j++) {
            const int64_t c = per_g * u[j];
            if (c > 0 && run <= target && target < run + c) {
                const int64_t g0 = (int64_t)(lane * kPer + j) * per_g;
                split[x] = 16 * c <= share ? g0 + (2 * (target - run) >= c ? per_g : 0)
                                           : g0 + (target - run + u[j] - 1) / u[j];
            }
            run += c;
        }
    }
    if (lane == 0) split[kNumXcd] = tiles;
}

constexpr size_t kLdsBytes = (size_t)(kSlotsFar + kSlotsNear) * kOpBytes;   // 163,840 bytes

template <typename T, typename OutT, int EPI, bool AA, int LAY, bool SPLIT = false>
hipError_t launch_aa(const GemmParams& p, int grid, hipStream_t s) {
    // opting in to more than 64 KB of dynamic LDS is idempotent and cheap
    hipError_t e = hipFuncSetAttribute((const void*)gemm_kernel<T, OutT, EPI, AA, LAY, SPLIT>,
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)kLdsBytes);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((gemm_kernel<T, OutT, EPI, AA, LAY, SPLIT>), dim3(grid), dim3(kThreads),
                       kLdsBytes, s, p);
    return hipGetLastError();
}

// Whether a dense GEMM's last round of tiles is at most half full on some XCD
// (then the row-split variant keeps more CUs busy in that round).
bool dense_split_pays(const GemmParams& p, int epi, int grid) {
    if (p.offsets || p.layout != LAY_NN) return false;
    const int64_t cols = epi == EPI_SWIGLU ? kBN / 2 : kBN;
    const int64_t total = ((p.M + kBM - 1) / kBM) * ((p.N + cols - 1) / cols);
    const int nslots = grid / kNumXcd;
    for (int x = 0; x < kNumXcd; x++) {
        const int64_t n_x = total * (x + 1) / kNumXcd - total * x / kNumXcd;
        const int64_t rem = n_x % nslots;
        if (rem > 0 && 2 * rem <= nslots) return true;
    }
    return false;
}

template <typename T, typename OutT, int EPI, int LAY = LAY_NN>
hipError_t launch_t(const GemmParams& p, int grid, hipStream_t s) {
    return p.a_ahead ? launch_aa<T, OutT, EPI, true, LAY>(p, grid, s)
                     : launch_aa<T, OutT, EPI, false, LAY>(p, grid, s);
}

// The backward layouts: LAY_BT stores C in the input type (plain, or the SwiGLU
// derivative); LAY_DW stores C in the input type or float32.
template <typename T>
hipError_t launch_bwd(const GemmParams& p, bool out_f32, int epi, int grid, hipStream_t s) {
    if (p.layout == LAY_DW)
        return out_f32 ? launch_t<T, float, EPI_STORE, LAY_DW>(p, grid, s)
                       : launch_t<T, T, EPI_STORE, LAY_DW>(p, grid, s);
    if (epi == EPI_SWIGLU_BWD) return launch_t<T, T, EPI_SWIGLU_BWD, LAY_BT>(p, grid, s);
    return launch_t<T, T, EPI_STORE, LAY_BT>(p, grid, s);
}

}  // namespace

int gemm_block_m() { return kBM; }

int gemm_k_bytes() { return kRowBytes; }

bool gemm_offsets_fit(const GemmParams& p, int es) {
    const int64_t lim = (int64_t)1 << 32;
    const int64_t kstep = kRowBytes / es;
    for (int s = 0; s < p.nseg; s++) {
        const GemmSeg& g = p.seg[s];
        // [reduction][column] operands: offsets span one K step of rows and a tile
        if (p.layout == LAY_DW) {
            if (((kstep - 1) * g.lda + kBM) * es >= lim) return false;
            if (((kstep - 1) * g.ldb + kBN) * es >= lim) return false;
            continue;
        }
        if (p.layout == LAY_BT) {
            if (((kstep - 1) * g.ldb + kBN) * es >= lim) return false;
            const int64_t a_rows = p.a_rows ? p.a_src_rows : kBM;
            if ((a_rows * g.lda + g.K) * es >= lim) return false;
            if (((int64_t)g.K * es) % kRowBytes) return false;
            continue;
        }
        // A: offsets from the gather base (any source row) or from the tile's row 0
        const int64_t a_rows = p.a_rows ? p.a_src_rows : kBM;
        if ((a_rows * g.lda + g.K) * es >= lim) return false;
        // B: offsets from the group's first row (a dense SwiGLU B has 2N rows)
        const int64_t b_rows = p.offsets ? p.b_group_rows : 2 * p.N;
        if ((b_rows * g.ldb + g.K) * es >= lim) return false;
        if (((int64_t)g.K * es) % kRowBytes) return false;
    }
    return true;
}

int gemm_cols_per_tile(int epi) { return epi == EPI_SWIGLU ? kBN / 2 : kBN; }

hipError_t launch_dw_split(const int32_t* offsets, int G, int64_t M, int64_t N, int elem_bytes,
                           bool out_f32, int64_t* split, hipStream_t s) {
    const int64_t per_g = ((M + kBM - 1) / kBM) * ((N + kBN - 1) / kBN);
    hipLaunchKernelGGL(dw_split_kernel, dim3(1), dim3(64), 0, s, offsets, G, per_g,
                       kRowBytes / elem_bytes, out_f32 ? 8 : 5, split);
    return hipGetLastError();
}

hipError_t launch_tile_prefix(const int32_t* offsets, int G, int BM, int32_t* tp, hipStream_t s) {
    hipLaunchKernelGGL(tile_prefix_kernel, dim3(1), dim3(1024), 0, s, offsets, G, BM, tp);
    return hipGetLastError();
}

hipError_t launch_gemm(const GemmParams& p, moe_dtype in_dt, bool out_f32, int epi,
                       int64_t max_tiles, hipStream_t s) {
    // the C ABI has checked these already; a violation here is a library bug
    if (!gemm_offsets_fit(p, in_dt == MOE_BF16 ? 2 : in_dt == MOE_E4M3 ? 1 : 4))
        return hipErrorInvalidValue;
    int dev = 0, cus = 256;
    if (hipGetDevice(&dev) != hipSuccess) return hipErrorInvalidDevice;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
        return hipErrorInvalidDevice;
    int64_t grid = cus;
    if (max_tiles < grid) grid = max_tiles;
    grid = ((grid + kNumXcd - 1) / kNumXcd) * kNumXcd;
    if (grid < kNumXcd) grid = kNumXcd;
    if (p.layout != LAY_NN)
        return in_dt == MOE_BF16 ? launch_bwd<bf16_t>(p, out_f32, epi, (int)grid, s)
                                 : launch_bwd<float>(p, out_f32, epi, (int)grid, s);
    if (in_dt == MOE_E4M3) {
        if (epi != EPI_STORE) return hipErrorInvalidValue;    // E4M3 operands: plain stores
        return out_f32 ? launch_t<fp8_t, float, EPI_STORE>(p, (int)grid, s)
                       : launch_t<fp8_t, bf16_t, EPI_STORE>(p, (int)grid, s);
    }
    if (in_dt == MOE_BF16 && p.a_ahead && dense_split_pays(p, epi, (int)grid)) {
        if (epi == EPI_STORE)
            return out_f32 ? launch_aa<bf16_t, float, EPI_STORE, true, LAY_NN, true>(p, (int)grid, s)
                           : launch_aa<bf16_t, bf16_t, EPI_STORE, true, LAY_NN, true>(p, (int)grid, s);
        if (epi == EPI_SWIGLU)
            return launch_aa<bf16_t, bf16_t, EPI_SWIGLU, true, LAY_NN, true>(p, (int)grid, s);
        return launch_aa<bf16_t, bf16_t, EPI_ADD, true, LAY_NN, true>(p, (int)grid, s);
    }
    if (in_dt == MOE_BF16) {
        if (epi == EPI_STORE)
            return out_f32 ? launch_t<bf16_t, float, EPI_STORE>(p, (int)grid, s)
                           : launch_t<bf16_t, bf16_t, EPI_STORE>(p, (int)grid, s);
        if (epi == EPI_SWIGLU) return launch_t<bf16_t, bf16_t, EPI_SWIGLU>(p, (int)grid, s);
        return launch_t<bf16_t, bf16_t, EPI_ADD>(p, (int)grid, s);
    }
    if (epi == EPI_STORE) return launch_t<float, float, EPI_STORE>(p, (int)grid, s);
    if (epi == EPI_SWIGLU) return launch_t<float, float, EPI_SWIGLU>(p, (int)grid, s);
    return launch_t<float, float, EPI_ADD>(p, (int)grid, s);
}

}  // namespace moe
