// Internal launch interface between the C-ABI layer (abi.hip) and the kernels.
// Not part of the public ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/moe.h"

namespace moe {

// ------------------------------------------------------------------ GEMM ---
enum { EPI_STORE = 0, EPI_SWIGLU = 1, EPI_ADD = 2, EPI_SWIGLU_BWD = 3 };
// Operand layouts.  By default A rows and B rows hold the reduction index
// contiguously (C = A B^T).  LAY_BT: B is stored [reduction][column] (a weight
// contracted over its rows: the input gradient of a grouped matmul).  LAY_DW:
// both operands are stored [reduction][column] and the reduction runs over each
// group's rows (the weight gradient of a grouped matmul).
enum { LAY_NN = 0, LAY_BT = 2, LAY_DW = 7 };
constexpr int kMaxSeg = 4;

struct GemmSeg {
    const void* A;     // A row r: A + r * lda (elements)
    int64_t lda;
    const void* B;     // B row n: B + n * ldb (elements)
    int64_t ldb;
    int32_t K;         // reduction length of this segment (multiple of 64 bytes)
};

// C[r, n] = epi(sum over segments s of A_s[arow(r), :] . B_s[brow(g, n), :]).
struct GemmParams {
    int64_t M;                   // rows when offsets == nullptr
    const int32_t* offsets;      // [G+1] row groups (device) or nullptr
    const int32_t* tile_prefix;  // [G+1] row-tile prefix for the GEMM's BM (device)
    int32_t G;
    int64_t b_group_rows;        // B rows between consecutive groups' weights
    const int32_t* a_rows;       // gather: A row of output row r = a_rows[r] / a_div
    int32_t a_div;
    int64_t N;                   // output columns
    int64_t n_per;               // SwiGLU: hidden columns per [gate; up] block of B
    int64_t a_src_rows;          // gather: rows of the A matrix a_rows indexes (host check)
    int32_t group_m;             // row tiles per swizzle group
    int32_t a_ahead;             // 1: A's K steps run two ahead (else B's)
    int32_t nt_store;            // 1: non-temporal output stores
    GemmSeg seg[kMaxSeg];
    int32_t nseg;
    void* C;                     // output row r: C + r * ldc
    int64_t ldc;
    const void* addend;          // EPI_ADD: added row r: addend + r * ld_add
    int64_t ld_add;              //   (EPI_SWIGLU_BWD: the [gate | up] pre-activations)
    void* C2;                    // EPI_SWIGLU_BWD: h row r: C2 + r * ldc2
    int64_t ldc2;
    int32_t layout;              // LAY_*
    const int64_t* xcd_split;    // LAY_DW: [9] tile range of each XCD (device), or nullptr
    // fp8 operands: the accumulators are multiplied by scale_a[0] * scale_b[0]
    // (device memory, each nullable = 1) before the epilogue
    const float* scale_a;
    const float* scale_b;
};

int gemm_block_m();
// Bytes of each row per K step: every segment's K * element size must be a
// multiple of it.
int gemm_k_bytes();
// True if every per-lane DMA byte offset of the GEMM fits in 32 bits.
bool gemm_offsets_fit(const GemmParams& p, int elem_bytes);
int gemm_cols_per_tile(int epi);
hipError_t launch_tile_prefix(const int32_t* offsets, int G, int BM, int32_t* tp, hipStream_t s);
// LAY_DW: XCD tile ranges balanced by each group's reduction length (device, [9]).
hipError_t launch_dw_split(const int32_t* offsets, int G, int64_t M, int64_t N, int elem_bytes,
                           bool out_f32, int64_t* split, hipStream_t s);
hipError_t launch_gemm(const GemmParams& p, moe_dtype in_dt, bool out_f32, int epi,
                       int64_t max_tiles, hipStream_t s);

// ------------------------------------------------------------------- fp8 ---
hipError_t launch_quantize_e4m3(const void* x, moe_dtype dt, int64_t n, const float* scale,
                                uint8_t* q, float* amax, hipStream_t s);
hipError_t launch_swiglu_quantize_e4m3(const void* gu, moe_dtype dt, const int32_t* offsets,
                                       int E, int64_t R_phys, int64_t H, const float* scale,
                                       uint8_t* hq, float* amax, hipStream_t s);
hipError_t launch_zero_u32(uint32_t* p, hipStream_t s);
hipError_t launch_fp8_scale_update(float* history, int len, const float* amax, float* scale,
                                   hipStream_t s);

// ----------------------------------------------------------------- route ---
hipError_t launch_route(const void* h, moe_dtype h_dt, int64_t T, int64_t d, const float* g,
                        float eps, int apply_norm, const float* W_r, const float* b_r, int E,
                        int k, void* r_out, moe_dtype r_dt, float* logits, int32_t* ids, float* w,
                        hipStream_t s);

// --------------------------------------------------------------- permute ---
size_t permute_ws_bytes(int64_t n, int E);
// expert-parallel dispatch, sender side: peer[i] = ids[i] / epp (-1 stays -1), and
// payload[r] = ids[row_src[r]] % epp for r < offsets[P], -1 past it
hipError_t launch_peer_of(const int32_t* ids, int64_t n, int epp, int32_t* peer, hipStream_t s);
hipError_t launch_payload_ids(const int32_t* ids, const int32_t* row_src, const int32_t* offsets,
                              int P, int64_t R_phys, int epp, int32_t* payload, hipStream_t s);
hipError_t launch_permute(const int32_t* ids, int64_t n, int E, int64_t capacity, const void* src,
                          int elem_bytes, int64_t width, int src_div, void* dst, int64_t R_phys,
                          int32_t* slot_row, int32_t* row_src, int32_t* counts, int32_t* offsets,
                          int64_t* n_dropped, int32_t* tile_prefix, int tile_bm, void* ws,
                          hipStream_t s, bool out_e4m3 = false, const float* scale = nullptr,
                          float* amax = nullptr);

// moe_permute's host-side argument checks (all but the workspace's), shared by
// the entry points that group assignments (abi.hip)
moe_status permute_check(const int32_t* ids, int64_t n_assign, int32_t E, int64_t capacity,
                         const void* src, moe_dtype dt, int64_t width, int32_t src_div,
                         const void* dst, int64_t R_phys, const int32_t* slot_row,
                         const int32_t* row_src, const int32_t* counts, const int32_t* offsets,
                         const int64_t* n_dropped);

// --------------------------------------------------------------- combine ---
hipError_t launch_combine(const void* Y, moe_dtype dt, const int32_t* slot_row, const float* w,
                          int64_t T, int k, int64_t width, void* out, int flags, hipStream_t s);

}  // namespace moe
