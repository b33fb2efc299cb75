// C ABI of libmoe: host-side validation, workspace carving and the order in
// which the layer's kernels are enqueued.  Every check runs before anything
// is enqueued; nothing here allocates, frees or synchronises device memory,
// and no mutable global state is kept.
#include <string.h>

#include "common.h"
#include "kernels.h"

using namespace moe;

namespace {

constexpr int kAbiVersion = 2;

inline size_t a256(size_t x) { return (x + 255) & ~(size_t)255; }
inline bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }
inline bool aligned4(const void* p) { return ((uintptr_t)p & 3u) == 0; }
inline int esize(moe_dtype dt) { return dt == MOE_BF16 ? 2 : dt == MOE_E4M3 ? 1 : 4; }
inline bool dt_ok(moe_dtype dt) { return dt == MOE_F32 || dt == MOE_BF16; }
inline hipStream_t hs(moe_stream s) { return (hipStream_t)s; }
// A GEMM reduction or output width: whole 128-byte K steps and 32-column blocks.
inline bool width_ok(int64_t w, moe_dtype dt) {
    return w > 0 && w % 32 == 0 && (w * esize(dt)) % gemm_k_bytes() == 0;
}
// Every DMA source offset of the GEMMs is a 32-bit byte offset from a base.
inline bool under4g(int64_t rows, int64_t width, moe_dtype dt) {
    return rows * width * esize(dt) < ((int64_t)1 << 32);
}

#define MOE_TRY(expr)                              \
    do {                                           \
        if ((expr) != hipSuccess) return MOE_ELAUNCH; \
    } while (0)

// Carves consecutive 256-byte-aligned regions out of a workspace (or, with a
// null base, only measures them).
struct Carver {
    char* base;
    size_t off = 0;
    explicit Carver(void* b) : base((char*)b) {}
    template <typename P>
    P* take(size_t bytes) {
        P* p = base ? (P*)(base + off) : nullptr;
        off += a256(bytes > 0 ? bytes : 1);
        return p;
    }
};

int64_t grouped_tile_bound(int64_t rows, int G, int64_t N, int epi) {
    const int64_t BM = gemm_block_m();
    const int64_t cols = gemm_cols_per_tile(epi);
    return ((rows + BM - 1) / BM + G) * ((N + cols - 1) / cols);
}
int64_t dense_tiles(int64_t rows, int64_t N, int epi) {
    const int64_t BM = gemm_block_m();
    const int64_t cols = gemm_cols_per_tile(epi);
    return ((rows + BM - 1) / BM) * ((N + cols - 1) / cols);
}

// Row tiles per swizzle group.  An XCD's 32 CUs work on consecutive tiles in
// near lockstep along K, so with 8 row tiles per group each B slice is shared by
// 8 concurrent tiles and each A slice by 4 (dense GEMMs).  Grouped GEMMs whose
// experts have few row tiles keep one row tile and walk the columns innermost,
// so the expert's rows stay in L2 across its column tiles while its weights
// stream past: faster than groups of 8 at the 535B shape (one row tile per
// expert) and at 65,536 tokens (about five; gate/up GEMM 19.7 vs 20.5 ms).
// Experts with many row tiles (the 6-expert receiver pool, about 43 each) take
// groups of 8 as the dense GEMMs do (pool FFN 3.00 vs 3.02 ms, three rounds).
constexpr int kGroupDense = 8;
constexpr int kGroupGroupedFew = 1;
constexpr int kGroupGroupedMany = 8;
constexpr int kManyTilesPerExpert = 16;

GemmParams gemm_base() {
    GemmParams p;
    memset(&p, 0, sizeof p);
    p.a_div = 1;
    p.group_m = kGroupDense;
    p.a_ahead = 1;
    return p;
}

// Which operand's K steps run two ahead in the GEMM's three-slot LDS ring: the
// one whose slices come from farthest away.  A grouped GEMM whose experts hold
// under two row tiles on average streams each expert's weights from HBM once,
// so B does; otherwise both operands are reused across tiles and A does.
// Measured at the 535B shape (gate/up GEMM 3.2 ms with B ahead, 3.4 with A) and
// on the shared experts' dense GEMM (1.05 ms with A ahead, 1.12 with B).
int grouped_a_ahead(int64_t R_rows, int E) {
    return R_rows >= (int64_t)2 * gemm_block_m() * E ? 1 : 0;
}

int grouped_group_m(int64_t R_rows, int E) {
    return R_rows >= (int64_t)kManyTilesPerExpert * gemm_block_m() * E ? kGroupGroupedMany
                                                                       : kGroupGroupedFew;
}

// The grouped GEMMs' outputs (the expert hidden and output rows, hundreds of MB
// at the 535B shape) are read back from HBM by the next kernel anyway, so they
// are written non-temporally (down GEMM 1.72 -> 1.66 ms, gate/up 3.23 -> 3.19 ms
// there); the dense GEMMs' smaller outputs keep the cached path, which lets the
// next GEMM find part of them in cache.
constexpr int kGroupedNtStore = 1;

// Grouped gated MLP over row groups: h = SwiGLU(X W_gu[g]^T), Y = h W_d[g]^T.
// X rows optionally gathered (a_rows / a_div).
moe_status grouped_ffn_impl(const void* X, int64_t ldx, const int32_t* a_rows, int a_div,
                            int64_t a_src_rows, const int32_t* offsets,
                            const int32_t* tile_prefix, int E, int64_t R_rows, const void* W_gu,
                            const void* W_d, int64_t d, int64_t H, moe_dtype dt, void* h,
                            void* Y, hipStream_t s) {
    GemmParams p = gemm_base();
    p.group_m = grouped_group_m(R_rows, E);
    p.a_ahead = grouped_a_ahead(R_rows, E);
    p.nt_store = kGroupedNtStore;
    p.a_src_rows = a_src_rows;
    p.offsets = offsets;
    p.tile_prefix = tile_prefix;
    p.G = E;
    p.a_rows = a_rows;
    p.a_div = a_div;
    p.b_group_rows = 2 * H;
    p.N = H;
    p.n_per = H;
    p.seg[0] = GemmSeg{X, ldx, W_gu, d, (int32_t)d};
    p.nseg = 1;
    p.C = h;
    p.ldc = H;
    MOE_TRY(launch_gemm(p, dt, false, EPI_SWIGLU, grouped_tile_bound(R_rows, E, H, EPI_SWIGLU), s));
    return MOE_OK;
}

moe_status grouped_down_impl(const void* h, const int32_t* offsets, const int32_t* tile_prefix,
                             int E, int64_t R_rows, const void* W_d, int64_t d, int64_t H,
                             moe_dtype dt, void* Y, hipStream_t s) {
    GemmParams p = gemm_base();
    p.group_m = grouped_group_m(R_rows, E);
    p.a_ahead = grouped_a_ahead(R_rows, E);
    p.nt_store = kGroupedNtStore;
    p.offsets = offsets;
    p.tile_prefix = tile_prefix;
    p.G = E;
    p.b_group_rows = d;
    p.N = d;
    p.seg[0] = GemmSeg{h, H, W_d, H, (int32_t)H};
    p.nseg = 1;
    p.C = Y;
    p.ldc = d;
    MOE_TRY(launch_gemm(p, dt, dt == MOE_F32, EPI_STORE,
                        grouped_tile_bound(R_rows, E, d, EPI_STORE), s));
    return MOE_OK;
}

// Input gradient of the grouped matmul Z[r] = X[r] W[g]^T (W [G, N, K]):
// dX[r] = dZ[r] W[g], a grouped GEMM that reads W[g] along its rows.  With
// EPI_SWIGLU_BWD the reduction result is dh of the gated MLP (K = H columns) and
// the epilogue turns it into [dG | dU] (C, 2H wide) and h (h_out) using the
// forward's pre-activations gu [rows, 2H] (float32).
moe_status dlhs_impl(const void* dZ, const int32_t* offsets, const int32_t* tile_prefix, int E,
                     int64_t R_rows, const void* W, int64_t N, int64_t K, moe_dtype dt, int epi,
                     void* C, int64_t ldc, const void* gu, void* h_out, hipStream_t s) {
    GemmParams p = gemm_base();
    p.layout = LAY_BT;
    p.group_m = grouped_group_m(R_rows, E);
    p.a_ahead = grouped_a_ahead(R_rows, E);
    p.offsets = offsets;
    p.tile_prefix = tile_prefix;
    p.G = E;
    p.b_group_rows = N;
    p.N = K;
    p.seg[0] = GemmSeg{dZ, N, W, K, (int32_t)N};
    p.nseg = 1;
    p.C = C;
    p.ldc = ldc;
    if (epi == EPI_SWIGLU_BWD) {
        p.addend = gu;
        p.ld_add = 2 * K;
        p.n_per = K;
        p.C2 = h_out;
        p.ldc2 = K;
    }
    MOE_TRY(launch_gemm(p, dt, false, epi, grouped_tile_bound(R_rows, E, K, EPI_STORE), s));
    return MOE_OK;
}

// Weight gradient of the grouped matmul: dW[g] = dZ[rows of g]^T X[rows of g],
// [N, K] per group, the reduction running over each group's rows.  `split`
// ([9] int64, device) receives the XCD tile ranges balanced by group length.
moe_status drhs_impl(const void* X, const void* dZ, const int32_t* offsets, int E, int64_t N,
                     int64_t K, moe_dtype dt, void* dW, bool out_f32, int64_t* split,
                     hipStream_t s) {
    MOE_TRY(launch_dw_split(offsets, E, N, K, esize(dt), out_f32 || dt == MOE_F32, split, s));
    GemmParams p = gemm_base();
    p.xcd_split = split;
    p.layout = LAY_DW;
    p.group_m = 1;
    p.offsets = offsets;
    p.G = E;
    p.M = N;
    p.N = K;
    p.seg[0] = GemmSeg{dZ, N, X, K, 0};
    p.nseg = 1;
    p.C = dW;
    p.ldc = K;
    const int64_t BM = gemm_block_m();
    MOE_TRY(launch_gemm(p, dt, out_f32, EPI_STORE,
                        (int64_t)E * ((N + BM - 1) / BM) * ((K + BM - 1) / BM), s));
    return MOE_OK;
}

// The grouped matmul Z[r] = scale * W[g] X[r] over row groups (the pages'
// ragged_dot forward in this library's output-major convention), in bf16, fp32
// or E4M3 operands; Z in bf16 or fp32.
moe_status ragged_dot_impl(const void* X, const int32_t* offsets, int E, int64_t R_phys,
                           const void* W, int64_t N, int64_t K, moe_dtype dt,
                           const float* scale_a, const float* scale_b, void* Z, bool out_f32,
                           int32_t* tile_prefix, hipStream_t s) {
    MOE_TRY(launch_tile_prefix(offsets, E, gemm_block_m(), tile_prefix, s));
    GemmParams p = gemm_base();
    p.group_m = grouped_group_m(R_phys, E);
    p.a_ahead = grouped_a_ahead(R_phys, E);
    p.nt_store = kGroupedNtStore;
    p.offsets = offsets;
    p.tile_prefix = tile_prefix;
    p.G = E;
    p.b_group_rows = N;
    p.N = N;
    p.seg[0] = GemmSeg{X, K, W, K, (int32_t)K};
    p.nseg = 1;
    p.C = Z;
    p.ldc = N;
    p.scale_a = scale_a;
    p.scale_b = scale_b;
    MOE_TRY(launch_gemm(p, dt, out_f32, EPI_STORE, grouped_tile_bound(R_phys, E, N, EPI_STORE), s));
    return MOE_OK;
}

moe_status check_ragged_dot(const void* X, const int32_t* offsets, int32_t E, int64_t R_phys,
                            const void* W, int64_t N, int64_t K, moe_dtype dt, void* Z,
                            moe_dtype z_dt, void* ws, size_t ws_bytes) {
    if (E < 1 || E > 1024 || R_phys < 0 || R_phys >= ((int64_t)1 << 31)) return MOE_ESHAPE;
    if (!dt_ok(z_dt)) return MOE_EDTYPE;
    if (!width_ok(K, dt) || !width_ok(N, z_dt) || N % 64) return MOE_ESHAPE;
    if (!under4g(gemm_block_m() + 1, K, dt) || !under4g(N + 1, K, dt)) return MOE_ESHAPE;
    if (!offsets || !W || (R_phys > 0 && (!X || !Z))) return MOE_EINVAL;
    const void* ptrs[] = {X, offsets, W, Z, ws};
    for (const void* p : ptrs)
        if (p && !aligned16(p)) return MOE_EALIGN;
    if (!ws || ws_bytes < a256((size_t)(E + 1) * 4)) return MOE_EWORKSPACE;
    return MOE_OK;
}

struct LayerBufs {
    float* z_pre;
    void* z_e;
    float* logits;
    int32_t* ids;
    float* w;
    void* perm_ws;
    int32_t* counts;
    int32_t* offsets;
    int64_t* n_dropped;
    int32_t* slot_row;
    int32_t* row_src;
    int32_t* tile_prefix;
    void* h;
    void* Y;
    void* c;
    void* h_s;
};

}  // namespace

namespace moe {

// moe_permute's argument checks, shared with its allocation-free variant (every
// check except the workspace's).
moe_status permute_check(const int32_t* ids, int64_t n_assign, int32_t E, int64_t capacity,
                         const void* src, moe_dtype dt, int64_t width, int32_t src_div,
                         const void* dst, int64_t R_phys, const int32_t* slot_row,
                         const int32_t* row_src, const int32_t* counts, const int32_t* offsets,
                         const int64_t* n_dropped) {
    if (E < 1 || E > 1024) return MOE_ESHAPE;
    if (n_assign < 0 || n_assign >= ((int64_t)1 << 31) || R_phys < 0) return MOE_ESHAPE;
    const int64_t max_kept = capacity < 0 ? n_assign
                                          : (capacity * E < n_assign ? capacity * E : n_assign);
    if (R_phys < max_kept || R_phys >= ((int64_t)1 << 31)) return MOE_ESHAPE;
    if (!counts || !offsets || !n_dropped) return MOE_EINVAL;
    if (n_assign > 0 && (!ids || !slot_row)) return MOE_EINVAL;
    if (R_phys > 0 && !row_src) return MOE_EINVAL;
    if ((src == nullptr) != (dst == nullptr)) return MOE_EINVAL;
    if (src) {
        if (!dt_ok(dt)) return MOE_EDTYPE;
        if (width <= 0 || (width * esize(dt)) % 16 || src_div < 1) return MOE_ESHAPE;
    }
    const void* ptrs[] = {ids, src, dst, slot_row, row_src, counts, offsets, n_dropped};
    for (const void* p : ptrs)
        if (p && !aligned16(p)) return MOE_EALIGN;
    return MOE_OK;
}

}  // namespace moe

namespace {

LayerBufs carve_layer(const moe_layer_desc* d, void* ws, size_t* total) {
    Carver cv(ws);
    LayerBufs b;
    const int64_t T = d->T, R = d->T * d->k;
    const int64_t de = d->L > 0 ? d->L : d->D;
    const int es = esize(d->dtype);
    b.z_pre = d->L > 0 ? cv.take<float>((size_t)T * d->L * 4) : nullptr;
    b.z_e = d->L > 0 ? cv.take<char>((size_t)T * d->L * es) : nullptr;
    b.logits = cv.take<float>((size_t)T * d->E * 4);
    b.ids = cv.take<int32_t>((size_t)R * 4);
    b.w = cv.take<float>((size_t)R * 4);
    b.perm_ws = cv.take<char>(permute_ws_bytes(R, d->E));
    b.counts = cv.take<int32_t>((size_t)d->E * 4);
    b.offsets = cv.take<int32_t>((size_t)(d->E + 1) * 4);
    b.n_dropped = cv.take<int64_t>(8);
    b.slot_row = cv.take<int32_t>((size_t)R * 4);
    b.row_src = cv.take<int32_t>((size_t)R * 4);
    b.tile_prefix = cv.take<int32_t>((size_t)(d->E + 1) * 4);
    b.h = cv.take<char>((size_t)R * d->H * es);
    b.Y = cv.take<char>((size_t)R * de * es);
    b.c = cv.take<char>((size_t)T * de * es);
    b.h_s = d->n_shared > 0 ? cv.take<char>((size_t)T * d->n_shared * d->Hs * es) : nullptr;
    *total = cv.off;
    return b;
}

moe_status check_layer(const moe_layer_desc* d, const moe_layer_weights* W, const void* x,
                       const void* y) {
    if (!d || !W || !x || !y) return MOE_EINVAL;
    if (!dt_ok(d->dtype)) return MOE_EDTYPE;
    if (d->T < 0 || d->D <= 0 || d->L < 0 || d->H <= 0) return MOE_ESHAPE;
    if (d->E < 1 || d->E > 512 || d->k < 1 || d->k > 16 || d->k > d->E) return MOE_ESHAPE;
    if (d->n_shared < 0 || d->n_shared > 3 || (d->n_shared > 0 && d->Hs <= 0)) return MOE_ESHAPE;
    if (!width_ok(d->D, d->dtype) || (d->L > 0 && !width_ok(d->L, d->dtype)) ||
        !width_ok(d->H, d->dtype) || (d->n_shared > 0 && !width_ok(d->Hs, d->dtype)))
        return MOE_ESHAPE;
    {
        const int64_t de = d->L > 0 ? d->L : d->D;
        // the routed GEMM gathers its rows from the [T, de] expert input, and an
        // expert's weights span 2H rows
        if (!under4g(d->T + 1, de, d->dtype) || !under4g(2 * d->H + 1, de, d->dtype) ||
            !under4g(de + 1, d->H, d->dtype))
            return MOE_ESHAPE;
    }
    if (d->T * d->k >= ((int64_t)1 << 31)) return MOE_ESHAPE;
    if (!(d->eps >= 0.0f)) return MOE_EINVAL;
    if (!W->W_r || !W->W_gu || !W->W_d) return MOE_EINVAL;
    if (d->L > 0 && (!W->W_dn || !W->W_up)) return MOE_EINVAL;
    if (d->n_shared > 0 && (!W->W_gu_s || !W->W_d_s)) return MOE_EINVAL;
    const void* ptrs[] = {x, y, W->W_dn, W->norm_g, W->W_r, W->b_r, W->W_gu, W->W_d, W->W_up,
                          W->W_gu_s, W->W_d_s};
    for (const void* p : ptrs)
        if (p && !aligned16(p)) return MOE_EALIGN;
    return MOE_OK;
}

}  // namespace

extern "C" {

int moe_abi_version(void) { return kAbiVersion; }

const char* moe_status_str(moe_status s) {
    switch (s) {
        case MOE_OK: return "ok";
        case MOE_EINVAL: return "invalid argument";
        case MOE_ESHAPE: return "unsupported shape";
        case MOE_EDTYPE: return "unsupported dtype";
        case MOE_EALIGN: return "pointer not 16-byte aligned";
        case MOE_EWORKSPACE: return "workspace too small";
        case MOE_ELAUNCH: return "kernel launch failed";
    }
    return "unknown status";
}

// ---------------------------------------------------------------- route ----
moe_status moe_route(const void* h, moe_dtype h_dt, int64_t T, int64_t d_r, const float* norm_g,
                     float eps, int32_t apply_norm, const float* W_r, const float* b_r, int32_t E,
                     int32_t k, void* r_out, moe_dtype r_dt, float* logits_out, int32_t* topk_ids,
                     float* topk_w, moe_stream stream) {
    if (T < 0 || d_r < 32 || d_r % 16) return MOE_ESHAPE;
    if (E < 1 || E > 512 || k < 1 || k > 16 || k > E) return MOE_ESHAPE;
    if (!dt_ok(h_dt) || (r_out && !dt_ok(r_dt))) return MOE_EDTYPE;
    if (T > 0 && (!h || !W_r || !topk_ids || !topk_w)) return MOE_EINVAL;
    if (!(eps >= 0.0f)) return MOE_EINVAL;
    const void* ptrs[] = {h, norm_g, W_r, b_r, r_out, logits_out, topk_ids, topk_w};
    for (const void* p : ptrs)
        if (p && !aligned16(p)) return MOE_EALIGN;
    if (T == 0) return MOE_OK;
    MOE_TRY(launch_route(h, h_dt, T, d_r, norm_g, eps, apply_norm, W_r, b_r, E, k, r_out, r_dt,
                         logits_out, topk_ids, topk_w, hs(stream)));
    return MOE_OK;
}

// -------------------------------------------------------------- permute ----
size_t moe_permute_workspace_size(int64_t n_assign, int32_t E) {
    if (n_assign < 0 || E < 1) return 0;
    return permute_ws_bytes(n_assign, E);
}

moe_status moe_permute(const int32_t* ids, int64_t n_assign, int32_t E, int64_t capacity,
                       const void* src, moe_dtype dt, int64_t width, int32_t src_div, void* dst,
                       int64_t R_phys, int32_t* slot_row, int32_t* row_src, int32_t* counts,
                       int32_t* offsets, int64_t* n_dropped, void* ws, size_t ws_bytes,
                       moe_stream stream) {
    const moe_status st = permute_check(ids, n_assign, E, capacity, src, dt, width, src_div, dst,
                                        R_phys, slot_row, row_src, counts, offsets, n_dropped);
    if (st != MOE_OK) return st;
    if (ws && !aligned16(ws)) return MOE_EALIGN;
    if (!ws || ws_bytes < permute_ws_bytes(n_assign, E)) return MOE_EWORKSPACE;
    MOE_TRY(launch_permute(ids, n_assign, E, capacity, src, src ? esize(dt) : 0, width, src_div,
                           dst, R_phys, slot_row, row_src, counts, offsets, n_dropped, nullptr, 0,
                           ws, hs(stream)));
    return MOE_OK;
}

moe_status moe_permute_e4m3(const int32_t* ids, int64_t n_assign, int32_t E, int64_t capacity,
                            const void* src, moe_dtype dt, int64_t width, int32_t src_div,
                            uint8_t* dst, int64_t R_phys, int32_t* slot_row, int32_t* row_src,
                            int32_t* counts, int32_t* offsets, int64_t* n_dropped,
                            const float* scale, float* amax, void* ws, size_t ws_bytes,
                            moe_stream stream) {
    if (E < 1 || E > 1024) return MOE_ESHAPE;
    if (n_assign < 0 || n_assign >= ((int64_t)1 << 31) || R_phys < 0) return MOE_ESHAPE;
    const int64_t max_kept = capacity < 0 ? n_assign
                                          : (capacity * E < n_assign ? capacity * E : n_assign);
    if (R_phys < max_kept || R_phys >= ((int64_t)1 << 31)) return MOE_ESHAPE;
    if (!dt_ok(dt)) return MOE_EDTYPE;
    if (width <= 0 || width % 16 || src_div < 1) return MOE_ESHAPE;
    if (!counts || !offsets || !n_dropped || !src || !dst) return MOE_EINVAL;
    if (n_assign > 0 && (!ids || !slot_row)) return MOE_EINVAL;
    if (R_phys > 0 && !row_src) return MOE_EINVAL;
    const void* ptrs[] = {ids, src, dst, slot_row, row_src, counts, offsets, n_dropped, ws};
    for (const void* p : ptrs)
        if (p && !aligned16(p)) return MOE_EALIGN;
    if (!aligned4(scale) || !aligned4(amax)) return MOE_EALIGN;
    if (!ws || ws_bytes < permute_ws_bytes(n_assign, E)) return MOE_EWORKSPACE;
    MOE_TRY(launch_permute(ids, n_assign, E, capacity, src, esize(dt), width, src_div, dst,
                           R_phys, slot_row, row_src, counts, offsets, n_dropped, nullptr, 0, ws,
                           hs(stream), true, scale, amax));
    return MOE_OK;
}

// ------------------------------------------------ EP dispatch, sender side ----
size_t moe_dispatch_pack_workspace_size(int64_t n_assign, int32_t n_peers) {
    if (n_assign < 0 || n_peers < 1) return 0;
    return a256((size_t)(n_assign > 0 ? n_assign : 1) * 4) + permute_ws_bytes(n_assign, n_peers);
}

namespace {
moe_status dispatch_pack_impl(const int32_t* expert_ids, int64_t T, int32_t k, int32_t E,
                              int32_t n_peers, int64_t capacity_per_peer, const void* x,
                              moe_dtype dt, int64_t width, void* send_rows, int32_t* send_expert,
                              int64_t R_phys, int32_t* slot_row, int32_t* row_src,
                              int32_t* counts, int32_t* offsets, int64_t* n_dropped, void* ws,
                              size_t ws_bytes, moe_stream stream, bool e4m3, const float* scale,
                              float* amax) {
    if (T < 0 || k < 1 || k > 16) return MOE_ESHAPE;
    if (n_peers < 1 || n_peers > 1024 || E < n_peers || E % n_peers) return MOE_ESHAPE;
    const int64_t n = T * k;
    if (n >= ((int64_t)1 << 31) || R_phys < 0) return MOE_ESHAPE;
    const int64_t max_kept = capacity_per_peer < 0
                                 ? n
                                 : (capacity_per_peer * n_peers < n ? capacity_per_peer * n_peers
                                                                    : n);
    if (R_phys < max_kept || R_phys >= ((int64_t)1 << 31)) return MOE_ESHAPE;
    if (!dt_ok(dt)) return MOE_EDTYPE;
    if (width <= 0 || (width * (e4m3 ? 1 : esize(dt))) % 16) return MOE_ESHAPE;
    if (!aligned4(scale) || !aligned4(amax)) return MOE_EALIGN;
    if (!counts || !offsets || !n_dropped || !x || !send_rows) return MOE_EINVAL;
    if (n > 0 && (!expert_ids || !slot_row)) return MOE_EINVAL;
    if (R_phys > 0 && (!row_src || !send_expert)) return MOE_EINVAL;
    const void* ptrs[] = {expert_ids, x, send_rows, send_expert, slot_row, row_src, counts,
                          offsets, n_dropped, ws};
    for (const void* p : ptrs)
        if (p && !aligned16(p)) return MOE_EALIGN;
    if (!ws || ws_bytes < moe_dispatch_pack_workspace_size(n, n_peers)) return MOE_EWORKSPACE;
    const int epp = E / n_peers;
    hipStream_t s = hs(stream);
    int32_t* peer = (int32_t*)ws;
    void* pws = (char*)ws + a256((size_t)(n > 0 ? n : 1) * 4);
    MOE_TRY(launch_peer_of(expert_ids, n, epp, peer, s));
    MOE_TRY(launch_permute(peer, n, n_peers, capacity_per_peer, x, esize(dt), width, k, send_rows,
                           R_phys, slot_row, row_src, counts, offsets, n_dropped, nullptr, 0, pws,
                           s, e4m3, scale, amax));
    MOE_TRY(launch_payload_ids(expert_ids, row_src, offsets, n_peers, R_phys, epp, send_expert,
                               s));
    return MOE_OK;
}
}  // namespace

moe_status moe_dispatch_pack(const int32_t* expert_ids, int64_t T, int32_t k, int32_t E,
                             int32_t n_peers, int64_t capacity_per_peer, const void* x,
                             moe_dtype dt, int64_t width, void* send_rows, int32_t* send_expert,
                             int64_t R_phys, int32_t* slot_row, int32_t* row_src, int32_t* counts,
                             int32_t* offsets, int64_t* n_dropped, void* ws, size_t ws_bytes,
                             moe_stream stream) {
    return dispatch_pack_impl(expert_ids, T, k, E, n_peers, capacity_per_peer, x, dt, width,
                              send_rows, send_expert, R_phys, slot_row, row_src, counts, offsets,
                              n_dropped, ws, ws_bytes, stream, false, nullptr, nullptr);
}

moe_status moe_dispatch_pack_e4m3(const int32_t* expert_ids, int64_t T, int32_t k, int32_t E,
                                  int32_t n_peers, int64_t capacity_per_peer, const void* x,
                                  moe_dtype dt, int64_t width, uint8_t* send_rows,
                                  int32_t* send_expert, int64_t R_phys, int32_t* slot_row,
                                  int32_t* row_src, int32_t* counts, int32_t* offsets,
                                  int64_t* n_dropped, const float* scale, float* amax, void* ws,
                                  size_t ws_bytes, moe_stream stream) {
    return dispatch_pack_impl(expert_ids, T, k, E, n_peers, capacity_per_peer, x, dt, width,
                              send_rows, send_expert, R_phys, slot_row, row_src, counts, offsets,
                              n_dropped, ws, ws_bytes, stream, true, scale, amax);
}

// ---------------------------------------------------------- grouped FFN ----
size_t moe_grouped_ffn_workspace_size(int32_t E, int64_t R_phys, int64_t H, moe_dtype dt) {
    if (E < 1 || R_phys < 0 || H <= 0 || !dt_ok(dt)) return 0;
    Carver cv(nullptr);
    cv.take<int32_t>((size_t)(E + 1) * 4);
    cv.take<char>((size_t)R_phys * H * esize(dt));
    return cv.off;
}

moe_status moe_grouped_ffn(const void* X, const int32_t* offsets, int32_t E, int64_t R_phys,
                           const void* W_gu, const void* W_d, int64_t d, int64_t H, moe_dtype dt,
                           void* Y, void* ws, size_t ws_bytes, moe_stream stream) {
    if (E < 1 || E > 1024 || R_phys < 0 || R_phys >= ((int64_t)1 << 31)) return MOE_ESHAPE;
    if (!dt_ok(dt)) return MOE_EDTYPE;
    if (!width_ok(d, dt) || !width_ok(H, dt)) return MOE_ESHAPE;
    if (!under4g(2 * H + 1, d, dt) || !under4g(d + 1, H, dt)) return MOE_ESHAPE;
    if (!offsets || !W_gu || !W_d || (R_phys > 0 && (!X || !Y))) return MOE_EINVAL;
    const void* ptrs[] = {X, offsets, W_gu, W_d, Y, ws};
    for (const void* p : ptrs)
        if (p && !aligned16(p)) return MOE_EALIGN;
    const size_t need = moe_grouped_ffn_workspace_size(E, R_phys, H, dt);
    if (!ws || ws_bytes < need) return MOE_EWORKSPACE;
    Carver cv(ws);
    int32_t* tp = cv.take<int32_t>((size_t)(E + 1) * 4);
    void* h = cv.take<char>((size_t)R_phys * H * esize(dt));
    hipStream_t s = hs(stream);
    MOE_TRY(launch_tile_prefix(offsets, E, gemm_block_m(), tp, s));
    moe_status st = grouped_ffn_impl(X, d, nullptr, 1, 0, offsets, tp, E, R_phys, W_gu, W_d, d,
                                     H, dt, h, Y, s);
    if (st != MOE_OK) return st;
    return grouped_down_impl(h, offsets, tp, E, R_phys, W_d, d, H, dt, Y, s);
}

// ---------------------------------------------------- ragged dot forward ----
size_t moe_ragged_dot_workspace_size(int32_t E) {
    if (E < 1) return 0;
    return a256((size_t)(E + 1) * 4);
}

moe_status moe_ragged_dot(const void* X, const int32_t* offsets, int32_t E, int64_t R_phys,
                          const void* W, int64_t N, int64_t K, moe_dtype dt, void* Z,
                          moe_dtype z_dt, void* ws, size_t ws_bytes, moe_stream stream) {
    if (!dt_ok(dt) || (z_dt != dt && z_dt != MOE_F32)) return MOE_EDTYPE;
    moe_status st = check_ragged_dot(X, offsets, E, R_phys, W, N, K, dt, Z, z_dt, ws, ws_bytes);
    if (st != MOE_OK) return st;
    return ragged_dot_impl(X, offsets, E, R_phys, W, N, K, dt, nullptr, nullptr, Z,
                           z_dt == MOE_F32, (int32_t*)ws, hs(stream));
}

moe_status moe_ragged_dot_e4m3(const uint8_t* Xq, const int32_t* offsets, int32_t E,
                               int64_t R_phys, const uint8_t* Wq, int64_t N, int64_t K,
                               const float* scale_x, const float* scale_w, void* Z,
                               moe_dtype z_dt, void* ws, size_t ws_bytes, moe_stream stream) {
    if (z_dt != MOE_BF16 && z_dt != MOE_F32) return MOE_EDTYPE;
    if (!aligned4(scale_x) || !aligned4(scale_w)) return MOE_EALIGN;
    moe_status st = check_ragged_dot(Xq, offsets, E, R_phys, Wq, N, K, MOE_E4M3, Z, z_dt, ws,
                                     ws_bytes);
    if (st != MOE_OK) return st;
    return ragged_dot_impl(Xq, offsets, E, R_phys, Wq, N, K, MOE_E4M3, scale_x, scale_w, Z,
                           z_dt == MOE_F32, (int32_t*)ws, hs(stream));
}

moe_status moe_quantize_e4m3(const void* x, moe_dtype dt, int64_t n, const float* scale,
                             uint8_t* q, float* amax, moe_stream stream) {
    if (!dt_ok(dt)) return MOE_EDTYPE;
    if (n < 0) return MOE_ESHAPE;
    if (n > 0 && (!x || !q)) return MOE_EINVAL;
    if ((x && !aligned16(x)) || (q && !aligned16(q)) || !aligned4(amax) || !aligned4(scale))
        return MOE_EALIGN;
    MOE_TRY(launch_quantize_e4m3(x, dt, n, scale, q, amax, hs(stream)));
    return MOE_OK;
}

moe_status moe_swiglu_quantize_e4m3(const void* gu, moe_dtype dt, const int32_t* offsets,
                                    int32_t E, int64_t R_phys, int64_t H, const float* scale,
                                    uint8_t* hq, float* amax, moe_stream stream) {
    if (!dt_ok(dt)) return MOE_EDTYPE;
    if (E < 1 || E > 1024 || R_phys < 0 || H <= 0 || H % 16) return MOE_ESHAPE;
    if (R_phys * (H / 16) >= ((int64_t)1 << 31)) return MOE_ESHAPE;
    if (!offsets || (R_phys > 0 && (!gu || !hq))) return MOE_EINVAL;
    const void* ptrs[] = {gu, offsets, hq};
    for (const void* p : ptrs)
        if (p && !aligned16(p)) return MOE_EALIGN;
    if (!aligned4(amax) || !aligned4(scale)) return MOE_EALIGN;
    MOE_TRY(launch_swiglu_quantize_e4m3(gu, dt, offsets, E, R_phys, H, scale, hq, amax,
                                        hs(stream)));
    return MOE_OK;
}

size_t moe_grouped_ffn_e4m3_workspace_size(int32_t E, int64_t R_phys, int64_t H) {
    if (E < 1 || R_phys < 0 || H <= 0) return 0;
    Carver cv(nullptr);
    cv.take<int32_t>((size_t)(E + 1) * 4);
    cv.take<char>((size_t)R_phys * 2 * H * 2);      // [g | u] in bf16
    cv.take<char>((size_t)R_phys * H);              // h in E4M3
    return cv.off;
}

// The gated expert MLP on E4M3 operands: gate/up ragged dot (bf16 out), the
// activation fused with h's quantisation, down ragged dot.
moe_status moe_grouped_ffn_e4m3(const uint8_t* Xq, const int32_t* offsets, int32_t E,
                                int64_t R_phys, const uint8_t* W_gu_q, const uint8_t* W_d_q,
                                int64_t d, int64_t H, const float* scale_x,
                                const float* scale_gu, const float* scale_h,
                                const float* scale_d, void* Y, moe_dtype y_dt, float* amax_h,
                                void* ws, size_t ws_bytes, moe_stream stream) {
    if (E < 1 || E > 1024 || R_phys < 0 || R_phys >= ((int64_t)1 << 31)) return MOE_ESHAPE;
    if (y_dt != MOE_BF16 && y_dt != MOE_F32) return MOE_EDTYPE;
    if (!width_ok(d, MOE_E4M3) || !width_ok(H, MOE_E4M3)) return MOE_ESHAPE;
    if (!under4g(2 * H + 1, d, MOE_E4M3) || !under4g(d + 1, H, MOE_E4M3)) return MOE_ESHAPE;
    if (R_phys * (H / 16) >= ((int64_t)1 << 31)) return MOE_ESHAPE;
    if (!offsets || !W_gu_q || !W_d_q || (R_phys > 0 && (!Xq || !Y))) return MOE_EINVAL;
    const void* ptrs[] = {Xq, offsets, W_gu_q, W_d_q, Y, ws};
    for (const void* p : ptrs)
        if (p && !aligned16(p)) return MOE_EALIGN;
    if (!aligned4(amax_h) || !aligned4(scale_x) || !aligned4(scale_gu) || !aligned4(scale_h) ||
        !aligned4(scale_d))
        return MOE_EALIGN;
    if (!ws || ws_bytes < moe_grouped_ffn_e4m3_workspace_size(E, R_phys, H))
        return MOE_EWORKSPACE;
    Carver cv(ws);
    int32_t* tp = cv.take<int32_t>((size_t)(E + 1) * 4);
    void* gu = cv.take<char>((size_t)R_phys * 2 * H * 2);
    uint8_t* hq = cv.take<uint8_t>((size_t)R_phys * H);
    hipStream_t s = hs(stream);
    moe_status st = ragged_dot_impl(Xq, offsets, E, R_phys, W_gu_q, 2 * H, d, MOE_E4M3, scale_x,
                                    scale_gu, gu, false, tp, s);
    if (st != MOE_OK) return st;
    MOE_TRY(launch_swiglu_quantize_e4m3(gu, MOE_BF16, offsets, E, R_phys, H, scale_h, hq, amax_h,
                                        s));
    return ragged_dot_impl(hq, offsets, E, R_phys, W_d_q, d, H, MOE_E4M3, scale_h, scale_d, Y,
                           y_dt == MOE_F32, tp, s);
}

moe_status moe_fp8_scale_update(float* history, int32_t len, const float* amax, float* scale,
                                moe_stream stream) {
    if (len < 1 || len > 1024) return MOE_ESHAPE;
    if (!history || !amax || !scale) return MOE_EINVAL;
    if (!aligned4(history) || !aligned4(amax) || !aligned4(scale)) return MOE_EALIGN;
    MOE_TRY(launch_fp8_scale_update(history, len, amax, scale, hs(stream)));
    return MOE_OK;
}

// ------------------------------------------------- ragged dot backward ----
size_t moe_ragged_dot_dlhs_workspace_size(int32_t E) {
    if (E < 1) return 0;
    return a256((size_t)(E + 1) * 4);
}

moe_status moe_ragged_dot_dlhs(const void* dZ, const int32_t* offsets, int32_t E, int64_t R_phys,
                               const void* W, int64_t N, int64_t K, moe_dtype dt, void* dX,
                               void* ws, size_t ws_bytes, moe_stream stream) {
    if (E < 1 || E > 1024 || R_phys < 0 || R_phys >= ((int64_t)1 << 31)) return MOE_ESHAPE;
    if (!dt_ok(dt)) return MOE_EDTYPE;
    if (!width_ok(N, dt) || !width_ok(K, dt)) return MOE_ESHAPE;
    if (!under4g(gemm_block_m() + 1, N, dt) || !under4g(gemm_k_bytes() + 1, K, dt))
        return MOE_ESHAPE;
    if (!offsets || !W || (R_phys > 0 && (!dZ || !dX))) return MOE_EINVAL;
    const void* ptrs[] = {dZ, offsets, W, dX, ws};
    for (const void* p : ptrs)
        if (p && !aligned16(p)) return MOE_EALIGN;
    if (!ws || ws_bytes < moe_ragged_dot_dlhs_workspace_size(E)) return MOE_EWORKSPACE;
    int32_t* tp = (int32_t*)ws;
    hipStream_t s = hs(stream);
    MOE_TRY(launch_tile_prefix(offsets, E, gemm_block_m(), tp, s));
    return dlhs_impl(dZ, offsets, tp, E, R_phys, W, N, K, dt, EPI_STORE, dX, K, nullptr, nullptr,
                     s);
}

size_t moe_ragged_dot_drhs_workspace_size(int32_t E) {
    if (E < 1) return 0;
    return a256(9 * sizeof(int64_t));
}

moe_status moe_ragged_dot_drhs(const void* X, const void* dZ, const int32_t* offsets, int32_t E,
                               int64_t R_phys, int64_t N, int64_t K, moe_dtype dt, void* dW,
                               moe_dtype dw_dt, void* ws, size_t ws_bytes, moe_stream stream) {
    if (E < 1 || E > 1024 || R_phys < 0 || R_phys >= ((int64_t)1 << 31)) return MOE_ESHAPE;
    if (!dt_ok(dt) || (dw_dt != dt && dw_dt != MOE_F32)) return MOE_EDTYPE;
    if (!width_ok(N, dt) || !width_ok(K, dt)) return MOE_ESHAPE;
    if (!under4g(gemm_k_bytes() + 1, N, dt) || !under4g(gemm_k_bytes() + 1, K, dt))
        return MOE_ESHAPE;
    if (!offsets || !dW || (R_phys > 0 && (!X || !dZ))) return MOE_EINVAL;
    const void* ptrs[] = {X, dZ, offsets, dW, ws};
    for (const void* p : ptrs)
        if (p && !aligned16(p)) return MOE_EALIGN;
    if (!ws || ws_bytes < moe_ragged_dot_drhs_workspace_size(E)) return MOE_EWORKSPACE;
    return drhs_impl(X, dZ, offsets, E, N, K, dt, dW, dw_dt == MOE_F32 && dt != MOE_F32,
                     (int64_t*)ws, hs(stream));
}

// ---------------------------------------------------- grouped FFN backward ----
size_t moe_grouped_ffn_bwd_workspace_size(int32_t E, int64_t R_phys, int64_t H, moe_dtype dt) {
    if (E < 1 || R_phys < 0 || H <= 0 || !dt_ok(dt)) return 0;
    Carver cv(nullptr);
    cv.take<int32_t>((size_t)(E + 1) * 4);
    cv.take<char>((size_t)R_phys * 2 * H * 4);             // [g | u], float32
    cv.take<char>((size_t)R_phys * 2 * H * esize(dt));     // [dg | du]
    cv.take<char>((size_t)R_phys * H * esize(dt));         // h
    cv.take<int64_t>(2 * 9 * sizeof(int64_t));             // XCD splits of dW_d, dW_gu
    return cv.off;
}

moe_status moe_grouped_ffn_bwd(const void* X, const void* dY, const int32_t* offsets, int32_t E,
                               int64_t R_phys, const void* W_gu, const void* W_d, int64_t d,
                               int64_t H, moe_dtype dt, void* dX, void* dW_gu, void* dW_d,
                               moe_dtype dw_dt, void* ws, size_t ws_bytes, moe_stream stream) {
    if (E < 1 || E > 1024 || R_phys < 0 || R_phys >= ((int64_t)1 << 31)) return MOE_ESHAPE;
    if (!dt_ok(dt) || (dw_dt != dt && dw_dt != MOE_F32)) return MOE_EDTYPE;
    if (!width_ok(d, dt) || !width_ok(H, dt)) return MOE_ESHAPE;
    if (!under4g(2 * H + 1, d, dt) || !under4g(d + 1, H, dt) ||
        !under4g(gemm_block_m() + 1, 2 * H, dt))
        return MOE_ESHAPE;
    if (!offsets || !W_gu || !W_d || !dW_gu || !dW_d || (R_phys > 0 && (!X || !dY || !dX)))
        return MOE_EINVAL;
    const void* ptrs[] = {X, dY, offsets, W_gu, W_d, dX, dW_gu, dW_d, ws};
    for (const void* p : ptrs)
        if (p && !aligned16(p)) return MOE_EALIGN;
    const size_t need = moe_grouped_ffn_bwd_workspace_size(E, R_phys, H, dt);
    if (!ws || ws_bytes < need) return MOE_EWORKSPACE;
    Carver cv(ws);
    int32_t* tp = cv.take<int32_t>((size_t)(E + 1) * 4);
    void* gu = cv.take<char>((size_t)R_phys * 2 * H * 4);
    void* dgu = cv.take<char>((size_t)R_phys * 2 * H * esize(dt));
    void* h = cv.take<char>((size_t)R_phys * H * esize(dt));
    int64_t* split = cv.take<int64_t>(2 * 9 * sizeof(int64_t));
    hipStream_t s = hs(stream);
    const bool w32 = dw_dt == MOE_F32 && dt != MOE_F32;
    MOE_TRY(launch_tile_prefix(offsets, E, gemm_block_m(), tp, s));
    // 1. the forward's pre-activations [g | u] = X W_gu[e]^T, kept in float32:
    //    rounding them to bfloat16 as well as [dg | du] took the weight
    //    gradients past the bf16 bound on ordinary inputs
    {
        GemmParams p = gemm_base();
        p.group_m = grouped_group_m(R_phys, E);
        p.a_ahead = grouped_a_ahead(R_phys, E);
        p.offsets = offsets;
        p.tile_prefix = tp;
        p.G = E;
        p.b_group_rows = 2 * H;
        p.N = 2 * H;
        p.seg[0] = GemmSeg{X, d, W_gu, d, (int32_t)d};
        p.nseg = 1;
        p.C = gu;
        p.ldc = 2 * H;
        MOE_TRY(launch_gemm(p, dt, true, EPI_STORE,
                            grouped_tile_bound(R_phys, E, 2 * H, EPI_STORE), s));
    }
    // 2. dh = dY W_d[e]; the epilogue writes [dg | du] and h
    moe_status st = dlhs_impl(dY, offsets, tp, E, R_phys, W_d, d, H, dt, EPI_SWIGLU_BWD, dgu,
                              2 * H, gu, h, s);
    if (st != MOE_OK) return st;
    // 3. dW_d[e] = dY[rows]^T h[rows]
    st = drhs_impl(h, dY, offsets, E, d, H, dt, dW_d, w32, split, s);
    if (st != MOE_OK) return st;
    // 4. dX = [dg | du] W_gu[e]
    st = dlhs_impl(dgu, offsets, tp, E, R_phys, W_gu, 2 * H, d, dt, EPI_STORE, dX, d, nullptr,
                   nullptr, s);
    if (st != MOE_OK) return st;
    // 5. dW_gu[e] = [dg | du][rows]^T X[rows]
    return drhs_impl(X, dgu, offsets, E, 2 * H, d, dt, dW_gu, w32, split + 9, s);
}

// -------------------------------------------------------------- combine ----
moe_status moe_combine(const void* Y, moe_dtype dt, const int32_t* slot_row, const float* w,
                       int64_t T, int32_t k, int64_t width, void* out, int32_t flags,
                       moe_stream stream) {
    if (!dt_ok(dt)) return MOE_EDTYPE;
    if (T < 0 || k < 1 || k > 64 || width <= 0 || (width * esize(dt)) % 16) return MOE_ESHAPE;
    if (flags & ~MOE_COMBINE_KEEP_UNROUTED) return MOE_EINVAL;
    if (T > 0 && (!Y || !slot_row || !out)) return MOE_EINVAL;
    const void* ptrs[] = {Y, slot_row, w, out};
    for (const void* p : ptrs)
        if (p && !aligned16(p)) return MOE_EALIGN;
    MOE_TRY(launch_combine(Y, dt, slot_row, w, T, k, width, out, flags, hs(stream)));
    return MOE_OK;
}

// ----------------------------------------------------------- full layer ----
size_t moe_layer_workspace_size(const moe_layer_desc* d) {
    if (!d || d->T < 0 || d->E < 1 || d->k < 1 || !dt_ok(d->dtype)) return 0;
    size_t total = 0;
    carve_layer(d, nullptr, &total);
    return total;
}

moe_status moe_layer_workspace_layout(const moe_layer_desc* d, moe_layer_ws_layout* out) {
    if (!d || !out) return MOE_EINVAL;
    if (d->T < 0 || d->E < 1 || d->k < 1) return MOE_ESHAPE;
    if (!dt_ok(d->dtype)) return MOE_EDTYPE;
    // carve from a fake base of 0, so each pointer is its region's offset
    constexpr size_t kNone = ~(size_t)0;
    char* const base = (char*)(uintptr_t)4096;
    size_t total = 0;
    const LayerBufs b = carve_layer(d, base, &total);
    auto off = [&](const void* p) { return p ? (size_t)((const char*)p - base) : kNone; };
    out->z_pre = off(b.z_pre);
    out->z_e = off(b.z_e);
    out->row_src = off(b.row_src);
    out->h = off(b.h);
    out->Y = off(b.Y);
    // without a latent or shared experts the combine writes y itself
    out->c = (d->L == 0 && d->n_shared == 0) ? kNone : off(b.c);
    out->h_s = off(b.h_s);
    out->total = total;
    return MOE_OK;
}

moe_status moe_layer_fwd(const moe_layer_desc* d, const moe_layer_weights* W, const void* x,
                         void* y, const moe_layer_aux* aux, void* ws, size_t ws_bytes,
                         moe_stream stream) {
    moe_status st = check_layer(d, W, x, y);
    if (st != MOE_OK) return st;
    if (aux) {
        const void* ptrs[] = {aux->logits, aux->ids, aux->w, aux->counts, aux->offsets,
                              aux->n_dropped, aux->slot_row};
        for (const void* p : ptrs)
            if (p && !aligned16(p)) return MOE_EALIGN;
    }
    size_t need = 0;
    carve_layer(d, nullptr, &need);
    if (!ws || ws_bytes < need || !aligned16(ws)) return MOE_EWORKSPACE;
    if (d->T == 0) return MOE_OK;

    size_t dummy;
    LayerBufs b = carve_layer(d, ws, &dummy);
    hipStream_t s = hs(stream);
    const moe_dtype dt = d->dtype;
    const int64_t T = d->T, D = d->D, L = d->L, H = d->H, Hs = d->Hs;
    const int E = d->E, k = d->k, ns = d->n_shared;
    const int64_t R = T * k;
    const int64_t de = L > 0 ? L : D;
    const int es = esize(dt);
    float* logits = (aux && aux->logits) ? aux->logits : b.logits;
    int32_t* ids = (aux && aux->ids) ? aux->ids : b.ids;
    float* w = (aux && aux->w) ? aux->w : b.w;
    int32_t* counts = (aux && aux->counts) ? aux->counts : b.counts;
    int32_t* offsets = (aux && aux->offsets) ? aux->offsets : b.offsets;
    int64_t* n_dropped = (aux && aux->n_dropped) ? aux->n_dropped : b.n_dropped;
    int32_t* slot_row = (aux && aux->slot_row) ? aux->slot_row : b.slot_row;
    void** ev = (aux && aux->events) ? aux->events : nullptr;
    auto mark = [&](int i) -> bool {
        return !ev || hipEventRecord((hipEvent_t)ev[i], s) == hipSuccess;
    };

    if (!mark(MOE_EV_START)) return MOE_ELAUNCH;
    // 1. down-projection to the latent (float32 out, normalised by the router)
    if (L > 0) {
        GemmParams p = gemm_base();
        p.M = T;
        p.N = L;
        p.seg[0] = GemmSeg{x, D, W->W_dn, D, (int32_t)D};
        p.nseg = 1;
        p.C = b.z_pre;
        p.ldc = L;
        MOE_TRY(launch_gemm(p, dt, true, EPI_STORE, dense_tiles(T, L, EPI_STORE), s));
    }
    if (!mark(MOE_EV_DOWNPROJ)) return MOE_ELAUNCH;
    // 2. RMSNorm + router + top-k; the normalised latent is stored in dt for the experts
    const void* e_in = L > 0 ? b.z_e : x;
    MOE_TRY(launch_route(L > 0 ? (const void*)b.z_pre : x, L > 0 ? MOE_F32 : dt, T, de, W->norm_g,
                         d->eps, L > 0 ? 1 : 0, W->W_r, W->b_r, E, k, L > 0 ? b.z_e : nullptr, dt,
                         logits, ids, w, s));
    if (!mark(MOE_EV_ROUTE)) return MOE_ELAUNCH;
    // 3. group by expert (no row copy: the expert GEMM gathers its rows)
    MOE_TRY(launch_permute(ids, R, E, d->capacity, nullptr, 0, 0, 1, nullptr, R, slot_row,
                           b.row_src, counts, offsets, n_dropped, b.tile_prefix, gemm_block_m(),
                           b.perm_ws, s));
    if (!mark(MOE_EV_PERMUTE)) return MOE_ELAUNCH;
    // 4-5. routed experts
    st = grouped_ffn_impl(e_in, de, b.row_src, k, T, offsets, b.tile_prefix, E, R, W->W_gu,
                          W->W_d, de, H, dt, b.h, b.Y, s);
    if (st != MOE_OK) return st;
    if (!mark(MOE_EV_GEMM1)) return MOE_ELAUNCH;
    st = grouped_down_impl(b.h, offsets, b.tile_prefix, E, R, W->W_d, de, H, dt, b.Y, s);
    if (st != MOE_OK) return st;
    if (!mark(MOE_EV_GEMM2)) return MOE_ELAUNCH;
    // 6. ordered weighted combine (straight into y when nothing follows)
    const bool c_is_y = (L == 0 && ns == 0);
    MOE_TRY(launch_combine(b.Y, dt, slot_row, w, T, k, de, c_is_y ? y : b.c, 0, s));
    if (!mark(MOE_EV_COMBINE)) return MOE_ELAUNCH;
    // 7. shared experts' gate/up + SwiGLU, all shared experts in one GEMM
    if (ns > 0) {
        GemmParams p = gemm_base();
        p.M = T;
        p.N = ns * Hs;
        p.n_per = Hs;
        p.seg[0] = GemmSeg{x, D, W->W_gu_s, D, (int32_t)D};
        p.nseg = 1;
        p.C = b.h_s;
        p.ldc = ns * Hs;
        MOE_TRY(launch_gemm(p, dt, false, EPI_SWIGLU, dense_tiles(T, ns * Hs, EPI_SWIGLU), s));
    }
    if (!mark(MOE_EV_SHARED)) return MOE_ELAUNCH;
    // 8. y = c W_up^T + sum_i h_s,i W_d_s,i^T in one K-concatenated GEMM (one
    //    rounding of y); without a latent, y = c + shared part.
    if (!c_is_y) {
        GemmParams p = gemm_base();
        p.M = T;
        p.N = D;
        int nseg = 0;
        if (L > 0) p.seg[nseg++] = GemmSeg{b.c, L, W->W_up, L, (int32_t)L};
        for (int i = 0; i < ns; i++)
            p.seg[nseg++] = GemmSeg{(const char*)b.h_s + (size_t)i * Hs * es, ns * Hs,
                                    (const char*)W->W_d_s + (size_t)i * D * Hs * es, Hs,
                                    (int32_t)Hs};
        p.nseg = nseg;
        p.C = y;
        p.ldc = D;
        int epi = EPI_STORE;
        if (L == 0) {
            epi = EPI_ADD;
            p.addend = b.c;
            p.ld_add = D;
        }
        MOE_TRY(launch_gemm(p, dt, dt == MOE_F32, epi, dense_tiles(T, D, epi), s));
    }
    if (!mark(MOE_EV_OUTPUT)) return MOE_ELAUNCH;
    return MOE_OK;
}

}  // extern "C"
