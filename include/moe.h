/*
 * moe.h -- C ABI of the MI355X (gfx950) routed mixture-of-experts layer forward,
 * its expert backward and its fp8 expert path.
 *
 * The layer (Marin 535B-A23B: the half of a training run nobody usually shows
 * you, section "What is actually being trained"; Marin Begins Open Training of a
 * 535B-Parameter MoE Model, section 2 "How the Sparse Model Is Organized"):
 *   z   = RMSNorm(x W_dn^T) * g                 latent (optional)
 *   l   = z W_r^T + b_r                          router logits, float32
 *   ids = top-k of l; w = softmax(l) over all experts, renormalised over the k
 *   Y_a = W_d[e] (silu(W_g[e] z) * (W_u[e] z))   per kept assignment a = (t, j)
 *   c_t = sum_j w_tj Y_(t,j)                      ordered, dropped j contribute 0
 *   y   = c W_up^T + sum_i SwiGLU_i(x)            shared experts see every token
 *
 * Beside the forward, the grouped expert matmuls' backward (Marin: Week of April
 * 26th summary, the custom-VJP paragraph) and the expert MLP on OCP E4M3 operands
 * with per-tensor delayed scaling kept on the device (Marin: Week of July 6th
 * summary, the fp8 compute-lane paragraph), including the E4M3 permutation leg.
 *
 * Conventions for every entry point:
 *   - Pointers marked (device) are device memory on the current HIP device; the
 *     caller owns every buffer.  The library never allocates, frees or
 *     synchronises; all work is enqueued on `stream` (a hipStream_t, NULL = the
 *     null stream) in call order, and device-written outputs are valid once that
 *     stream has been synchronised.
 *   - Matrices are row-major and contiguous.  Projections use the [out, in]
 *     layout, so both operands of every product are contiguous along the
 *     reduction.  Pointers must be 16-byte aligned.
 *   - Every shape, dtype, alignment and workspace check runs on the host before
 *     anything is enqueued; a failed check returns an error code, enqueues
 *     nothing and writes nothing.  MOE_ELAUNCH reports a launch failure seen by
 *     hipGetLastError; faults inside a kernel surface at the caller's next sync.
 *   - The library keeps no mutable global state: calls on different streams or
 *     devices may run concurrently (a shared handle that hung under concurrent
 *     calls is reported in Marin: Week of July 6th summary, JaxPP paragraph).
 *   - Workspaces are scratch owned by the caller; their contents on entry do not
 *     matter and on return are unspecified.
 */
#ifndef MOE_H
#define MOE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    MOE_OK = 0,
    MOE_EINVAL = 1,     /* null pointer where one is required, bad flag */
    MOE_ESHAPE = 2,     /* a size out of range or not a supported multiple */
    MOE_EDTYPE = 3,     /* unsupported dtype combination */
    MOE_EALIGN = 4,     /* pointer not 16-byte aligned */
    MOE_EWORKSPACE = 5, /* workspace missing or smaller than required */
    MOE_ELAUNCH = 6     /* a kernel launch failed */
} moe_status;

/* MOE_E4M3 (OCP 8-bit E4M3) is taken only by the fp8 entry points below. */
typedef enum { MOE_F32 = 0, MOE_BF16 = 1, MOE_E4M3 = 2 } moe_dtype;

/* A hipStream_t, passed as an opaque pointer so that this header needs no HIP
 * headers.  NULL is the null stream. */
typedef void *moe_stream;

/* Version of this ABI (changes when a signature or struct changes). */
int moe_abi_version(void);

/* Name of a status code (static string). */
const char *moe_status_str(moe_status s);

/* ------------------------------------------------------------------ route -- */
/* Router: optional RMSNorm, float32 logits, top-k, routing weights.
 * Follows the spec's order: softmax over all E experts, keep the k largest,
 * renormalise them to sum to one.  The largest logits are the largest
 * probabilities, so selection is taken on the float32 logits: larger first,
 * equal values (+0 and -0 are equal) to the lower expert id, NaN below all.
 * Router weight and bias are free parameters (Marin 535B-A23B article, section
 * "The one knob nobody pinned"); a more accurate router changed top-8 for ~9%
 * of tokens there (section "What I'd take from it"), which is why the router is
 * float32 throughout.
 *   h          (device) [T, d_r] in h_dt (MOE_F32 or MOE_BF16)
 *   norm_g     (device) [d_r] float32 gain, NULL = ones; used if apply_norm
 *   apply_norm nonzero: r = h / sqrt(mean(h^2) + eps) * g, else r = h
 *   W_r        (device) [E, d_r] float32;  b_r (device) [E] float32 or NULL
 *   r_out      (device) [T, d_r] in r_dt, or NULL: the router input r, stored
 *   logits_out (device) [T, E] float32, or NULL
 *   topk_ids   (device) [T, k] int32: j-th best expert of token t
 *   topk_w     (device) [T, k] float32 routing weights
 * With logits_out given and E > 256 the router runs as two kernels (logits for
 * 64 tokens x half of the experts per workgroup, then top-k per token); topk_w then
 * carries each token's inverse RMS from the first to the second.
 * Limits: 1 <= E <= 512, 1 <= k <= min(E, 16), d_r a multiple of 16 and at
 * least 32, T >= 0. */
moe_status moe_route(const void *h, moe_dtype h_dt, int64_t T, int64_t d_r,
                     const float *norm_g, float eps, int32_t apply_norm,
                     const float *W_r, const float *b_r, int32_t E, int32_t k,
                     void *r_out, moe_dtype r_dt, float *logits_out,
                     int32_t *topk_ids, float *topk_w, moe_stream stream);

/* ---------------------------------------------------------------- permute -- */
/* Group assignments by expert (the rows each expert's GEMM reads).
 * Source: expert group boundaries passed to the grouped GEMM as cu_seqlens
 * (Marin 535B-A23B article, section "21% to 27% MFU without stopping the run");
 * fixed capacity with overflow dropped and reported separately (launch blog,
 * section 2); integer capacity so no buffer overflows by a row (Marin weekly
 * summary of September 14, hero-run engineering).
 *   ids       (device) [n_assign] int32 expert of assignment a (a = t*k + j, or a
 *             pool row); a negative id is padding and takes part in nothing.
 *   capacity  rows kept per expert, < 0 = unlimited.  The kept assignments of an
 *             expert are its first `capacity` in ascending a.
 *   src, dst  (device) optional row copy: dst[row(a)] = src[a / src_div], rows of
 *             `width` elements of dt.  Both NULL = no copy.
 *   R_phys    rows of dst / row_src; must be >= the kept rows (n_assign suffices)
 * Outputs (device): slot_row [n_assign] (row of a, -1 if padding or dropped),
 *   row_src [R_phys] (assignment in each row, -1 past the last kept row),
 *   counts [E] (before the capacity cut), offsets [E+1] (exclusive prefix sum of
 *   kept rows), n_dropped [1] int64.  Integer outputs are deterministic.
 *   ws        (device) workspace of moe_permute_workspace_size(n_assign, E) bytes.
 * Limits: 1 <= E <= 1024, 0 <= n_assign < 2^31. */
moe_status moe_permute(const int32_t *ids, int64_t n_assign, int32_t E, int64_t capacity,
                       const void *src, moe_dtype dt, int64_t width, int32_t src_div,
                       void *dst, int64_t R_phys, int32_t *slot_row, int32_t *row_src,
                       int32_t *counts, int32_t *offsets, int64_t *n_dropped,
                       void *ws, size_t ws_bytes, moe_stream stream);
size_t moe_permute_workspace_size(int64_t n_assign, int32_t E);

/* moe_permute_noalloc: moe_permute for callers that cannot allocate device memory
 * (code under HIP graph capture, tight serving loops, harnesses that forbid
 * allocation), so cannot provide a workspace.  Arguments, outputs, limits and errors
 * are moe_permute's, without ws and ws_bytes: the scratch of the grouping passes
 * lives in a device array inside the library, MOE_PERMUTE_NOALLOC_SCRATCH_BYTES
 * (16 MiB) on each device, held until the process ends.  It serves every (n_assign,
 * E) with moe_permute_workspace_size(n_assign, E) <= that size (for example
 * 1,048,576 assignments over up to 768 experts); larger sizes return
 * MOE_EWORKSPACE and enqueue nothing.  The call allocates nothing; the first call on
 * a device looks up that device's copy of the array (host only) and returns
 * MOE_ELAUNCH if that fails.  Every call on a device shares its copy, which keeps
 * the last call's contents: calls that overlap on one device (on different streams,
 * or from several threads without ordering) race, so order them on one stream. */
#define MOE_PERMUTE_NOALLOC_SCRATCH_BYTES ((size_t)16 << 20)
moe_status moe_permute_noalloc(const int32_t *ids, int64_t n_assign, int32_t E,
                               int64_t capacity, const void *src, moe_dtype dt, int64_t width,
                               int32_t src_div, void *dst, int64_t R_phys, int32_t *slot_row,
                               int32_t *row_src, int32_t *counts, int32_t *offsets,
                               int64_t *n_dropped, moe_stream stream);

/* ------------------------------------------------------------ grouped FFN -- */
/* Per-expert gated MLP over contiguous row groups (the pages' ragged_dot with
 * group sizes: Marin: Week of April 26th summary; the gated expert MLP: Marin:
 * Week of July 6th summary, JaxPP paragraph).  Rows [offsets[e], offsets[e+1])
 * of X go through expert e:
 *   Y[r] = W_d[e] (silu(G) * U),  [G | U] = W_gu[e] X[r]
 * with G the first H rows of W_gu[e] and U the last H.  silu is computed with
 * an accurate exp and division (an approximate activation broke parity on the
 * pages).  Only active rows are computed; rows >= offsets[E] are not touched.
 *   X      (device) [R_phys, d] in dt;  offsets (device) [E+1] int32, ascending,
 *          offsets[0] = 0, offsets[E] <= R_phys
 *   W_gu   (device) [E, 2H, d];  W_d (device) [E, d, H]  (dt)
 *   Y      (device) [R_phys, d] in dt
 *   ws     (device) moe_grouped_ffn_workspace_size(E, R_phys, H, dt) bytes: the
 *          row-tile prefix ([E+1] int32, padded to 256 bytes), then the hidden
 *          h [R_phys, H] in dt (rows past offsets[E] unwritten), which the caller
 *          may read back once the stream has synchronised
 * Accumulation is float32; the hidden h is stored in dt.
 * Limits: d and H multiples of 64 for MOE_BF16 and of 32 for MOE_F32 (whole
 * 128-byte steps along each reduction), E <= 1024, and every expert's weight
 * matrix under 4 GiB; otherwise MOE_ESHAPE. */
moe_status moe_grouped_ffn(const void *X, const int32_t *offsets, int32_t E, int64_t R_phys,
                           const void *W_gu, const void *W_d, int64_t d, int64_t H,
                           moe_dtype dt, void *Y, void *ws, size_t ws_bytes, moe_stream stream);
size_t moe_grouped_ffn_workspace_size(int32_t E, int64_t R_phys, int64_t H, moe_dtype dt);

/* --------------------------------------------------- ragged dot forward -- */
/* The grouped matmul on its own (the pages' ragged_dot with group sizes: Marin:
 * Week of April 26th summary), in this library's output-major convention:
 *   Z[r] = W[e] X[r]  for the rows r of group e = [offsets[e], offsets[e+1]),
 *   X (device) [R_phys, K] dt;  W (device) [E, N, K] dt;  Z (device) [R_phys, N] in
 *   z_dt (dt or MOE_F32).  Rows >= offsets[E] of Z are not touched.
 *   ws (device) moe_ragged_dot_workspace_size(E) bytes (the row-tile prefix).
 * Accumulation is float32.  Limits: K a multiple of 64 for MOE_BF16 and of 32 for
 * MOE_F32, N a multiple of 64, 1 <= E <= 1024, each expert's matrix under 4 GiB. */
moe_status moe_ragged_dot(const void *X, const int32_t *offsets, int32_t E, int64_t R_phys,
                          const void *W, int64_t N, int64_t K, moe_dtype dt, void *Z,
                          moe_dtype z_dt, void *ws, size_t ws_bytes, moe_stream stream);
size_t moe_ragged_dot_workspace_size(int32_t E);

/* -------------------------------------------------------------------- fp8 -- */
/* OCP E4M3 operands for the expert GEMMs (Marin: Week of July 6th summary, the fp8
 * compute-lane paragraph: fp8 ragged dots, E4M3 in the forward, delayed scaling).
 * E4M3: sign, 4 exponent bits with bias 7, 3 mantissa bits, no infinity,
 * S.1111.111 = NaN, largest finite magnitude 448.
 *
 * Scales are per tensor and live in device memory, so that a training loop keeps its
 * delayed-scaling state on the GPU and never waits for the host.  A scale s is a
 * dequantisation scale: a code c stands for s * E4M3(c).  Every scale pointer below
 * is a device float (4-byte aligned); NULL means s = 1.
 *
 * moe_quantize_e4m3:  q[i] = E4M3(x[i] * inv), inv = 1 / scale[0] rounded to float32,
 *   the product rounded to float32 first, then the nearest code with ties to the even
 *   mantissa; magnitudes of 464 and up (and infinities) saturate to 448, NaN becomes
 *   0x7F.  amax (device, nullable) receives max |x[i]| (NaN ignored), the value the
 *   delayed-scaling history records.  x (device) [n] in dt (MOE_F32 or MOE_BF16);
 *   q (device) [n] bytes.  No workspace.
 * moe_ragged_dot_e4m3:  Z[r] = (scale_x[0] * scale_w[0]) * W[e] X[r] with X [R_phys, K]
 *   and W [E, N, K] as E4M3 codes (the product of the scales rounded to float32); the
 *   fp8 matrix instruction sums each run of 64 products below float32 precision
 *   (measured: within 2^-14 of the sum of their magnitudes), the runs accumulate in
 *   float32, then the scale is applied; Z in z_dt (MOE_BF16 or MOE_F32), rows >=
 *   offsets[E] untouched.  ws as moe_ragged_dot.  Limits: K a multiple of 128, N a
 *   multiple of 64, 1 <= E <= 1024.
 * moe_swiglu_quantize_e4m3:  the expert MLP's gated activation (the JaxPP paragraph of
 *   the same summary: SwiGLU with the exact activation) quantised for an E4M3 down
 *   projection.  For the rows r < offsets[E] (at most R_phys) of gu = [g | u] (device,
 *   [R_phys, 2H] in dt, gate columns first):
 *     h = silu(g) u in float32,  hq[r, c] = E4M3(h * inv) as moe_quantize_e4m3 with
 *     scale,  amax (device, nullable) = max |h|.
 *   hq (device) [R_phys, H]; its rows past offsets[E] are not touched.
 *   Limits: H a multiple of 16, R_phys * H / 16 < 2^31.  No workspace.
 * moe_grouped_ffn_e4m3:  the gated expert MLP with E4M3 operands in both ragged dots
 *   (the same paragraph: the fp8 ragged dots threaded through the expert MLP), for the
 *   rows of group e = [offsets[e], offsets[e+1]):
 *     [g | u] = (scale_x[0] * scale_gu[0]) * W_gu_q[e] Xq[r], stored in bf16 (workspace);
 *     hq = moe_swiglu_quantize_e4m3([g | u], scale_h), amax_h = max |h|;
 *     Y[r] = (scale_h[0] * scale_d[0]) * W_d_q[e] hq[r]  in y_dt (MOE_BF16 or MOE_F32).
 *   Xq [R_phys, d], W_gu_q [E, 2H, d], W_d_q [E, d, H] E4M3 codes (device); scale_x,
 *   scale_gu, scale_d the scales they were quantised with; scale_h the scale for h
 *   (from earlier steps' amax_h: delayed scaling).  Rows >= offsets[E] of Y are not
 *   touched.  ws (device) moe_grouped_ffn_e4m3_workspace_size(E, R_phys, H) bytes.
 *   Limits: d and H multiples of 128, 1 <= E <= 1024.  Accumulation as
 *   moe_ragged_dot_e4m3.
 * moe_fp8_scale_update:  delayed scaling's state update for one tensor.  history
 *   (device float [len], in/out) holds the amax of the last len steps, newest first;
 *   it is shifted by one with amax[0] (device) in front, and scale[0] (device, out)
 *   becomes m / 448 for m the largest finite entry (the value that maps to E4M3's
 *   largest code), or 1 when m is 0.  1 <= len <= 1024.
 * Pointers 16-byte aligned unless stated; nothing is allocated; calls on one stream
 * run in order, so a scale written by moe_fp8_scale_update is the one the next
 * call on that stream reads. */
moe_status moe_quantize_e4m3(const void *x, moe_dtype dt, int64_t n, const float *scale,
                             uint8_t *q, float *amax, moe_stream stream);
moe_status moe_ragged_dot_e4m3(const uint8_t *Xq, const int32_t *offsets, int32_t E,
                               int64_t R_phys, const uint8_t *Wq, int64_t N, int64_t K,
                               const float *scale_x, const float *scale_w, void *Z,
                               moe_dtype z_dt, void *ws, size_t ws_bytes, moe_stream stream);
moe_status moe_swiglu_quantize_e4m3(const void *gu, moe_dtype dt, const int32_t *offsets,
                                    int32_t E, int64_t R_phys, int64_t H, const float *scale,
                                    uint8_t *hq, float *amax, moe_stream stream);
moe_status moe_grouped_ffn_e4m3(const uint8_t *Xq, const int32_t *offsets, int32_t E,
                                int64_t R_phys, const uint8_t *W_gu_q, const uint8_t *W_d_q,
                                int64_t d, int64_t H, const float *scale_x,
                                const float *scale_gu, const float *scale_h,
                                const float *scale_d, void *Y, moe_dtype y_dt, float *amax_h,
                                void *ws, size_t ws_bytes, moe_stream stream);
size_t moe_grouped_ffn_e4m3_workspace_size(int32_t E, int64_t R_phys, int64_t H);
moe_status moe_fp8_scale_update(float *history, int32_t len, const float *amax, float *scale,
                                moe_stream stream);

/* moe_dispatch_pack:  the sender's half of the expert-parallel dispatch (Marin Begins
 *   Open Training of a 535B-Parameter MoE Model, section 2: routed rows travel to the
 *   GPU that owns their expert, with the expert id carried beside the row and a
 *   sender-side capacity; the exchange itself needs the peers and is not here).
 *   Experts are dealt to n_peers peers in contiguous blocks of epp = E / n_peers.  The
 *   T*k assignments expert_ids [T, k] (device, int32, -1 = none) are grouped by peer as
 *   moe_permute groups them by expert (ids / epp), with capacity_per_peer (-1 = none):
 *   counts, offsets [n_peers + 1], slot_row, row_src and n_dropped as there; each kept
 *   row r < offsets[n_peers] of send_rows (device, [R_phys, width] in dt) is token
 *   row_src[r] / k of x (device, [T, width] in dt), and send_expert[r] (device, int32
 *   [R_phys]) is its expert's local id, expert_ids[row_src[r]] % epp (-1 past the kept
 *   rows): the payload a receiver groups by.  ws (device)
 *   moe_dispatch_pack_workspace_size(T * k, n_peers) bytes.  Limits: E a multiple of
 *   n_peers, 1 <= n_peers <= 1024, k <= 16, width * element size a multiple of 16. */
moe_status moe_dispatch_pack(const int32_t *expert_ids, int64_t T, int32_t k, int32_t E,
                             int32_t n_peers, int64_t capacity_per_peer, const void *x,
                             moe_dtype dt, int64_t width, void *send_rows, int32_t *send_expert,
                             int64_t R_phys, int32_t *slot_row, int32_t *row_src, int32_t *counts,
                             int32_t *offsets, int64_t *n_dropped, void *ws, size_t ws_bytes,
                             moe_stream stream);
size_t moe_dispatch_pack_workspace_size(int64_t n_assign, int32_t n_peers);
/* moe_dispatch_pack_e4m3:  moe_dispatch_pack with the rows sent as E4M3 codes, the fp8
 *   wire format of the forward's permutation leg (Marin: Week of July 6th summary, the
 *   fp8 compute-lane paragraph: E4M3 forward on the permutation legs): send_rows
 *   (device, [R_phys, width] bytes) holds E4M3(x / scale[0]) as moe_quantize_e4m3
 *   converts, and amax (device, nullable) max |x| over the token rows sent.  scale is a
 *   device float (NULL = 1).  Limits as moe_dispatch_pack, and width a multiple of 16. */
moe_status moe_dispatch_pack_e4m3(const int32_t *expert_ids, int64_t T, int32_t k, int32_t E,
                                  int32_t n_peers, int64_t capacity_per_peer, const void *x,
                                  moe_dtype dt, int64_t width, uint8_t *send_rows,
                                  int32_t *send_expert, int64_t R_phys, int32_t *slot_row,
                                  int32_t *row_src, int32_t *counts, int32_t *offsets,
                                  int64_t *n_dropped, const float *scale, float *amax, void *ws,
                                  size_t ws_bytes, moe_stream stream);

/* moe_permute_e4m3:  moe_permute whose row copy writes E4M3 codes: the grouping
 *   outputs exactly as moe_permute's, and dst[r] = E4M3(src[row_src[r] / src_div] * inv)
 *   for r < offsets[E] as moe_quantize_e4m3 converts (inv = 1 / scale[0]), so the rows
 *   enter the E4M3 expert MLP already quantised: the local part of the fp8
 *   permutation leg (Marin: Week of July 6th summary, the fp8 compute-lane paragraph:
 *   E4M3 in the forward on the permutation legs).  amax (device, nullable) receives
 *   max |x| over the source rows read, those with at least one kept assignment.
 *   src (device) [n_src, width] in dt (MOE_F32 or MOE_BF16); dst (device) [R_phys,
 *   width] bytes.  Limits as moe_permute, and width a multiple of 16. */
moe_status moe_permute_e4m3(const int32_t *ids, int64_t n_assign, int32_t E, int64_t capacity,
                            const void *src, moe_dtype dt, int64_t width, int32_t src_div,
                            uint8_t *dst, int64_t R_phys, int32_t *slot_row, int32_t *row_src,
                            int32_t *counts, int32_t *offsets, int64_t *n_dropped,
                            const float *scale, float *amax, void *ws, size_t ws_bytes,
                            moe_stream stream);

/* ------------------------------------------------------- ragged dot VJP -- */
/* Backward of the grouped matmul (the pages' ragged_dot), split as the pages
 * split their custom VJP (Marin: Week of April 26th summary, the paragraph on
 * moving the backward pass onto Triton): an input-gradient kernel with the
 * grouped right-hand side transposed and a separate ragged-contracting kernel
 * for the weight gradient.  The forward convention is this library's:
 *   Z[r] = W[e] X[r]  for the rows r of group e = [offsets[e], offsets[e+1]),
 *   X [R_phys, K], W [E, N, K] (each group's matrix output-major), Z [R_phys, N].
 * Accumulation is float32.
 *
 * moe_ragged_dot_dlhs:  dX[r] = W[e]^T dZ[r], i.e. dX[r, k] = sum_n dZ[r, n] W[e][n, k]
 *   dZ (device) [R_phys, N] dt;  W (device) [E, N, K] dt;  dX (device) [R_phys, K] dt.
 *   Rows >= offsets[E] of dX are not touched.
 *   ws (device) moe_ragged_dot_dlhs_workspace_size(E) bytes (the row-tile prefix).
 * moe_ragged_dot_drhs:  dW[e] = sum over the rows r of group e of dZ[r] X[r]^T
 *   X (device) [R_phys, K] dt;  dZ (device) [R_phys, N] dt;  dW (device) [E, N, K]
 *   in dw_dt (dt or MOE_F32).  An empty group's dW[e] is written as zeros.
 *   ws (device) moe_ragged_dot_drhs_workspace_size(E) bytes (the XCD tile ranges,
 *   balanced by each group's row count).
 * Both: offsets (device) [E+1] int32 ascending, offsets[0] = 0, offsets[E] <=
 * R_phys.  Limits: N and K multiples of 64 for MOE_BF16 and of 32 for MOE_F32,
 * 1 <= E <= 1024, R_phys < 2^31; otherwise MOE_ESHAPE.  Pointers 16-byte
 * aligned (MOE_EALIGN).  Nothing is allocated; work is enqueued on `stream`. */
moe_status moe_ragged_dot_dlhs(const void *dZ, const int32_t *offsets, int32_t E, int64_t R_phys,
                               const void *W, int64_t N, int64_t K, moe_dtype dt, void *dX,
                               void *ws, size_t ws_bytes, moe_stream stream);
size_t moe_ragged_dot_dlhs_workspace_size(int32_t E);
moe_status moe_ragged_dot_drhs(const void *X, const void *dZ, const int32_t *offsets, int32_t E,
                               int64_t R_phys, int64_t N, int64_t K, moe_dtype dt, void *dW,
                               moe_dtype dw_dt, void *ws, size_t ws_bytes, moe_stream stream);
size_t moe_ragged_dot_drhs_workspace_size(int32_t E);

/* Backward of moe_grouped_ffn (the gated expert MLP over row groups; the same
 * VJP pieces as above, chained through SwiGLU's derivative).  Given the
 * gradient dY of Y:
 *   [g | u] = W_gu[e] x  (recomputed),  h = silu(g) u,  dh = W_d[e]^T dy,
 *   dg = dh u silu'(g),  du = dh silu(g),  silu'(g) = s (1 + g (1 - s)), s = sigmoid(g),
 *   dx = W_gu[e]^T [dg | du],  dW_d[e] = sum dy h^T,  dW_gu[e] = sum [dg | du] x^T.
 *   X, dY (device) [R_phys, d] dt;  W_gu [E, 2H, d], W_d [E, d, H] (dt).
 *   dX (device) [R_phys, d] dt (rows >= offsets[E] not touched);  dW_gu [E, 2H, d]
 *   and dW_d [E, d, H] in dw_dt (dt or MOE_F32); empty groups get zeros.
 *   ws (device) moe_grouped_ffn_bwd_workspace_size(E, R_phys, H, dt) bytes: holds
 *   [g | u] in float32 and [dg | du] and h in dt (both are operands of the
 *   weight-gradient and input-gradient GEMMs, so they are rounded to dt), and the
 *   weight-gradient GEMMs' XCD tile ranges.
 * Limits as moe_grouped_ffn. */
moe_status moe_grouped_ffn_bwd(const void *X, const void *dY, const int32_t *offsets, int32_t E,
                               int64_t R_phys, const void *W_gu, const void *W_d, int64_t d,
                               int64_t H, moe_dtype dt, void *dX, void *dW_gu, void *dW_d,
                               moe_dtype dw_dt, void *ws, size_t ws_bytes, moe_stream stream);
size_t moe_grouped_ffn_bwd_workspace_size(int32_t E, int64_t R_phys, int64_t H, moe_dtype dt);

/* ---------------------------------------------------------------- combine -- */
/* Ordered weighted gather (Marin weekly summary of September 14: an ordered
 * gather replaced an atomic scatter-add so repeated scoring is bitwise exact):
 *   out[t] = sum over j = 0..k-1 in order of w[t*k+j] * Y[slot_row[t*k+j]],
 * skipping slots < 0 (a dropped assignment contributes zero; the others are not
 * renormalised -- launch blog, section 4).  float32 accumulation.
 *   Y (device) [*, width] dt;  slot_row (device) [T*k];  w (device) [T*k] float32
 *   or NULL (weights 1);  out (device) [T, width] dt.
 *   flags: MOE_COMBINE_KEEP_UNROUTED leaves out[t] untouched when every slot of t
 *   is < 0 (unpermute of a receiver pool whose padding rows must survive);
 *   otherwise such a row is written as zeros. */
#define MOE_COMBINE_KEEP_UNROUTED 1
moe_status moe_combine(const void *Y, moe_dtype dt, const int32_t *slot_row, const float *w,
                       int64_t T, int32_t k, int64_t width, void *out, int32_t flags,
                       moe_stream stream);

/* ------------------------------------------------------------ full layer -- */
typedef struct {
    int64_t T;          /* tokens */
    int64_t D;          /* model width */
    int64_t L;          /* latent width; 0 = no latent (routing and experts act on x) */
    int32_t E;          /* routed experts */
    int32_t k;          /* experts per token */
    int64_t H;          /* routed expert hidden width */
    int32_t n_shared;   /* shared experts (0..3) */
    int64_t Hs;         /* shared expert hidden width */
    moe_dtype dtype;    /* storage of x, weights, intermediates and y */
    float eps;          /* RMSNorm epsilon */
    int64_t capacity;   /* rows kept per expert, < 0 = unlimited (dropless) */
} moe_layer_desc;

typedef struct {
    const void *W_dn;    /* [L, D] dtype (latent only) */
    const float *norm_g; /* [L] float32 or NULL = ones (latent only) */
    const float *W_r;    /* [E, d_r] float32, d_r = L or D */
    const float *b_r;    /* [E] float32 or NULL */
    const void *W_gu;    /* [E, 2H, d_e] dtype, d_e = L or D; gate rows then up rows */
    const void *W_d;     /* [E, d_e, H] dtype */
    const void *W_up;    /* [D, L] dtype (latent only) */
    const void *W_gu_s;  /* [n_shared, 2Hs, D] dtype */
    const void *W_d_s;   /* [n_shared, D, Hs] dtype */
} moe_layer_weights;

/* Stage boundaries at which moe_layer_fwd records caller-supplied events. */
enum {
    MOE_EV_START = 0,      /* before the first kernel */
    MOE_EV_DOWNPROJ = 1,   /* after x W_dn^T */
    MOE_EV_ROUTE = 2,      /* after RMSNorm + router + top-k */
    MOE_EV_PERMUTE = 3,    /* after grouping */
    MOE_EV_GEMM1 = 4,      /* after gate/up + SwiGLU */
    MOE_EV_GEMM2 = 5,      /* after the down projection of the experts */
    MOE_EV_COMBINE = 6,    /* after the weighted combine */
    MOE_EV_SHARED = 7,     /* after the shared experts' gate/up + SwiGLU */
    MOE_EV_OUTPUT = 8,     /* after up-projection + shared down (the output) */
    MOE_EV_COUNT = 9
};

typedef struct {
    float *logits;        /* [T, E] or NULL */
    int32_t *ids;         /* [T, k] or NULL */
    float *w;             /* [T, k] or NULL */
    int32_t *counts;      /* [E] or NULL */
    int32_t *offsets;     /* [E+1] or NULL */
    int64_t *n_dropped;   /* [1] or NULL */
    int32_t *slot_row;    /* [T*k] or NULL */
    void **events;        /* MOE_EV_COUNT hipEvent_t handles, or NULL: each is
                             recorded on `stream` at its stage boundary (timing) */
} moe_layer_aux;

/* The whole layer forward.  x (device) [T, D] dtype -> y (device) [T, D] dtype.
 * aux may be NULL; each of its pointers may be NULL.  ws: device workspace of
 * moe_layer_workspace_size(d) bytes.  Limits: those of the parts, plus D, L, H,
 * Hs multiples of 64 for MOE_BF16 and of 32 for MOE_F32, n_shared <= 3, and the
 * expert input [T, L] (or [T, D] without a latent) under 4 GiB; otherwise
 * MOE_ESHAPE. */
moe_status moe_layer_fwd(const moe_layer_desc *d, const moe_layer_weights *W, const void *x,
                         void *y, const moe_layer_aux *aux, void *ws, size_t ws_bytes,
                         moe_stream stream);
size_t moe_layer_workspace_size(const moe_layer_desc *d);

/* Where moe_layer_fwd keeps its intermediate stages inside ws, as byte offsets
 * from ws (SIZE_MAX where the configuration has no such stage), so that a
 * caller can read each stage back after the stream has synchronised (the
 * per-kernel parity checks do).  Valid for calls with the same desc; the
 * contents are those of the last call that used the workspace.
 *   z_pre   [T, L] float32    latent before RMSNorm (latent only)
 *   z_e     [T, L] dtype      normalised latent: the routed experts' input
 *                             (latent only; without one they read x)
 *   row_src [T*k] int32       assignment a = t*k + j held by each grouped row
 *   h       [T*k, H] dtype    routed experts' hidden silu(G) * U, rows grouped
 *                             by expert as offsets says (rows past offsets[E]
 *                             hold nothing)
 *   Y       [T*k, d_e] dtype  routed experts' outputs, the same rows
 *   c       [T, d_e] dtype    the ordered weighted combine (SIZE_MAX when there
 *                             is neither a latent nor a shared expert: the
 *                             combine then writes y)
 *   h_s     [T, n_shared*Hs] dtype  the shared experts' hidden, expert i in
 *                             columns [i Hs, (i + 1) Hs)
 *   total   moe_layer_workspace_size(d)
 * The ids, weights, counts, offsets, n_dropped and slot_row are read through
 * moe_layer_aux instead.  Host only; returns MOE_EINVAL for a NULL argument,
 * MOE_ESHAPE / MOE_EDTYPE for a desc moe_layer_workspace_size rejects. */
typedef struct {
    size_t z_pre, z_e, row_src, h, Y, c, h_s;
    size_t total;
} moe_layer_ws_layout;
moe_status moe_layer_workspace_layout(const moe_layer_desc *d, moe_layer_ws_layout *out);

#ifdef __cplusplus
}
#endif
#endif /* MOE_H */
