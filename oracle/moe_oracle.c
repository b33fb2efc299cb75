/*
 * moe_oracle.c -- plain, slow, obviously-correct CPU oracle for the forward pass
 * of one routed mixture-of-experts layer, and for the backward of its grouped
 * expert matmuls and gated expert MLP.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
 * benchmark's CPU-baseline leg may load this library.  The GPU library never
 * includes, links or calls anything in this directory, and this file includes
 * nothing from the GPU library.
 *
 * Arithmetic: every sum and product is done in IEEE double, in the order the
 * loops below state (no blocking, no reordering, no fused multiply-add: build
 * with -ffp-contract=off).  Storage roundings to bfloat16 / float32 are applied
 * exactly where the layer stores a tensor in that precision, using the
 * round-to-nearest-even rule implemented below from its definition.
 *
 * What the layer computes (sources):
 *   - Marin 535B-A23B: the half of a training run nobody usually shows you,
 *     section "What is actually being trained": a 6,144-wide token is projected
 *     to a 3,072-wide latent, normalised, sent to 8 of 384 routed experts,
 *     weighted-combined, projected back up; two shared experts see every token.
 *   - Marin Begins Open Training of a 535B-Parameter MoE Model, section 2
 *     "How the Sparse Model Is Organized": the up-projected routed output is
 *     added to the shared-expert path; capacity overflow is dropped and counted.
 *   - same page, section 4: a dropped assignment skips only that expert; the
 *     shared experts still process the token.
 *   - Marin 535B-A23B article, section "The one knob nobody pinned": the router
 *     has a weight and a bias (both free parameters).
 *   - Marin: Week of July 6th summary, JaxPP paragraph: the expert MLP is gated
 *     (SwiGLU) and an approximate activation broke parity, so the activation here
 *     is the exact silu(v) = v / (1 + exp(-v)).
 *   - Marin weekly summary of September 14 (post-training section): the combine
 *     is an ordered gather, summed in a fixed order, not an atomic scatter-add.
 *   - same summary (hero-run engineering): capacity is an integer computation
 *     so that it can never exceed the buffer by a row.
 *   - Marin: Week of July 6th summary, the fp8 compute-lane paragraph: fp8 ragged
 *     dots with E4M3 in the forward and delayed (per-tensor, history-based)
 *     scaling.
 *   - Marin: Week of April 26th summary, the paragraph on moving the backward
 *     pass onto Triton: the grouped matmul's backward is an input-gradient
 *     grouped GEMM against the transposed weights plus a ragged-contracting
 *     weight-gradient GEMM.
 * Readings where the pages are silent (router input, tie rule, capacity rounding,
 * gate/up halves, eps) are stated next to the function that takes them.
 *
 * Parity status: every exported function is pinned by CPU tests against
 * closed forms, brute force and library routines (see tests/test_oracle_*.py).
 */
#include <math.h>
#include <omp.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define DT_F32 0
#define DT_BF16 1

/* Threads the parallel loops below use (timing plumbing for the CPU baseline;
 * results do not depend on it: each loop iteration writes its own outputs). */
void moe_ref_set_threads(int n)
{
    omp_set_num_threads(n > 0 ? n : 1);
}

int moe_ref_max_threads(void)
{
    return omp_get_max_threads();
}

/* ---------------------------------------------------------------- storage --- */

/* bfloat16 bits -> exact value.  A bfloat16 is the upper half of a float32. */
static double bf16_val(uint16_t b)
{
    uint32_t u = (uint32_t)b << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

/* Round a double to the nearest bfloat16, ties to even, straight from the
 * double (no intermediate float).  bfloat16 has an 8-bit significand and the
 * float32 exponent range; below 2^-126 the quantum is fixed at 2^-133. */
uint16_t moe_ref_to_bf16(double x)
{
    if (isnan(x))
        return 0x7FC0;
    int neg = signbit(x) ? 1 : 0;
    double a = fabs(x);
    if (isinf(a) || a == 0.0) {
        uint16_t mag = isinf(a) ? 0x7F80 : 0x0000;
        return (uint16_t)(mag | (neg << 15));
    }
    int e;
    (void)frexp(a, &e);               /* a = m * 2^e, m in [0.5, 1) */
    int qe = e - 8;                   /* quantum exponent of an 8-bit significand */
    if (qe < -133)
        qe = -133;                    /* subnormal range */
    double q = ldexp(a, -qe);         /* exact: a power-of-two scaling */
    double r = nearbyint(q);          /* current rounding mode = to nearest, ties even */
    double v = ldexp(r, qe);
    uint16_t out;
    if (v >= 0x1p128) {
        out = 0x7F80;                 /* overflow to infinity */
    } else {
        float f = (float)v;           /* exact: v has at most 8 significant bits */
        uint32_t u;
        memcpy(&u, &f, sizeof u);
        out = (uint16_t)(u >> 16);
    }
    return (uint16_t)(out | (neg << 15));
}

/* Value of a double after storage in the given precision. */
static double store_as(double v, int dt)
{
    if (dt == DT_BF16)
        return bf16_val(moe_ref_to_bf16(v));
    return (double)(float)v;          /* float32: C's conversion rounds to nearest even */
}

/* Element i of a float32 or bfloat16 array, as an exact double. */
static double ld(const void *p, int dt, int64_t i)
{
    if (dt == DT_BF16)
        return bf16_val(((const uint16_t *)p)[i]);
    return (double)((const float *)p)[i];
}

/* ------------------------------------------------------------------ norm --- */

/* RMSNorm of one row: z = v / sqrt(mean(v^2) + eps) * g.  g may be NULL (= 1).
 * Reading: eps = 1e-5 unless the caller passes another; the pages only say the
 * latent is "normalised" and that norm gains are free parameters. */
void moe_ref_rmsnorm_row(const double *v, int64_t n, const float *g, double eps, double *z)
{
    double ss = 0.0;
    for (int64_t i = 0; i < n; i++)
        ss += v[i] * v[i];
    double inv = 1.0 / sqrt(ss / (double)n + eps);
    for (int64_t i = 0; i < n; i++)
        z[i] = v[i] * inv * (g ? (double)g[i] : 1.0);
}

/* ------------------------------------------------------------------ top-k --- */

/* Does (va, ia) rank above (vb, ib)?  Larger value first; equal values (and
 * +0 == -0, which C's == already treats as equal) go to the lower expert id;
 * a NaN ranks below every number, NaNs among themselves by id. */
static int ranks_above(float va, int ia, float vb, int ib)
{
    int na = isnan(va), nb = isnan(vb);
    if (na || nb) {
        if (na && nb)
            return ia < ib;
        return nb;                    /* the non-NaN one is above */
    }
    if (va > vb)
        return 1;
    if (va < vb)
        return 0;
    return ia < ib;
}

/* Top-k selection and routing weights for T tokens.
 *   logits [T, E] float32 -> ids [T, k] int32, w [T, k] float32.
 * The spec's order: softmax over all E in double, select k experts, renormalise
 * the selected probabilities to sum to one.  Selection is taken on the float32
 * logits themselves (softmax is strictly increasing, so this is the same set in
 * exact arithmetic, and it avoids ties that rounded probabilities would create).
 * ids[t, j] is the j-th best expert.  Selection is k passes, each taking the
 * best expert not yet taken. */
void moe_ref_topk(const float *logits, int64_t T, int32_t E, int32_t k, int32_t *ids, float *w)
{
    double *p = (double *)malloc(sizeof(double) * (size_t)E);
    char *taken = (char *)malloc((size_t)E);
    for (int64_t t = 0; t < T; t++) {
        const float *l = logits + t * E;
        /* softmax over all experts, double precision */
        double m = -INFINITY;
        for (int32_t e = 0; e < E; e++)
            if ((double)l[e] > m)
                m = (double)l[e];
        double s = 0.0;
        for (int32_t e = 0; e < E; e++) {
            p[e] = exp((double)l[e] - m);
            s += p[e];
        }
        for (int32_t e = 0; e < E; e++)
            p[e] /= s;
        /* selection */
        memset(taken, 0, (size_t)E);
        double ps = 0.0;
        for (int32_t j = 0; j < k; j++) {
            int best = -1;
            for (int32_t e = 0; e < E; e++) {
                if (taken[e])
                    continue;
                if (best < 0 || ranks_above(l[e], e, l[best], best))
                    best = e;
            }
            taken[best] = 1;
            ids[t * k + j] = best;
            ps += p[best];
        }
        /* renormalise over the selected set */
        for (int32_t j = 0; j < k; j++)
            w[t * k + j] = (float)(p[ids[t * k + j]] / ps);
    }
    free(p);
    free(taken);
}

/* -------------------------------------------------------------- capacity --- */

/* Per-expert capacity C = ceil(cf * n_assign / E) with cf = num/den, computed
 * in integers so that no rounding can add a row (the pages report a float
 * capacity rounding that could exceed the buffer by one row). */
int64_t moe_ref_capacity(int64_t cf_num, int64_t cf_den, int64_t n_assign, int64_t E)
{
    return (cf_num * n_assign + cf_den * E - 1) / (cf_den * E);
}

/* ---------------------------------------------------------------- permute --- */

/* Group assignments by expert.
 *   ids [n] int32: expert of assignment a (a = t*k + j for routed tokens, or a
 *       pool row); a negative id is padding and takes part in nothing.
 *   capacity: rows kept per expert, or < 0 for no limit.
 * Outputs:
 *   counts [E]     assignments per expert (before the capacity cut)
 *   offsets [E+1]  exclusive prefix sum of kept rows: expert e owns rows
 *                  [offsets[e], offsets[e+1])
 *   slot_row [n]   row of assignment a, or -1 if a is padding or dropped
 *   row_src [R_phys] assignment that fills each row, -1 beyond offsets[E]
 *   n_dropped      assignments cut by the capacity
 * The kept assignments of an expert are its first `capacity` ones in ascending
 * a (arrival order), and they fill its rows in that order.
 * Returns 0, or -1 on an id >= E or too few physical rows. */
int moe_ref_permute(const int32_t *ids, int64_t n, int32_t E, int64_t capacity,
                    int32_t *counts, int32_t *offsets, int32_t *slot_row,
                    int32_t *row_src, int64_t R_phys, int64_t *n_dropped)
{
    for (int32_t e = 0; e < E; e++)
        counts[e] = 0;
    for (int64_t a = 0; a < n; a++) {
        if (ids[a] >= E)
            return -1;
        if (ids[a] >= 0)
            counts[ids[a]]++;
    }
    offsets[0] = 0;
    int64_t dropped = 0;
    for (int32_t e = 0; e < E; e++) {
        int64_t kept = counts[e];
        if (capacity >= 0 && kept > capacity)
            kept = capacity;
        dropped += counts[e] - kept;
        offsets[e + 1] = (int32_t)(offsets[e] + kept);
    }
    if (offsets[E] > R_phys)
        return -1;
    for (int64_t r = 0; r < R_phys; r++)
        row_src[r] = -1;
    int32_t *seen = (int32_t *)calloc((size_t)E, sizeof(int32_t));
    for (int64_t a = 0; a < n; a++) {
        int32_t e = ids[a];
        if (e < 0) {
            slot_row[a] = -1;
            continue;
        }
        int32_t rank = seen[e]++;
        if (rank < offsets[e + 1] - offsets[e]) {
            int32_t row = offsets[e] + rank;
            slot_row[a] = row;
            row_src[row] = (int32_t)a;
        } else {
            slot_row[a] = -1;
        }
    }
    free(seen);
    *n_dropped = dropped;
    return 0;
}

/* ------------------------------------------------------------- expert FFN --- */

/* One expert applied to one row: the gated (SwiGLU) MLP.
 *   x [d] exact values, W_gu [2H, d] (rows [0, H) are the gate projection,
 *   rows [H, 2H) the up projection -- a reading: the pages name a w13 layout
 *   without fixing the order), W_d [d, H].
 *   u = W_gu x;  h_i = silu(u_i) * u_{H+i} stored in dt;  y = W_d h.
 * y is returned unrounded (the caller stores it). */
static void expert_row(const double *x, int64_t d, int64_t H, const void *W_gu,
                       const void *W_d, int dt, double *h, double *y)
{
    for (int64_t i = 0; i < H; i++) {
        double g = 0.0, u = 0.0;
        for (int64_t c = 0; c < d; c++) {
            g += ld(W_gu, dt, i * d + c) * x[c];
            u += ld(W_gu, dt, (H + i) * d + c) * x[c];
        }
        double silu = g / (1.0 + exp(-g));
        h[i] = store_as(silu * u, dt);
    }
    for (int64_t o = 0; o < d; o++) {
        double s = 0.0;
        for (int64_t i = 0; i < H; i++)
            s += ld(W_d, dt, o * H + i) * h[i];
        y[o] = s;
    }
}

/* Expert FFN over rows, each with its own expert:
 *   X [n, d] (dt), expert [n] (row r uses expert expert[r]; < 0 = skip),
 *   W_gu_e[e] -> [2H, d], W_d_e[e] -> [d, H]  (per-expert pointers, so callers
 *   can pass only the experts they use).
 *   Y [n, d] double, unrounded; h_out [n, H] double (stored values), nullable. */
void moe_ref_expert_rows(const void *X, int dt, int64_t n, int64_t d, int64_t H,
                         const int32_t *expert, const void *const *W_gu_e,
                         const void *const *W_d_e, double *Y, double *h_out)
{
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t r = 0; r < n; r++) {
        double *x = (double *)malloc(sizeof(double) * (size_t)d);
        double *h = (double *)malloc(sizeof(double) * (size_t)H);
        if (expert[r] >= 0) {
            for (int64_t c = 0; c < d; c++)
                x[c] = ld(X, dt, r * d + c);
            expert_row(x, d, H, W_gu_e[expert[r]], W_d_e[expert[r]], dt, h, Y + r * d);
            if (h_out)
                memcpy(h_out + r * H, h, sizeof(double) * (size_t)H);
        } else {
            for (int64_t c = 0; c < d; c++)
                Y[r * d + c] = 0.0;
        }
        free(x);
        free(h);
    }
}

/* ------------------------------------------------- backward of the experts --- */

/* The backward of a grouped matmul, as the pages split it (Marin: Week of April
 * 26th summary, the paragraph on moving the backward pass onto Triton with a
 * custom VJP: one kernel for the input gradient with the grouped right-hand side
 * transposed, a separate ragged-contracting kernel for the weight gradient).  The forward is Z[r] = W[e(r)] X[r] for the rows r of
 * group e = [offsets[e], offsets[e+1]), W [E, N, K], X [R, K], Z [R, N]; for a
 * scalar loss with dZ = dLoss/dZ:
 *   dX[r, k]    = sum over n = 0..N-1 (ascending) of dZ[r, n] * W[e(r)][n, k]
 *   dW[e][n, k] = sum over rows r of group e (ascending) of dZ[r, n] * X[r, k]
 * Inputs in dt, sums in double, results unrounded.  Rows r >= offsets[E] of dX
 * are not written; an empty group's dW is zero. */
void moe_ref_ragged_dlhs(const void *dZ, const void *W, int dt, const int32_t *offsets,
                         int32_t E, int64_t N, int64_t K, double *dX)
{
    for (int32_t e = 0; e < E; e++) {
#pragma omp parallel for schedule(static)
        for (int64_t r = offsets[e]; r < offsets[e + 1]; r++) {
            for (int64_t k = 0; k < K; k++) {
                double s = 0.0;
                for (int64_t n = 0; n < N; n++)
                    s += ld(dZ, dt, r * N + n) * ld(W, dt, ((int64_t)e * N + n) * K + k);
                dX[r * K + k] = s;
            }
        }
    }
}

void moe_ref_ragged_drhs(const void *X, const void *dZ, int dt, const int32_t *offsets,
                         int32_t E, int64_t N, int64_t K, double *dW)
{
    for (int32_t e = 0; e < E; e++) {
#pragma omp parallel for schedule(static)
        for (int64_t n = 0; n < N; n++) {
            for (int64_t k = 0; k < K; k++) {
                double s = 0.0;
                for (int64_t r = offsets[e]; r < offsets[e + 1]; r++)
                    s += ld(dZ, dt, r * N + n) * ld(X, dt, r * K + k);
                dW[((int64_t)e * N + n) * K + k] = s;
            }
        }
    }
}

/* Backward of the gated expert MLP of expert_row for the rows of each group
 * (rows r of group e use expert e; rows >= offsets[E] take no part), given the
 * gradient dY [R, d] of its output.  The forward is recomputed row by row:
 *   g = W_gate x, u = W_up x (rows [0, H) and [H, 2H) of W_gu), h = silu(g) u
 *   stored in dt as the forward stores it, y = W_d h.
 * Chain rule, with silu'(v) = s (1 + v (1 - s)), s = 1 / (1 + exp(-v)), and the
 * storage rounding of h taken as the identity (it has no derivative):
 *   dh = W_d^T dy;  dg = dh * u * silu'(g);  du = dh * silu(g)
 *   dx = W_gate^T dg + W_up^T du
 *   dW_d[e]  = sum over the group's rows (ascending) of dy h^T      [d, H]
 *   dW_gu[e] = sum over the group's rows (ascending) of [dg; du] x^T [2H, d]
 * All in double; dX [R, d], dW_gu [E, 2H, d], dW_d [E, d, H] unrounded. */
static void expert_row_grad(const double *x, const double *dy, int64_t d, int64_t H,
                            const void *W_gu, const void *W_d, int dt, double *h,
                            double *dgu, double *dx)
{
    for (int64_t i = 0; i < H; i++) {
        double g = 0.0, u = 0.0, dh = 0.0;
        for (int64_t c = 0; c < d; c++) {
            g += ld(W_gu, dt, i * d + c) * x[c];
            u += ld(W_gu, dt, (H + i) * d + c) * x[c];
        }
        for (int64_t o = 0; o < d; o++)
            dh += ld(W_d, dt, o * H + i) * dy[o];
        double s = 1.0 / (1.0 + exp(-g));
        double silu = g / (1.0 + exp(-g));
        h[i] = store_as(silu * u, dt);
        dgu[i] = dh * u * (s * (1.0 + g * (1.0 - s)));
        dgu[H + i] = dh * silu;
    }
    for (int64_t c = 0; c < d; c++) {
        double s = 0.0;
        for (int64_t i = 0; i < 2 * H; i++)
            s += ld(W_gu, dt, i * d + c) * dgu[i];
        dx[c] = s;
    }
}

void moe_ref_expert_rows_bwd(const void *X, const void *dY, int dt, const int32_t *offsets,
                             int32_t E, int64_t d, int64_t H, const void *W_gu,
                             const void *W_d, double *dX, double *dW_gu, double *dW_d)
{
    const int64_t R = offsets[E];
    double *hh = (double *)malloc(sizeof(double) * (size_t)(R > 0 ? R : 1) * (size_t)H);
    double *gg = (double *)malloc(sizeof(double) * (size_t)(R > 0 ? R : 1) * (size_t)(2 * H));
    for (int32_t e = 0; e < E; e++) {
        const void *Wg = (const char *)W_gu + (size_t)e * (size_t)(2 * H * d) * (dt == DT_BF16 ? 2 : 4);
        const void *Wd = (const char *)W_d + (size_t)e * (size_t)(d * H) * (dt == DT_BF16 ? 2 : 4);
#pragma omp parallel for schedule(dynamic, 1)
        for (int64_t r = offsets[e]; r < offsets[e + 1]; r++) {
            double *x = (double *)malloc(sizeof(double) * (size_t)d);
            double *dy = (double *)malloc(sizeof(double) * (size_t)d);
            for (int64_t c = 0; c < d; c++) {
                x[c] = ld(X, dt, r * d + c);
                dy[c] = ld(dY, dt, r * d + c);
            }
            expert_row_grad(x, dy, d, H, Wg, Wd, dt, hh + r * H, gg + r * 2 * H, dX + r * d);
            free(x);
            free(dy);
        }
        /* weight gradients: each element sums its group's rows in ascending order */
#pragma omp parallel for schedule(static)
        for (int64_t o = 0; o < d; o++)
            for (int64_t i = 0; i < H; i++) {
                double s = 0.0;
                for (int64_t r = offsets[e]; r < offsets[e + 1]; r++)
                    s += ld(dY, dt, r * d + o) * hh[r * H + i];
                dW_d[((int64_t)e * d + o) * H + i] = s;
            }
#pragma omp parallel for schedule(static)
        for (int64_t i = 0; i < 2 * H; i++)
            for (int64_t c = 0; c < d; c++) {
                double s = 0.0;
                for (int64_t r = offsets[e]; r < offsets[e + 1]; r++)
                    s += gg[r * 2 * H + i] * ld(X, dt, r * d + c);
                dW_gu[((int64_t)e * 2 * H + i) * d + c] = s;
            }
    }
    free(hh);
    free(gg);
}

/* ------------------------------------------------------------------- fp8 --- */

/* OCP 8-bit floating point E4M3 (the format the pages name for the fp8 expert
 * GEMMs' forward: Marin: Week of July 6th summary, the fp8 compute-lane
 * paragraph).  Sign bit, 4 exponent bits with bias 7, 3 mantissa bits; exponent
 * field 0 holds subnormals m/8 * 2^-6; S.1111.111 is NaN and there is no
 * infinity, so the largest finite magnitude is 1.75 * 2^8 = 448. */
double moe_ref_e4m3_value(uint8_t code)
{
    int s = code >> 7, e = (code >> 3) & 15, m = code & 7;
    if (e == 15 && m == 7)
        return NAN;
    double v = e == 0 ? ldexp((double)m / 8.0, -6) : ldexp(1.0 + (double)m / 8.0, e - 7);
    return s ? -v : v;
}

/* Nearest E4M3 code to x, ties to the code with an even mantissa, magnitudes
 * beyond 448 (and infinities) saturated to +-448 (the saturating conversion
 * used for training tensors), NaN to NaN.  Found by comparing x with every
 * finite positive code's value, so it follows from the definition alone. */
uint8_t moe_ref_to_e4m3(double x)
{
    if (isnan(x))
        return 0x7F;
    uint8_t sign = signbit(x) ? 0x80 : 0;
    double a = fabs(x);
    int best = 0;
    double best_d = INFINITY;
    for (int c = 0; c <= 0x7E; c++) {
        double d = fabs(moe_ref_e4m3_value((uint8_t)c) - a);
        if (d < best_d || (d == best_d && (c & 1) == 0)) {
            best = c;
            best_d = d;
        }
    }
    return (uint8_t)(sign | best);
}

/* Quantisation with a per-tensor scale, decided in float32 as a kernel does:
 *   q[i] = E4M3( (float)(x[i] * inv_scale) ),  x in dt, the product rounded to
 * float32 first.  amax (nullable) receives max |x[i]| over the tensor (the value
 * a delayed-scaling history records), NaN ignored. */
void moe_ref_quantize_e4m3(const void *x, int dt, int64_t n, float inv_scale, uint8_t *q,
                           float *amax)
{
    float m = 0.0f;
#pragma omp parallel for schedule(static) reduction(max : m)
    for (int64_t i = 0; i < n; i++) {
        float v = (float)ld(x, dt, i);
        float p = v * inv_scale;          /* one float32 rounding */
        q[i] = moe_ref_to_e4m3((double)p);
        if (fabsf(v) > m)
            m = fabsf(v);
    }
    if (amax)
        *amax = m;
}

/* Delayed scaling's state update for one tensor (the train-step state of the fp8
 * lane in the same summary): the history holds the amax of the last len steps,
 * newest first.  The update shifts it by one and puts this step's amax first; the
 * next step's dequantisation scale is m / 448 for m the largest finite entry (the
 * value that maps to E4M3's largest code), or 1 when m is 0.  scale[1] receives the
 * quantisation factor 1 / scale[0], rounded to float32. */
void moe_ref_fp8_scale_update(float *history, int32_t len, float amax, float *scale)
{
    for (int32_t i = len - 1; i > 0; i--)
        history[i] = history[i - 1];
    if (len > 0)
        history[0] = amax;
    float m = 0.0f;
    for (int32_t i = 0; i < len; i++)
        if (isfinite(history[i]) && history[i] > m)
            m = history[i];
    scale[0] = m > 0.0f ? m / 448.0f : 1.0f;
    scale[1] = 1.0f / scale[0];
}

/* The grouped matmul on E4M3 operands: Z[r] = scale * W[e] X[r] for the rows r of
 * group e, X [R, K] and W [E, N, K] as E4M3 codes, the products of the decoded
 * values summed in double (ascending k), Z [R, N] unrounded; rows >= offsets[E]
 * are not written. */
void moe_ref_ragged_dot_e4m3(const uint8_t *X, const uint8_t *W, const int32_t *offsets,
                             int32_t E, int64_t N, int64_t K, double scale, double *Z)
{
    for (int32_t e = 0; e < E; e++) {
#pragma omp parallel for schedule(static)
        for (int64_t r = offsets[e]; r < offsets[e + 1]; r++)
            for (int64_t n = 0; n < N; n++) {
                double s = 0.0;
                for (int64_t k = 0; k < K; k++)
                    s += moe_ref_e4m3_value(X[r * K + k]) *
                         moe_ref_e4m3_value(W[((int64_t)e * N + n) * K + k]);
                Z[r * N + n] = scale * s;
            }
    }
}

/* The gated activation quantised for an E4M3 down projection (the expert MLP of
 * the fp8 lane; SwiGLU with the exact activation as in the JaxPP paragraph of the
 * same summary): for each of n rows of gu = [g | u] (2H wide, in dt, gate first),
 *   h = silu(g) * u in double, rounded once to float32 (hf, the activation a
 *   float32 kernel holds), q = E4M3( (float)(hf * inv_scale) ) as
 *   moe_ref_quantize_e4m3 decides it, amax = max |hf|.
 * h (nullable) receives the double values before the rounding. */
void moe_ref_swiglu_quantize_e4m3(const void *gu, int dt, int64_t n, int64_t H, float inv_scale,
                                  uint8_t *q, float *amax, double *h)
{
    float m = 0.0f;
#pragma omp parallel for schedule(static) reduction(max : m)
    for (int64_t r = 0; r < n; r++)
        for (int64_t i = 0; i < H; i++) {
            double g = ld(gu, dt, r * 2 * H + i);
            double u = ld(gu, dt, r * 2 * H + H + i);
            double v = g / (1.0 + exp(-g)) * u;
            float hf = (float)v;
            float p = hf * inv_scale;     /* one float32 rounding */
            q[r * H + i] = moe_ref_to_e4m3((double)p);
            if (fabsf(hf) > m)
                m = fabsf(hf);
            if (h)
                h[r * H + i] = v;
        }
    if (amax)
        *amax = m;
}

/* The grouped matmul itself in dt (the forward of the pages' ragged_dot in this
 * library's convention): Z[r] = W[e] X[r], summed in double, unrounded. */
void moe_ref_ragged_dot(const void *X, const void *W, int dt, const int32_t *offsets, int32_t E,
                        int64_t N, int64_t K, double *Z)
{
    for (int32_t e = 0; e < E; e++) {
#pragma omp parallel for schedule(static)
        for (int64_t r = offsets[e]; r < offsets[e + 1]; r++)
            for (int64_t n = 0; n < N; n++) {
                double s = 0.0;
                for (int64_t k = 0; k < K; k++)
                    s += ld(X, dt, r * K + k) * ld(W, dt, ((int64_t)e * N + n) * K + k);
                Z[r * N + n] = s;
            }
    }
}

/* Weighted combine, ordered gather: c_t = sum over j = 0..k-1 (ascending) of
 * w[t,j] * Y[slot_row[t*k+j]], skipping slots < 0 (dropped: contributes zero,
 * the survivors are not renormalised).  w may be NULL (weight 1).  Y [*, d] in
 * dt; c [T, d] double, unrounded. */
void moe_ref_combine(const void *Y, int dt, const int32_t *slot_row, const float *w,
                     int64_t T, int32_t k, int64_t d, double *c)
{
#pragma omp parallel for schedule(static)
    for (int64_t t = 0; t < T; t++) {
        for (int64_t o = 0; o < d; o++)
            c[t * d + o] = 0.0;
        for (int32_t j = 0; j < k; j++) {
            int32_t row = slot_row[t * k + j];
            if (row < 0)
                continue;
            double wj = w ? (double)w[t * k + j] : 1.0;
            for (int64_t o = 0; o < d; o++)
                c[t * d + o] += wj * ld(Y, dt, (int64_t)row * d + o);
        }
    }
}

/* ------------------------------------------------------------- full layer --- */

typedef struct {
    int64_t T, D, L;      /* L = 0: no latent; routing and experts act on x */
    int32_t E, k;
    int64_t H;            /* routed expert hidden width */
    int32_t n_shared;
    int64_t Hs;           /* shared expert hidden width */
    int32_t dtype;        /* DT_F32 or DT_BF16: storage of activations and weights */
    double eps;
} moe_ref_dims;

typedef struct {
    const void *W_dn;             /* [L, D] */
    const float *norm_g;          /* [L], NULL = ones */
    const float *W_r;             /* [E, d_r] float32 (d_r = L, or D without latent) */
    const float *b_r;             /* [E], NULL = zeros */
    const void *const *W_gu_e;    /* E pointers to [2H, d_e] */
    const void *const *W_d_e;     /* E pointers to [d_e, H] */
    const void *W_up;             /* [D, L] */
    const void *W_gu_s;           /* [n_shared, 2Hs, D] */
    const void *W_d_s;            /* [n_shared, D, Hs] */
} moe_ref_weights;

/* Router/expert input of token t as exact doubles (length d_r = L, or D
 * without latent):
 *   without latent: x_t;
 *   with latent:    z = RMSNorm(W_dn x_t) * g, computed in double. */
static void token_input(const moe_ref_dims *dm, const moe_ref_weights *W, const void *x,
                        int64_t t, double *r)
{
    const int dt = dm->dtype;
    if (dm->L > 0) {
        double *zp = (double *)malloc(sizeof(double) * (size_t)dm->L);
        for (int64_t o = 0; o < dm->L; o++) {
            double s = 0.0;
            for (int64_t c = 0; c < dm->D; c++)
                s += ld(W->W_dn, dt, o * dm->D + c) * ld(x, dt, t * dm->D + c);
            zp[o] = s;
        }
        moe_ref_rmsnorm_row(zp, dm->L, W->norm_g, dm->eps, r);
        free(zp);
    } else {
        for (int64_t c = 0; c < dm->D; c++)
            r[c] = ld(x, dt, t * dm->D + c);
    }
}

/* Router part of the layer for a list of tokens.
 *   x [T, D] (dt); tok [n] token indices.
 * Per token t (outputs indexed by position i in tok):
 *   without latent: r = x_t;
 *   with latent:    z_pre = W_dn x_t;  z = RMSNorm(z_pre) * g  (double);
 *   router input    h32 = float32(r or z);  expert input h_e = dt(r or z).
 *   logits = W_r h32 + b_r, summed in double from float32 operands and stored
 *   as float32 (logits64 keeps the double sum).
 *   ids/w from moe_ref_topk on the float32 logits.
 * Reading: the router reads the normalised latent (project, normalise, route),
 * in float32, as the spec fixes the router's precision.
 * Any output pointer may be NULL except ids and w. */
void moe_ref_route_tokens(const moe_ref_dims *dm, const moe_ref_weights *W, const void *x,
                          const int32_t *tok, int64_t n, double *z_out, float *logits32,
                          double *logits64, int32_t *ids, float *w)
{
    const int64_t d_r = dm->L > 0 ? dm->L : dm->D;
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t i = 0; i < n; i++) {
        const int64_t t = tok[i];
        double *r = (double *)malloc(sizeof(double) * (size_t)d_r);
        float *l32 = (float *)malloc(sizeof(float) * (size_t)dm->E);
        token_input(dm, W, x, t, r);
        if (z_out)
            memcpy(z_out + i * d_r, r, sizeof(double) * (size_t)d_r);
        for (int32_t e = 0; e < dm->E; e++) {
            double s = 0.0;
            for (int64_t c = 0; c < d_r; c++)
                s += (double)W->W_r[(int64_t)e * d_r + c] * (double)(float)r[c];
            if (W->b_r)
                s += (double)W->b_r[e];
            l32[e] = (float)s;
            if (logits32)
                logits32[i * dm->E + e] = (float)s;
            if (logits64)
                logits64[i * dm->E + e] = s;
        }
        moe_ref_topk(l32, 1, dm->E, dm->k, ids + i * dm->k, w + i * dm->k);
        free(r);
        free(l32);
    }
}

/* Output part of the layer for a list of tokens, given each token's routing.
 *   ids/w [n, k] for the tokens in tok (position i), keep [n, k] (1 kept,
 *   0 dropped by capacity; NULL = all kept).
 * Per token:
 *   h_e = dt(r or z)  (r = x_t without latent; z from moe_ref_route_tokens' rule)
 *   Y_j = dt(FFN_{ids_j}(h_e)) for kept j
 *   c   = dt(sum_j w_j Y_j)    (ordered, ascending j)
 *   routed = W_up c  (latent)  or  c  (no latent)
 *   shared = sum_i W_d_s[i] * dt(silu(W1_i x) * (W3_i x)),  W_gu_s[i] = [W1_i; W3_i]
 *   y = routed + shared, unrounded double.
 * c_out [n, d_e] (the stored c) may be NULL. */
void moe_ref_output_tokens(const moe_ref_dims *dm, const moe_ref_weights *W, const void *x,
                           const int32_t *tok, int64_t n, const int32_t *ids, const float *w,
                           const int32_t *keep, double *y, double *c_out)
{
    const int64_t d_e = dm->L > 0 ? dm->L : dm->D;
    const int dt = dm->dtype;
    const int32_t k = dm->k;
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t i = 0; i < n; i++) {
        const int64_t t = tok[i];
        double *he = (double *)malloc(sizeof(double) * (size_t)d_e);
        double *xv = (double *)malloc(sizeof(double) * (size_t)dm->D);
        double *Yj = (double *)malloc(sizeof(double) * (size_t)d_e);
        double *hbuf = (double *)malloc(sizeof(double) * (size_t)(dm->H > dm->Hs ? dm->H : dm->Hs));
        double *c = (double *)calloc((size_t)d_e, sizeof(double));
        for (int64_t cc = 0; cc < dm->D; cc++)
            xv[cc] = ld(x, dt, t * dm->D + cc);
        token_input(dm, W, x, t, he);
        for (int64_t o = 0; o < d_e; o++)
            he[o] = store_as(he[o], dt);   /* expert input is stored in dt */
        /* routed experts and the ordered weighted combine */
        for (int32_t j = 0; j < k; j++) {
            if (keep && !keep[i * k + j])
                continue;
            int32_t e = ids[i * k + j];
            expert_row(he, d_e, dm->H, W->W_gu_e[e], W->W_d_e[e], dt, hbuf, Yj);
            double wj = (double)w[i * k + j];
            for (int64_t o = 0; o < d_e; o++)
                c[o] += wj * store_as(Yj[o], dt);
        }
        for (int64_t o = 0; o < d_e; o++)
            c[o] = store_as(c[o], dt);
        if (c_out)
            memcpy(c_out + i * d_e, c, sizeof(double) * (size_t)d_e);
        double *yo = y + i * dm->D;
        /* up-projection */
        for (int64_t o = 0; o < dm->D; o++) {
            if (dm->L > 0) {
                double s = 0.0;
                for (int64_t cc = 0; cc < dm->L; cc++)
                    s += ld(W->W_up, dt, o * dm->L + cc) * c[cc];
                yo[o] = s;
            } else {
                yo[o] = c[o];
            }
        }
        /* shared experts: unweighted, every token */
        for (int32_t si = 0; si < dm->n_shared; si++) {
            const int64_t Hs = dm->Hs, D = dm->D;
            const int64_t gu_off = (int64_t)si * 2 * Hs * D;
            const int64_t d_off = (int64_t)si * D * Hs;
            for (int64_t q = 0; q < Hs; q++) {
                double g = 0.0, u = 0.0;
                for (int64_t cc = 0; cc < D; cc++) {
                    g += ld(W->W_gu_s, dt, gu_off + q * D + cc) * xv[cc];
                    u += ld(W->W_gu_s, dt, gu_off + (Hs + q) * D + cc) * xv[cc];
                }
                hbuf[q] = store_as(g / (1.0 + exp(-g)) * u, dt);
            }
            for (int64_t o = 0; o < D; o++) {
                double s = 0.0;
                for (int64_t q = 0; q < Hs; q++)
                    s += ld(W->W_d_s, dt, d_off + o * Hs + q) * hbuf[q];
                yo[o] += s;
            }
        }
        free(he);
        free(xv);
        free(Yj);
        free(hbuf);
        free(c);
    }
}
