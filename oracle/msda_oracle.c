/*
 * Plain fp64 CPU oracle for the multi-scale deformable attention (MSDA) core
 * operator: the forward and its three gradients.
 *
 * TEST INFRASTRUCTURE ONLY.  It exists so that the GPU library can be checked
 * against an obviously correct definition.  Only the test suite, the smoke
 * check and the CPU-baseline leg of the benchmark may load it.  It shares no
 * code, header, table or helper with the GPU library, and neither includes
 * nor links the other.
 *
 * Source of the definition: "1. Deformable attention, from scratch" (the
 * msda-triton course, chapter 1):
 *   - section "The equation, term by term": the tensor shapes
 *       value               (B, S, M, D)   flattened pyramid, per head
 *       spatial_shapes      (L, 2)         rows are (H_l, W_l)
 *       sampling_locations  (B, Q, M, L, K, 2), last axis (x, y), normalised
 *       attention_weights   (B, Q, M, L, K)
 *       output              (B, Q, M*D)
 *   - section "Bilinear interpolation: reading between the pixels": the four
 *     corners and their weights, the pixel-centre mapping x = loc_x*W - 0.5,
 *     and zero contribution from corners outside the map;
 *   - section "The simplest possible implementation": the six nested loops,
 *     the use of floor, the per-corner bounds test and the row index
 *     start_l + yy*W_l + xx into the flattened pyramid.
 * The pages use the attention weights as given by default (DeformOps page,
 * section "Multi-scale deformable attention"); the same section names a
 * second method, "softmax", that normalises raw logits jointly over levels
 * and points.  That normalisation and its derivative are the two functions at
 * the end of this file; the operator itself never normalises.
 *
 * The gradients are not printed on the pages (the course's backward chapter
 * is not among them).  They are derived here by differentiating the forward
 * loop by hand; every formula is stated where it is used.
 *
 * Arithmetic: all inputs arrive as fp64 (exact upcasts of fp32 or bf16), and
 * every accumulation is fp64.  The pixel coordinate is computed as in the
 * naive loop, a float multiply then a subtraction, in fp64.  The product of a
 * 24-bit significand and an integer size below 2^29 is exact in fp64, so the
 * floor decision is the exact one.  Build with -ffp-contract=off so that no
 * other expression is fused either.
 */
#include <math.h>
#include <omp.h>
#include <stdint.h>
#include <string.h>

/* Threads the oracle's parallel loops use (reported beside its timings). */
int msda_oracle_threads(void) { return omp_get_max_threads(); }

/* Geometry of one bilinear sample at one pyramid level. */
typedef struct {
    int64_t row[4]; /* flattened-pyramid row of corners 00, 01, 10, 11; -1 = outside */
    double w[4];    /* bilinear weight of each corner */
    double lx, ly;  /* fractional parts of the pixel coordinate */
    int any_valid;  /* at least one corner lies inside the map */
} corner_set;

/*
 * Corners of the sample at normalised (u, v) on a level of H x W pixels whose
 * rows start at `start` in the flattened pyramid.
 * Chapter 1, "Bilinear interpolation": x = u*W - 0.5, y = v*H - 0.5;
 * x0 = floor(x), y0 = floor(y), lx = x - x0, ly = y - y0;
 * corner 00 = (y0, x0) with weight (1-lx)(1-ly), 01 = (y0, x0+1) with
 * lx(1-ly), 10 = (y0+1, x0) with (1-lx)ly, 11 = (y0+1, x0+1) with lx*ly.
 * A corner is used only when 0 <= xx < W and 0 <= yy < H.  The test is made
 * on the floating-point corner position, so a NaN or infinite coordinate
 * fails it and no integer conversion of such a value ever happens.
 */
static void level_corners(double u, double v, int64_t H, int64_t W, int64_t start,
                          corner_set *cs)
{
    double x = u * (double)W - 0.5;
    double y = v * (double)H - 0.5;
    double x0 = floor(x);
    double y0 = floor(y);
    double lx = x - x0;
    double ly = y - y0;
    double cy[4] = {y0, y0, y0 + 1.0, y0 + 1.0};
    double cx[4] = {x0, x0 + 1.0, x0, x0 + 1.0};

    cs->w[0] = (1.0 - lx) * (1.0 - ly);
    cs->w[1] = lx * (1.0 - ly);
    cs->w[2] = (1.0 - lx) * ly;
    cs->w[3] = lx * ly;
    cs->lx = lx;
    cs->ly = ly;
    cs->any_valid = 0;
    for (int c = 0; c < 4; ++c) {
        int inside = cx[c] >= 0.0 && cx[c] < (double)W && cy[c] >= 0.0 && cy[c] < (double)H;
        if (inside) {
            cs->row[c] = start + (int64_t)cy[c] * W + (int64_t)cx[c];
            cs->any_valid = 1;
        } else {
            cs->row[c] = -1;
        }
    }
}

/*
 * Forward.  For every (b, q, m):
 *   out[b, q, m*D + d] = sum over l, k, valid corners c of
 *                        a[b,q,m,l,k] * w_c * value[b, row_c, m, d].
 * Loop order and product order follow the naive loop of chapter 1.
 * Parallel over (b, q): each pair writes its own output rows only.
 */
void msda_oracle_forward(const double *value, const int64_t *spatial_shapes,
                         const int64_t *level_start_index, const double *sampling_locations,
                         const double *attention_weights, double *out, int64_t B, int64_t S,
                         int64_t M, int64_t D, int64_t L, int64_t Q, int64_t K)
{
#pragma omp parallel for collapse(2) schedule(dynamic, 16)
    for (int64_t b = 0; b < B; ++b) {
        for (int64_t q = 0; q < Q; ++q) {
            for (int64_t m = 0; m < M; ++m) {
                double *o = out + ((b * Q + q) * M + m) * D;
                for (int64_t d = 0; d < D; ++d)
                    o[d] = 0.0;
                for (int64_t l = 0; l < L; ++l) {
                    int64_t H = spatial_shapes[2 * l];
                    int64_t W = spatial_shapes[2 * l + 1];
                    int64_t start = level_start_index[l];
                    for (int64_t k = 0; k < K; ++k) {
                        int64_t s = (((b * Q + q) * M + m) * L + l) * K + k;
                        double a = attention_weights[s];
                        corner_set cs;
                        level_corners(sampling_locations[2 * s], sampling_locations[2 * s + 1],
                                      H, W, start, &cs);
                        for (int c = 0; c < 4; ++c) {
                            if (cs.row[c] < 0)
                                continue;
                            const double *vr = value + ((b * S + cs.row[c]) * M + m) * D;
                            for (int64_t d = 0; d < D; ++d)
                                o[d] += a * cs.w[c] * vr[d];
                        }
                    }
                }
            }
        }
    }
}

/*
 * Backward, by differentiating the forward above.  With g = grad_out[b,q,m,:]
 * and, per sample, V_c the value row of corner c (zero when outside):
 *   p_c                      = <g, V_c>
 *   grad_attention_weights   = sum_c w_c p_c
 *   grad_value[b, row_c, m]  += a * w_c * g                 (valid corners)
 *   d out / d lx             = a * ((1-ly)(V01 - V00) + ly (V11 - V10))
 *   d out / d ly             = a * ((1-lx)(V10 - V00) + lx (V11 - V01))
 *   dx/du = W, dy/dv = H  (from x = u*W - 0.5), so
 *   grad_loc_x = a * W * ((1-ly)(p01 - p00) + ly (p11 - p10))
 *   grad_loc_y = a * H * ((1-lx)(p10 - p00) + lx (p11 - p01)).
 * The mask of valid corners is piecewise constant, so outside corners enter
 * as V_c = 0.  On a cell edge (lx or ly exactly 0) these are the derivatives
 * from the right, the side that floor assigns the point to.  A sample with no
 * corner inside the map (including NaN or infinite coordinates) contributes
 * nothing and gets zero gradients.
 *
 * grad_value is overwritten: zeroed, then accumulated.  Parallel over (b, m):
 * grad_value[b, :, m, :] receives contributions from head m of batch b only,
 * so the slices are disjoint and every element is summed in increasing
 * (q, l, k) order, deterministically.
 */
void msda_oracle_backward(const double *value, const int64_t *spatial_shapes,
                          const int64_t *level_start_index, const double *sampling_locations,
                          const double *attention_weights, const double *grad_out,
                          double *grad_value, double *grad_loc, double *grad_attn, int64_t B,
                          int64_t S, int64_t M, int64_t D, int64_t L, int64_t Q, int64_t K)
{
    memset(grad_value, 0, (size_t)(B * S * M * D) * sizeof(double));
#pragma omp parallel for collapse(2) schedule(dynamic, 1)
    for (int64_t b = 0; b < B; ++b) {
        for (int64_t m = 0; m < M; ++m) {
            for (int64_t q = 0; q < Q; ++q) {
                const double *g = grad_out + ((b * Q + q) * M + m) * D;
                for (int64_t l = 0; l < L; ++l) {
                    int64_t H = spatial_shapes[2 * l];
                    int64_t W = spatial_shapes[2 * l + 1];
                    int64_t start = level_start_index[l];
                    for (int64_t k = 0; k < K; ++k) {
                        int64_t s = (((b * Q + q) * M + m) * L + l) * K + k;
                        double a = attention_weights[s];
                        corner_set cs;
                        level_corners(sampling_locations[2 * s], sampling_locations[2 * s + 1],
                                      H, W, start, &cs);
                        if (!cs.any_valid) {
                            grad_attn[s] = 0.0;
                            grad_loc[2 * s] = 0.0;
                            grad_loc[2 * s + 1] = 0.0;
                            continue;
                        }
                        double p[4];
                        for (int c = 0; c < 4; ++c) {
                            p[c] = 0.0;
                            if (cs.row[c] < 0)
                                continue;
                            const double *vr = value + ((b * S + cs.row[c]) * M + m) * D;
                            for (int64_t d = 0; d < D; ++d)
                                p[c] += g[d] * vr[d];
                        }
                        double lx = cs.lx, ly = cs.ly;
                        grad_attn[s] = cs.w[0] * p[0] + cs.w[1] * p[1] + cs.w[2] * p[2] +
                                       cs.w[3] * p[3];
                        grad_loc[2 * s] =
                            a * (double)W * ((1.0 - ly) * (p[1] - p[0]) + ly * (p[3] - p[2]));
                        grad_loc[2 * s + 1] =
                            a * (double)H * ((1.0 - lx) * (p[2] - p[0]) + lx * (p[3] - p[1]));
                        for (int c = 0; c < 4; ++c) {
                            if (cs.row[c] < 0)
                                continue;
                            double *gv = grad_value + ((b * S + cs.row[c]) * M + m) * D;
                            double aw = a * cs.w[c];
                            for (int64_t d = 0; d < D; ++d)
                                gv[d] += aw * g[d];
                        }
                    }
                }
            }
        }
    }
}

/*
 * The "softmax" method of the DeformOps page (section "Multi-scale deformable
 * attention"): the L*K raw logits z of every head-query (b, q, m) become the
 * attention weights
 *     A_j = exp(z_j - max_i z_i) / sum_i exp(z_i - max_i z_i)
 * (the usual softmax; subtracting the maximum changes nothing but the range).
 * logits and weights are [n_hq][lk], contiguous.
 */
void msda_oracle_softmax(const double *logits, double *weights, int64_t n_hq, int64_t lk) {
#pragma omp parallel for schedule(static)
    for (int64_t h = 0; h < n_hq; ++h) {
        const double *z = logits + h * lk;
        double *a = weights + h * lk;
        double mx = z[0];
        for (int64_t j = 1; j < lk; ++j)
            if (z[j] > mx)
                mx = z[j];
        double sum = 0.0;
        for (int64_t j = 0; j < lk; ++j) {
            a[j] = exp(z[j] - mx);
            sum += a[j];
        }
        for (int64_t j = 0; j < lk; ++j)
            a[j] = a[j] / sum;
    }
}

/*
 * Derivative through that softmax.  With gA_j = dLoss/dA_j (the grad_attn of
 * the operator) and dA_i/dz_j = A_i (delta_ij - A_j):
 *     dLoss/dz_j = sum_i gA_i A_i (delta_ij - A_j) = A_j (gA_j - sum_i A_i gA_i).
 */
void msda_oracle_softmax_backward(const double *weights, const double *grad_weights,
                                  double *grad_logits, int64_t n_hq, int64_t lk) {
#pragma omp parallel for schedule(static)
    for (int64_t h = 0; h < n_hq; ++h) {
        const double *a = weights + h * lk;
        const double *ga = grad_weights + h * lk;
        double dot = 0.0;
        for (int64_t i = 0; i < lk; ++i)
            dot += a[i] * ga[i];
        for (int64_t j = 0; j < lk; ++j)
            grad_logits[h * lk + j] = a[j] * (ga[j] - dot);
    }
}
