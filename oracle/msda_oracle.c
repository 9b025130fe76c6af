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
 *   - section "The equation, term by term": the output of head m of query q is
 *     the sum over levels l and points k of the attention weight A[b,q,m,l,k]
 *     times the value of level l sampled at the point's location, with shapes
 *       value               (B, S, M, D)   flattened pyramid, per head
 *       spatial_shapes      (L, 2)         rows are (H_l, W_l)
 *       level_start_index   (L,)           first pyramid row of each level
 *       sampling_locations  (B, Q, M, L, K, 2), last axis (x, y), normalised
 *       attention_weights   (B, Q, M, L, K)
 *       output              (B, Q, M*D);
 *   - section "Bilinear interpolation: reading between the pixels": a sample
 *     between pixels blends the four surrounding pixels, each weighted by the
 *     product of the fractional distances along x and y, with pixel centres
 *     at integer coordinates x = loc_x * W - 0.5 and pixels outside the map
 *     contributing zero.  Written out, that is the tent (hat) kernel:
 *       sample(x, y) = sum over pixels (i, j) inside the map of
 *                      tent(x - j) * tent(y - i) * V[i, j],   tent(t) = max(0, 1 - |t|),
 *     whose non-zero terms are the (at most) four pixels of the cell
 *     floor(x) .. floor(x) + 1, floor(y) .. floor(y) + 1.  A pixel (i, j) of
 *     level l is pyramid row level_start_index[l] + i * W_l + j.
 * The pages use the attention weights as given by default (DeformOps page,
 * section "Multi-scale deformable attention"); the same section names a
 * second method, "softmax", that normalises raw logits jointly over levels
 * and points.  That normalisation and its derivative are the two functions at
 * the end of this file; the operator itself never normalises.
 *
 * The gradients are not printed on the pages (the course's backward chapter
 * is not among them).  They follow from the sum above: it is linear in the
 * weights and in the value, and its x-derivative takes the slope of each tent
 * factor; every formula is stated where it is used.
 *
 * Arithmetic: all inputs arrive as fp64 (exact upcasts of fp32 or bf16), and
 * every accumulation is fp64.  The pixel coordinate is a multiply then a
 * subtraction in fp64; the product of a 24-bit significand and an integer
 * size below 2^29 is exact in fp64, so the cell is the exact one.  Built with
 * -ffp-contract=off so that no expression is fused.
 */
#include <math.h>
#include <omp.h>
#include <stdint.h>
#include <string.h>

/* Threads the oracle's parallel loops use (reported beside its timings). */
int msda_oracle_threads(void) { return omp_get_max_threads(); }

/* The tent (hat) kernel of bilinear interpolation. */
static double tent(double t)
{
    double a = fabs(t);
    return a < 1.0 ? 1.0 - a : 0.0;
}

/* The pixels of an H x W map that lie in the cell of (x, y) (pixel
 * coordinates, centres at integers), with their tent factors along x and y
 * and the slopes of those factors: on the cell [floor(x), floor(x) + 1] the
 * factor of the left column falls with slope -1 and that of the right column
 * rises with slope +1 (the derivative from the right at an integer x, the
 * side floor() puts the point on; likewise along y). */
typedef struct {
    int n;                /* pixels of the cell inside the map (0 to 4) */
    int64_t pix[4];       /* i * W + j of each */
    double wx[4], wy[4];  /* tent(x - j), tent(y - i) */
    double sx[4], sy[4];  /* d tent(x - j) / dx, d tent(y - i) / dy */
} cell_taps;

static void cell_of(double x, double y, int64_t H, int64_t W, cell_taps *t)
{
    double xc = floor(x);
    double yc = floor(y);
    t->n = 0;
    for (int dy = 0; dy < 2; ++dy) {
        for (int dx = 0; dx < 2; ++dx) {
            double px = xc + (double)dx;
            double py = yc + (double)dy;
            /* the test is made on the floating-point pixel position: a NaN or
             * infinite coordinate fails it, and no integer conversion of such
             * a value ever happens */
            if (!(px >= 0.0 && px < (double)W && py >= 0.0 && py < (double)H))
                continue;
            t->pix[t->n] = (int64_t)py * W + (int64_t)px;
            t->wx[t->n] = tent(x - px);
            t->wy[t->n] = tent(y - py);
            t->sx[t->n] = (px == xc) ? -1.0 : 1.0;
            t->sy[t->n] = (py == yc) ? -1.0 : 1.0;
            t->n += 1;
        }
    }
}

/*
 * Forward.  For every (b, q, m): first the bilinear samples of all levels and
 * points, then their sum weighted by the attention weights:
 *   out[b, q, m*D + d] = sum_{l,k} A[b,q,m,l,k] * sample_l(x_lk, y_lk)[d],
 *   x = u * W_l - 0.5, y = v * H_l - 0.5 for the sample's location (u, v).
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
            double smp[L * K][D];  /* the sample of every (level, point) */
            for (int64_t m = 0; m < M; ++m) {
                const int64_t hq = (b * Q + q) * M + m;
                for (int64_t l = 0; l < L; ++l) {
                    const int64_t H = spatial_shapes[2 * l];
                    const int64_t W = spatial_shapes[2 * l + 1];
                    /* level l of head m of image b: its pixel p is pyramid row start + p */
                    const double *img = value + ((b * S + level_start_index[l]) * M + m) * D;
                    for (int64_t k = 0; k < K; ++k) {
                        const int64_t s = hq * L * K + l * K + k;
                        double u = sampling_locations[2 * s], v = sampling_locations[2 * s + 1];
                        double x = u * (double)W - 0.5;
                        double y = v * (double)H - 0.5;
                        cell_taps t;
                        cell_of(x, y, H, W, &t);
                        double *dst = smp[l * K + k];
                        for (int64_t d = 0; d < D; ++d)
                            dst[d] = 0.0;
                        for (int c = 0; c < t.n; ++c) {
                            const double *vr = img + t.pix[c] * M * D;
                            for (int64_t d = 0; d < D; ++d)
                                dst[d] += t.wx[c] * t.wy[c] * vr[d];
                        }
                    }
                }
                double *o = out + hq * D;
                for (int64_t d = 0; d < D; ++d)
                    o[d] = 0.0;
                for (int64_t j = 0; j < L * K; ++j) {
                    const double a = attention_weights[hq * L * K + j];
                    for (int64_t d = 0; d < D; ++d)
                        o[d] += a * smp[j][d];
                }
            }
        }
    }
}

/*
 * Backward of <out, g>, g = grad_out[b,q,m,:], from the sum above.  For each
 * sample, with s = sample(x, y) and its partial derivatives
 *   ds/dx = sum over the cell's pixels of tent'(x - j) tent(y - i) V[i, j],
 *   ds/dy = sum over the cell's pixels of tent(x - j) tent'(y - i) V[i, j]
 * (tent' the slopes of cell_of; outside pixels are zero, a piecewise-constant
 * mask, so they drop out of the derivatives too):
 *   grad_attention_weights = <g, s>                       (out is linear in A)
 *   grad_loc_x             = A * W * <g, ds/dx>            (dx/du = W)
 *   grad_loc_y             = A * H * <g, ds/dy>            (dy/dv = H)
 *   grad_value[pixel]     += A * tent(x - j) tent(y - i) * g   (out is linear in V)
 * A sample whose cell has no pixel inside the map (NaN or infinite
 * coordinates included) has s = 0 and zero derivatives: it contributes
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
            double smp[D], dsx[D], dsy[D];
            for (int64_t q = 0; q < Q; ++q) {
                const int64_t hq = (b * Q + q) * M + m;
                const double *g = grad_out + hq * D;
                for (int64_t l = 0; l < L; ++l) {
                    const int64_t H = spatial_shapes[2 * l];
                    const int64_t W = spatial_shapes[2 * l + 1];
                    const int64_t row0 = b * S + level_start_index[l];
                    const double *img = value + (row0 * M + m) * D;
                    double *gimg = grad_value + (row0 * M + m) * D;
                    for (int64_t k = 0; k < K; ++k) {
                        const int64_t s = hq * L * K + l * K + k;
                        const double a = attention_weights[s];
                        double u = sampling_locations[2 * s], v = sampling_locations[2 * s + 1];
                        double x = u * (double)W - 0.5;
                        double y = v * (double)H - 0.5;
                        cell_taps t;
                        cell_of(x, y, H, W, &t);
                        for (int64_t d = 0; d < D; ++d) {
                            smp[d] = 0.0;
                            dsx[d] = 0.0;
                            dsy[d] = 0.0;
                        }
                        for (int c = 0; c < t.n; ++c) {
                            const double *vr = img + t.pix[c] * M * D;
                            for (int64_t d = 0; d < D; ++d) {
                                smp[d] += t.wx[c] * t.wy[c] * vr[d];
                                dsx[d] += t.sx[c] * t.wy[c] * vr[d];
                                dsy[d] += t.wx[c] * t.sy[c] * vr[d];
                            }
                        }
                        double ga = 0.0, gx = 0.0, gy = 0.0;
                        for (int64_t d = 0; d < D; ++d) {
                            ga += g[d] * smp[d];
                            gx += g[d] * dsx[d];
                            gy += g[d] * dsy[d];
                        }
                        grad_attn[s] = ga;
                        grad_loc[2 * s] = a * (double)W * gx;
                        grad_loc[2 * s + 1] = a * (double)H * gy;
                        for (int c = 0; c < t.n; ++c) {
                            double *gv = gimg + t.pix[c] * M * D;
                            double aw = a * t.wx[c] * t.wy[c];
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
