/*
 * oracle/conv_oracle.c -- plain CPU reference for the 2-D convolution forward
 * pass (FPROP), its gradients (backward passes with respect to x and F), the
 * pooling forward pass and the batch-reduce GEMM.  TEST INFRASTRUCTURE ONLY: only the tests, the smoke check and
 * the CPU-baseline leg of the benchmark may load this library.  It shares no
 * code, header, table or helper with the GPU path.
 *
 * What it computes (direct convolution, cross-correlation form, zero padding):
 *
 *   acc[n,k,p,q] = sum_{c<C} sum_{r<R} sum_{s<S}  X(n, c, p*u + r - pad_top,
 *                                                       q*v + s - pad_left)
 *                                                 * F[k, c, r, s]
 *   X(n,c,h,w)   = x[n*sn + c*sc + h*sh + w*sw]  if 0 <= h < H and 0 <= w < W,
 *                  0 otherwise
 *   y[n,k,p,q]   = alpha * acc + beta * y_old[n,k,p,q]   (y_old unread if beta == 0)
 *   B[n,k,p,q]   = sum_{c,r,s} |X(...) * F[k,c,r,s]|      (error-bound weight)
 *
 *   P = floor((H + pad_top + pad_bottom - R) / u) + 1
 *   Q = floor((W + pad_left + pad_right - S) / v) + 1
 *
 * Sources: the maxDNN page (Lavin, "maxDNN: An Efficient Convolution Kernel
 * for Deep Learning with Maxwell GPUs"), section "Proposed Method": every
 * output feature-map coordinate is the product of the input receptive field
 * with the filter weights; the zero-memory direct-convolution page (Zhang,
 * Franchetti et al., "High Performance Zero-Memory Overhead Direct
 * Convolutions"), Abstract and "Proposed Method": the convolution is computed
 * directly, with no packing or copying; the cuDNN page (Chetlur et al.,
 * "cuDNN: Efficient Primitives for Deep Learning"), "Proposed Method":
 * tensors are described by dimensions plus arbitrary strides, and padding may
 * be asymmetric (non-square inputs, asymmetric padding).  The pages print no
 * formula: no filter flip, zero padding, floor output size, BLAS-style
 * alpha/beta and element (not byte) strides are the plain readings taken.
 *
 * Arithmetic: everything in IEEE double, accumulated in the fixed order
 * c, r, s.  Build with -ffp-contract=off so no fused multiply-add changes the
 * rounding.  Inputs of lower precision (fp32, bf16) are widened to double by
 * the caller, which is exact.
 */
#include <math.h>
#include <stdint.h>
#include <stddef.h>

#ifdef _OPENMP
#include <omp.h>
#endif

/* One convolution problem.  Mirrored field by field by a ctypes Structure in
 * oracle/__init__.py; keep the two in the same order. */
typedef struct {
    int64_t N, C, H, W;            /* input dims */
    int64_t sn, sc, sh, sw;        /* input element strides */
    int64_t K, R, S;               /* filter dims; filter is packed K,C,R,S */
    int64_t pad_top, pad_bottom, pad_left, pad_right;
    int64_t u, v;                  /* stride along H, along W */
} oracle_conv_problem;

/* 0 on success, -1 if the problem is malformed or the output would be empty. */
int oracle_output_dims(const oracle_conv_problem* pb, int64_t* P, int64_t* Q)
{
    if (pb->N < 1 || pb->C < 1 || pb->H < 1 || pb->W < 1) return -1;
    if (pb->K < 1 || pb->R < 1 || pb->S < 1) return -1;
    if (pb->u < 1 || pb->v < 1) return -1;
    if (pb->pad_top < 0 || pb->pad_bottom < 0 || pb->pad_left < 0 || pb->pad_right < 0) return -1;
    int64_t hspan = pb->H + pb->pad_top + pb->pad_bottom - pb->R;
    int64_t wspan = pb->W + pb->pad_left + pb->pad_right - pb->S;
    if (hspan < 0 || wspan < 0) return -1;
    *P = hspan / pb->u + 1;      /* both spans are >= 0 here, so '/' is floor */
    *Q = wspan / pb->v + 1;
    return 0;
}

/* Input value with zero padding outside the H x W plane. */
static double input_at(const oracle_conv_problem* pb, const double* x,
                       int64_t n, int64_t c, int64_t h, int64_t w)
{
    if (h < 0 || h >= pb->H || w < 0 || w >= pb->W) return 0.0;
    return x[n * pb->sn + c * pb->sc + h * pb->sh + w * pb->sw];
}

/* The sum for one output coordinate, and its absolute-value twin. */
static void one_output(const oracle_conv_problem* pb, const double* x, const double* f,
                       int64_t n, int64_t k, int64_t p, int64_t q,
                       double* acc_out, double* bound_out)
{
    double acc = 0.0, bound = 0.0;
    for (int64_t c = 0; c < pb->C; ++c) {
        for (int64_t r = 0; r < pb->R; ++r) {
            for (int64_t s = 0; s < pb->S; ++s) {
                int64_t h = p * pb->u + r - pb->pad_top;
                int64_t w = q * pb->v + s - pb->pad_left;
                double xv = input_at(pb, x, n, c, h, w);
                double fv = f[((k * pb->C + c) * pb->R + r) * pb->S + s];
                double prod = xv * fv;
                acc += prod;
                bound += fabs(prod);
            }
        }
    }
    *acc_out = acc;
    *bound_out = bound;
}

/*
 * Full output.  y and bound (either may be NULL) are packed N,K,P,Q.
 * y_old is packed N,K,P,Q and read only when beta != 0.
 * nthreads <= 0 means the OpenMP default.  Returns 0, or -1 on a bad problem.
 */
int oracle_conv2d_fprop(const oracle_conv_problem* pb,
                        const double* x, const double* f,
                        double alpha, double beta, const double* y_old,
                        double* y, double* bound, int nthreads)
{
    int64_t P, Q;
    if (oracle_output_dims(pb, &P, &Q) != 0) return -1;
    if (beta != 0.0 && y_old == NULL) return -1;
    const int64_t N = pb->N, K = pb->K;
#ifdef _OPENMP
    if (nthreads <= 0) nthreads = omp_get_max_threads();
#pragma omp parallel for collapse(2) schedule(dynamic, 1) num_threads(nthreads)
#endif
    for (int64_t n = 0; n < N; ++n) {
        for (int64_t k = 0; k < K; ++k) {
            for (int64_t p = 0; p < P; ++p) {
                for (int64_t q = 0; q < Q; ++q) {
                    double acc, bnd;
                    one_output(pb, x, f, n, k, p, q, &acc, &bnd);
                    int64_t o = ((n * K + k) * P + p) * Q + q;
                    double val = alpha * acc;
                    if (beta != 0.0) val += beta * y_old[o];
                    if (y) y[o] = val;
                    if (bound) bound[o] = bnd;
                }
            }
        }
    }
    (void)nthreads;
    return 0;
}

/*
 * Selected outputs only.  idx holds count coordinates as (n, k, p, q) int64
 * quadruples.  y_old_vals (read only when beta != 0) holds y_old at those
 * coordinates, in the same order; y and bound receive count values each.
 * Returns 0, or -1 on a bad problem or a coordinate out of range.
 */
int oracle_conv2d_fprop_at(const oracle_conv_problem* pb,
                           const double* x, const double* f,
                           double alpha, double beta, const double* y_old_vals,
                           const int64_t* idx, int64_t count,
                           double* y, double* bound, int nthreads)
{
    int64_t P, Q;
    if (oracle_output_dims(pb, &P, &Q) != 0) return -1;
    if (beta != 0.0 && y_old_vals == NULL) return -1;
    for (int64_t i = 0; i < count; ++i) {
        const int64_t* t = idx + 4 * i;
        if (t[0] < 0 || t[0] >= pb->N || t[1] < 0 || t[1] >= pb->K ||
            t[2] < 0 || t[2] >= P || t[3] < 0 || t[3] >= Q) return -1;
    }
#ifdef _OPENMP
    if (nthreads <= 0) nthreads = omp_get_max_threads();
#pragma omp parallel for schedule(dynamic, 64) num_threads(nthreads)
#endif
    for (int64_t i = 0; i < count; ++i) {
        const int64_t* t = idx + 4 * i;
        double acc, bnd;
        one_output(pb, x, f, t[0], t[1], t[2], t[3], &acc, &bnd);
        double val = alpha * acc;
        if (beta != 0.0) val += beta * y_old_vals[i];
        if (y) y[i] = val;
        if (bound) bound[i] = bnd;
    }
    (void)nthreads;
    return 0;
}

/*
 * Backward pass with respect to the input (data gradient).  The pages name
 * the backward pass (cuDNN page, "Proposed Method": forward and backward
 * routines for convolution; maxDNN page, Abstract and research question RQ4:
 * the same techniques are expected to carry over to BPROP) but print no
 * formula.  The plain reading taken: the gradient of the forward sum above
 * with respect to x, i.e. its adjoint, for the same geometry:
 *
 *   dacc[n,c,h,w] = sum_{k<K} sum_{r<R} sum_{s<S}  dY(n, k, p, q) * F[k, c, r, s]
 *                   over the (r, s) with  p*u = h + pad_top - r,   0 <= p < P,
 *                                         q*v = w + pad_left - s,  0 <= q < Q
 *   dY(n,k,p,q)   = dy[n*sdy[0] + k*sdy[1] + p*sdy[2] + q*sdy[3]]
 *   dx[n,c,h,w]   = alpha * dacc + beta * dx_old[n,c,h,w]   (dx_old unread if beta == 0)
 *   B[n,c,h,w]    = sum of |dY * F| over the same terms     (error-bound weight)
 *
 * with P, Q the forward output size of the problem (oracle_output_dims) and
 * N, C, H, W the input (= dx) dims.  Accumulated in double in the fixed
 * order k, r, s.
 */
static void one_dgrad(const oracle_conv_problem* pb, int64_t P, int64_t Q,
                      const double* dy, const int64_t* sdy, const double* f,
                      int64_t n, int64_t c, int64_t h, int64_t w,
                      double* acc_out, double* bound_out)
{
    double acc = 0.0, bound = 0.0;
    for (int64_t k = 0; k < pb->K; ++k) {
        for (int64_t r = 0; r < pb->R; ++r) {
            int64_t hh = h + pb->pad_top - r;
            if (hh < 0 || hh % pb->u != 0 || hh / pb->u >= P) continue;
            int64_t p = hh / pb->u;
            for (int64_t s = 0; s < pb->S; ++s) {
                int64_t ww = w + pb->pad_left - s;
                if (ww < 0 || ww % pb->v != 0 || ww / pb->v >= Q) continue;
                int64_t q = ww / pb->v;
                double dv = dy[n * sdy[0] + k * sdy[1] + p * sdy[2] + q * sdy[3]];
                double fv = f[((k * pb->C + c) * pb->R + r) * pb->S + s];
                double prod = dv * fv;
                acc += prod;
                bound += fabs(prod);
            }
        }
    }
    *acc_out = acc;
    *bound_out = bound;
}

/*
 * Whole data gradient.  dx and bound (either may be NULL) are packed N,C,H,W;
 * dx_old is packed N,C,H,W and read only when beta != 0.  dy is read through
 * the element strides sdy[4] (n, k, p, q).  Returns 0, or -1 on a bad problem.
 */
int oracle_conv2d_bwd_data(const oracle_conv_problem* pb,
                           const double* dy, const int64_t* sdy, const double* f,
                           double alpha, double beta, const double* dx_old,
                           double* dx, double* bound, int nthreads)
{
    int64_t P, Q;
    if (oracle_output_dims(pb, &P, &Q) != 0) return -1;
    if (beta != 0.0 && dx_old == NULL) return -1;
    const int64_t N = pb->N, C = pb->C, H = pb->H, W = pb->W;
#ifdef _OPENMP
    if (nthreads <= 0) nthreads = omp_get_max_threads();
#pragma omp parallel for collapse(2) schedule(dynamic, 1) num_threads(nthreads)
#endif
    for (int64_t n = 0; n < N; ++n) {
        for (int64_t c = 0; c < C; ++c) {
            for (int64_t h = 0; h < H; ++h) {
                for (int64_t w = 0; w < W; ++w) {
                    double acc, bnd;
                    one_dgrad(pb, P, Q, dy, sdy, f, n, c, h, w, &acc, &bnd);
                    int64_t o = ((n * C + c) * H + h) * W + w;
                    double val = alpha * acc;
                    if (beta != 0.0) val += beta * dx_old[o];
                    if (dx) dx[o] = val;
                    if (bound) bound[o] = bnd;
                }
            }
        }
    }
    (void)nthreads;
    return 0;
}

/*
 * Selected data-gradient values.  idx holds count (n, c, h, w) int64
 * quadruples; dx_old_vals (read only when beta != 0) the old values there.
 * Returns 0, or -1 on a bad problem or a coordinate out of range.
 */
int oracle_conv2d_bwd_data_at(const oracle_conv_problem* pb,
                              const double* dy, const int64_t* sdy, const double* f,
                              double alpha, double beta, const double* dx_old_vals,
                              const int64_t* idx, int64_t count,
                              double* dx, double* bound, int nthreads)
{
    int64_t P, Q;
    if (oracle_output_dims(pb, &P, &Q) != 0) return -1;
    if (beta != 0.0 && dx_old_vals == NULL) return -1;
    for (int64_t i = 0; i < count; ++i) {
        const int64_t* t = idx + 4 * i;
        if (t[0] < 0 || t[0] >= pb->N || t[1] < 0 || t[1] >= pb->C ||
            t[2] < 0 || t[2] >= pb->H || t[3] < 0 || t[3] >= pb->W) return -1;
    }
#ifdef _OPENMP
    if (nthreads <= 0) nthreads = omp_get_max_threads();
#pragma omp parallel for schedule(dynamic, 64) num_threads(nthreads)
#endif
    for (int64_t i = 0; i < count; ++i) {
        const int64_t* t = idx + 4 * i;
        double acc, bnd;
        one_dgrad(pb, P, Q, dy, sdy, f, t[0], t[1], t[2], t[3], &acc, &bnd);
        double val = alpha * acc;
        if (beta != 0.0) val += beta * dx_old_vals[i];
        if (dx) dx[i] = val;
        if (bound) bound[i] = bnd;
    }
    (void)nthreads;
    return 0;
}

/*
 * Backward pass with respect to the filter (filter gradient): the gradient
 * of the forward sum with respect to F, i.e. its adjoint in F (same reading
 * as the data gradient above; the pages print no formula):
 *
 *   dacc[k,c,r,s] = sum_{n<N} sum_{p<P} sum_{q<Q}  dY(n, k, p, q) * X(n, c, p*u + r - pad_top,
 *                                                                         q*v + s - pad_left)
 *   dw[k,c,r,s]   = alpha * dacc + beta * dw_old[k,c,r,s]   (dw_old unread if beta == 0)
 *   B[k,c,r,s]    = sum of |dY * X| over the same terms     (error-bound weight)
 *
 * X is x read through the problem's element strides with zero padding, dY
 * is dy read through sdy[4]; dw is packed K,C,R,S.  Accumulated in double in
 * the fixed order n, p, q.
 */
static void one_wgrad(const oracle_conv_problem* pb, int64_t P, int64_t Q,
                      const double* x, const double* dy, const int64_t* sdy,
                      int64_t k, int64_t c, int64_t r, int64_t s,
                      double* acc_out, double* bound_out)
{
    double acc = 0.0, bound = 0.0;
    for (int64_t n = 0; n < pb->N; ++n) {
        for (int64_t p = 0; p < P; ++p) {
            for (int64_t q = 0; q < Q; ++q) {
                double xv = input_at(pb, x, n, c, p * pb->u + r - pb->pad_top, q * pb->v + s - pb->pad_left);
                double dv = dy[n * sdy[0] + k * sdy[1] + p * sdy[2] + q * sdy[3]];
                double prod = dv * xv;
                acc += prod;
                bound += fabs(prod);
            }
        }
    }
    *acc_out = acc;
    *bound_out = bound;
}

/*
 * Whole filter gradient.  dw and bound (either may be NULL) are packed
 * K,C,R,S; dw_old is packed K,C,R,S and read only when beta != 0.  x is read
 * through the problem's strides, dy through sdy[4] (n, k, p, q).
 * Returns 0, or -1 on a bad problem.
 */
int oracle_conv2d_bwd_filter(const oracle_conv_problem* pb,
                             const double* x, const double* dy, const int64_t* sdy,
                             double alpha, double beta, const double* dw_old,
                             double* dw, double* bound, int nthreads)
{
    int64_t P, Q;
    if (oracle_output_dims(pb, &P, &Q) != 0) return -1;
    if (beta != 0.0 && dw_old == NULL) return -1;
    const int64_t K = pb->K, C = pb->C, R = pb->R, S = pb->S;
#ifdef _OPENMP
    if (nthreads <= 0) nthreads = omp_get_max_threads();
#pragma omp parallel for collapse(2) schedule(dynamic, 1) num_threads(nthreads)
#endif
    for (int64_t k = 0; k < K; ++k) {
        for (int64_t c = 0; c < C; ++c) {
            for (int64_t r = 0; r < R; ++r) {
                for (int64_t s = 0; s < S; ++s) {
                    double acc, bnd;
                    one_wgrad(pb, P, Q, x, dy, sdy, k, c, r, s, &acc, &bnd);
                    int64_t o = ((k * C + c) * R + r) * S + s;
                    double val = alpha * acc;
                    if (beta != 0.0) val += beta * dw_old[o];
                    if (dw) dw[o] = val;
                    if (bound) bound[o] = bnd;
                }
            }
        }
    }
    (void)nthreads;
    return 0;
}

/*
 * Selected filter-gradient values.  idx holds count (k, c, r, s) int64
 * quadruples; dw_old_vals (read only when beta != 0) the old values there.
 * Returns 0, or -1 on a bad problem or a coordinate out of range.
 */
int oracle_conv2d_bwd_filter_at(const oracle_conv_problem* pb,
                                const double* x, const double* dy, const int64_t* sdy,
                                double alpha, double beta, const double* dw_old_vals,
                                const int64_t* idx, int64_t count,
                                double* dw, double* bound, int nthreads)
{
    int64_t P, Q;
    if (oracle_output_dims(pb, &P, &Q) != 0) return -1;
    if (beta != 0.0 && dw_old_vals == NULL) return -1;
    for (int64_t i = 0; i < count; ++i) {
        const int64_t* t = idx + 4 * i;
        if (t[0] < 0 || t[0] >= pb->K || t[1] < 0 || t[1] >= pb->C ||
            t[2] < 0 || t[2] >= pb->R || t[3] < 0 || t[3] >= pb->S) return -1;
    }
#ifdef _OPENMP
    if (nthreads <= 0) nthreads = omp_get_max_threads();
#pragma omp parallel for schedule(dynamic, 4) num_threads(nthreads)
#endif
    for (int64_t i = 0; i < count; ++i) {
        const int64_t* t = idx + 4 * i;
        double acc, bnd;
        one_wgrad(pb, P, Q, x, dy, sdy, t[0], t[1], t[2], t[3], &acc, &bnd);
        double val = alpha * acc;
        if (beta != 0.0) val += beta * dw_old_vals[i];
        if (dw) dw[i] = val;
        if (bound) bound[i] = bnd;
    }
    (void)nthreads;
    return 0;
}

/*
 * Pooling forward pass.  The cuDNN page ("Proposed Method") lists pooling
 * among the library's forward and backward routines; it prints no formula.
 * The plain reading taken, over the same window geometry as the convolution
 * (window R x S, strides u, v, per-side padding; output size P x Q by the
 * same floor rule), with C channels pooled independently:
 *
 *   mode 0 (max):           acc = max of X over the window positions inside
 *                            the H x W plane (padding never wins), 0 if none
 *   mode 1 (average, pad):  acc = (sum of X over the window positions inside
 *                            the plane) / (R * S)     (padding counts as 0)
 *   mode 2 (average):       acc = that sum / (number of positions inside the
 *                            plane), 0 if none
 *   y[n,c,p,q] = alpha * acc + beta * y_old[n,c,p,q]   (y_old unread if beta == 0)
 *
 * X is x read through the problem's strides.  The problem's K is unused.
 * y is packed N,C,P,Q.  Sums run in the fixed order r, s in double.
 */
static double one_pool(const oracle_conv_problem* pb, const double* x, int mode,
                       int64_t n, int64_t c, int64_t p, int64_t q)
{
    double best = 0.0, sum = 0.0;
    int64_t inside = 0;
    for (int64_t r = 0; r < pb->R; ++r) {
        for (int64_t s = 0; s < pb->S; ++s) {
            int64_t h = p * pb->u + r - pb->pad_top;
            int64_t w = q * pb->v + s - pb->pad_left;
            if (h < 0 || h >= pb->H || w < 0 || w >= pb->W) continue;
            double v = x[n * pb->sn + c * pb->sc + h * pb->sh + w * pb->sw];
            if (inside == 0 || v > best) best = v;
            sum += v;
            ++inside;
        }
    }
    if (mode == 0) return inside ? best : 0.0;
    if (mode == 1) return sum / (double)(pb->R * pb->S);
    return inside ? sum / (double)inside : 0.0;
}

/* Whole pooled output; y packed N,C,P,Q.  Returns 0, or -1 on a bad problem or mode. */
int oracle_pool_forward(const oracle_conv_problem* pb, const double* x, int mode,
                        double alpha, double beta, const double* y_old, double* y, int nthreads)
{
    int64_t P, Q;
    if (oracle_output_dims(pb, &P, &Q) != 0) return -1;
    if (mode < 0 || mode > 2) return -1;
    if (beta != 0.0 && y_old == NULL) return -1;
    const int64_t N = pb->N, C = pb->C;
#ifdef _OPENMP
    if (nthreads <= 0) nthreads = omp_get_max_threads();
#pragma omp parallel for collapse(2) schedule(dynamic, 1) num_threads(nthreads)
#endif
    for (int64_t n = 0; n < N; ++n) {
        for (int64_t c = 0; c < C; ++c) {
            for (int64_t p = 0; p < P; ++p) {
                for (int64_t q = 0; q < Q; ++q) {
                    int64_t o = ((n * C + c) * P + p) * Q + q;
                    double val = alpha * one_pool(pb, x, mode, n, c, p, q);
                    if (beta != 0.0) val += beta * y_old[o];
                    y[o] = val;
                }
            }
        }
    }
    (void)nthreads;
    return 0;
}

/*
 * Batch-reduce GEMM, the single-building-block page's kernel ("Proposed
 * Method": the products of a batch of input sub-tensor blocks reduced into
 * one output block), written out:
 *
 *   C[m,n] = alpha * sum_{i<batch} sum_{k<K} A_i[m,k] * B_i[k,n] + beta * C_old[m,n]
 *   A_i[m,k] = a[i*sa_i + m*sa_m + k*sa_k],  B_i[k,n] = b[i*sb_i + k*sb_k + n*sb_n]
 *   bound[m,n] = sum of |A_i[m,k] * B_i[k,n]|
 *
 * C and bound are packed M x N row-major; C_old (read only when beta != 0)
 * likewise.  Order i, k, in double.  Returns 0, or -1 on bad sizes.
 */
int oracle_brgemm(int64_t M, int64_t N, int64_t K, int64_t batch,
                  const double* a, int64_t sa_i, int64_t sa_m, int64_t sa_k,
                  const double* b, int64_t sb_i, int64_t sb_k, int64_t sb_n,
                  double alpha, double beta, const double* c_old,
                  double* c, double* bound, int nthreads)
{
    if (M < 1 || N < 1 || K < 1 || batch < 1) return -1;
    if (beta != 0.0 && c_old == NULL) return -1;
#ifdef _OPENMP
    if (nthreads <= 0) nthreads = omp_get_max_threads();
#pragma omp parallel for collapse(2) schedule(dynamic, 16) num_threads(nthreads)
#endif
    for (int64_t m = 0; m < M; ++m) {
        for (int64_t n = 0; n < N; ++n) {
            double acc = 0.0, bnd = 0.0;
            for (int64_t i = 0; i < batch; ++i) {
                for (int64_t k = 0; k < K; ++k) {
                    double prod = a[i * sa_i + m * sa_m + k * sa_k] * b[i * sb_i + k * sb_k + n * sb_n];
                    acc += prod;
                    bnd += fabs(prod);
                }
            }
            double val = alpha * acc;
            if (beta != 0.0) val += beta * c_old[m * N + n];
            if (c) c[m * N + n] = val;
            if (bound) bound[m * N + n] = bnd;
        }
    }
    (void)nthreads;
    return 0;
}

/* Number of OpenMP threads a call with nthreads <= 0 would use. */
int oracle_default_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}
