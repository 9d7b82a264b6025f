/*
 * einsum_ref.c -- CPU oracle for the extended EinSum (TEST INFRASTRUCTURE).
 *
 * This file is part of the oracle that the HIP path is checked against. It is
 * loaded only by the test-suite, the smoke entry point and the bench's CPU
 * baseline leg; the product library never links it, and it shares no code,
 * header or table with the HIP kernels.
 *
 * Definition followed (page "EinDecomp：基于爱因斯坦求和与张量关系代数的自动张量并行分解算法",
 * section 2.1 on the extended Einstein notation): a label that appears on the
 * right-hand side but not on the left is contracted; the extension replaces
 * the sum by any associative and commutative aggregate (sum, max, min,
 * logsumexp) and the product by any binary scalar function, e.g. (x-y)^2.
 * So, for every output index z,
 *
 *     Z[z] = post_scale * AGG over all contracted index tuples c of
 *                          JOIN( X[(z,c) restricted to X's labels],
 *                                Y[(z,c) restricted to Y's labels] )
 *
 * and, with no contracted label, Z[z] = JOIN(...) (aggregate NONE).
 * The contracted tuples are visited in ascending lexicographic order of the
 * contracted labels as the caller lists them. Floating point is carried in
 * double throughout; integers in int64. logsumexp is evaluated as
 * m + log(sum exp(v - m)) with m the maximum, which is the definition
 * log(sum exp v) written so that it does not overflow.
 *
 * Nothing here is blocked, fused or reordered: one output element at a time,
 * one contracted tuple at a time, offsets recomputed from the strides for
 * every term. OpenMP only splits the list of output elements among threads.
 */
#include <math.h>
#include <stdint.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define OR_MAX_LABELS 26

enum { OR_JOIN_MUL = 0, OR_JOIN_SQDIFF = 1, OR_JOIN_ADD = 2, OR_JOIN_IDENT = 3, OR_JOIN_EXP_SUB = 4, OR_JOIN_SUB = 5 };
enum { OR_AGG_NONE = 0, OR_AGG_SUM = 1, OR_AGG_MAX = 2, OR_AGG_MIN = 3, OR_AGG_LSE = 4 };

static double join_f(int op, double x, double y)
{
    switch (op) {
    case OR_JOIN_MUL: return x * y;
    case OR_JOIN_SQDIFF: return (x - y) * (x - y);
    case OR_JOIN_ADD: return x + y;
    case OR_JOIN_IDENT: return x;
    case OR_JOIN_EXP_SUB: return exp(x - y);
    case OR_JOIN_SUB: return x - y;
    }
    return NAN;
}

static int64_t join_i(int op, int64_t x, int64_t y)
{
    switch (op) {
    case OR_JOIN_MUL: return x * y;
    case OR_JOIN_SQDIFF: return (x - y) * (x - y);
    case OR_JOIN_ADD: return x + y;
    case OR_JOIN_IDENT: return x;
    case OR_JOIN_SUB: return x - y;
    }
    return 0;
}

/* Row-major strides of a tensor whose dimensions are the listed labels. */
static void strides_of(int n, const int32_t *labels, const int64_t *bounds, int64_t *st)
{
    int64_t s = 1;
    for (int p = n - 1; p >= 0; --p) {
        st[p] = s;
        s *= bounds[labels[p]];
    }
}

static int64_t offset_of(int n, const int32_t *labels, const int64_t *st, const int64_t *idx)
{
    int64_t o = 0;
    for (int p = 0; p < n; ++p)
        o += idx[labels[p]] * st[p];
    return o;
}

/* Advance the odometer over the contracted labels (last label fastest).
 * Returns 0 once every tuple has been visited. */
static int next_tuple(int nc, const int32_t *cl, const int64_t *bounds, int64_t *idx)
{
    for (int p = nc - 1; p >= 0; --p) {
        if (++idx[cl[p]] < bounds[cl[p]])
            return 1;
        idx[cl[p]] = 0;
    }
    return 0;
}

/* 1 when some contracted label has extent 0: the fold then runs over no
   terms and the result is the aggregate's identity. */
static int empty_range(int nc, const int32_t *cl, const int64_t *bounds)
{
    for (int p = 0; p < nc; ++p)
        if (bounds[cl[p]] == 0)
            return 1;
    return 0;
}

static int check_args(int n_labels, int nx, int ny, int nz, int nc, int join, int agg)
{
    if (n_labels < 1 || n_labels > OR_MAX_LABELS || nx < 0 || ny < 0 || nz < 0 || nc < 0)
        return -1;
    if (agg == OR_AGG_NONE && nc != 0)
        return -2;
    if (ny == 0 && join != OR_JOIN_IDENT)
        return -3;
    return 0;
}

/* Decompose output element `zi` (row-major over the output labels). */
static void out_index(int nz, const int32_t *zl, const int64_t *bounds, int64_t zi, int64_t *idx)
{
    for (int p = nz - 1; p >= 0; --p) {
        idx[zl[p]] = zi % bounds[zl[p]];
        zi /= bounds[zl[p]];
    }
}

int oracle_einsum_f64(int n_labels, const int64_t *bounds,
                      int nx, const int32_t *xl, const double *x,
                      int ny, const int32_t *yl, const double *y,
                      int nz, const int32_t *zl, int nc, const int32_t *cl,
                      int join, int agg, double post_scale,
                      int64_t n_out, const int64_t *out_idx, double *z, int threads)
{
    int rc = check_args(n_labels, nx, ny, nz, nc, join, agg);
    if (rc)
        return rc;
    int64_t xs[OR_MAX_LABELS], ys[OR_MAX_LABELS];
    strides_of(nx, xl, bounds, xs);
    strides_of(ny, yl, bounds, ys);
    const int empty = empty_range(nc, cl, bounds);
#ifdef _OPENMP
    if (threads > 0)
        omp_set_num_threads(threads);
#pragma omp parallel for schedule(dynamic, 64)
#endif
    for (int64_t o = 0; o < n_out; ++o) {
        int64_t idx[OR_MAX_LABELS];
        memset(idx, 0, sizeof(idx));
        out_index(nz, zl, bounds, out_idx ? out_idx[o] : o, idx);
        double r;
        if (agg == OR_AGG_NONE) {
            double xv = x[offset_of(nx, xl, xs, idx)];
            double yv = ny ? y[offset_of(ny, yl, ys, idx)] : 0.0;
            r = join_f(join, xv, yv);
        } else if (agg == OR_AGG_LSE) {
            /* pass 1: the maximum term; pass 2: the sum of exp(v - max). */
            double m = -INFINITY;
            if (!empty) do {
                double yv = ny ? y[offset_of(ny, yl, ys, idx)] : 0.0;
                double v = join_f(join, x[offset_of(nx, xl, xs, idx)], yv);
                if (v > m) m = v;
            } while (next_tuple(nc, cl, bounds, idx));
            if (m == -INFINITY) {
                r = -INFINITY;
            } else {
                double s = 0.0;
                do {
                    double yv = ny ? y[offset_of(ny, yl, ys, idx)] : 0.0;
                    s += exp(join_f(join, x[offset_of(nx, xl, xs, idx)], yv) - m);
                } while (next_tuple(nc, cl, bounds, idx));
                r = m + log(s);
            }
        } else {
            double acc = agg == OR_AGG_SUM ? 0.0 : (agg == OR_AGG_MAX ? -INFINITY : INFINITY);
            if (!empty) do {
                double yv = ny ? y[offset_of(ny, yl, ys, idx)] : 0.0;
                double v = join_f(join, x[offset_of(nx, xl, xs, idx)], yv);
                if (agg == OR_AGG_SUM) acc += v;
                else if (agg == OR_AGG_MAX) acc = v > acc ? v : acc;
                else acc = v < acc ? v : acc;
            } while (next_tuple(nc, cl, bounds, idx));
            r = acc;
        }
        z[o] = post_scale * r;
    }
    return 0;
}

int oracle_einsum_i64(int n_labels, const int64_t *bounds,
                      int nx, const int32_t *xl, const int64_t *x,
                      int ny, const int32_t *yl, const int64_t *y,
                      int nz, const int32_t *zl, int nc, const int32_t *cl,
                      int join, int agg,
                      int64_t n_out, const int64_t *out_idx, int64_t *z, int threads)
{
    int rc = check_args(n_labels, nx, ny, nz, nc, join, agg);
    if (rc)
        return rc;
    if (join == OR_JOIN_EXP_SUB || agg == OR_AGG_LSE)
        return -4; /* not defined on integers */
    int64_t xs[OR_MAX_LABELS], ys[OR_MAX_LABELS];
    strides_of(nx, xl, bounds, xs);
    strides_of(ny, yl, bounds, ys);
    const int empty = empty_range(nc, cl, bounds);
#ifdef _OPENMP
    if (threads > 0)
        omp_set_num_threads(threads);
#pragma omp parallel for schedule(dynamic, 64)
#endif
    for (int64_t o = 0; o < n_out; ++o) {
        int64_t idx[OR_MAX_LABELS];
        memset(idx, 0, sizeof(idx));
        out_index(nz, zl, bounds, out_idx ? out_idx[o] : o, idx);
        int64_t r;
        if (agg == OR_AGG_NONE) {
            int64_t yv = ny ? y[offset_of(ny, yl, ys, idx)] : 0;
            r = join_i(join, x[offset_of(nx, xl, xs, idx)], yv);
        } else {
            int64_t acc = agg == OR_AGG_SUM ? 0 : (agg == OR_AGG_MAX ? INT64_MIN : INT64_MAX);
            if (!empty) do {
                int64_t yv = ny ? y[offset_of(ny, yl, ys, idx)] : 0;
                int64_t v = join_i(join, x[offset_of(nx, xl, xs, idx)], yv);
                if (agg == OR_AGG_SUM) acc += v;
                else if (agg == OR_AGG_MAX) acc = v > acc ? v : acc;
                else acc = v < acc ? v : acc;
            } while (next_tuple(nc, cl, bounds, idx));
            r = acc;
        }
        z[o] = r;
    }
    return 0;
}

int oracle_max_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}
