/*
 * CPU float64 oracle for batched weighted isotonic regression.
 *
 * TEST INFRASTRUCTURE ONLY.  This file is the checker, not the product: it is
 * built into liboracle.so and may be loaded only by the test suite, by the
 * package smoke check and by the CPU-baseline leg of the benchmark.  It shares
 * no code, header, table or helper with the GPU library, and it never reads a
 * value produced by the GPU library except where a caller passes a partition
 * in explicitly (iso_oracle_vjp takes block starts as an input).
 *
 * What it computes (page "Merge Hulls Without Copying Vertices: GPU Isotonic
 * Regression", Sec. 2.1, Eq. (1)): for each row, the non-decreasing z that
 * minimises sum_i w_i (z_i - y_i)^2 with strictly positive weights.  The
 * algorithm is pool adjacent violators (same page, Sec. 1: scan once and merge
 * neighbouring blocks while they violate the order), the sequential method the
 * page names as the standard one, written plainly in float64:
 *
 *   - blocks keep (sum of w*y, sum of w) with Neumaier compensation, so a block
 *     of millions of elements keeps its mean to a few ulp;
 *   - a new element is pushed as its own block; while the block below the top
 *     has a mean >= the top's mean, the two are pooled.  Pooling equal means
 *     gives the canonical partition (the page, Sec. 2.1, drops collinear
 *     points of the cumulative sum diagram, i.e. it pools equal neighbouring
 *     block means);
 *   - each element takes its block's mean.
 *
 * Semantics on the page "torchisotonic" (PyPI), section "Semantics":
 *   - weights must be strictly positive: a finite weight <= 0 makes the call
 *     report ORACLE_EWEIGHT and that row comes back NaN;
 *   - a row holding a NaN (in y or in w; also +-Inf, outside the contract)
 *     comes back all NaN, without an error;
 *   - the result is clipped to [y_min, y_max] after the fit;
 *   - increasing = 0 asks for the non-increasing fit, computed here by
 *     reversing the row, fitting non-decreasing, and reversing back.
 *
 * Block starts: block_start[i] = 1 iff element i begins a block of the pooled
 * partition (in the row's own order).  clipped[i] = 1 iff the unclipped fit z_i
 * lies strictly outside [y_min, y_max], so the clip is active there.
 *
 * The vector-Jacobian product of the fit with respect to y (same page as
 * above, Appendix C, where the product averages over the blocks; weighted
 * form derived from Eq. (1)): within a block B with fit value
 * sum_{i in B} w_i y_i / sum_{i in B} w_i, d z_B / d y_j = w_j / W_B, so
 *   grad_y_j = w_j * (sum_{i in B(j)} g_i [clip inactive at i]) / W_B.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORACLE_OK 0
#define ORACLE_EINVAL (-1)
#define ORACLE_EWEIGHT (-3)

/* Neumaier-compensated accumulator: value = s + c. */
typedef struct {
    double s, c;
} acc_t;

static void acc_add(acc_t* a, double x) {
    double t = a->s + x;
    if (fabs(a->s) >= fabs(x))
        a->c += (a->s - t) + x;
    else
        a->c += (x - t) + a->s;
    a->s = t;
}

static void acc_merge(acc_t* a, const acc_t* b) {
    acc_add(a, b->s);
    acc_add(a, b->c);
}

static double acc_value(const acc_t* a) { return a->s + a->c; }

typedef struct {
    acc_t sw;    /* sum of w over the block */
    acc_t swy;   /* sum of w*y over the block */
    int64_t start; /* first element of the block (in fitting order) */
} block_t;

static double block_mean(const block_t* b) { return acc_value(&b->swy) / acc_value(&b->sw); }

/*
 * Non-decreasing PAVA on one row given in fitting order (already reversed for
 * the non-increasing case).  Writes z (unclipped) and the block starts in
 * fitting order.  stack must hold n blocks.
 */
static void pava_row(const double* y, const double* w, int64_t n, double* z, uint8_t* start,
                     block_t* stack) {
    int64_t top = -1;
    for (int64_t i = 0; i < n; ++i) {
        double wi = w ? w[i] : 1.0;
        ++top;
        stack[top].sw.s = wi;
        stack[top].sw.c = 0.0;
        stack[top].swy.s = wi * y[i];
        stack[top].swy.c = 0.0;
        stack[top].start = i;
        while (top >= 1 && block_mean(&stack[top - 1]) >= block_mean(&stack[top])) {
            acc_merge(&stack[top - 1].sw, &stack[top].sw);
            acc_merge(&stack[top - 1].swy, &stack[top].swy);
            --top;
        }
    }
    for (int64_t b = 0; b <= top; ++b) {
        int64_t lo = stack[b].start;
        int64_t hi = (b == top) ? n : stack[b + 1].start;
        double m = block_mean(&stack[b]);
        for (int64_t i = lo; i < hi; ++i) {
            z[i] = m;
            start[i] = (uint8_t)(i == lo);
        }
    }
}

typedef struct {
    const double* y;
    const double* w;
    int64_t n;
    int increasing;
    double y_min, y_max;
    double* out;
    uint8_t* block_start;
    uint8_t* clipped;
    uint8_t* row_nan;
    int64_t row_lo, row_hi;
    int status;
} fit_job_t;

static void fit_one_row(const fit_job_t* jb, int64_t r, double* ybuf, double* wbuf, double* zbuf,
                        uint8_t* sbuf, block_t* stack, int* status) {
    const int64_t n = jb->n;
    const double* y = jb->y + r * n;
    const double* w = jb->w ? jb->w + r * n : NULL;
    double* out = jb->out + r * n;
    uint8_t* bs = jb->block_start ? jb->block_start + r * n : NULL;
    uint8_t* cl = jb->clipped ? jb->clipped + r * n : NULL;

    int nonfinite = 0, badweight = 0;
    for (int64_t i = 0; i < n; ++i) {
        if (!isfinite(y[i])) nonfinite = 1;
        if (w) {
            if (!isfinite(w[i]))
                nonfinite = 1;
            else if (!(w[i] > 0.0))
                badweight = 1;
        }
    }
    if (nonfinite || badweight) {
        for (int64_t i = 0; i < n; ++i) {
            out[i] = NAN;
            if (bs) bs[i] = 0;
            if (cl) cl[i] = 0;
        }
        if (jb->row_nan) jb->row_nan[r] = 1;
        if (badweight && !nonfinite) *status = ORACLE_EWEIGHT;
        return;
    }
    if (jb->row_nan) jb->row_nan[r] = 0;

    /* fitting order: reversed for the non-increasing fit */
    for (int64_t i = 0; i < n; ++i) {
        int64_t src = jb->increasing ? i : n - 1 - i;
        ybuf[i] = y[src];
        wbuf[i] = w ? w[src] : 1.0;
    }
    pava_row(ybuf, wbuf, n, zbuf, sbuf, stack);

    for (int64_t i = 0; i < n; ++i) {
        int64_t src = jb->increasing ? i : n - 1 - i;
        double z = zbuf[src];
        /* block start in the row's own order: element i starts a block iff it
           is the first element of its block when read left to right */
        uint8_t st;
        if (jb->increasing)
            st = sbuf[i];
        else
            st = (uint8_t)(i == 0 || sbuf[src + 1]); /* reversed: block ends at src */
        int clip = (z < jb->y_min) || (z > jb->y_max);
        double v = z;
        if (v < jb->y_min) v = jb->y_min;
        if (v > jb->y_max) v = jb->y_max;
        out[i] = v;
        if (bs) bs[i] = st;
        if (cl) cl[i] = (uint8_t)clip;
    }
}

static void* fit_worker(void* arg) {
    fit_job_t* jb = (fit_job_t*)arg;
    int64_t n = jb->n;
    double* ybuf = (double*)malloc(sizeof(double) * (size_t)(n > 0 ? n : 1));
    double* wbuf = (double*)malloc(sizeof(double) * (size_t)(n > 0 ? n : 1));
    double* zbuf = (double*)malloc(sizeof(double) * (size_t)(n > 0 ? n : 1));
    uint8_t* sbuf = (uint8_t*)malloc((size_t)(n > 0 ? n : 1) + 1);
    block_t* stack = (block_t*)malloc(sizeof(block_t) * (size_t)(n > 0 ? n : 1));
    int status = ORACLE_OK;
    if (!ybuf || !wbuf || !zbuf || !sbuf || !stack) {
        status = ORACLE_EINVAL;
    } else {
        for (int64_t r = jb->row_lo; r < jb->row_hi; ++r) {
            fit_one_row(jb, r, ybuf, wbuf, zbuf, sbuf, stack, &status);
        }
    }
    free(ybuf);
    free(wbuf);
    free(zbuf);
    free(sbuf);
    free(stack);
    jb->status = status;
    return NULL;
}

/*
 * y, w: [rows, n] float64, row-major; w may be NULL (unit weights).
 * y_min / y_max: clip bounds; pass -INFINITY / +INFINITY for none (a NaN bound
 * also means none).  out: [rows, n].  block_start, clipped: [rows, n] bytes or
 * NULL.  row_nan: [rows] bytes or NULL.  nthreads: host threads (rows are split
 * evenly; one row is always one thread, PAVA being sequential in a row).
 * Returns ORACLE_OK, ORACLE_EINVAL, or ORACLE_EWEIGHT if some row had a finite
 * weight <= 0 (that row is NaN).
 */
int iso_oracle_fit(const double* y, const double* w, int64_t rows, int64_t n, int increasing,
                   double y_min, double y_max, double* out, uint8_t* block_start,
                   uint8_t* clipped, uint8_t* row_nan, int nthreads) {
    if (rows < 0 || n < 0) return ORACLE_EINVAL;
    if (rows == 0 || n == 0) return ORACLE_OK;
    if (!y || !out) return ORACLE_EINVAL;
    if (isnan(y_min)) y_min = -INFINITY;
    if (isnan(y_max)) y_max = INFINITY;
    if (y_min > y_max) return ORACLE_EINVAL;
    if (nthreads < 1) nthreads = 1;
    if (nthreads > rows) nthreads = (int)rows;

    fit_job_t* jobs = (fit_job_t*)calloc((size_t)nthreads, sizeof(fit_job_t));
    pthread_t* th = (pthread_t*)calloc((size_t)nthreads, sizeof(pthread_t));
    if (!jobs || !th) {
        free(jobs);
        free(th);
        return ORACLE_EINVAL;
    }
    for (int t = 0; t < nthreads; ++t) {
        fit_job_t* jb = &jobs[t];
        jb->y = y;
        jb->w = w;
        jb->n = n;
        jb->increasing = increasing ? 1 : 0;
        jb->y_min = y_min;
        jb->y_max = y_max;
        jb->out = out;
        jb->block_start = block_start;
        jb->clipped = clipped;
        jb->row_nan = row_nan;
        jb->row_lo = rows * t / nthreads;
        jb->row_hi = rows * (t + 1) / nthreads;
    }
    for (int t = 1; t < nthreads; ++t) pthread_create(&th[t], NULL, fit_worker, &jobs[t]);
    fit_worker(&jobs[0]);
    for (int t = 1; t < nthreads; ++t) pthread_join(th[t], NULL);
    int status = ORACLE_OK;
    for (int t = 0; t < nthreads; ++t) {
        if (jobs[t].status == ORACLE_EINVAL) status = ORACLE_EINVAL;
        else if (jobs[t].status == ORACLE_EWEIGHT && status == ORACLE_OK) status = ORACLE_EWEIGHT;
    }
    free(jobs);
    free(th);
    return status;
}

/*
 * Vector-Jacobian product of the (clipped) fit with respect to y, for the
 * partition given by block_start (block_start[i] = 1 where a block begins;
 * element 0 always begins one) and the clip flags.  g, w, out: [rows, n]
 * float64; w may be NULL.  row_nan may be NULL; rows flagged there come back
 * NaN.  Block sums use the same compensated accumulator as the fit.
 */
int iso_oracle_vjp(const double* g, const uint8_t* block_start, const uint8_t* clipped,
                   const uint8_t* row_nan, const double* w, int64_t rows, int64_t n, double* out) {
    if (rows < 0 || n < 0) return ORACLE_EINVAL;
    if (rows == 0 || n == 0) return ORACLE_OK;
    if (!g || !block_start || !out) return ORACLE_EINVAL;
    for (int64_t r = 0; r < rows; ++r) {
        const double* gr = g + r * n;
        const uint8_t* bs = block_start + r * n;
        const uint8_t* cl = clipped ? clipped + r * n : NULL;
        const double* wr = w ? w + r * n : NULL;
        double* o = out + r * n;
        if (row_nan && row_nan[r]) {
            for (int64_t i = 0; i < n; ++i) o[i] = NAN;
            continue;
        }
        int64_t lo = 0;
        while (lo < n) {
            int64_t hi = lo + 1;
            while (hi < n && !bs[hi]) ++hi;
            acc_t sg = {0.0, 0.0}, sw = {0.0, 0.0};
            for (int64_t i = lo; i < hi; ++i) {
                if (!(cl && cl[i])) acc_add(&sg, gr[i]);
                acc_add(&sw, wr ? wr[i] : 1.0);
            }
            double G = acc_value(&sg), W = acc_value(&sw);
            for (int64_t i = lo; i < hi; ++i) o[i] = (wr ? wr[i] : 1.0) * G / W;
            lo = hi;
        }
    }
    return ORACLE_OK;
}

/*
 * Vector-Jacobian product of the (clipped) fit with respect to the weights
 * (the PyPI page, "Semantics": the fit is differentiable in y and in the
 * weights), for the partition given by block_start and the clip flags.  A
 * block B takes the value mean_B = sum_B w y / sum_B w, whose derivative in
 * w_j (j in B) is (y_j - mean_B) / sum_B w; so
 *     grad_w[j] = (sum_{i in B, not clipped} g_i) * (y_j - mean_B) / sum_B w.
 * The same formula holds for the non-increasing fit (its blocks' values are
 * the same weighted means).  g, y, w, out: [rows, n] float64; w may be NULL
 * (unit weights).  row_nan may be NULL; rows flagged there come back NaN.
 */
int iso_oracle_vjp_w(const double* g, const double* y, const uint8_t* block_start, const uint8_t* clipped,
                     const uint8_t* row_nan, const double* w, int64_t rows, int64_t n, double* out) {
    if (rows < 0 || n < 0) return ORACLE_EINVAL;
    if (rows == 0 || n == 0) return ORACLE_OK;
    if (!g || !y || !block_start || !out) return ORACLE_EINVAL;
    for (int64_t r = 0; r < rows; ++r) {
        const double* gr = g + r * n;
        const double* yr = y + r * n;
        const uint8_t* bs = block_start + r * n;
        const uint8_t* cl = clipped ? clipped + r * n : NULL;
        const double* wr = w ? w + r * n : NULL;
        double* o = out + r * n;
        if (row_nan && row_nan[r]) {
            for (int64_t i = 0; i < n; ++i) o[i] = NAN;
            continue;
        }
        int64_t lo = 0;
        while (lo < n) {
            int64_t hi = lo + 1;
            while (hi < n && !bs[hi]) ++hi;
            acc_t sg = {0.0, 0.0}, sw = {0.0, 0.0}, sy = {0.0, 0.0};
            for (int64_t i = lo; i < hi; ++i) {
                const double wi = wr ? wr[i] : 1.0;
                if (!(cl && cl[i])) acc_add(&sg, gr[i]);
                acc_add(&sw, wi);
                acc_add(&sy, wi * yr[i]);
            }
            const double G = acc_value(&sg), W = acc_value(&sw), mean = acc_value(&sy) / W;
            for (int64_t i = lo; i < hi; ++i) o[i] = G * (yr[i] - mean) / W;
            lo = hi;
        }
    }
    return ORACLE_OK;
}
