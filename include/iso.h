/*
 * iso.h - C ABI of the batched weighted isotonic-regression library (libiso.so)
 * for AMD Instinct MI355X (gfx950).
 *
 * What is computed.  For every row r of a rows x n matrix y with positive
 * weights w, the fit z_r is the non-decreasing (or non-increasing) sequence
 * closest to y_r in weighted least squares, Eq. (1) of "Merge Hulls Without
 * Copying Vertices: GPU Isotonic Regression", Sec. 2.1.  It is computed as the
 * slope sequence of the lower convex hull of the cumulative sum diagram
 * P_k = (W_k, S_k), W_k = sum_{i<=k} w_i, S_k = sum_{i<=k} w_i y_i (same page,
 * Sec. 2.1 Eq. (2), Sec. 3 and 4): element i takes the slope of the hull edge
 * over [W_{i-1}, W_i].  The semantics are those of the "torchisotonic" PyPI
 * page, section "Semantics": strictly positive weights, optional clipping of
 * the result to [y_min, y_max] after the fit, and a row holding a NaN comes
 * back as NaN.
 *
 * Memory and streams.  Every pointer argument named *_dev is device memory
 * owned by the caller.  The library allocates nothing and never synchronises
 * inside iso_fit / iso_vjp: their kernels are queued on `stream` (a
 * hipStream_t passed as void*; NULL = the legacy default stream) and read the
 * inputs / write the outputs in stream order.  Matrices are row-major and
 * contiguous: element (r, i) is at index r * n + i.  Supported element types
 * are float32 and float64; all accumulation is in float64.
 *
 * Errors.  Functions return ISO_OK (0) or a negative code.  Argument errors
 * (ISO_EINVAL) are detected on the host before anything is queued.  Data
 * errors are found on the device: a finite weight <= 0 makes the row come back
 * NaN and records ISO_EWEIGHT, which iso_status reports after the call has
 * completed.  A NaN or infinity in y or w is not an error: the row comes back
 * all NaN (an infinity is outside the contract and is treated like a NaN).
 */
#ifndef ISO_H
#define ISO_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* element types */
#define ISO_F32 0
#define ISO_F64 1
#define ISO_F16 2  /* IEEE binary16; views only (iso_fit_view, iso_vjp_view)      */
#define ISO_BF16 3 /* bfloat16 (the high half of a binary32); views only          */
#define ISO_I32 4  /* int32 inputs of views (converted to float32)                */
#define ISO_I64 5  /* int64 inputs of views (converted to float32)                */

/* return codes */
#define ISO_OK 0
#define ISO_EINVAL (-1)  /* bad argument, detected on the host; nothing queued   */
#define ISO_EHIP (-2)    /* a HIP launch or runtime call failed                   */
#define ISO_EWEIGHT (-3) /* a finite weight <= 0 in some row (that row is NaN)    */
#define ISO_ETOOBIG (-4) /* iso_fit_noalloc: the problem needs more workspace than
                            the library's static scratch holds; nothing queued   */

/*
 * Partition handle for the backward pass: which elements start a pooled block
 * of the fit, which elements were clipped, and which rows came back NaN.  The
 * struct lives in host memory and only holds pointers into caller-owned
 * device memory (`blocks_mem` of iso_fit) plus sizes; iso_fit fills it in
 * without synchronising.  `w_dev` is borrowed from the iso_fit call and must
 * stay valid until the last iso_vjp that uses the handle.
 *
 *   start_bits_dev[r * words + q] bit b = 1 iff element 64q + b of row r starts
 *       a block (its left point P_{i} is a vertex of the row's hull; element 0
 *       always starts one);
 *   clip_bits_dev[r * words + q] bit b = 1 iff the unclipped fit of that
 *       element lies strictly outside [y_min, y_max];
 *   row_nan_dev[r] = 1 iff row r came back NaN;
 *   words = ceil(n / 64).
 */
typedef struct iso_blocks {
    uint64_t* start_bits_dev;
    uint64_t* clip_bits_dev;
    uint32_t* row_nan_dev;
    const void* w_dev;
    int64_t rows;
    int64_t n;
    int64_t words;
    int dtype;
    int valid;
} iso_blocks;

/*
 * Bytes of device workspace iso_fit needs for a rows x n problem of the given
 * dtype (at least 256; 256-byte alignment is required).  The workspace holds
 * the status word read by iso_status and, for rows longer than one chunk, the
 * chunk hulls, segment descriptors and per-chunk records of the merge tree
 * (first page, Sec. 3.3-3.4).  Returns 0 for invalid sizes.
 */
size_t iso_workspace_bytes(int64_t rows, int64_t n, int dtype);

/*
 * Bytes of device memory backing an iso_blocks handle for rows x n: the
 * block-start and clip bit words and the row-NaN flags described above, which
 * record the partition of each row into the pooled blocks of its fit (first
 * page, Sec. 2.1: the hull's vertices split the row into blocks sharing one
 * value) and the elements that clipping changed (PyPI page, "Semantics").
 * The backward pass averages over exactly these blocks (first page,
 * Appendix C).  Returns 0 for negative sizes.
 */
size_t iso_blocks_bytes(int64_t rows, int64_t n);

/*
 * Fit every row (first page, Sec. 2-4; PyPI page, "Semantics").
 *
 *   y_dev        [rows, n] of dtype, read only.
 *   w_dev        [rows, n] of dtype, read only, or NULL for unit weights.
 *                Weights must be strictly positive.
 *   increasing   1 for a non-decreasing fit, 0 for non-increasing.
 *   y_min, y_max clip bounds applied after the fit; -INFINITY / +INFINITY (or
 *                NaN) mean "no bound".  y_min > y_max is ISO_EINVAL.
 *   dtype        ISO_F32 or ISO_F64, the type of y, w and fit.
 *   fit_dev      [rows, n] of dtype, written.  May not alias y or w.
 *   blocks_out   host struct filled with the partition handle, or NULL.
 *   blocks_mem_dev  iso_blocks_bytes(rows, n) bytes of device memory backing
 *                the handle, or NULL (then blocks_out must be NULL too, and no
 *                block bits are written).
 *   workspace_dev   iso_workspace_bytes(rows, n, dtype) bytes, 256-aligned.
 *                One workspace may serve only one call in flight at a time.
 *   stream       hipStream_t as void*.
 *
 * rows == 0 or n == 0 queues nothing and returns ISO_OK.
 */
int iso_fit(const void* y_dev, const void* w_dev, int64_t rows, int64_t n, int increasing,
            double y_min, double y_max, int dtype, void* fit_dev, iso_blocks* blocks_out,
            void* blocks_mem_dev, void* workspace_dev, size_t workspace_bytes, void* stream);

/*
 * iso_fit without a workspace argument, for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops, harnesses
 * that forbid hipMalloc).  It runs exactly iso_fit's checks and kernels, with
 * the workspace in a static array of ISO_NOALLOC_SCRATCH_BYTES bytes that the
 * library holds on each GPU it runs on until the process ends.  It calls no
 * allocating routine.
 *
 *   Arguments as for iso_fit; the caller still passes y, w, fit and, when it
 *   wants the partition, blocks_out and blocks_mem_dev.
 *   Returns ISO_ETOOBIG, queuing nothing, when iso_workspace_bytes(rows, n,
 *   dtype) exceeds ISO_NOALLOC_SCRATCH_BYTES (128 MiB: any batch of rows of
 *   at most 32 elements, up to about 3e7 rows of 33 to 512, every batch of
 *   rows of several waves up to 1000 x 6144 elements, and single rows of up
 *   to about 1.2e7 elements).
 *
 * Every call on one GPU shares that GPU's array, and the array keeps the last
 * call's contents: calls that overlap on one GPU (other streams, other host
 * threads) race and must be ordered by the caller.  Nothing needs to start
 * at zero (each call writes what it reads).  iso_status cannot read this
 * entry point's data errors (the caller has no workspace pointer); a row with
 * a weight <= 0 still comes back NaN, with its row-NaN flag set in the
 * partition handle.
 */
#define ISO_NOALLOC_SCRATCH_BYTES (128ull << 20)

int iso_fit_noalloc(const void* y_dev, const void* w_dev, int64_t rows, int64_t n, int increasing,
                    double y_min, double y_max, int dtype, void* fit_dev, iso_blocks* blocks_out,
                    void* blocks_mem_dev, void* stream);

/*
 * Vector-Jacobian product of the fit with respect to y (first page,
 * Appendix C: the product averages over the solver's blocks; weighted form
 * derived from Eq. (1)): for j in block B,
 *     grad_y[j] = w_j * sum_{i in B, clip inactive at i} grad[i] / sum_{i in B} w_i,
 * which is the block mean of the unclipped gradient when w = 1.  Rows that
 * came back NaN give NaN.
 *
 *   grad_dev      [rows, n] of blocks->dtype, read only.
 *   blocks        handle filled by iso_fit (host struct).
 *   grad_y_dev    [rows, n] of blocks->dtype, written.
 *   workspace_dev iso_workspace_bytes(rows, n, dtype) bytes (may be the fit's).
 */
int iso_vjp(const void* grad_dev, const iso_blocks* blocks, void* grad_y_dev, void* workspace_dev,
            size_t workspace_bytes, void* stream);

/*
 * Vector-Jacobian products of the fit with respect to y and to the weights
 * (page "torchisotonic", "Semantics": the fit is differentiable in y and in
 * the weights).  A block B takes the value mean_B = sum_B w y / sum_B w, so
 * for j in B, with G_B = sum_{i in B, clip inactive at i} grad[i] and
 * W_B = sum_B w:
 *     grad_y[j] = w_j * G_B / W_B                 (as iso_vjp),
 *     grad_w[j] = G_B * (y_j - mean_B) / W_B.
 * The non-increasing fit has the same form over its own blocks.  Unit weights
 * (blocks->w_dev == NULL) give the derivative in weights that are all 1.
 * Rows that came back NaN give NaN in both.
 *
 *   grad_dev      [rows, n] of blocks->dtype, read only.
 *   blocks        handle filled by iso_fit (host struct).
 *   y_dev         the y that iso_fit was given ([rows, n] of blocks->dtype,
 *                 read only); required when grad_w_dev is not NULL.
 *   grad_y_dev    [rows, n] of blocks->dtype, written, or NULL.
 *   grad_w_dev    [rows, n] of blocks->dtype, written, or NULL.
 *   workspace_dev iso_workspace_bytes(rows, n, dtype) bytes (may be the fit's).
 *
 * Both outputs NULL, or grad_w_dev without y_dev, is ISO_EINVAL (unless rows
 * or n is 0: then nothing is queued and ISO_OK is returned).
 */
int iso_vjp_yw(const void* grad_dev, const iso_blocks* blocks, const void* y_dev, void* grad_y_dev,
               void* grad_w_dev, void* workspace_dev, size_t workspace_bytes, void* stream);

/*
 * Strided, typed views: the operator's full input semantics (page
 * "torchisotonic", "Semantics": weights of y's shape or broadcast to it, `dim`
 * picks the axis, float input keeps its dtype with float16 and bfloat16
 * computed in float32, integer input becomes the default float dtype).
 *
 * A view describes a logical [outer, inner, n] array: row r = o * inner + j
 * (o < outer, j < inner) and its element i live at element offset
 *     o * stride_outer + j * stride_inner + i * stride_elem
 * from data, counted in elements of the view's dtype.  Strides are >= 0; a
 * stride of 0 repeats the data along that axis (broadcasting).  Every tensor
 * layout whose non-fit axes fold into at most two strides is one view: a
 * fit along any axis of a 2-D or 3-D tensor, a weight vector shared by every
 * row (stride_outer = stride_inner = 0), one weight per row (stride_elem = 0),
 * an expanded y.
 *
 * Computation.  The compute type is float64 when y or the fit's output view
 * is float64, else float32 (float16, bfloat16, float32 and integer y with an
 * output of float32, float16 or bfloat16); accumulation is float64 as in
 * iso_fit.  Weights are converted to the compute type.  Inputs that are not already contiguous rows of the compute
 * type are converted into the workspace by a gather kernel (a tiled transpose
 * through LDS when stride_elem != 1); the fit then runs exactly as iso_fit on
 * those rows, and a scatter kernel converts the result to the output view
 * (float16: round to nearest even by the hardware conversion; bfloat16: round
 * to nearest even of the float32 bits, NaN kept NaN).
 */
typedef struct iso_view {
    void* data;           /* device memory (read only for inputs)                  */
    int dtype;            /* ISO_F16, ISO_BF16, ISO_F32, ISO_F64; inputs also ISO_I32, ISO_I64 */
    int64_t stride_outer; /* elements from row (o, j) to row (o + 1, j)            */
    int64_t stride_inner; /* elements from row (o, j) to row (o, j + 1)            */
    int64_t stride_elem;  /* elements from element i to element i + 1 of a row     */
} iso_view;

/* Bytes of device workspace iso_fit_view and iso_vjp_view need for
 * outer * inner = rows rows of n elements in the compute type compute_dtype
 * (ISO_F32 or ISO_F64; 0 for invalid sizes or dtype): the solver's workspace
 * and four [rows, n] arrays for converted inputs and outputs. */
size_t iso_view_workspace_bytes(int64_t rows, int64_t n, int compute_dtype);

/* Bytes of device memory backing the partition handle of iso_fit_view:
 * iso_blocks_bytes(rows, n) plus, when weighted, room for the weights
 * converted to the compute type (the backward pass reads them from there
 * when the caller's weights are not already contiguous rows of that type). */
size_t iso_view_blocks_bytes(int64_t rows, int64_t n, int compute_dtype, int weighted);

/*
 * iso_fit on views (first page, Sec. 2-4; PyPI page, "Semantics").
 *   y            view of the data (required).
 *   w            view of the weights, or NULL for unit weights.
 *   outer, inner the logical row shape: rows = outer * inner.
 *   fit          view written with the result: ISO_F32, ISO_F64, or, when y
 *                is not float64, ISO_F16 / ISO_BF16.  Its strides must not map
 *                two elements to one place (stride_elem 0 is ISO_EINVAL for
 *                n > 1; other repeats are not checked), and it may not
 *                overlap y or w.
 *   blocks_out, blocks_mem_dev  as for iso_fit, with
 *                iso_view_blocks_bytes(rows, n, compute type, w != NULL) bytes;
 *                the handle's rows are the logical rows r = o * inner + j, its
 *                dtype the compute type, and its w_dev the caller's weights
 *                or their converted copy inside blocks_mem_dev.
 *   workspace_dev  iso_view_workspace_bytes(rows, n, compute type) bytes,
 *                256-aligned; iso_status reads it as for iso_fit.
 * ISO_EINVAL for a bad dtype or stride, NULL pointers, misaligned or short
 * buffers.  rows == 0 or n == 0 queues nothing.
 */
int iso_fit_view(const iso_view* y, const iso_view* w, int64_t outer, int64_t inner, int64_t n, int increasing,
                 double y_min, double y_max, const iso_view* fit, iso_blocks* blocks_out, void* blocks_mem_dev,
                 void* workspace_dev, size_t workspace_bytes, void* stream);

/*
 * iso_vjp_yw on views: the products in y and in the weights of a fit made by
 * iso_fit_view (the same formulas), computed in the fit's compute type
 * (blocks->dtype).  grad and y are input views (any input dtype), grad_y and
 * grad_w output views (ISO_F32 or ISO_F64, or ISO_F16 / ISO_BF16 when the
 * compute type is float32), each NULL when not wanted; y is required with
 * grad_w and is the y the fit was given.  grad_w is written at every element of the logical [rows, n] array:
 * for weights that were broadcast, the product in the caller's weights is
 * its sum over the broadcast axes, which the library leaves to the caller.
 *   workspace_dev  iso_view_workspace_bytes(rows, n, blocks->dtype) bytes
 *                  (may be the fit's workspace: the calls are stream-ordered).
 * ISO_EINVAL for a bad handle, dtype or stride, NULL pointers, both outputs
 * NULL, outer * inner != blocks->rows, a short or misaligned workspace.
 */
int iso_vjp_view(const iso_view* grad, const iso_blocks* blocks, const iso_view* y, const iso_view* grad_y,
                 const iso_view* grad_w, int64_t outer, int64_t inner, void* workspace_dev, size_t workspace_bytes,
                 void* stream);

/*
 * Soft rank with quadratic regularization of strength eps (first page,
 * Sec. 7.9, after Blondel et al.): for each row, theta = x / eps is sorted in
 * decreasing order into s, the non-increasing fit v of z = s - (n, n-1, ..., 1)
 * is computed with unit weights by the same solver as iso_fit, and the element
 * at sorted position i gets the rank s_i - v_i.  This is the Euclidean
 * projection of theta onto the permutahedron of (1, ..., n): ranks sum to
 * n(n+1)/2, keep the order of x, are the hard ranks (n for the largest value)
 * when eps is small enough, and tied values share one rank.  Equal values are
 * sorted in index order.  A row holding a NaN comes back NaN.
 *
 * Rows of any length up to INT32_MAX elements: rows of at most 8192 are
 * sorted by one workgroup each, longer rows (the first page's Table 6 runs
 * rows of 10^4 to 10^6) by tiles of 2048 and merge passes, as the
 * calibration scores are.  The state keeps what the backward pass needs: the sorting permutation, its
 * inverse, and the fit's partition over the sorted positions.
 *   blocks     partition of the fit of z in sorted order (w_dev is NULL, no
 *              clipping);
 *   perm_dev   [rows, n] int32: perm[r * n + i] = index of the element at
 *              sorted position i of row r;
 *   rank_dev   [rows, n] int32: the inverse of perm within each row;
 *   eps        the strength the ranks were computed with.
 */
typedef struct iso_soft_rank_state {
    iso_blocks blocks;
    int32_t* perm_dev;
    int32_t* rank_dev;
    double eps;
    int valid;
} iso_soft_rank_state;

/* Bytes of device memory backing an iso_soft_rank_state for rows x n. */
size_t iso_soft_rank_state_bytes(int64_t rows, int64_t n);

/* Bytes of device workspace iso_soft_rank and iso_soft_rank_vjp need
 * (256-byte aligned; 0 for invalid sizes, n > INT32_MAX or a bad dtype):
 * the solver's workspace, z and its fit, and for rows longer than 8192 the
 * sort's keys and indices (24 bytes per element). */
size_t iso_soft_rank_workspace_bytes(int64_t rows, int64_t n, int dtype);

/*
 * Soft ranks of every row.
 *   x_dev          [rows, n] of dtype, read only.
 *   eps            regularization strength, finite and > 0.
 *   r_dev          [rows, n] of dtype, written.  May not alias x.
 *   state_out      host struct filled with the backward state (required).
 *   state_mem_dev  iso_soft_rank_state_bytes(rows, n) bytes, 256-aligned.
 *   workspace_dev  iso_soft_rank_workspace_bytes(rows, n, dtype) bytes,
 *                  256-aligned; one call in flight per workspace.
 * ISO_EINVAL for n or rows > INT32_MAX, a bad eps or dtype, NULL pointers,
 * misaligned or short buffers.  rows == 0 or n == 0 queues nothing.
 */
int iso_soft_rank(const void* x_dev, int64_t rows, int64_t n, double eps, int dtype, void* r_dev,
                  iso_soft_rank_state* state_out, void* state_mem_dev, void* workspace_dev,
                  size_t workspace_bytes, void* stream);

/*
 * Vector-Jacobian product of the soft ranks in x: with g_s the upstream
 * gradient in sorted order and A the block averaging of the fit,
 *     grad_x[perm[i]] = (g_s[i] - (A g_s)[i]) / eps.
 * Rows that came back NaN give NaN.
 *   grad_dev       [rows, n] of the forward's dtype, read only.
 *   state          filled by iso_soft_rank (its memory still alive).
 *   grad_x_dev     [rows, n] of that dtype, written.
 *   workspace_dev  iso_soft_rank_workspace_bytes(rows, n, dtype) bytes (may be
 *                  the forward's once it has completed in stream order).
 */
int iso_soft_rank_vjp(const void* grad_dev, const iso_soft_rank_state* state, void* grad_x_dev,
                      void* workspace_dev, size_t workspace_bytes, void* stream);

/*
 * Calibration curve of every row (first page, Sec. 7.7; page "torchisotonic",
 * "What it is for": scikit-learn's IsotonicRegression curve).  The row's
 * scores are sorted in increasing order, equal scores are pooled (their labels
 * summed and counted), and the curve is the non-decreasing fit of the pooled
 * means with the counts as weights, computed by the same solver as iso_fit.
 *   scores_dev, labels_dev  [rows, n] of dtype, read only.
 *   xs_dev         [rows, n] of dtype, written: the m[r] distinct scores of
 *                  row r in increasing order (-0 and +0 are one score, kept as
 *                  +0); entries past m[r] are NaN.
 *   fit_dev        [rows, n] of dtype, written: the curve at xs (entries past
 *                  m[r] are unspecified).
 *   m_dev          [rows] int32, written: the number of distinct scores, 0 for
 *                  a row holding a NaN score or label (which has no curve).
 *   workspace_dev  iso_calibration_workspace_bytes(rows, n, dtype) bytes,
 *                  256-aligned; one call in flight per workspace.
 * Scores and labels must be finite apart from NaN.  ISO_EINVAL for a bad
 * dtype, NULL pointers, misaligned or short buffers, n above INT32_MAX.
 * rows == 0 or n == 0 queues nothing.
 */
size_t iso_calibration_workspace_bytes(int64_t rows, int64_t n, int dtype);

int iso_calibration_fit(const void* scores_dev, const void* labels_dev, int64_t rows, int64_t n, int dtype,
                        void* xs_dev, void* fit_dev, int32_t* m_dev, void* workspace_dev, size_t workspace_bytes,
                        void* stream);

/*
 * Calibrated values (page "torchisotonic", "What it is for"): each query of
 * row r is placed on row r's curve, linearly between its points (the first
 * point at or above the query and the one before it) and constant beyond the
 * first and last points.  A NaN query, or a row without a curve (m = 0),
 * gives NaN.
 *   xs_dev, fit_dev, m_dev  as written by iso_calibration_fit ([rows, n],
 *                  [rows, n], [rows]).
 *   q_dev          [rows, k] of dtype, read only; out_dev [rows, k], written.
 */
int iso_calibrate(const void* xs_dev, const void* fit_dev, const int32_t* m_dev, int64_t rows, int64_t n,
                  const void* q_dev, int64_t k, int dtype, void* out_dev, void* stream);

/*
 * Data errors of a fit (PyPI page, "Semantics": the weights must be strictly
 * positive).  The kernels cannot return an error to the host without a
 * synchronisation, so a row holding a finite weight <= 0 comes back NaN and
 * the error is recorded in the workspace.  iso_status synchronises `stream`
 * and returns the data error of the most recent iso_fit that used this
 * workspace: ISO_OK or ISO_EWEIGHT (ISO_EHIP if the read fails, ISO_EINVAL
 * for a NULL workspace).  The answer is defined only for a workspace that an
 * iso_fit has used; the library keeps no host state per workspace (the call's
 * epoch and error live in the workspace's first 16 bytes).
 */
int iso_status(const void* workspace_dev, void* stream);

/*
 * Static, human-readable text for a return code of this library (ISO_OK,
 * ISO_EINVAL, ISO_EHIP, ISO_EWEIGHT: the PyPI page's "Semantics" rule that
 * weights be strictly positive, ISO_ETOOBIG); "unknown error" for any other.
 */
const char* iso_strerror(int code);

#ifdef __cplusplus
}
#endif

#endif /* ISO_H */
