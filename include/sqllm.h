/*
 * sqllm.h -- C ABI of the dense-and-sparse LUT matrix-vector product
 * y = (D + S) x on AMD Instinct MI355X (gfx950).
 *
 * The operation (SqueezeLLM: Dense-and-Sparse Quantization, summary page):
 *   - §3.4 "The Dense-and-Sparse Decomposition": W = D + S.  S holds the few
 *     outlier / sensitive weights in CSR form with fp16 values, 16-bit column
 *     indices and row pointers (nnz of row i = row_ptr[i+1] - row_ptr[i]).
 *   - §3.4 "Kernel Implementation": D is stored as a 2-D array of b-bit
 *     indices (b = 3 or 4; b = 2 as in Appendix F, Tables F.8 and F.10);
 *     index code[r][c] selects one of 2^b fp16
 *     centroids in the lookup table of output channel r; the dequantized
 *     weights multiply an fp16 activation vector.  A balanced sparse kernel
 *     computes S x, fused with the dense part into one output.
 *   - §3.4 "The 3/4-bit storage format": every index takes exactly b bits.
 *   - §3.4 "The Memory-Bound Analysis": batch-1 generation is a
 *     matrix-vector product; batches up to 16 are accepted here.
 *
 *   y[b][r] = sum_c LUT[r][code[r][c]] * x[b][c]
 *           + sum_{i=row_ptr[r]}^{row_ptr[r+1]-1} val[i] * x[b][col_idx[i]]
 *
 * Arithmetic: every product of two fp16 values is formed exactly and summed
 * in fp32; the fused call rounds each output once to fp16 (round to nearest
 * even).  For a given shape, batch and workspace size the launch shape is
 * fixed and every sum is taken in a fixed order (including the combine of a
 * row's column split, below), so repeated calls give identical bits.
 *
 * Conventions shared by every call
 *   - All data pointers are DEVICE pointers owned by the caller.  The library
 *     never allocates or frees memory on the hot calls and keeps no state
 *     between calls (the workspace below is the caller's).
 *   - fp16 values are passed as raw IEEE binary16 bit patterns (uint16_t).
 *   - Layouts are row-major and contiguous:
 *       lut  [rows][2^bits]          16-byte aligned
 *       x    [batch][cols]           16-byte aligned
 *       y    [batch][rows]           4-byte aligned
 *       row_ptr [rows+1] int32, col_idx [nnz] uint16, val [nnz] fp16
 *     i.e. y = x W^T with W = [rows][cols] = out x in features.
 *   - Hot calls are asynchronous on `stream` (NULL = default stream), never
 *     synchronise, and report only argument errors (checked on the host
 *     before any HIP call) and launch errors.
 *   - Preconditions not checked on the hot path (violations are undefined
 *     behaviour): row_ptr[0] == 0, row_ptr[rows] == nnz, row_ptr
 *     non-decreasing, col_idx[i] < cols, x and y do not overlap, inputs finite.
 *     Duplicate (row, column) outlier entries are summed.
 *   - rows >= 1; cols >= 256 and a multiple of 256; cols <= 65536 when
 *     outliers are given (16-bit column indices); nnz < 2^31; 1 <= batch <= 16.
 *
 * Packed code layout (the pages fix only that every index takes exactly b bits; the
 * arrangement below is this library's, chosen so that each 64-lane wave
 * streams 1 KiB of codes per 128-bit load instruction and every code byte
 * turns into a table address with one byte-permute):
 *   rows are grouped in tiles of 64 (tile t = r / 64, lane l = r % 64), the
 *   columns of a row in groups of 256 (g = c / 256, j = c % 256).  The 32*b
 *   bytes that hold the 256 codes of (r, g) form the group's byte string,
 *   cut into 2*b pieces of 16 bytes; piece q of (r, g) is stored at byte
 *       ((t * G + g) * 2b + q) * 1024 + l * 16,      G = cols / 256.
 *   Codes go in pairs: pair p (0..127) holds codes 2p and 2p+1 as the
 *   2b-bit value code[2p] | code[2p+1] << b.
 *     4-bit: byte p of the string is pair p.
 *     2-bit: byte p of the string holds pair 2p in its low four bits and
 *       pair 2p+1 in its high four bits.
 *     3-bit: the string is 8 units of 12 bytes; unit u holds pairs
 *       16u .. 16u+15.  Pair 16u+p for p < 12 is the low six bits of unit
 *       byte p.  Pair 16u+12+q (q = 0..3) stores its bits [2k, 2k+2) in the
 *       top two bits of unit byte 4k + q, for k = 0, 1, 2.
 *   Example (3-bit, codes 0,1,2,...,7 repeating along the row): the pair
 *   values cycle 0x08, 0x1A, 0x2C, 0x3E, and every 12-byte unit reads
 *   08 9A 2C BE 88 9A EC FE 08 5A AC FE.
 *   Rows of the last tile beyond `rows` are padding (zero after sqllm_pack).
 *   Total size: sqllm_packed_bytes() = ceil(rows / 64) * 64 * cols * b / 8.
 *   The packed buffer must be 16-byte aligned.
 *
 * Workspace: the hot calls may split a row's columns over several
 * workgroups (at most 16), which then combine their fp32 partial sums on the
 * device.  They take a caller-owned workspace of at least
 * sqllm_workspace_bytes(rows, cols, batch) bytes, 256-byte aligned,
 * ZERO-FILLED before its first use.  With the columns split over s > 1
 * workgroups a call uses s - 1 eight-byte words per output: the partial sums
 * meet in a binary tree (splits 2j and 2j+1 pair up, one atomic OR each sets
 * its half of the pair's word, the second arrival adds left + right), so
 * the order of the fp32 additions does not depend on which workgroup
 * arrives first; every word is reset by the workgroup that completes it.
 * Every call therefore leaves the workspace ready for the next one, so one
 * workspace serves any sequence of calls, of any shapes it is large enough
 * for, that are ordered on one stream.  Calls that may run concurrently
 * need separate workspaces.  At batch >= 5 the workspace also holds, after
 * the words of the largest split, a transposed copy of x ([cols][8] fp16,
 * [cols][16] above batch 8) from which the outliers read all batch columns
 * of a column in one load; the call writes it before its product kernel and
 * clears it after, so the whole workspace is zero again when the call's work
 * on the stream is done.  A call that does not split (small shapes) needs no
 * words: the workspace may then be NULL, and a workspace with room for the
 * words of the call's split but smaller than sqllm_workspace_bytes() makes
 * the outliers read x in place.
 */
#ifndef SQLLM_H
#define SQLLM_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    SQLLM_OK = 0,
    SQLLM_ERR_NULL = 1,       /* a required pointer is NULL */
    SQLLM_ERR_BITS = 2,       /* bits not 2, 3 or 4 */
    SQLLM_ERR_SHAPE = 3,      /* rows / cols / nnz out of range */
    SQLLM_ERR_BATCH = 4,      /* batch not in [1, 16] */
    SQLLM_ERR_ALIGN = 5,      /* a pointer is not aligned as required */
    SQLLM_ERR_CODE_RANGE = 6, /* sqllm_pack: a code is >= 2^bits */
    SQLLM_ERR_HIP = 7,        /* a HIP runtime call or kernel launch failed */
    SQLLM_ERR_WORKSPACE = 8,  /* workspace missing, misaligned or too small */
    SQLLM_ERR_CAPACITY = 9,   /* sqllm_outlier_extract: more outliers than the CSR buffers hold */
    SQLLM_ERR_SCRATCH = 10    /* sqllm_dense_sparse_gemv_noalloc: the launch needs more than its fixed scratch */
} sqllm_status;

/* Human-readable name of a status code (static string, never NULL). */
const char *sqllm_status_string(sqllm_status s);

/* Bytes of the packed code buffer for a rows x cols matrix of `bits`-bit
 * codes (see the layout above); 0 if the arguments are out of range. */
size_t sqllm_packed_bytes(int64_t rows, int64_t cols, int bits);

/* Bytes of workspace the hot calls need for this shape and batch (the same
 * bound covers sqllm_gemv, sqllm_spmv_add and sqllm_dense_sparse_gemv): the
 * words of the largest split, ceil(rows / 64) * 64 * batch * 8 * 15, plus at
 * batch >= 5 the transposed x, cols * 16 (cols * 32 above batch 8) rounded
 * up to 256; 0 if the arguments are out of range. */
size_t sqllm_workspace_bytes(int64_t rows, int64_t cols, int batch);

/*
 * sqllm_pack -- offline step: unpacked codes -> packed layout.
 * Stores the b-bit indices with exactly b bits each (§3.4 "The 3/4-bit
 * storage format").
 *   codes:  device uint8 [rows][cols], every value < 2^bits
 *   packed: device buffer of sqllm_packed_bytes(rows, cols, bits) bytes,
 *           16-byte aligned; padding rows are written as zeros
 *   workspace: caller-owned device memory of at least 4 bytes, 4-byte
 *           aligned, for the call's error flag; its first 4 bytes are zero
 *           again when the call returns (so a hot-call workspace may serve);
 *           the library allocates nothing
 * The code range is checked on the device; the call SYNCHRONISES `stream`
 * to report SQLLM_ERR_CODE_RANGE (packed contents are then unspecified).
 * A missing or too small workspace is SQLLM_ERR_WORKSPACE.
 */
sqllm_status sqllm_pack(const uint8_t *codes, int64_t rows, int64_t cols, int bits, void *packed, void *workspace,
                        size_t workspace_bytes, hipStream_t stream);

/*
 * sqllm_gemv -- dense part only: y = D x.
 * §3.4 "Kernel Implementation", LUT-based dense kernel: stream the packed
 * indices, look each one up in its row's fp16 table, multiply-add against
 * the fp16 activations.
 *   packed: sqllm_pack output; lut: fp16 [rows][2^bits]; x: fp16 [batch][cols]
 *   y: fp16 [batch][rows], overwritten
 */
sqllm_status sqllm_gemv(const void *packed, const uint16_t *lut, int bits, int64_t rows, int64_t cols,
                        const uint16_t *x, int batch, uint16_t *y, void *workspace, size_t workspace_bytes,
                        hipStream_t stream);

/*
 * sqllm_spmv_add -- sparse part only: y += S x (read y, add, round once to
 * fp16, write y).  §3.4 "Kernel Implementation", balanced sparse kernel:
 * a fixed share of the nonzeros per thread, rows split across threads and
 * their partial sums combined (here: in a fixed order).
 *   nnz == 0 is a no-op; row_ptr / col_idx / val may then be NULL.
 * With sqllm_gemv before it on the same stream this is the stream-ordered
 * form of sqllm_dense_sparse_gemv (two fp16 roundings instead of one).
 */
sqllm_status sqllm_spmv_add(const int32_t *row_ptr, const uint16_t *col_idx, const uint16_t *val, int64_t nnz,
                            int64_t rows, int64_t cols, const uint16_t *x, int batch, uint16_t *y,
                            void *workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * sqllm_dense_sparse_gemv -- the fused product y = (D + S) x in one launch.
 * §3.2 "Big-Picture Architecture" and §3.4 "Kernel Implementation" (kernel
 * fusion): the dense and sparse contributions are summed on chip and each
 * output is written once.  nnz == 0 gives exactly sqllm_gemv's result.
 *   Arguments as for sqllm_gemv and sqllm_spmv_add; y is overwritten.
 */
sqllm_status sqllm_dense_sparse_gemv(const void *packed, const uint16_t *lut, int bits, const int32_t *row_ptr,
                                     const uint16_t *col_idx, const uint16_t *val, int64_t nnz, int64_t rows,
                                     int64_t cols, const uint16_t *x, int batch, uint16_t *y, void *workspace,
                                     size_t workspace_bytes, hipStream_t stream);

/*
 * sqllm_dense_sparse_gemv_group -- n independent fused products
 * y_i = (D_i + S_i) x_i in one launch (1 <= n <= 8), all with the same
 * `bits` and `batch`: for instance the query, key and value projections of
 * one attention block, or the gate and up projections of one MLP, which the
 * pages' decoder layers (§5 "Experiments", LLaMA) compute from one input.
 * Each product is the one sqllm_dense_sparse_gemv computes, within the same
 * tolerance; the launch lets one product's start-up and tail overlap the
 * others' code streams.
 *   items: HOST array of n descriptors (read during the call only); each
 *          holds device pointers laid out as for sqllm_dense_sparse_gemv,
 *          nnz == 0 allowed (row_ptr / col_idx / val may then be NULL).
 *          No product's y may overlap any product's inputs or another y.
 *          plan / plan_helpers: see sqllm_outlier_plan below (NULL / 0: no
 *          plan; a plan with plan_helpers > 0 needs a NULL-free plan, 4-byte
 *          aligned, plan_helpers <= 8 * ceil(rows / 64), else
 *          SQLLM_ERR_NULL / SQLLM_ERR_ALIGN / SQLLM_ERR_SHAPE).
 *   workspace: at least sqllm_group_workspace_bytes(items, n, batch) bytes,
 *          256-byte aligned, zero-filled before first use, left zeroed; the
 *          products use disjoint parts of it in item order.
 * Products with and without outliers are launched separately (at most two
 * launches, in stream order).  Argument errors are reported before any
 * launch.
 */
typedef struct {
    const void *packed;       /* sqllm_pack output, 16-byte aligned */
    const uint16_t *lut;      /* fp16 [rows][2^bits], 16-byte aligned */
    const int32_t *row_ptr;   /* int32 [rows + 1] */
    const uint16_t *col_idx;  /* uint16 [nnz] */
    const uint16_t *val;      /* fp16 [nnz] */
    int64_t nnz;
    int64_t rows;
    int64_t cols;
    const uint16_t *x;        /* fp16 [batch][cols], 16-byte aligned */
    uint16_t *y;              /* fp16 [batch][rows], overwritten */
    const int32_t *plan;      /* device copy of sqllm_outlier_plan's output for this CSR, or NULL */
    int64_t plan_helpers;     /* plan[0]: the plan's extra workgroups (0 without a plan) */
} sqllm_product;

size_t sqllm_group_workspace_bytes(const sqllm_product *items, int n, int batch);

/*
 * sqllm_outlier_plan -- offline, host only: the preprocessing step of the
 * balanced sparse kernel (§3.4 "Kernel Implementation": a fixed share of the
 * nonzeros per thread, decided ahead of time; Appendix C, Figure C.1: a few
 * output channels hold far more outliers than the rest).  The product
 * kernels share a row tile's nonzeros evenly among the workgroups that own
 * the tile; a tile holding far more than the others would keep its
 * workgroups busy after the rest have finished.  The plan gives such tiles
 * extra workgroups ("helpers") that take shares of the tile's nonzeros and
 * nothing else, and whose partial sums join the tile's fixed-order combine.
 *   Rule: with tiles = ceil(rows / 64) and q = 2 * ceil(nnz / tiles), tile t
 *   holding n_t > q nonzeros gets min(8, ceil(n_t / q) - 1) helpers.
 *   row_ptr: HOST int32 [rows + 1], the CSR's row pointers (row_ptr[0] == 0,
 *            non-decreasing); read only.
 *   plan:    HOST int32 buffer of plan_len entries.  Written: plan[0] = H,
 *            the number of helpers; plan[1 + t] = helpers of tile t (0..8);
 *            then H entries (t << 4) | e, e = 0 .. helpers of t - 1, in
 *            tile order.
 *   Returns the entries written (1 + tiles + H), or 0 when an argument is
 *   out of range (rows < 1, a NULL pointer, row pointers not
 *   non-decreasing from 0) or plan_len is below sqllm_outlier_plan_len().
 * The caller copies the plan to the device (int32, 4-byte aligned) and sets
 * sqllm_product.plan and .plan_helpers = plan[0] for the group call.  A
 * planned product needs the full sqllm_workspace_bytes() region (its tiles
 * combine up to 16 partial sums), runs its row tiles over at most 8
 * workgroups each besides the helpers, and gives the same result as without
 * the plan within the stated tolerance; repeated calls give identical bits.
 * A plan with no helpers changes nothing.  The single-product calls take no
 * plan; a group of one product does.
 */
size_t sqllm_outlier_plan_len(int64_t rows);
size_t sqllm_outlier_plan(const int32_t *row_ptr, int64_t rows, int32_t *plan, size_t plan_len);

sqllm_status sqllm_dense_sparse_gemv_group(const sqllm_product *items, int n, int bits, int batch, void *workspace,
                                           size_t workspace_bytes, hipStream_t stream);

/*
 * sqllm_dense_sparse_gemv_noalloc -- sqllm_dense_sparse_gemv without a
 * workspace argument, for callers that cannot allocate device memory or
 * pass a workspace (code under HIP graph capture, fixed serving loops,
 * hosts that forbid allocation).  Same arguments (minus the workspace),
 * checks, launch and result: for any shape it takes, its output equals
 * sqllm_dense_sparse_gemv's with a workspace of sqllm_workspace_bytes()
 * bit for bit.  The call itself allocates nothing.
 *   Scratch: the words and the transposed x live in a device array of
 *   SQLLM_NOALLOC_SCRATCH_BYTES (16 MiB) that the library holds on every GPU
 *   it runs on, from its first use there until the process ends.  The first
 *   call on a GPU looks the array up and zero-fills it on `stream` (make that
 *   first call outside graph capture, or the fill joins the captured graph);
 *   each call leaves it zero again, as with a caller's workspace.
 *   Size: at the library's own launch shapes every accepted shape fits (a
 *   call splits at most 256 row tiles' worth of outputs, whose words take at
 *   most 2 MiB at batch 16).  The transposed x of batch >= 5 is used only
 *   when sqllm_workspace_bytes(rows, cols, batch) <= the scratch size; larger
 *   products read x in place (same result).  A launch that needs more words
 *   than the scratch holds (only a launch shape forced through
 *   sqllm_test_tuning) is refused with SQLLM_ERR_SCRATCH before any launch.
 *   Concurrency: all calls on one GPU share its array.  Calls on one stream
 *   are safe; calls that can overlap on the GPU (several streams, several
 *   host threads with their own streams) race and give wrong results.
 */
#define SQLLM_NOALLOC_SCRATCH_BYTES ((size_t)16 << 20)
sqllm_status sqllm_dense_sparse_gemv_noalloc(const void *packed, const uint16_t *lut, int bits,
                                             const int32_t *row_ptr, const uint16_t *col_idx, const uint16_t *val,
                                             int64_t nnz, int64_t rows, int64_t cols, const uint16_t *x, int batch,
                                             uint16_t *y, hipStream_t stream);

/*
 * Offline steps upstream of the product (not timed on the hot path): the
 * dense-and-sparse split of an fp16 weight matrix W and the per-row
 * (optionally sensitivity-weighted) k-means that yields the codes and the
 * tables.  SqueezeLLM: Dense-and-Sparse Quantization, summary page, §3.4
 * "The Dense-and-Sparse Decomposition" (W = D + S, S the weights outside
 * the [T_min, T_max] percentile range, in CSR) and §3.3, Eq. 1 / Eq. 6 with
 * "The weighted k-means algorithm in practice" (per output channel: assign
 * each weight to the nearest centroid, move each centroid to the
 * sensitivity-weighted mean of its weights); that subsection's paragraph
 * on sensitive values adds the most sensitive weights (0.05%) to S.
 * Device pointers owned by the
 * caller; W is fp16 [rows][cols] row-major, 1 <= cols <= 65536 and
 * rows * cols <= 2^31 - 1 (else SQLLM_ERR_SHAPE, and workspace bytes 0).
 *
 * sqllm_quantize_workspace_bytes: device scratch the two split calls need.
 */
size_t sqllm_quantize_workspace_bytes(int64_t rows, int64_t cols);

/*
 * sqllm_outlier_thresholds: T_min and T_max of W at tail_ppm parts per
 * million on each side (2000 = the pages' 0.2 / 99.8 percentiles): the
 * values of rank floor(rows * cols * tail_ppm / 1e6) from the low and the
 * high end of W's fp16 values ordered as IEEE total order (-0 before +0).
 * Given sensitivities `sens` (fp32 [rows][cols], e.g. a Fisher diagonal;
 * NULL for none), also T_s: with n_top = floor(rows * cols * top_ppm / 1e6),
 * the sensitivity of rank rows * cols - 1 - n_top in ascending total order
 * (500 = the pages' 0.05% most sensitive values); else T_s = +infinity.
 * *nnz is the number of weights S will hold: those comparing below T_min
 * or above T_max, and those whose sensitivity is above T_s.  Ranges:
 * 0 <= tail_ppm < 500000, 0 <= top_ppm < 1000000.  t_min, t_max (fp16
 * bits), t_s (may be NULL when sens is) and nnz are HOST outputs; the call
 * synchronises `stream`.
 */
sqllm_status sqllm_outlier_thresholds(const uint16_t *w, const float *sens, int64_t rows, int64_t cols, int tail_ppm,
                                      int top_ppm, void *workspace, size_t workspace_bytes, uint16_t *t_min,
                                      uint16_t *t_max, float *t_s, int64_t *nnz, hipStream_t stream);

/*
 * sqllm_outlier_extract: S = the weights below t_min or above t_max, or
 * (sens given) with sensitivity above t_s, as CSR (row_ptr int32
 * [rows + 1]; col_idx uint16 and val fp16 [nnz], columns ascending within a
 * row) and D = W with zeros at S's entries (fp16 [rows][cols], must not
 * overlap W).  sens_dense (optional, needs sens): the sensitivities with
 * zeros at S's entries, the weights to give sqllm_kmeans_lut so that S's
 * positions take no part in D's clustering.  Writes past nnz_capacity are
 * dropped and reported as SQLLM_ERR_CAPACITY; the call synchronises
 * `stream`.
 */
sqllm_status sqllm_outlier_extract(const uint16_t *w, const float *sens, int64_t rows, int64_t cols, uint16_t t_min,
                                   uint16_t t_max, float t_s, int32_t *row_ptr, uint16_t *col_idx, uint16_t *val,
                                   int64_t nnz_capacity, uint16_t *dense, float *sens_dense, void *workspace,
                                   size_t workspace_bytes, hipStream_t stream);

/*
 * sqllm_kmeans_lut: per row of D, 2^bits centroids by `iters` k-means steps
 * from uniformly spaced starts over the row's range (each weight to the
 * nearest centroid, ties to the lower; each centroid to the weighted mean
 * of its weights, unchanged when it has none; sens = NULL weighs all
 * equally, else fp32 [rows][cols] non-negative sensitivities), then the
 * centroids rounded to fp16 into lut [rows][2^bits] and every weight's code
 * (uint8 [rows][cols]) = its nearest fp16 centroid, ties to the lower.
 * Asynchronous on `stream`; 0 <= iters <= 1000.
 */
sqllm_status sqllm_kmeans_lut(const uint16_t *dense, const float *sens, int64_t rows, int64_t cols, int bits, int iters,
                              uint8_t *codes, uint16_t *lut, hipStream_t stream);

/*
 * Test-only exports (not part of the stable contract).  The readers are
 * asynchronous on `stream`.
 *   sqllm_test_unpack: packed -> uint8 codes [rows][cols]
 *   sqllm_test_decode: packed + lut -> fp16 weights LUT[r][code[r][c]],
 *                      [rows][cols] (exact bit copies of table entries)
 */
sqllm_status sqllm_test_unpack(const void *packed, int64_t rows, int64_t cols, int bits, uint8_t *codes,
                               hipStream_t stream);
/*   sqllm_test_tuning: launch shape of later calls in this process: the
 *   workgroup count the column split aims for, the fewest 256-column groups
 *   per workgroup, a forced split (1..16) and forced waves per workgroup
 *   (1..16).  0 restores a value's built-in default (no environment
 *   variable changes any launch).  sparse_naive
 *   = 1 switches the outliers to the unbalanced form for the ablation of the
 *   balanced kernel (summary page, Appendix C, Table C.1): one thread per
 *   row walks the row's nonzeros; 0 restores the balanced form.  dot_only =
 *   1 computes the dense part in the v_dot2c form instead of the default
 *   matrix-core form (for the comparison of the two); 0 restores the
 *   default.  Shapes that no compiled kernel fits fail with
 *   SQLLM_ERR_SHAPE.  Results agree within the stated tolerance for every
 *   shape; not thread-safe against concurrent calls. */
sqllm_status sqllm_test_tuning(int target_wgs, int min_gps, int split, int waves, int sparse_naive, int dot_only);
/*   sqllm_test_launch_plan: the launch the hot calls would make, without
 *   making it (no device is touched; stand-in addresses are never read):
 *   mode 0 = sqllm_dense_sparse_gemv (n = 1), 1 = sqllm_dense_sparse_gemv_group
 *   with a separate x per product, 2 = the group with one x shared by all
 *   products (equal cols).  rows / cols / nnz: HOST arrays of n; workspace_bytes
 *   as the call would get it (0: no workspace).  plan: HOST array of 5 n + 1
 *   ints; for product i, plan[5 i ..] = split (workgroups per row tile), column
 *   groups per workgroup, waves per workgroup of its launch, where its
 *   outliers read x (0 in place, 1 a transposed copy, 2 staged in LDS), and
 *   for a single call run as two
 *   row slices the row tiles of the first slice (which runs at the split
 *   given; the rest runs whole), else 0; plan[5 n]: bit 0 set for the
 *   matrix-core form, bit 1 set when the outlier launch takes the compact
 *   3-bit pair table (64 pair entries per lane instead of 256, which leaves
 *   room in LDS for x).  Argument and workspace errors as the calls report
 *   them. */
sqllm_status sqllm_test_launch_plan(int mode, int n, const int64_t *rows, const int64_t *cols, const int64_t *nnz,
                                    int batch, size_t workspace_bytes, int *plan);
sqllm_status sqllm_test_decode(const void *packed, const uint16_t *lut, int64_t rows, int64_t cols, int bits,
                               uint16_t *w, hipStream_t stream);

/*
 * sqllm_test_stream_read -- test-only reference for the HBM roofline (§3.4
 * "The Memory-Bound Analysis": the product is bound by the bytes it loads):
 * reads `bytes` of device memory at `src` (16-byte aligned, a multiple of
 * 1024) once with wide non-temporal loads, 1024 workgroups of 4 waves each
 * streaming a contiguous range with 8 loads in flight, no arithmetic beyond
 * an XOR of the 32-bit words.  sink: device uint32 [4096], entry w = the XOR
 * of the words wave w read (the XOR of all entries is that of the whole
 * range).  Timed as one launch per product it gives the rate a launch with
 * no decode could reach at the same launch count.
 * Async on `stream`; SQLLM_ERR_SHAPE for bytes not a positive multiple of
 * 1024, SQLLM_ERR_NULL / SQLLM_ERR_ALIGN for src or sink.
 */
sqllm_status sqllm_test_stream_read(const void *src, size_t bytes, uint32_t *sink, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* SQLLM_H */
