/*
 * sqllm_oracle.c -- plain, slow CPU oracle for the dense-and-sparse LUT
 * matrix-vector product y = (D + S) x.
 *
 * TEST INFRASTRUCTURE.  Only the test suite, the smoke check and the
 * benchmark's CPU-baseline leg may load this library.  It shares no code with
 * the HIP path: its own packed-layout reader, its own binary16 decoder and
 * encoder, its own fp64 multiply-adds.
 *
 * What it computes (SqueezeLLM: Dense-and-Sparse Quantization, summary page):
 *   - §3.4 "The Dense-and-Sparse Decomposition": W = D + S, S stored in CSR
 *     (values fp16, column indices, row pointers, nnz of row i =
 *     row_ptr[i+1] - row_ptr[i]).
 *   - §3.4 "Kernel Implementation", LUT-based dense kernel: D is a 2-D array
 *     of b-bit indices; each index selects an fp16 centroid from the lookup
 *     table of its output channel (row); the dequantized weights multiply the
 *     fp16 activation vector.
 *   - §3.2 "Big-Picture Architecture": the dense product and the sparse
 *     product SX are summed into one output.
 *   - §3.4 "The 3/4-bit storage format": exactly b bits per index.
 * So, for batch column b and row r:
 *   y[b][r] = sum_c LUT[r][code[r][c]] * x[b][c]
 *           + sum_{i = row_ptr[r]}^{row_ptr[r+1]-1} val[i] * x[b][col[i]]
 * evaluated here in fp64 with c ascending, then i ascending.  Every product
 * of two fp16 values is exact in fp64.
 *
 * Tolerance normaliser (the accepted error bound scales with it):
 *   scale[b][r] = sum_c |What[r][c]| * |x[b][c]|,  What = LUT[code] + dense(S)
 * where dense(S) scatters the row's CSR entries into a length-cols row,
 * adding duplicates.
 *
 * Packed layout read by oracle_unpack (the storage format of the library;
 * the pages fix only that every index takes exactly b bits; the rest is this library's
 * choice):
 *   tiles of 64 rows (t = r / 64, lane l = r % 64), groups of 256 columns
 *   (g = c / 256, j = c % 256), 2b pieces of 16 bytes per (row, group).
 *   Piece q of (r, g) sits at byte ((t*G + g)*2b + q)*1024 + l*16, G = cols/256.
 *   The 32b bytes of (r, g), pieces in order, form the group's byte string.
 *   Codes pair up: pair p holds codes 2p and 2p+1 as
 *   value = code[2p] | code[2p+1] << b.
 *   2-bit: byte p of the string holds pair 2p in its low four bits and
 *   pair 2p+1 in its high four bits.
 *   4-bit: byte p of the string is pair p.
 *   3-bit: the string is 8 units of 12 bytes, unit u holding codes
 *   32u .. 32u+31 as pairs p = 0..15 of that unit; pair p < 12 is the low
 *   six bits of unit byte p; pair 12+q (q = 0..3) keeps its bits [2k, 2k+2)
 *   in the top two bits of unit byte 4k + q, for k = 0, 1, 2.
 *   Rows past `rows` in the last tile are padding.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* ---- IEEE-754 binary16 ------------------------------------------------ */

/* binary16 bits -> double, written from the format: 1 sign bit, 5 exponent
 * bits (bias 15), 10 fraction bits; exponent 0 = zero/subnormal
 * (value = fraction * 2^-24), exponent 31 = inf/NaN. */
double oracle_f16_to_f64(uint16_t h)
{
    int sign = (h >> 15) & 1;
    int e = (h >> 10) & 0x1F;
    int f = h & 0x3FF;
    double v;
    if (e == 0) v = ldexp((double)f, -24);
    else if (e == 31) v = f ? NAN : INFINITY;
    else v = ldexp((double)(1024 + f), e - 25);
    return sign ? -v : v;
}

/* double -> binary16 bits, round to nearest, ties to even, written on the
 * double's own bit fields (53-bit significand cut to 11 bits with guard and
 * sticky bits).  Overflow goes to infinity. */
uint16_t oracle_f64_to_f16(double v)
{
    uint64_t u;
    memcpy(&u, &v, 8);
    uint16_t sign = (uint16_t)((u >> 48) & 0x8000u);
    int e = (int)((u >> 52) & 0x7FF);
    uint64_t m = u & ((1ULL << 52) - 1);
    if (e == 0x7FF) return (uint16_t)(sign | (m ? 0x7E00u : 0x7C00u));
    if (e == 0) return sign; /* double subnormals are far below half's range */
    uint64_t sig = m | (1ULL << 52); /* value = sig * 2^(e - 1075) */
    int ue = e - 1023;              /* unbiased exponent */
    /* target: half significand s (11 bits incl. hidden) with exponent he, or
     * subnormal units of 2^-24 */
    int shift; /* bits of sig dropped */
    int he;
    if (ue >= -14) { he = ue; shift = 52 - 10; }
    else { he = -15; shift = 52 - 10 + (-14 - ue); } /* subnormal: fewer bits */
    if (shift > 63) return sign;
    uint64_t kept = sig >> shift;
    uint64_t rem = sig & ((1ULL << shift) - 1);
    uint64_t half = 1ULL << (shift - 1);
    if (rem > half || (rem == half && (kept & 1))) kept += 1;
    if (he == -15) {
        /* kept counts units of 2^-24; 1024 of them is the smallest normal */
        return (uint16_t)(sign | (uint16_t)kept);
    }
    if (kept == 2048) { kept = 1024; he += 1; }
    if (he > 15) return (uint16_t)(sign | 0x7C00u);
    return (uint16_t)(sign | (uint16_t)((he + 15) << 10) | (uint16_t)(kept - 1024));
}

/* ---- packed layout ---------------------------------------------------- */

int64_t oracle_packed_bytes(int64_t rows, int64_t cols, int bits)
{
    int64_t tiles = (rows + 63) / 64;
    return tiles * 64 * cols * bits / 8;
}

/* byte offset of byte k (0 <= k < 32*bits) of the bit string of (row, group) */
static int64_t string_byte_offset(int64_t row, int64_t group, int64_t k, int64_t cols, int bits)
{
    int64_t G = cols / 256, P = 2 * bits;
    int64_t t = row / 64, l = row % 64;
    int64_t q = k / 16, m = k % 16;
    return ((t * G + group) * P + q) * 1024 + l * 16 + m;
}

/* The b-bit pair value (codes 2p and 2p+1) of pair p (0..127) of (row, group). */
static unsigned pair_value(const uint8_t *packed, int64_t row, int64_t group, int64_t p, int64_t cols, int bits)
{
    if (bits == 4) return packed[string_byte_offset(row, group, p, cols, bits)];
    if (bits == 2) return (packed[string_byte_offset(row, group, p / 2, cols, bits)] >> (4 * (p % 2))) & 0xFu;
    int64_t unit = p / 16, pu = p % 16, base = 12 * unit;
    if (pu < 12) return packed[string_byte_offset(row, group, base + pu, cols, bits)] & 0x3Fu;
    int64_t q = pu - 12;
    unsigned v = 0;
    for (int k = 0; k < 3; ++k) {
        unsigned byte = packed[string_byte_offset(row, group, base + 4 * k + q, cols, bits)];
        v |= ((byte >> 6) & 3u) << (2 * k);
    }
    return v;
}

/* Every code of a rows x cols matrix from its packed bytes (uint8 out,
 * row-major). */
void oracle_unpack(const uint8_t *packed, int64_t rows, int64_t cols, int bits, uint8_t *codes)
{
    const unsigned mask = (1u << bits) - 1u;
    for (int64_t r = 0; r < rows; ++r) {
        for (int64_t c = 0; c < cols; ++c) {
            int64_t g = c / 256, j = c % 256;
            unsigned v = pair_value(packed, r, g, j / 2, cols, bits);
            codes[r * cols + c] = (uint8_t)((j % 2 ? v >> bits : v) & mask);
        }
    }
}

/* Dequantized fp16 weights What_D[r][c] = LUT[r][code[r][c]] (bit copies). */
void oracle_decode(const uint8_t *codes, const uint16_t *lut, int64_t rows, int64_t cols, int bits, uint16_t *w)
{
    const int64_t k = (int64_t)1 << bits;
    for (int64_t r = 0; r < rows; ++r)
        for (int64_t c = 0; c < cols; ++c) w[r * cols + c] = lut[r * k + codes[r * cols + c]];
}

/* ---- the product ------------------------------------------------------ */

/*
 * One selected row: y and its normaliser for every batch column.
 *   with_dense:  add sum_c LUT[r][code[c]] * x[b][c]
 *   with_sparse: add sum_i val[i] * x[b][col[i]] over row r's CSR entries
 *   y_in:        if non-NULL, add the fp16 value y_in[b*rows + r] (and its
 *                magnitude to the normaliser)
 * w is a caller-provided scratch row of `cols` doubles.
 */
static void row_product(int64_t r, const uint8_t *code_row, const uint16_t *lut, int bits,
                        const int32_t *row_ptr, const uint16_t *col_idx, const uint16_t *val,
                        int64_t rows, int64_t cols, const uint16_t *x, int batch, const uint16_t *y_in,
                        int with_dense, int with_sparse, double *w, double *y_out, double *scale_out,
                        int64_t out_stride, int64_t out_index)
{
    const int64_t k = (int64_t)1 << bits;
    /* reconstructed row What[r][:] for the normaliser */
    for (int64_t c = 0; c < cols; ++c) w[c] = with_dense ? oracle_f16_to_f64(lut[r * k + code_row[c]]) : 0.0;
    int64_t i0 = 0, i1 = 0;
    if (with_sparse) {
        i0 = row_ptr[r];
        i1 = row_ptr[r + 1];
        for (int64_t i = i0; i < i1; ++i) w[col_idx[i]] += oracle_f16_to_f64(val[i]);
    }
    for (int b = 0; b < batch; ++b) {
        const uint16_t *xb = x + (int64_t)b * cols;
        double acc = 0.0, sc = 0.0;
        if (with_dense)
            for (int64_t c = 0; c < cols; ++c)
                acc += oracle_f16_to_f64(lut[r * k + code_row[c]]) * oracle_f16_to_f64(xb[c]);
        if (with_sparse)
            for (int64_t i = i0; i < i1; ++i) acc += oracle_f16_to_f64(val[i]) * oracle_f16_to_f64(xb[col_idx[i]]);
        for (int64_t c = 0; c < cols; ++c) sc += fabs(w[c]) * fabs(oracle_f16_to_f64(xb[c]));
        if (y_in) {
            double yi = oracle_f16_to_f64(y_in[(int64_t)b * rows + r]);
            acc += yi;
            sc += fabs(yi);
        }
        y_out[(int64_t)b * out_stride + out_index] = acc;
        scale_out[(int64_t)b * out_stride + out_index] = sc;
    }
}

/*
 * y = (D + S) x in fp64 for selected rows.
 *   codes:   uint8 [nsel][cols], the codes of the selected rows, in sel order
 *   lut:     fp16 bits [rows][2^bits]
 *   row_ptr, col_idx, val: CSR of all rows (row_ptr NULL: no sparse part)
 *   sel:     row indices (NULL: all rows, nsel must equal rows)
 *   x:       fp16 bits [batch][cols]
 *   y_in:    fp16 bits [batch][rows] added to the result, or NULL
 *   y, scale: fp64 [batch][nsel]
 *   threads: OpenMP threads over rows (<= 0: library default)
 * Returns 0, or -1 on bad arguments / allocation failure.
 */
static int product(const uint8_t *codes, const uint16_t *lut, int bits, const int32_t *row_ptr,
                   const uint16_t *col_idx, const uint16_t *val, int64_t rows, int64_t cols, const int64_t *sel,
                   int64_t nsel, const uint16_t *x, int batch, const uint16_t *y_in, int with_dense,
                   double *y, double *scale, int threads)
{
    if (rows < 1 || cols < 1 || batch < 1 || nsel < 0) return -1;
    if (!sel && nsel != rows) return -1;
    if (sel)
        for (int64_t i = 0; i < nsel; ++i)
            if (sel[i] < 0 || sel[i] >= rows) return -1;
    int with_sparse = row_ptr != NULL;
    int err = 0;
#ifdef _OPENMP
    if (threads <= 0) threads = omp_get_max_threads();
#pragma omp parallel num_threads(threads)
#endif
    {
        double *w = (double *)malloc((size_t)cols * sizeof(double));
        if (!w) {
#ifdef _OPENMP
#pragma omp atomic write
#endif
            err = 1;
        } else {
#ifdef _OPENMP
#pragma omp for schedule(static)
#endif
            for (int64_t i = 0; i < nsel; ++i) {
                int64_t r = sel ? sel[i] : i;
                row_product(r, with_dense ? codes + i * cols : NULL, lut, bits, row_ptr, col_idx, val, rows, cols,
                            x, batch, y_in, with_dense, with_sparse, w, y, scale, nsel, i);
            }
            free(w);
        }
    }
    (void)threads;
    return err ? -1 : 0;
}

/* y = (D + S) x  (row_ptr NULL: y = D x) */
int oracle_dense_sparse_gemv(const uint8_t *codes, const uint16_t *lut, int bits, const int32_t *row_ptr,
                             const uint16_t *col_idx, const uint16_t *val, int64_t rows, int64_t cols,
                             const int64_t *sel, int64_t nsel, const uint16_t *x, int batch, double *y,
                             double *scale, int threads)
{
    return product(codes, lut, bits, row_ptr, col_idx, val, rows, cols, sel, nsel, x, batch, NULL, 1, y, scale,
                   threads);
}

/* y = y_in + S x  (y_in fp16 [batch][rows]) */
int oracle_spmv_add(const int32_t *row_ptr, const uint16_t *col_idx, const uint16_t *val, int64_t rows,
                    int64_t cols, const int64_t *sel, int64_t nsel, const uint16_t *x, int batch,
                    const uint16_t *y_in, double *y, double *scale, int threads)
{
    if (!row_ptr || !y_in) return -1;
    return product(NULL, NULL, 3, row_ptr, col_idx, val, rows, cols, sel, nsel, x, batch, y_in, 0, y, scale,
                   threads);
}
