/*
 * synth.c -- seeded, counter-based synthetic inputs for the dense-and-sparse
 * LUT matrix-vector product y = (D + S) x.
 *
 * This module draws inputs only: b-bit codes, per-row fp16 lookup tables,
 * sparse outlier positions and values, and fp16 activations.  It holds none
 * of the product's arithmetic (no unpacking, no lookup, no multiply-add), so
 * both the HIP path and the CPU oracle can be fed from it.
 *
 * Shapes and distributions follow the workloads the method is evaluated on
 * (SqueezeLLM: Dense-and-Sparse Quantization, summary page, §3.4 "The
 * Dense-and-Sparse Decomposition" for the ~0.45% outlier budget, Appendix C /
 * Figure C.1 for the skewed per-row outlier counts): LLaMA layer shapes,
 * uniform codes, N(0, sigma) centroids, N(0, sigma_s) outliers.
 *
 * Every element is a pure function of (seed, stream, index): draw(key, i) is
 * the i-th output of SplitMix64 started at `key` (Steele, Lea & Flood,
 * "Fast splittable pseudorandom number generators", OOPSLA 2014; the
 * finalizer constants are the published mix64 variant).  Any row range can
 * therefore be regenerated on its own, which lets a checker rebuild sampled
 * rows of a multi-gigabyte weight stream without storing it.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define GOLDEN 0x9E3779B97F4A7C15ULL

static inline uint64_t mix64(uint64_t z)
{
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ULL;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBULL;
    return z ^ (z >> 31);
}

/* Key of one independent stream (one tensor of one matrix of one workload). */
uint64_t synth_key(uint64_t seed, uint64_t stream)
{
    return mix64(mix64(seed + GOLDEN) ^ mix64(stream ^ 0xD1B54A32D192ED03ULL));
}

/* i-th 64-bit draw of the stream. */
uint64_t synth_draw(uint64_t key, uint64_t i)
{
    return mix64(key + (i + 1) * GOLDEN);
}

/* Uniform in [0, n) by the multiply-high map (bias < n / 2^64). */
static inline uint64_t below(uint64_t h, uint64_t n)
{
    return (uint64_t)(((unsigned __int128)h * (unsigned __int128)n) >> 64);
}

/* Standard normal number i of the stream: Box-Muller on draws 2i, 2i+1. */
double synth_normal(uint64_t key, uint64_t i)
{
    const double two_pi = 6.283185307179586476925286766559;
    uint64_t h1 = synth_draw(key, 2 * i), h2 = synth_draw(key, 2 * i + 1);
    double u1 = (double)((h1 >> 11) + 1) * 0x1.0p-53; /* (0, 1] */
    double u2 = (double)(h2 >> 11) * 0x1.0p-53;       /* [0, 1) */
    return sqrt(-2.0 * log(u1)) * cos(two_pi * u2);
}

/* IEEE-754 binary16 bits of v, round to nearest, ties to even.  Used only to
 * store drawn values; scaling by powers of two is exact, rint() rounds in the
 * default nearest-even mode. */
uint16_t synth_f16(double v)
{
    uint16_t sign = signbit(v) ? 0x8000u : 0u;
    double a = fabs(v);
    if (isnan(v)) return (uint16_t)(sign | 0x7E00u);
    if (a < 0x1.0p-14) { /* subnormal range: units of 2^-24 */
        double m = rint(a * 0x1.0p24); /* 0..1024; 1024 encodes 2^-14 */
        return (uint16_t)(sign | (uint16_t)m);
    }
    int ex;
    frexp(a, &ex); /* a = f * 2^ex, f in [0.5, 1) */
    int e = ex - 1; /* a in [2^e, 2^(e+1)) */
    double m = rint(ldexp(a, 10 - e)); /* 1024..2048 */
    if (m >= 2048.0) { m = 1024.0; e += 1; }
    if (e + 15 > 30) return (uint16_t)(sign | 0x7C00u);
    return (uint16_t)(sign | (uint16_t)((e + 15) << 10) | (uint16_t)(m - 1024.0));
}

/* Codes of rows [row0, row0 + nrows) of a rows x cols matrix, row-major uint8,
 * uniform in [0, 2^bits).  Code (r, c) is byte (c mod 8) of draw((r*cols + c)/8),
 * masked to `bits` bits (cols is a multiple of 8). */
void synth_codes(uint64_t key, int64_t row0, int64_t nrows, int64_t cols, int bits, uint8_t *out)
{
    const uint8_t mask = (uint8_t)((1u << bits) - 1u);
    const int64_t words = nrows * cols / 8;
    const uint64_t base = (uint64_t)(row0 * cols / 8);
#pragma omp parallel for schedule(static)
    for (int64_t w = 0; w < words; ++w) {
        uint64_t h = synth_draw(key, base + (uint64_t)w);
        uint8_t *o = out + w * 8;
        for (int j = 0; j < 8; ++j) o[j] = (uint8_t)((h >> (8 * j)) & mask);
    }
}

/* n fp16 values sigma * N(0,1), normal numbers start .. start+n-1. */
void synth_normal_f16(uint64_t key, int64_t start, int64_t n, double sigma, uint16_t *out)
{
#pragma omp parallel for schedule(static) if (n > 65536)
    for (int64_t i = 0; i < n; ++i) out[i] = synth_f16(sigma * synth_normal(key, (uint64_t)(start + i)));
}

static int cmp_f16_value(const void *a, const void *b)
{
    /* order by numeric value; only finite values are drawn here */
    uint16_t x = *(const uint16_t *)a, y = *(const uint16_t *)b;
    int sx = x >> 15, sy = y >> 15;
    int kx = sx ? -(int)(x & 0x7FFF) : (int)(x & 0x7FFF);
    int ky = sy ? -(int)(y & 0x7FFF) : (int)(y & 0x7FFF);
    return (kx > ky) - (kx < ky);
}

/* Lookup tables for rows [row0, row0 + nrows): 2^bits fp16 centroids per row
 * drawn sigma * N(0,1) (normal number r * 2^bits + e), optionally sorted
 * ascending per row. */
void synth_lut(uint64_t key, int64_t row0, int64_t nrows, int bits, double sigma, int sorted, uint16_t *out)
{
    const int64_t k = (int64_t)1 << bits;
#pragma omp parallel for schedule(static) if (nrows > 4096)
    for (int64_t r = 0; r < nrows; ++r) {
        uint16_t *o = out + r * k;
        for (int64_t e = 0; e < k; ++e) o[e] = synth_f16(sigma * synth_normal(key, (uint64_t)((row0 + r) * k + e)));
        if (sorted) qsort(o, (size_t)k, sizeof(uint16_t), cmp_f16_value);
    }
}

/* Outlier count for a density given in basis points (1 bp = 0.01%), rounded
 * half up in integer arithmetic: round(rows * cols * bp / 10000). */
int64_t synth_nnz_bp(int64_t rows, int64_t cols, int64_t bp)
{
    return (rows * cols * bp + 5000) / 10000;
}

/* Fill CSR arrays from a row-major position bitmap; outlier values are
 * sigma_s * N(0,1) drawn at normal number (r * cols + c) of key_val. */
static void bitmap_to_csr(const uint64_t *bm, int64_t rows, int64_t cols, uint64_t key_val, double sigma_s,
                          int32_t *row_ptr, uint16_t *col, uint16_t *val)
{
    int64_t k = 0;
    row_ptr[0] = 0;
    for (int64_t r = 0; r < rows; ++r) {
        int64_t p0 = r * cols, p1 = p0 + cols;
        int64_t p = p0;
        while (p < p1) {
            uint64_t w = bm[p >> 6] >> (p & 63);
            if (w == 0) { p = (p | 63) + 1; continue; }
            p += __builtin_ctzll(w);
            if (p >= p1) break;
            col[k] = (uint16_t)(p - p0);
            val[k] = synth_f16(sigma_s * synth_normal(key_val, (uint64_t)p));
            ++k;
            ++p;
        }
        row_ptr[r + 1] = (int32_t)k;
    }
}

/* nnz distinct positions drawn uniformly from the rows x cols grid (a draw
 * that hits a taken position is skipped), stored as sorted CSR.
 * Returns 0, or -1 on bad arguments / allocation failure. */
int synth_csr_uniform(uint64_t key_pos, uint64_t key_val, int64_t rows, int64_t cols, int64_t nnz, double sigma_s,
                      int32_t *row_ptr, uint16_t *col, uint16_t *val)
{
    const int64_t cells = rows * cols;
    if (nnz < 0 || nnz > cells || cols > 65536) return -1;
    uint64_t *bm = (uint64_t *)calloc((size_t)((cells + 63) / 64), sizeof(uint64_t));
    if (!bm) return -1;
    int64_t got = 0;
    for (uint64_t i = 0; got < nnz; ++i) {
        uint64_t p = below(synth_draw(key_pos, i), (uint64_t)cells);
        uint64_t bit = 1ULL << (p & 63);
        if (!(bm[p >> 6] & bit)) { bm[p >> 6] |= bit; ++got; }
    }
    bitmap_to_csr(bm, rows, cols, key_val, sigma_s, row_ptr, col, val);
    free(bm);
    return 0;
}

struct frac_rank { double frac; int64_t rank; };

static int cmp_frac_rank(const void *a, const void *b)
{
    const struct frac_rank *x = (const struct frac_rank *)a, *y = (const struct frac_rank *)b;
    if (x->frac != y->frac) return x->frac > y->frac ? -1 : 1;
    return (x->rank > y->rank) - (x->rank < y->rank);
}

/* Per-row outlier counts following a rank-form Zipf law: the row holding rank
 * k (k = 1..rows, ranks assigned by a seeded Fisher-Yates permutation) gets
 * weight k^-s; counts are nnz * w / sum(w), capped at cols with the excess
 * spread over the remaining rows, then made integral by largest remainder. */
static int zipf_counts(uint64_t key_perm, int64_t rows, int64_t cols, int64_t nnz, double s, int64_t *count_of_row)
{
    int64_t *perm = (int64_t *)malloc((size_t)rows * sizeof(int64_t));
    double *ideal = (double *)malloc((size_t)rows * sizeof(double));
    int64_t *cnt = (int64_t *)malloc((size_t)rows * sizeof(int64_t));
    if (!perm || !ideal || !cnt) { free(perm); free(ideal); free(cnt); return -1; }
    for (int64_t i = 0; i < rows; ++i) perm[i] = i;
    for (int64_t i = rows - 1; i > 0; --i) { /* Fisher-Yates */
        int64_t j = (int64_t)below(synth_draw(key_perm, (uint64_t)i), (uint64_t)(i + 1));
        int64_t t = perm[i]; perm[i] = perm[j]; perm[j] = t;
    }
    /* cap the heaviest ranks at cols (weights fall with rank) */
    int64_t remaining = nnz, k0 = 0;
    for (;;) {
        if (k0 >= rows) break;
        double wsum = 0.0;
        for (int64_t k = k0; k < rows; ++k) wsum += pow((double)(k + 1), -s);
        double c = (double)remaining * pow((double)(k0 + 1), -s) / wsum;
        if (c < (double)cols) {
            for (int64_t k = k0; k < rows; ++k) ideal[k] = (double)remaining * pow((double)(k + 1), -s) / wsum;
            break;
        }
        ideal[k0] = (double)cols;
        remaining -= cols;
        ++k0;
    }
    int64_t assigned = 0;
    for (int64_t k = 0; k < rows; ++k) { cnt[k] = (int64_t)floor(ideal[k]); assigned += cnt[k]; }
    /* largest remainder: the leftover units go to the largest fractional
     * parts, ties to the lower rank */
    int64_t left = nnz - assigned;
    struct frac_rank *fr = (struct frac_rank *)malloc((size_t)rows * sizeof(struct frac_rank));
    if (!fr) { free(perm); free(ideal); free(cnt); return -1; }
    for (int64_t k = 0; k < rows; ++k) { fr[k].frac = ideal[k] - floor(ideal[k]); fr[k].rank = k; }
    qsort(fr, (size_t)rows, sizeof(struct frac_rank), cmp_frac_rank);
    for (int64_t i = 0; i < rows && left > 0; ++i)
        if (cnt[fr[i].rank] < cols) { cnt[fr[i].rank] += 1; --left; }
    free(fr);
    for (int64_t k = 0; k < rows; ++k) count_of_row[perm[k]] = cnt[k];
    free(perm); free(ideal); free(cnt);
    return 0;
}

/* Skewed outliers: per-row counts from zipf_counts, columns within a row
 * distinct and uniform, values sigma_s * N(0,1).  Returns 0 or -1. */
int synth_csr_zipf(uint64_t key_perm, uint64_t key_pos, uint64_t key_val, int64_t rows, int64_t cols, int64_t nnz,
                   double s, double sigma_s, int32_t *row_ptr, uint16_t *col, uint16_t *val)
{
    const int64_t cells = rows * cols;
    if (nnz < 0 || nnz > cells || cols > 65536) return -1;
    int64_t *cnt = (int64_t *)malloc((size_t)rows * sizeof(int64_t));
    uint64_t *bm = (uint64_t *)calloc((size_t)((cells + 63) / 64), sizeof(uint64_t));
    if (!cnt || !bm) { free(cnt); free(bm); return -1; }
    if (zipf_counts(key_perm, rows, cols, nnz, s, cnt) != 0) { free(cnt); free(bm); return -1; }
    for (int64_t r = 0; r < rows; ++r) {
        int64_t n = cnt[r];
        int invert = n > cols / 2; /* draw the absent columns instead */
        int64_t want = invert ? cols - n : n;
        uint64_t kr = mix64(key_pos ^ mix64((uint64_t)r + 1));
        uint64_t *row_bits = bm; /* positions are flat indices r*cols + c */
        int64_t got = 0;
        for (uint64_t i = 0; got < want; ++i) {
            uint64_t p = (uint64_t)(r * cols) + below(synth_draw(kr, i), (uint64_t)cols);
            uint64_t bit = 1ULL << (p & 63);
            if (!(row_bits[p >> 6] & bit)) { row_bits[p >> 6] |= bit; ++got; }
        }
        if (invert) {
            for (int64_t c = 0; c < cols; ++c) {
                uint64_t p = (uint64_t)(r * cols + c);
                bm[p >> 6] ^= 1ULL << (p & 63);
            }
        }
    }
    bitmap_to_csr(bm, rows, cols, key_val, sigma_s, row_ptr, col, val);
    free(cnt);
    free(bm);
    return 0;
}
