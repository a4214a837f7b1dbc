// sqllm_quantize.hip -- the offline steps upstream of the product: the
// dense-and-sparse split of an fp16 weight matrix and the per-row
// (optionally sensitivity-weighted) 1-D k-means that yields codes and
// fp16 lookup tables (SqueezeLLM: Dense-and-Sparse Quantization, summary
// page: §3.4 "The Dense-and-Sparse Decomposition"; §3.3, Eq. 1 and Eq. 6,
// "The weighted k-means algorithm in practice").
//
// Split: T_min / T_max are the values of rank floor(n p) from either end of
// the matrix's fp16 values in IEEE total order (-0 before +0), found exactly
// from a 65536-bin histogram of the bit patterns (one bin per fp16 value);
// a weight is an outlier when it compares below T_min or above T_max.  With
// sensitivities, T_s is the fp32 sensitivity of rank n - 1 - n_top, found
// exactly from two 16-bit histogram passes (high key halves, then low halves
// within the chosen high half), and a weight whose sensitivity is above T_s
// goes to S as well.  S goes to CSR (columns ascending), D keeps the rest
// with zeros there.
//
// k-means: one workgroup per row.  Centroids start uniformly spaced over the
// row's range; each step assigns every weight to the nearest centroid (the
// centroids stay sorted, so that is the interval between midpoints; a tie
// goes to the lower one) and moves each centroid to the sensitivity-weighted
// mean of its weights (unchanged when it has none).  Centroids and sums are
// fp64, reduced in a fixed order.  After the steps the centroids are rounded to
// fp16 and every weight takes the index of its nearest fp16 centroid.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "sqllm_internal.h"

namespace sqllm {
namespace {

__device__ __forceinline__ float h2f(uint16_t h) { return (float)__builtin_bit_cast(_Float16, h); }
__device__ __forceinline__ uint16_t f2h(float f) { return __builtin_bit_cast(uint16_t, (_Float16)f); }

// IEEE total order of binary16 / binary32 bit patterns as unsigned keys.
__device__ __forceinline__ uint32_t order_key(uint32_t b) { return (b & 0x8000u) ? (~b & 0xFFFFu) : (b | 0x8000u); }
__device__ __forceinline__ uint32_t order_key32(uint32_t b) { return (b & 0x80000000u) ? ~b : (b | 0x80000000u); }

constexpr int kHistThreads = 512;
constexpr int kHistChunk = 65535; // values per workgroup: a 16-bit LDS counter cannot overflow

enum HistMode { kHistF16 = 0, kHistF32High = 1, kHistF32Low = 2 };

// Histogram of 16-bit keys: the fp16 order key, the high half of the fp32
// order key, or the low half of the fp32 keys whose high half is *sel.
// Per-workgroup LDS counters (two 16-bit counts per word) added into the
// global 65536 bins.
template <int MODE>
__global__ void __launch_bounds__(kHistThreads) hist_kernel(const void *__restrict__ src, int64_t n,
                                                            const uint32_t *__restrict__ sel,
                                                            uint32_t *__restrict__ bins)
{
    __shared__ uint32_t h[32768];
    for (int i = threadIdx.x; i < 32768; i += kHistThreads) h[i] = 0;
    const uint32_t want = MODE == kHistF32Low ? *sel : 0u;
    __syncthreads();
    const int64_t beg = (int64_t)blockIdx.x * kHistChunk, end = min(beg + kHistChunk, n);
    for (int64_t i = beg + threadIdx.x; i < end; i += kHistThreads) {
        uint32_t k;
        if (MODE == kHistF16) {
            k = order_key(((const uint16_t *)src)[i]);
        } else {
            const uint32_t k32 = order_key32(((const uint32_t *)src)[i]);
            if (MODE == kHistF32Low && (k32 >> 16) != want) continue;
            k = MODE == kHistF32High ? k32 >> 16 : k32 & 0xFFFFu;
        }
        atomicAdd(&h[k >> 1], 1u << (16 * (k & 1)));
    }
    __syncthreads();
    for (int i = threadIdx.x; i < 32768; i += kHistThreads) {
        const uint32_t v = h[i];
        if (v & 0xFFFFu) atomicAdd(&bins[2 * i], v & 0xFFFFu);
        if (v >> 16) atomicAdd(&bins[2 * i + 1], v >> 16);
    }
}

// For ranks r[0], r[1] (ascending, from `rank` in device memory when given,
// else r0 / r1): the bin holding that rank and the rank within the bin.
// One workgroup.
__global__ void __launch_bounds__(1024) select_kernel(const uint32_t *__restrict__ bins, int64_t r0, int64_t r1,
                                                      const int64_t *__restrict__ rank,
                                                      uint32_t *__restrict__ out_bin, int64_t *__restrict__ out_rest)
{
    __shared__ int64_t part[1024];
    const int t = threadIdx.x;
    int64_t s = 0;
    for (int i = 0; i < 64; ++i) s += bins[t * 64 + i];
    part[t] = s;
    __syncthreads();
    // inclusive scan over the threads' sums (Hillis-Steele)
    for (int off = 1; off < 1024; off <<= 1) {
        const int64_t v = t >= off ? part[t - off] : 0;
        __syncthreads();
        part[t] += v;
        __syncthreads();
    }
    const int64_t before = t > 0 ? part[t - 1] : 0;
    for (int q = 0; q < 2; ++q) {
        const int64_t r = rank ? rank[q] : (q == 0 ? r0 : r1);
        if (before <= r && r < part[t]) {
            int64_t c = before;
            for (int i = 0; i < 64; ++i) {
                const int64_t next = c + bins[t * 64 + i];
                if (r < next) {
                    out_bin[q] = (uint32_t)(t * 64 + i);
                    out_rest[q] = r - c;
                    break;
                }
                c = next;
            }
        }
    }
}

// Whether a weight goes to S: outside [lo, hi], or more sensitive than t_s.
__device__ __forceinline__ bool to_sparse(uint16_t b, float lo, float hi, const float *srow, int c, float t_s)
{
    const float v = h2f(b);
    return v < lo || v > hi || (srow && srow[c] > t_s);
}

// Entries of S per row (one workgroup per row) and their total.
__global__ void __launch_bounds__(256) count_kernel(const uint16_t *__restrict__ w, const float *__restrict__ sens,
                                                    int cols, uint16_t t_min, uint16_t t_max, float t_s,
                                                    int32_t *__restrict__ counts,
                                                    unsigned long long *__restrict__ total)
{
    __shared__ int part[4];
    const float lo = h2f(t_min), hi = h2f(t_max);
    const uint16_t *row = w + (int64_t)blockIdx.x * cols;
    const float *srow = sens ? sens + (int64_t)blockIdx.x * cols : nullptr;
    int c = 0;
    for (int i = threadIdx.x; i < cols; i += 256) c += to_sparse(row[i], lo, hi, srow, i, t_s);
    for (int off = 32; off > 0; off >>= 1) c += __shfl_xor(c, off, 64);
    if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = c;
    __syncthreads();
    if (threadIdx.x == 0) {
        const int n = part[0] + part[1] + part[2] + part[3];
        counts[blockIdx.x] = n;
        if (total) atomicAdd(total, (unsigned long long)n);
    }
}

// row_ptr = exclusive prefix sum of the counts; one workgroup.
__global__ void __launch_bounds__(1024) scan_kernel(const int32_t *__restrict__ counts, int rows,
                                                    int32_t *__restrict__ row_ptr)
{
    __shared__ int64_t part[1024];
    const int t = threadIdx.x;
    const int per = (rows + 1023) / 1024;
    const int b = min(t * per, rows), e = min(b + per, rows);
    int64_t s = 0;
    for (int i = b; i < e; ++i) s += counts[i];
    part[t] = s;
    __syncthreads();
    for (int off = 1; off < 1024; off <<= 1) {
        const int64_t v = t >= off ? part[t - off] : 0;
        __syncthreads();
        part[t] += v;
        __syncthreads();
    }
    int64_t run = t > 0 ? part[t - 1] : 0;
    for (int i = b; i < e; ++i) {
        row_ptr[i] = (int32_t)run;
        run += counts[i];
    }
    if (t == 1023) row_ptr[rows] = (int32_t)part[1023];
}

// CSR entries of each row in column order, D, and (when asked) the
// sensitivities with zeros at S's entries; one workgroup of four waves per
// row, 256 columns per step.  Entries past the capacity are dropped and
// flagged.
__global__ void __launch_bounds__(256) fill_kernel(const uint16_t *__restrict__ w, const float *__restrict__ sens,
                                                   int cols, uint16_t t_min, uint16_t t_max, float t_s,
                                                   const int32_t *__restrict__ row_ptr,
                                                   uint16_t *__restrict__ col_idx, uint16_t *__restrict__ val,
                                                   int64_t capacity, uint16_t *__restrict__ dense,
                                                   float *__restrict__ sens_dense, int *__restrict__ overflow)
{
    __shared__ int wave_n[4];
    const float lo = h2f(t_min), hi = h2f(t_max);
    const int64_t r = blockIdx.x;
    const uint16_t *row = w + r * cols;
    const float *srow = sens ? sens + r * cols : nullptr;
    uint16_t *drow = dense + r * cols;
    float *sdrow = sens_dense ? sens_dense + r * cols : nullptr;
    const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
    int64_t base = row_ptr[r];
    for (int c0 = 0; c0 < cols; c0 += 256) {
        const int c = c0 + threadIdx.x;
        const uint16_t b = c < cols ? row[c] : 0;
        const bool out = c < cols && to_sparse(b, lo, hi, srow, c, t_s);
        const uint64_t m = __ballot(out);
        const int before_lane = __popcll(m & ((1ull << lane) - 1));
        if (lane == 0) wave_n[wv] = __popcll(m);
        __syncthreads();
        int before_wave = 0;
        for (int k = 0; k < wv; ++k) before_wave += wave_n[k];
        const int step_n = wave_n[0] + wave_n[1] + wave_n[2] + wave_n[3];
        if (c < cols) {
            drow[c] = out ? (uint16_t)0 : b;
            if (sdrow) sdrow[c] = out ? 0.f : srow[c];
        }
        if (out) {
            const int64_t at = base + before_wave + before_lane;
            if (at < capacity) {
                col_idx[at] = (uint16_t)c;
                val[at] = b;
            } else {
                *overflow = 1;
            }
        }
        base += step_n;
        __syncthreads();
    }
}

constexpr int kKmThreads = 256;

// Sum over the workgroup in a fixed order (wave shuffles, then the four waves).
__device__ __forceinline__ double block_sum(double v, double *scratch)
{
    for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off, 64);
    __syncthreads();
    if ((threadIdx.x & 63) == 0) scratch[threadIdx.x >> 6] = v;
    __syncthreads();
    return ((scratch[0] + scratch[1]) + scratch[2]) + scratch[3];
}

// One workgroup per row; all centroid arithmetic in fp64.  The fp16 weights
// and their differences are exact in fp64, so the final nearest-centroid
// choice is exact.
template <int K>
__global__ void __launch_bounds__(kKmThreads) kmeans_kernel(const uint16_t *__restrict__ dense,
                                                            const float *__restrict__ sens, int cols, int iters,
                                                            uint8_t *__restrict__ codes, uint16_t *__restrict__ lut)
{
    __shared__ double scratch[4];
    __shared__ float ext[8];
    const int64_t r = blockIdx.x;
    const uint16_t *row = dense + r * cols;
    const float *srow = sens ? sens + r * cols : nullptr;
    // range of the row
    float lo = INFINITY, hi = -INFINITY;
    for (int i = threadIdx.x; i < cols; i += kKmThreads) {
        const float v = h2f(row[i]);
        lo = fminf(lo, v);
        hi = fmaxf(hi, v);
    }
    for (int off = 32; off > 0; off >>= 1) {
        lo = fminf(lo, __shfl_xor(lo, off, 64));
        hi = fmaxf(hi, __shfl_xor(hi, off, 64));
    }
    if ((threadIdx.x & 63) == 0) {
        ext[threadIdx.x >> 6] = lo;
        ext[4 + (threadIdx.x >> 6)] = hi;
    }
    __syncthreads();
    const double dlo = fminf(fminf(ext[0], ext[1]), fminf(ext[2], ext[3]));
    const double dhi = fmaxf(fmaxf(ext[4], ext[5]), fmaxf(ext[6], ext[7]));
    double c[K];
#pragma unroll
    for (int j = 0; j < K; ++j) c[j] = dlo + (double)j * (dhi - dlo) / (double)(K - 1);
    for (int it = 0; it < iters; ++it) {
        // the centroids stay sorted, so the nearest one is found from the
        // midpoints; a weight on a midpoint goes to the lower centroid
        double mid[K - 1];
#pragma unroll
        for (int j = 0; j < K - 1; ++j) mid[j] = 0.5 * (c[j] + c[j + 1]);
        double sw[K], swx[K];
#pragma unroll
        for (int j = 0; j < K; ++j) sw[j] = swx[j] = 0.0;
        for (int i = threadIdx.x; i < cols; i += kKmThreads) {
            const double x = h2f(row[i]);
            const double f = srow ? (double)srow[i] : 1.0;
            int q = 0;
#pragma unroll
            for (int j = 0; j < K - 1; ++j) q += x > mid[j];
#pragma unroll
            for (int j = 0; j < K; ++j) {
                const bool s = q == j;
                sw[j] += s ? f : 0.0;
                swx[j] += s ? f * x : 0.0;
            }
        }
#pragma unroll
        for (int j = 0; j < K; ++j) {
            const double tw = block_sum(sw[j], scratch);
            const double twx = block_sum(swx[j], scratch);
            if (tw > 0.0) c[j] = twx / tw;
        }
    }
    uint16_t l[K];
    double lv[K];
#pragma unroll
    for (int j = 0; j < K; ++j) {
        l[j] = __builtin_bit_cast(uint16_t, (_Float16)c[j]); // one rounding, to nearest even
        lv[j] = h2f(l[j]);
    }
    if (threadIdx.x < K) {
#pragma unroll
        for (int j = 0; j < K; ++j)
            if (j == (int)threadIdx.x) lut[r * K + j] = l[j];
    }
    for (int i = threadIdx.x; i < cols; i += kKmThreads) {
        const double x = h2f(row[i]);
        int best = 0;
        double bd = fabs(x - lv[0]);
#pragma unroll
        for (int j = 1; j < K; ++j) {
            const double d = fabs(x - lv[j]);
            if (d < bd) {
                bd = d;
                best = j;
            }
        }
        codes[r * cols + i] = (uint8_t)best;
    }
}

} // namespace

hipError_t launch_rank_select(const void *src, bool fp32, int64_t n, int64_t r0, int64_t r1, uint32_t *bins,
                              SelectOut *out, hipStream_t stream)
{
    const unsigned blocks = (unsigned)((n + kHistChunk - 1) / kHistChunk);
    if (hipMemsetAsync(bins, 0, 65536 * sizeof(uint32_t), stream) != hipSuccess) return hipGetLastError();
    if (!fp32) {
        hipLaunchKernelGGL(hist_kernel<kHistF16>, dim3(blocks), dim3(kHistThreads), 0, stream, src, n,
                           (const uint32_t *)nullptr, bins);
        hipLaunchKernelGGL(select_kernel, dim3(1), dim3(1024), 0, stream, bins, r0, r1, (const int64_t *)nullptr,
                           out->bin, out->rest);
        return hipGetLastError();
    }
    // high halves of the keys, then the low halves within the selected high half
    hipLaunchKernelGGL(hist_kernel<kHistF32High>, dim3(blocks), dim3(kHistThreads), 0, stream, src, n,
                       (const uint32_t *)nullptr, bins);
    hipLaunchKernelGGL(select_kernel, dim3(1), dim3(1024), 0, stream, bins, r0, r1, (const int64_t *)nullptr,
                       out->bin, out->rest);
    if (hipMemsetAsync(bins, 0, 65536 * sizeof(uint32_t), stream) != hipSuccess) return hipGetLastError();
    hipLaunchKernelGGL(hist_kernel<kHistF32Low>, dim3(blocks), dim3(kHistThreads), 0, stream, src, n,
                       (const uint32_t *)out->bin, bins);
    hipLaunchKernelGGL(select_kernel, dim3(1), dim3(1024), 0, stream, bins, (int64_t)0, (int64_t)0,
                       (const int64_t *)out->rest, out->bin2, out->rest2);
    return hipGetLastError();
}

hipError_t launch_outlier_count(const uint16_t *w, const float *sens, int rows, int cols, uint16_t t_min,
                                uint16_t t_max, float t_s, int32_t *counts, unsigned long long *total,
                                hipStream_t stream)
{
    hipLaunchKernelGGL(count_kernel, dim3((unsigned)rows), dim3(256), 0, stream, w, sens, cols, t_min, t_max, t_s,
                       counts, total);
    return hipGetLastError();
}

hipError_t launch_outlier_extract(const uint16_t *w, const float *sens, int rows, int cols, uint16_t t_min,
                                  uint16_t t_max, float t_s, int32_t *counts, int32_t *row_ptr, uint16_t *col_idx,
                                  uint16_t *val, int64_t capacity, uint16_t *dense, float *sens_dense, int *overflow,
                                  hipStream_t stream)
{
    hipLaunchKernelGGL(count_kernel, dim3((unsigned)rows), dim3(256), 0, stream, w, sens, cols, t_min, t_max, t_s,
                       counts, (unsigned long long *)nullptr);
    hipLaunchKernelGGL(scan_kernel, dim3(1), dim3(1024), 0, stream, counts, rows, row_ptr);
    hipLaunchKernelGGL(fill_kernel, dim3((unsigned)rows), dim3(256), 0, stream, w, sens, cols, t_min, t_max, t_s,
                       row_ptr, col_idx, val, capacity, dense, sens_dense, overflow);
    return hipGetLastError();
}

hipError_t launch_kmeans(const uint16_t *dense, const float *sens, int rows, int cols, int bits, int iters,
                         uint8_t *codes, uint16_t *lut, hipStream_t stream)
{
    if (bits == 2)
        hipLaunchKernelGGL(kmeans_kernel<4>, dim3((unsigned)rows), dim3(kKmThreads), 0, stream, dense, sens, cols,
                           iters, codes, lut);
    else if (bits == 3)
        hipLaunchKernelGGL(kmeans_kernel<8>, dim3((unsigned)rows), dim3(kKmThreads), 0, stream, dense, sens, cols,
                           iters, codes, lut);
    else
        hipLaunchKernelGGL(kmeans_kernel<16>, dim3((unsigned)rows), dim3(kKmThreads), 0, stream, dense, sens, cols,
                           iters, codes, lut);
    return hipGetLastError();
}

} // namespace sqllm
