// sqllm_kernels.hip -- gfx950 kernels of the dense-and-sparse LUT GEMV
// y = (D + S) x (SqueezeLLM: Dense-and-Sparse Quantization, summary page,
// §3.4 "Kernel Implementation"; storage per §3.4 "The 3/4-bit storage
// format").
//
// Mapping (one wave = 64 rows, one lane = one output row):
//   * codes stream in as 128-bit loads: the packed layout puts the same
//     16-byte piece of 64 consecutive rows next to each other, so one
//     wave-wide load moves 1 KiB of contiguous codes;
//   * because every lane works on its own row, every lane owns its own copy
//     of that row's lookup table in LDS.  The table is a *pair* table: entry
//     e = (code_even | code_odd << b) holds both centroids as one half2, at
//     byte (e << 8) | (lane << 2).  A lookup is one 32-bit LDS read whose
//     bank is the lane number (conflict free), and it feeds one
//     v_dot2_f32_f16 (two fp16 products, fp32 accumulate);
//   * all lanes of a wave work on the same columns at the same time, so the
//     activation pairs are wave-uniform and come in through scalar loads
//     (SGPR operands of the dot product), not through LDS or VGPRs;
//   * long rows are split across workgroups along the columns; each
//     workgroup reduces its waves in LDS and the last workgroup of a row tile
//     to finish (device-scope counter) adds the partial sums in a fixed order
//     and writes fp16 y once;
//   * the outliers of the tile (CSR) are shared evenly by all threads of
//     the tile's workgroups (balanced, independent of per-row skew,
//     §3.4 "Kernel Implementation", balanced sparse kernel; Appendix C),
//     reduced per row with a segmented scan across the wave, and added to
//     the same fp32 accumulators before the single rounding (kernel fusion).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <utility>

#include "sqllm_internal.h"

namespace sqllm {
namespace {

typedef _Float16 half2_t __attribute__((ext_vector_type(2)));
typedef const __attribute__((address_space(4))) uint32_t *const_u32_ptr;
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float f16_to_f32(uint16_t h) { return (float)__builtin_bit_cast(_Float16, h); }
__device__ __forceinline__ uint16_t f32_to_f16_rne(float f) { return __builtin_bit_cast(uint16_t, (_Float16)f); }

template <int BITS>
struct Format {
    static constexpr int kEntries = 1 << BITS;            // centroids per row
    static constexpr int kPieces = 2 * BITS;              // 16-byte pieces per (row, group)
    static constexpr int kDwords = 4 * kPieces;           // dwords per (row, group)
    static constexpr int kPairs = 1 << (2 * BITS);        // pair-table entries
    static constexpr uint32_t kPairMask = (uint32_t)(kPairs - 1) << 8;
    static constexpr int kTableBytes = kPairs * 64 * 4;   // one half2 per (entry, lane)
};

// Byte address (in the pair table) of pair p of a 256-code group held in d[]:
// the 2b-bit field of codes 2p, 2p+1 is moved to bits [8, 8+2b) and the lane
// offset is or-ed in.  All shifts are compile-time constants.
template <int BITS, int P>
__device__ __forceinline__ uint32_t pair_address(const uint32_t *d, uint32_t lane4)
{
    if constexpr (BITS == 3) {
        constexpr int bit = 6 * P, i = bit >> 5, s = bit & 31;
        uint32_t v;
        if constexpr (s == 8) v = d[i];
        else if constexpr (s > 8 && s + 6 <= 32) v = d[i] >> (s - 8);
        else if constexpr (s > 8) v = __builtin_amdgcn_alignbit(d[i + 1], d[i], s - 8);
        else v = d[i] << (8 - s);
        return (v & Format<3>::kPairMask) | lane4;
    } else {
        // 4-bit: pair p is byte p; v_perm puts byte (p & 3) of d[p >> 2] into
        // bits [8, 16) and the lane offset byte into bits [0, 8).
        constexpr uint32_t sel = 0x0C0C0000u | ((4u + (P & 3)) << 8);
        return __builtin_amdgcn_perm(d[P >> 2], lane4, sel);
    }
}

template <int BITS, int B, int P>
__device__ __forceinline__ void mac_pair(const uint32_t *d, uint32_t lane4, const uint32_t *tab_bytes_base,
                                         const_u32_ptr xg, int xstride, float *acc)
{
    const uint32_t a = pair_address<BITS, P>(d, lane4);
    const uint32_t tv = *(const uint32_t *)((const char *)tab_bytes_base + a);
    const half2_t w = __builtin_bit_cast(half2_t, tv);
#pragma unroll
    for (int b = 0; b < B; ++b) {
        const uint32_t xv = xg[b * xstride + P];
        acc[b] = __builtin_amdgcn_fdot2(w, __builtin_bit_cast(half2_t, xv), acc[b], false);
    }
}

template <int BITS, int B, int P0, int... Ps>
__device__ __forceinline__ void mac_group_impl(const uint32_t *d, uint32_t lane4, const uint32_t *tab,
                                               const_u32_ptr xg, int xstride, float *acc,
                                               std::integer_sequence<int, P0, Ps...>)
{
    mac_pair<BITS, B, P0>(d, lane4, tab, xg, xstride, acc);
    if constexpr (sizeof...(Ps) > 0)
        mac_group_impl<BITS, B>(d, lane4, tab, xg, xstride, acc, std::integer_sequence<int, Ps...>{});
}

// 128 pairs (256 codes) of one group.
template <int BITS, int B>
__device__ __forceinline__ void mac_group(const uint32_t *d, uint32_t lane4, const uint32_t *tab, const_u32_ptr xg,
                                          int xstride, float *acc)
{
    mac_group_impl<BITS, B>(d, lane4, tab, xg, xstride, acc, std::make_integer_sequence<int, 128>{});
}

template <int BITS>
__device__ __forceinline__ void load_group(const u32x4 *__restrict__ src, uint32_t *d)
{
#pragma unroll
    for (int q = 0; q < Format<BITS>::kPieces; ++q) {
        const u32x4 v = __builtin_nontemporal_load(src + q * 64);
        d[4 * q + 0] = v.x;
        d[4 * q + 1] = v.y;
        d[4 * q + 2] = v.z;
        d[4 * q + 3] = v.w;
    }
}

// Pair table of the tile: entry e of lane l = LUT[row][e & (E-1)] | LUT[row][e >> b] << 16.
// Thread -> (lane l, high code h); it writes the E entries (lo = 0..E-1, h).
template <int BITS>
__device__ void build_pair_table(uint32_t *tab, const uint16_t *__restrict__ lut, int row0, int rows)
{
    constexpr int E = Format<BITS>::kEntries;
    const int nt = blockDim.x;
    for (int idx = threadIdx.x; idx < 64 * E; idx += nt) {
        const int l = idx & 63, h = idx >> 6;
        const int r = min(row0 + l, rows - 1);
        const uint4 *lrow = (const uint4 *)(lut + (int64_t)r * E);
        uint32_t lw[E / 2];
#pragma unroll
        for (int q = 0; q < E / 8; ++q) {
            const uint4 v = lrow[q];
            lw[4 * q + 0] = v.x;
            lw[4 * q + 1] = v.y;
            lw[4 * q + 2] = v.z;
            lw[4 * q + 3] = v.w;
        }
        const uint32_t hi = (uint32_t)lut[(int64_t)r * E + h] << 16;
#pragma unroll
        for (int lo = 0; lo < E; ++lo) {
            const uint32_t lov = (lo & 1) ? (lw[lo >> 1] >> 16) : (lw[lo >> 1] & 0xFFFFu);
            tab[((h << BITS) | lo) * 64 + l] = lov | hi;
        }
    }
}

// Row (0..63) of nonzero i of the tile: largest r with rps[r] <= i.
__device__ __forceinline__ int tile_row_of(const int *rps, int i)
{
    int lo = 0;
#pragma unroll
    for (int step = 32; step >= 1; step >>= 1)
        if (rps[lo + step] <= i) lo += step;
    return lo;
}

// Balanced share of the tile's outliers for this wave; per-row fp32 sums
// are added into acc_rows[b * 64 + row] (wave-private LDS slice).
template <int B>
__device__ void sparse_share(const KernelArgs &a, const int *rps, int s, int w, int nw, int lane, float *acc_rows)
{
    const int nz0 = rps[0], nz1 = rps[64];
    const int64_t len = nz1 - nz0;
    const int ws0 = nz0 + (int)(len * s / a.split), ws1 = nz0 + (int)(len * (s + 1) / a.split);
    const int64_t wlen = ws1 - ws0;
    const int v0 = ws0 + (int)(wlen * w / nw), v1 = ws0 + (int)(wlen * (w + 1) / nw);
    for (int base = v0; base < v1; base += 64) {
        const int i = base + lane;
        const bool valid = i < v1;
        int r = 64; // sentinel: never equal to a real row
        float prod[B];
#pragma unroll
        for (int b = 0; b < B; ++b) prod[b] = 0.f;
        if (valid) {
            const int c = a.col[i];
            const float v = f16_to_f32(a.val[i]);
            r = tile_row_of(rps, i);
#pragma unroll
            for (int b = 0; b < B; ++b) prod[b] = v * f16_to_f32(a.x[(int64_t)b * a.cols + c]);
        }
        // segmented inclusive scan over lanes (rows are non-decreasing in i)
#pragma unroll
        for (int off = 1; off < 64; off <<= 1) {
            const int ru = __shfl_up(r, off, 64);
            const bool same = lane >= off && ru == r;
#pragma unroll
            for (int b = 0; b < B; ++b) {
                const float pu = __shfl_up(prod[b], off, 64);
                if (same) prod[b] += pu;
            }
        }
        const int rn = __shfl_down(r, 1, 64);
        const bool last = valid && (lane == 63 || rn != r);
        if (last) {
#pragma unroll
            for (int b = 0; b < B; ++b) acc_rows[b * 64 + r] += prod[b];
        }
    }
}

} // namespace

// ---------------------------------------------------------------------------
// The fused kernel.  DENSE: y += D x;  SPARSE: y += S x;  ADDY: y += y_in.
// Grid: tiles * split workgroups (workgroup = (tile t, column split s)),
// blockDim = 64 * waves (waves <= kMaxWaves).
// LDS words of one instantiation: the pair table (DENSE) or the per-wave
// outlier row sums plus 65 row pointers (SPARSE), whichever is larger, and
// room for the final wave reduction.  Sized for kMaxWaves so it is static:
// the array then sits at LDS address 0 and a table address needs no base.
template <int BITS, int B, bool DENSE, bool SPARSE>
struct LdsWords {
    static constexpr int kTable = DENSE ? Format<BITS>::kTableBytes / 4 : 0;
    static constexpr int kSparse = SPARSE ? kMaxWaves * B * 64 + 68 : 0;
    static constexpr int kReduce = kMaxWaves * B * 64;
    static constexpr int kMax1 = kTable > kSparse ? kTable : kSparse;
    static constexpr int value = kMax1 > kReduce ? kMax1 : kReduce;
};

#ifndef SQLLM_MIN_WAVES_PER_SIMD
#define SQLLM_MIN_WAVES_PER_SIMD 3
#endif

template <int BITS, int B, bool DENSE, bool SPARSE, bool ADDY>
__global__ void __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(SQLLM_MIN_WAVES_PER_SIMD)))
dense_sparse_kernel(KernelArgs a)
{
    __shared__ __align__(16) uint32_t lds[LdsWords<BITS, B, DENSE, SPARSE>::value];
    const int nw = blockDim.x >> 6;
    // wave index, made visibly uniform so that addresses built from it
    // (the column group, hence the activation pairs) stay scalar
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    const int t = blockIdx.x / a.split, s = blockIdx.x - t * a.split;
    const int row0 = t * 64;
    const uint32_t lane4 = (uint32_t)lane << 2;

    float acc[B];
#pragma unroll
    for (int b = 0; b < B; ++b) acc[b] = 0.f;

    // -- first codes of this wave in flight before anything else
    constexpr int BITS_ = BITS == 4 ? 4 : 3;
    constexpr int ND = Format<BITS_>::kDwords;
    uint32_t cur[ND];
    int g = 0, g_end = 0;
    const u32x4 *tile_codes = nullptr;
    if constexpr (DENSE) {
        const int g_begin = s * a.gps;
        g_end = min(g_begin + a.gps, a.groups);
        g = g_begin + w;
        tile_codes = (const u32x4 *)a.packed + (int64_t)t * a.groups * Format<BITS_>::kPieces * 64 + lane;
        if (g < g_end) load_group<BITS_>(tile_codes + (int64_t)g * Format<BITS_>::kPieces * 64, cur);
    }

    // -- outliers: LDS = [waves][B][64] fp32 row sums, then 65 row pointers
    if constexpr (SPARSE) {
        float *rows_acc = (float *)lds;
        int *rps = (int *)(rows_acc + nw * B * 64);
        for (int i = threadIdx.x; i <= 64; i += blockDim.x) rps[i] = a.row_ptr[min(row0 + i, a.rows)];
#pragma unroll
        for (int b = 0; b < B; ++b) rows_acc[(w * B + b) * 64 + lane] = 0.f;
        __syncthreads();
        sparse_share<B>(a, rps, s, w, nw, lane, rows_acc + w * B * 64);
        __syncthreads();
#pragma unroll
        for (int b = 0; b < B; ++b) acc[b] = rows_acc[(w * B + b) * 64 + lane];
        __syncthreads(); // LDS is reused for the pair table
    }

    // -- dense: pair table, then stream the codes
    if constexpr (DENSE) {
        build_pair_table<BITS_>(lds, a.lut, row0, a.rows);
        __syncthreads();
        const const_u32_ptr xpairs = (const_u32_ptr)(const void *)a.x;
        const int xstride = a.cols >> 1;
        // the next group's codes are in flight while this one is multiplied
        for (; g < g_end; g += nw) {
            uint32_t nxt[ND];
            const int gn = g + nw;
            if (gn < g_end) load_group<BITS_>(tile_codes + (int64_t)gn * Format<BITS_>::kPieces * 64, nxt);
            mac_group<BITS_, B>(cur, lane4, lds, xpairs + g * 128, xstride, acc);
#pragma unroll
            for (int k = 0; k < ND; ++k) cur[k] = nxt[k];
        }
        __syncthreads(); // table dead from here on
    }

    // -- reduce the waves of this workgroup
    float *red = (float *)lds;
#pragma unroll
    for (int b = 0; b < B; ++b) red[(w * B + b) * 64 + lane] = acc[b];
    __syncthreads();
    if (w != 0) return;

    float tot[B];
#pragma unroll
    for (int b = 0; b < B; ++b) {
        float v = 0.f;
        for (int k = 0; k < nw; ++k) v += red[(k * B + b) * 64 + lane];
        tot[b] = v;
    }
    const int row = row0 + lane;

    if (a.split > 1) {
        // partial sums of (t, s) -> workspace; the last of the tile's
        // workgroups adds them in split order
        float *part = a.part + (int64_t)t * a.split * B * 64;
#pragma unroll
        for (int b = 0; b < B; ++b) part[(s * B + b) * 64 + lane] = tot[b];
        __threadfence();
        uint32_t prev = 0;
        if (lane == 0) prev = atomicAdd(a.counters + t, 1u);
        prev = __shfl(prev, 0, 64);
        if (prev != (uint32_t)(a.split - 1)) return;
        __threadfence();
#pragma unroll
        for (int b = 0; b < B; ++b) {
            float v = 0.f;
            for (int k = 0; k < a.split; ++k) v += part[(k * B + b) * 64 + lane];
            tot[b] = v;
        }
        if (lane == 0) __hip_atomic_store(a.counters + t, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }

    if (row < a.rows) {
#pragma unroll
        for (int b = 0; b < B; ++b) {
            float v = tot[b];
            if constexpr (ADDY) v += f16_to_f32(a.y[(int64_t)b * a.rows + row]);
            a.y[(int64_t)b * a.rows + row] = f32_to_f16_rne(v);
        }
    }
}

// ---------------------------------------------------------------------------
// Offline packing and the test-only readers.  One thread per (row, group);
// thread index -> (tile, group, lane) with the lane fastest, so the 16-byte
// pieces of 64 rows are written (read) contiguously.

template <int BITS>
__global__ void __launch_bounds__(256) pack_kernel(const uint8_t *__restrict__ codes, int rows, int cols, int groups,
                                                   int64_t total, uint4 *__restrict__ packed, int *__restrict__ bad)
{
    constexpr int NDW = Format<BITS>::kDwords;
    const int64_t id = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (id >= total) return;
    const int l = (int)(id & 63);
    const int64_t rest = id >> 6;
    const int g = (int)(rest % groups);
    const int64_t t = rest / groups;
    const int64_t r = t * 64 + l;
    uint32_t wv[NDW];
#pragma unroll
    for (int k = 0; k < NDW; ++k) wv[k] = 0;
    uint32_t oor = 0;
    if (r < rows) {
        const uint4 *src = (const uint4 *)(codes + r * cols + (int64_t)g * 256);
#pragma unroll
        for (int q = 0; q < 16; ++q) {
            const uint4 v = src[q];
            const uint32_t word[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
            for (int m = 0; m < 16; ++m) {
                const uint32_t c = (word[m >> 2] >> (8 * (m & 3))) & 0xFFu;
                oor |= c >> BITS;
                const int j = q * 16 + m, bit = BITS * j, i = bit >> 5, sh = bit & 31;
                wv[i] |= c << sh;
                if (sh + BITS > 32) wv[i + 1] |= c >> (32 - sh);
            }
        }
    }
    if (oor) atomicOr(bad, 1);
    uint4 *dst = packed + ((t * groups + g) * Format<BITS>::kPieces) * 64 + l;
#pragma unroll
    for (int q = 0; q < Format<BITS>::kPieces; ++q)
        dst[q * 64] = make_uint4(wv[4 * q], wv[4 * q + 1], wv[4 * q + 2], wv[4 * q + 3]);
}

template <int BITS, bool DECODE>
__global__ void __launch_bounds__(256) unpack_kernel(const uint4 *__restrict__ packed, const uint16_t *__restrict__ lut,
                                                     int rows, int cols, int groups, int64_t total,
                                                     uint8_t *__restrict__ codes, uint16_t *__restrict__ w)
{
    constexpr int NDW = Format<BITS>::kDwords;
    constexpr uint32_t mask = (1u << BITS) - 1u;
    const int64_t id = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (id >= total) return;
    const int l = (int)(id & 63);
    const int64_t rest = id >> 6;
    const int g = (int)(rest % groups);
    const int64_t t = rest / groups;
    const int64_t r = t * 64 + l;
    if (r >= rows) return;
    uint32_t d[NDW];
    const uint4 *src = packed + ((t * groups + g) * Format<BITS>::kPieces) * 64 + l;
#pragma unroll
    for (int q = 0; q < Format<BITS>::kPieces; ++q) {
        const uint4 v = src[q * 64];
        d[4 * q] = v.x;
        d[4 * q + 1] = v.y;
        d[4 * q + 2] = v.z;
        d[4 * q + 3] = v.w;
    }
#pragma unroll
    for (int q = 0; q < 16; ++q) {
        uint32_t out8[4] = {0, 0, 0, 0};
        uint32_t out16[8];
#pragma unroll
        for (int m = 0; m < 16; ++m) {
            const int j = q * 16 + m, bit = BITS * j, i = bit >> 5, sh = bit & 31;
            uint32_t c = d[i] >> sh;
            if (sh + BITS > 32) c |= d[i + 1] << (32 - sh);
            c &= mask;
            if constexpr (DECODE) {
                const uint32_t wv = lut[r * (1 << BITS) + c];
                if (m & 1) out16[m >> 1] |= wv << 16;
                else out16[m >> 1] = wv;
            } else {
                out8[m >> 2] |= c << (8 * (m & 3));
            }
        }
        if constexpr (DECODE) {
            uint4 *dst = (uint4 *)(w + r * cols + (int64_t)g * 256 + q * 16);
            dst[0] = make_uint4(out16[0], out16[1], out16[2], out16[3]);
            dst[1] = make_uint4(out16[4], out16[5], out16[6], out16[7]);
        } else {
            *(uint4 *)(codes + r * cols + (int64_t)g * 256 + q * 16) = make_uint4(out8[0], out8[1], out8[2], out8[3]);
        }
    }
}

// ---------------------------------------------------------------------------
// launchers

template <int BITS, int B, bool DENSE, bool SPARSE, bool ADDY>
static hipError_t launch_dsg(const KernelArgs &a, int waves, hipStream_t stream)
{
    const dim3 grid((unsigned)(a.tiles * a.split)), block((unsigned)(64 * waves));
    hipLaunchKernelGGL((dense_sparse_kernel<BITS, B, DENSE, SPARSE, ADDY>), grid, block, 0, stream, a);
    return hipGetLastError();
}

template <int BITS, bool DENSE, bool SPARSE, bool ADDY>
static hipError_t dispatch_batch(const KernelArgs &a, int batch, int waves, hipStream_t stream)
{
    switch (batch) {
    case 1: return launch_dsg<BITS, 1, DENSE, SPARSE, ADDY>(a, waves, stream);
    case 2: return launch_dsg<BITS, 2, DENSE, SPARSE, ADDY>(a, waves, stream);
    case 3: return launch_dsg<BITS, 3, DENSE, SPARSE, ADDY>(a, waves, stream);
    case 4: return launch_dsg<BITS, 4, DENSE, SPARSE, ADDY>(a, waves, stream);
    case 5: return launch_dsg<BITS, 5, DENSE, SPARSE, ADDY>(a, waves, stream);
    case 6: return launch_dsg<BITS, 6, DENSE, SPARSE, ADDY>(a, waves, stream);
    case 7: return launch_dsg<BITS, 7, DENSE, SPARSE, ADDY>(a, waves, stream);
    case 8: return launch_dsg<BITS, 8, DENSE, SPARSE, ADDY>(a, waves, stream);
    default: return hipErrorInvalidValue;
    }
}

hipError_t launch_dense_sparse(const KernelArgs &a, int bits, int batch, bool dense, bool sparse, bool add_y,
                               int waves, hipStream_t stream)
{
    if (dense && sparse) {
        return bits == 3 ? dispatch_batch<3, true, true, false>(a, batch, waves, stream)
                         : dispatch_batch<4, true, true, false>(a, batch, waves, stream);
    }
    if (dense) {
        return bits == 3 ? dispatch_batch<3, true, false, false>(a, batch, waves, stream)
                         : dispatch_batch<4, true, false, false>(a, batch, waves, stream);
    }
    if (sparse && add_y) return dispatch_batch<3, false, true, true>(a, batch, waves, stream);
    return hipErrorInvalidValue;
}

hipError_t launch_pack(const uint8_t *codes, int rows, int cols, int bits, void *packed, int *bad, hipStream_t stream)
{
    const int groups = cols / 256, tiles = (rows + 63) / 64;
    const int64_t total = (int64_t)tiles * groups * 64;
    const dim3 grid((unsigned)((total + 255) / 256)), block(256);
    if (bits == 3)
        hipLaunchKernelGGL(pack_kernel<3>, grid, block, 0, stream, codes, rows, cols, groups, total, (uint4 *)packed, bad);
    else
        hipLaunchKernelGGL(pack_kernel<4>, grid, block, 0, stream, codes, rows, cols, groups, total, (uint4 *)packed, bad);
    return hipGetLastError();
}

hipError_t launch_unpack(const void *packed, const uint16_t *lut, int rows, int cols, int bits, uint8_t *codes,
                         uint16_t *w, hipStream_t stream)
{
    const int groups = cols / 256, tiles = (rows + 63) / 64;
    const int64_t total = (int64_t)tiles * groups * 64;
    const dim3 grid((unsigned)((total + 255) / 256)), block(256);
    const uint4 *p = (const uint4 *)packed;
    if (w) {
        if (bits == 3)
            hipLaunchKernelGGL((unpack_kernel<3, true>), grid, block, 0, stream, p, lut, rows, cols, groups, total, codes, w);
        else
            hipLaunchKernelGGL((unpack_kernel<4, true>), grid, block, 0, stream, p, lut, rows, cols, groups, total, codes, w);
    } else {
        if (bits == 3)
            hipLaunchKernelGGL((unpack_kernel<3, false>), grid, block, 0, stream, p, lut, rows, cols, groups, total, codes, w);
        else
            hipLaunchKernelGGL((unpack_kernel<4, false>), grid, block, 0, stream, p, lut, rows, cols, groups, total, codes, w);
    }
    return hipGetLastError();
}

} // namespace sqllm
