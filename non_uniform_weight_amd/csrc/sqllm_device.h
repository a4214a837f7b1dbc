// sqllm_device.h -- gfx950 device code of the dense-and-sparse LUT GEMV
// y = (D + S) x (SqueezeLLM: Dense-and-Sparse Quantization, summary page,
// §3.4 "Kernel Implementation"; storage per §3.4 "The 3/4-bit storage
// format").  Included by the translation units that instantiate it.
//
// Mapping: one wave = 64 rows (one lane = one output row), so
//   * codes stream in as 128-bit loads: the packed layout puts the same
//     16-byte piece of 64 consecutive rows next to each other, one wave-wide
//     load moves 1 KiB of contiguous codes; a wave issues the loads of all
//     its column groups before it computes anything;
//   * every lane owns its own copy of its row's lookup table in LDS, as a
//     *pair* table: entry e holds the two centroids of code pair e as one
//     half2 at byte (e << 8) | (lane << 2) -- a lookup is one conflict-free
//     32-bit LDS read (the bank is the lane) feeding one v_dot2_f32_f16;
//     one v_perm_b32 turns a packed byte into that address (4-bit: every
//     pair is a byte; 3-bit: 12 of 16 pairs are the low six bits of a byte,
//     the table repeats over the two ignored top bits, and the other 4 pairs
//     are gathered from the top bits with 6 shifts/masks per 16 pairs);
//   * all lanes of a wave work on the same columns at the same time, so the
//     activation pairs are wave-uniform: the workgroup stages its columns of
//     x in LDS once and every wave reads them with broadcast 128-bit reads;
//   * a row tile's columns may be split over several workgroups; each one
//     adds its fp32 row sums into a (sum, count) word per output with a
//     compare-and-swap, and the one that completes the count rounds and
//     writes y -- no fences or cache flushes, one atomic round trip;
//   * the tile's CSR outliers are shared evenly by all waves of all its
//     workgroups (balanced regardless of per-row skew: §3.4 "Kernel
//     Implementation", balanced sparse kernel; Appendix C), reduced per row
//     with a segmented scan across the wave, and summed with the dense part
//     in fp32 before the single rounding (kernel fusion).
#ifndef SQLLM_DEVICE_H
#define SQLLM_DEVICE_H

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <utility>

#include "sqllm_internal.h"

namespace sqllm {
namespace dev {

typedef _Float16 half2_t __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float f16_to_f32(uint16_t h) { return (float)__builtin_bit_cast(_Float16, h); }
__device__ __forceinline__ uint16_t f32_to_f16_rne(float f) { return __builtin_bit_cast(uint16_t, (_Float16)f); }

template <int BITS>
struct Format {
    static constexpr int kEntries = 1 << BITS;   // centroids per row
    static constexpr int kPieces = 2 * BITS;     // 16-byte pieces per (row, group)
    static constexpr int kDwords = 8 * BITS;     // dwords per (row, group)
};

// v_perm_b32 selector: byte K of src0 -> result byte 1, byte 0 of src1 ->
// result byte 0, zeros above.
template <int K>
constexpr uint32_t addr_sel() { return 0x0C0C0000u | ((4u + K) << 8); }

// Pair-table byte address of pair P (0..127) of a group held in d[].
template <int BITS, int P>
__device__ __forceinline__ uint32_t pair_address(const uint32_t *d, uint32_t lane4)
{
    if constexpr (BITS == 4) {
        return __builtin_amdgcn_perm(d[P >> 2], lane4, addr_sel<P & 3>());
    } else {
        constexpr int u = P / 16, pu = P % 16;
        if constexpr (pu < 12) {
            return __builtin_amdgcn_perm(d[3 * u + pu / 4], lane4, addr_sel<pu % 4>());
        } else {
            // pair 12+q of the unit: bits [2k, 2k+2) are the top bits of unit byte 4k+q
            const uint32_t top = ((d[3 * u] >> 6) & 0x03030303u) | ((d[3 * u + 1] >> 4) & 0x0C0C0C0Cu) |
                                 ((d[3 * u + 2] >> 2) & 0x30303030u);
            return __builtin_amdgcn_perm(top, lane4, addr_sel<pu - 12>());
        }
    }
}

template <int BITS, int B, int P>
__device__ __forceinline__ void mac_pair(const uint32_t *d, uint32_t lane4, const uint32_t *tab, const u32x4 *xq,
                                         float *acc)
{
    const uint32_t a = pair_address<BITS, P>(d, lane4);
    const half2_t w = __builtin_bit_cast(half2_t, *(const uint32_t *)((const char *)tab + a));
#pragma unroll
    for (int b = 0; b < B; ++b) {
        const uint32_t xv = xq[b][P & 3];
        acc[b] = __builtin_amdgcn_fdot2(w, __builtin_bit_cast(half2_t, xv), acc[b], false);
    }
}

// Four pairs 4Q..4Q+3: one broadcast 128-bit LDS read of x per batch column.
template <int BITS, int B, int Q>
__device__ __forceinline__ void mac_quad(const uint32_t *d, uint32_t lane4, const uint32_t *tab, const uint32_t *xs,
                                         int xstride, float *acc)
{
    u32x4 xq[B];
#pragma unroll
    for (int b = 0; b < B; ++b) xq[b] = *(const u32x4 *)(xs + b * xstride + 4 * Q);
    mac_pair<BITS, B, 4 * Q + 0>(d, lane4, tab, xq, acc);
    mac_pair<BITS, B, 4 * Q + 1>(d, lane4, tab, xq, acc);
    mac_pair<BITS, B, 4 * Q + 2>(d, lane4, tab, xq, acc);
    mac_pair<BITS, B, 4 * Q + 3>(d, lane4, tab, xq, acc);
}

template <int BITS, int B, int... Qs>
__device__ __forceinline__ void mac_group_impl(const uint32_t *d, uint32_t lane4, const uint32_t *tab,
                                               const uint32_t *xs, int xstride, float *acc,
                                               std::integer_sequence<int, Qs...>)
{
    (mac_quad<BITS, B, Qs>(d, lane4, tab, xs, xstride, acc), ...);
}

// 128 pairs (256 codes) of one group; xs = the group's 128 x pairs (LDS),
// batch column b at xs + b * xstride.
template <int BITS, int B>
__device__ __forceinline__ void mac_group(const uint32_t *d, uint32_t lane4, const uint32_t *tab, const uint32_t *xs,
                                          int xstride, float *acc)
{
    mac_group_impl<BITS, B>(d, lane4, tab, xs, xstride, acc, std::make_integer_sequence<int, 32>{});
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

// Pair table of the tile (256 entries per lane).  Work item (lane l, low
// code h): lo = LUT[row][h]; for every high code c, entry h | c << b (3-bit:
// also with both ignored top bits set every way) = lo | LUT[row][c] << 16.
// An item's loads (the row's table and lo) are issued apart from its stores
// so that they can go out ahead of the bulk code loads.
template <int BITS>
struct TableItem {
    uint32_t lw[Format<BITS>::kEntries / 2];
    uint32_t lo;
};

template <int BITS>
__device__ __forceinline__ void table_item_load(TableItem<BITS> &it, const uint16_t *__restrict__ lut, int idx,
                                                int row0, int rows)
{
    constexpr int E = Format<BITS>::kEntries;
    const int l = idx & 63, h = idx >> 6;
    const int r = min(row0 + l, rows - 1);
    const u32x4 *lrow = (const u32x4 *)(lut + (int64_t)r * E);
#pragma unroll
    for (int q = 0; q < E / 8; ++q) {
        const u32x4 v = lrow[q];
        it.lw[4 * q + 0] = v.x;
        it.lw[4 * q + 1] = v.y;
        it.lw[4 * q + 2] = v.z;
        it.lw[4 * q + 3] = v.w;
    }
    it.lo = lut[(int64_t)r * E + h];
}

template <int BITS>
__device__ __forceinline__ void table_item_store(const TableItem<BITS> &it, uint32_t *tab, int idx)
{
    constexpr int E = Format<BITS>::kEntries;
    const int l = idx & 63, h = idx >> 6;
#pragma unroll
    for (int c = 0; c < E; ++c) {
        const uint32_t hi = (c & 1) ? (it.lw[c >> 1] & 0xFFFF0000u) : (it.lw[c >> 1] << 16);
        const uint32_t v = it.lo | hi;
        if constexpr (BITS == 4) {
            tab[(h | (c << 4)) * 64 + l] = v;
        } else {
#pragma unroll
            for (int j = 0; j < 4; ++j) tab[(h | (c << 3) | (j << 6)) * 64 + l] = v;
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

// A batch of up to kSparseBatch chunks of 64 nonzeros: column, value, row.
struct SparseBatch {
    int col[kSparseBatch];
    int row[kSparseBatch];
    float val[kSparseBatch];
};

// Loads of nonzeros [base, base + kSparseBatch*64) clipped to v1.
__device__ __forceinline__ void sparse_batch_load(SparseBatch &sb, const KernelArgs &a, int base, int v1, int lane)
{
#pragma unroll
    for (int k = 0; k < kSparseBatch; ++k) {
        const int i = base + k * 64 + lane;
        sb.col[k] = 0;
        sb.val[k] = 0.f;
        if (i < v1) {
            sb.col[k] = a.col[i];
            sb.val[k] = f16_to_f32(a.val[i]);
        }
    }
}

// Row (0..63) of each nonzero of the batch, products with x, summed per row
// (segmented scan over the wave: rows are non-decreasing along the CSR) into
// the wave's LDS row sums rsum[b * 64 + r].  x from LDS (xh, all columns,
// batch column b at xh + b * xhs) when staged there, else from global memory.
template <int B>
__device__ __forceinline__ void sparse_batch_finish(const SparseBatch &sb, const KernelArgs &a, const int *rps,
                                                    const uint16_t *xh, int xhs, int base, int v1, int lane,
                                                    float *rsum)
{
    float xv[kSparseBatch][B];
    int row[kSparseBatch];
#pragma unroll
    for (int k = 0; k < kSparseBatch; ++k) {
        const int i = base + k * 64 + lane;
        row[k] = i < v1 ? tile_row_of(rps, i) : 64; // 64: never a real row
#pragma unroll
        for (int b = 0; b < B; ++b)
            xv[k][b] = f16_to_f32(xh ? xh[b * xhs + sb.col[k]] : a.x[(int64_t)b * a.cols + sb.col[k]]);
    }
#pragma unroll
    for (int k = 0; k < kSparseBatch; ++k) {
        if (base + k * 64 >= v1) break;
        float prod[B];
#pragma unroll
        for (int b = 0; b < B; ++b) prod[b] = sb.val[k] * xv[k][b];
        const int r = row[k];
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
        if (r < 64 && (lane == 63 || rn != r)) {
#pragma unroll
            for (int b = 0; b < B; ++b) rsum[b * 64 + r] += prod[b];
        }
    }
}

// Round and store (or hand over) this workgroup's fp32 row sums.
template <int B, bool ADDY>
__device__ __forceinline__ void finish_rows(const KernelArgs &a, int t, int lane, const float *tot)
{
    const int row = t * 64 + lane;
    if (a.split == 1) {
        if (row < a.rows) {
#pragma unroll
            for (int b = 0; b < B; ++b) {
                float v = tot[b];
                if constexpr (ADDY) v += f16_to_f32(a.y[(int64_t)b * a.rows + row]);
                a.y[(int64_t)b * a.rows + row] = f32_to_f16_rne(v);
            }
        }
        return;
    }
    // (fp32 sum | count << 32) per output; the empty word is 0.  -0.0 is the
    // additive identity, so a lone partial keeps its sign of zero.  With two
    // workgroups per tile the result does not depend on arrival order.
#pragma unroll
    for (int b = 0; b < B; ++b) {
        unsigned long long *slot = a.slots + ((int64_t)t * B + b) * 64 + lane;
        unsigned long long expected = 0ull, desired = 0ull;
        for (;;) {
            const uint32_t cnt = (uint32_t)(expected >> 32);
            const float sum = cnt ? __uint_as_float((uint32_t)expected) : -0.0f;
            desired = ((unsigned long long)(cnt + 1) << 32) | __float_as_uint(sum + tot[b]);
            const unsigned long long got = atomicCAS(slot, expected, desired);
            if (got == expected) break;
            expected = got;
        }
        if ((int)(desired >> 32) == a.split) {
            if (row < a.rows) {
                float v = __uint_as_float((uint32_t)desired);
                if constexpr (ADDY) v += f16_to_f32(a.y[(int64_t)b * a.rows + row]);
                a.y[(int64_t)b * a.rows + row] = f32_to_f16_rne(v);
            }
            __hip_atomic_store(slot, 0ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
    }
}

// ---------------------------------------------------------------------------
// The kernel.  MODE: kFused y = (D+S)x; kDenseOnly y = Dx; kSparseAdd y += Sx.
// Grid: tiles * split workgroups, workgroup (tile t, split s) owns column
// groups [s*gps, min((s+1)*gps, groups)); wave w of it owns gpw <= GW of
// them.  Dynamic LDS: x [B][xstride pairs] -- every column when a.x_full,
// else only the workgroup's -- then (outlier modes) 65 row pointers and
// [waves][B][64] fp32 row sums.
//
// Order of work: the small loads (x, the pair-table rows, row pointers) go
// out first, the codes right behind them; the table is built while the
// codes stream in; outlier loads are issued before the dense work and used
// after it.
// Register room: with 16 waves per workgroup (128 VGPRs each) a wave holds
// its codes plus ~8 registers per batch column only up to 96 dwords; beyond
// that the kernel is compiled for at most 8 waves.
template <int BITS, int B, int GW>
constexpr int max_threads() { return max_waves(BITS, B, GW) * 64; }

template <int BITS, int B, int MODE, int GW>
__global__ void __launch_bounds__((max_threads<BITS, B, GW>())) dense_sparse_kernel(KernelArgs a)
{
    constexpr bool DENSE = MODE != kSparseAdd;
    constexpr bool SPARSE = MODE != kDenseOnly;
    constexpr bool ADDY = MODE == kSparseAdd;
    constexpr int ND = Format<BITS>::kDwords;
    constexpr int E = Format<BITS>::kEntries;
    __shared__ __align__(16) uint32_t tab[DENSE ? kTableBytes / 4 : kMaxWaves * B * 64];
    extern __shared__ __align__(16) uint32_t dyn[];

    const int nt = blockDim.x;
    const int nw = nt >> 6;
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    const int t = blockIdx.x / a.split, s = blockIdx.x - t * a.split;
    const int row0 = t * 64;
    const uint32_t lane4 = (uint32_t)lane << 2;
    const int gb = s * a.gps;
    const int ge = min(gb + a.gps, a.groups);
    // staged x: pairs [xg0*128, xg1*128) of every batch column
    const int xg0 = a.x_full ? 0 : gb, xg1 = a.x_full ? a.groups : ge;
    const int xstride = (a.x_full ? a.groups : a.gps) * 128;
    uint32_t *xs = dyn;
    int *rps = (int *)(dyn + ((DENSE || a.x_full) ? B * xstride : 0));
    float *rsum = (float *)(rps + 68) + w * B * 64;

    float acc[B];
#pragma unroll
    for (int b = 0; b < B; ++b) acc[b] = 0.f;

    // -- 1. small loads first: one x quad per batch column, one table item
    //       and one row pointer per thread (the rest, if any, after the codes)
    const int nq = (DENSE || a.x_full) ? (xg1 - xg0) * 32 : 0;
    u32x4 xq[B];
    if (threadIdx.x < nq) {
#pragma unroll
        for (int b = 0; b < B; ++b)
            xq[b] = *((const u32x4 *)(a.x + (int64_t)b * a.cols + (int64_t)xg0 * 256) + threadIdx.x);
    }
    TableItem<BITS> item;
    if constexpr (DENSE) {
        if (threadIdx.x < 64 * E) table_item_load<BITS>(item, a.lut, threadIdx.x, row0, a.rows);
    }
    // row pointers of the tile: rps[0..63] by the first wave, rps[64] (the
    // tile's end) by thread 0 too, so any block size loads all 65
    int rpv = 0, rpv_end = 0;
    if constexpr (SPARSE) {
        if (threadIdx.x < 64) rpv = a.row_ptr[min(row0 + (int)threadIdx.x, a.rows)];
        if (threadIdx.x == 0) rpv_end = a.row_ptr[min(row0 + 64, a.rows)];
    }

    // -- 2. every code load of this wave
    uint32_t buf[GW][ND];
    int ng = 0;
    if constexpr (DENSE) {
        const int g0 = gb + w * a.gpw;
        ng = max(0, min(a.gpw, ge - g0));
        const u32x4 *wave_codes =
            (const u32x4 *)a.packed + ((int64_t)t * a.groups + g0) * Format<BITS>::kPieces * 64 + lane;
#pragma unroll
        for (int j = 0; j < GW; ++j)
            if (j < ng) load_group<BITS>(wave_codes + j * Format<BITS>::kPieces * 64, buf[j]);
    }

    // -- 3. fill LDS: x, pair table, row pointers, zeroed row sums
    if (threadIdx.x < nq) {
#pragma unroll
        for (int b = 0; b < B; ++b) ((u32x4 *)(xs + b * xstride))[threadIdx.x] = xq[b];
    }
    for (int i = threadIdx.x + nt; i < nq; i += nt) {
#pragma unroll
        for (int b = 0; b < B; ++b)
            ((u32x4 *)(xs + b * xstride))[i] = *((const u32x4 *)(a.x + (int64_t)b * a.cols + (int64_t)xg0 * 256) + i);
    }
    if constexpr (DENSE) {
        if (threadIdx.x < 64 * E) table_item_store<BITS>(item, tab, threadIdx.x);
        for (int idx = threadIdx.x + nt; idx < 64 * E; idx += nt) {
            TableItem<BITS> it2;
            table_item_load<BITS>(it2, a.lut, idx, row0, a.rows);
            table_item_store<BITS>(it2, tab, idx);
        }
    }
    if constexpr (SPARSE) {
        if (threadIdx.x < 64) rps[threadIdx.x] = rpv;
        if (threadIdx.x == 0) rps[64] = rpv_end;
#pragma unroll
        for (int b = 0; b < B; ++b) rsum[b * 64 + lane] = 0.f;
    }
    __syncthreads();

    // -- 4. outliers: the tile's nonzeros cut into shares of about 256, dealt
    //       round-robin over the tile's workgroups, one share per wave at most;
    //       the first batch's loads go out before the dense work
    int v0 = 0, v1 = 0;
    SparseBatch sb;
    if constexpr (SPARSE) {
        const int nz0 = rps[0];
        const int64_t len = rps[64] - nz0;
        int64_t parts = (int64_t)a.split * nw;
        const int64_t want = (len + 255) / 256;
        if (want < parts) parts = want > 0 ? want : 1;
        const int64_t part = (int64_t)w * a.split + s;
        if (part < parts) {
            v0 = nz0 + (int)(len * part / parts);
            v1 = nz0 + (int)(len * (part + 1) / parts);
        }
        if (v0 < v1) sparse_batch_load(sb, a, v0, v1, lane);
    }

    // -- 5. dense: look up and multiply every loaded group
    if constexpr (DENSE) {
        const int g0 = gb + w * a.gpw;
#pragma unroll
        for (int j = 0; j < GW; ++j)
            if (j < ng) mac_group<BITS, B>(buf[j], lane4, tab, xs + (g0 + j - xg0) * 128, xstride, acc);
    }

    // -- 6. outliers: finish the first batch, then any further ones
    if constexpr (SPARSE) {
        const uint16_t *xh = a.x_full ? (const uint16_t *)xs : nullptr;
        const int xhs = 2 * xstride;
        if (v0 < v1) sparse_batch_finish<B>(sb, a, rps, xh, xhs, v0, v1, lane, rsum);
        for (int base = v0 + kSparseBatch * 64; base < v1; base += kSparseBatch * 64) {
            sparse_batch_load(sb, a, base, v1, lane);
            sparse_batch_finish<B>(sb, a, rps, xh, xhs, base, v1, lane, rsum);
        }
    }
    __syncthreads(); // pair table and x no longer needed

    // -- 7. reduce the waves (fixed order), then round and store / hand over
    float *red = (float *)tab;
#pragma unroll
    for (int b = 0; b < B; ++b) {
        float v = acc[b];
        if constexpr (SPARSE) v += rsum[b * 64 + lane];
        red[(w * B + b) * 64 + lane] = v;
    }
    __syncthreads();
    if (w != 0) return;
    float tot[B];
#pragma unroll
    for (int b = 0; b < B; ++b) {
        float v = 0.f;
        for (int k = 0; k < nw; ++k) v += red[(k * B + b) * 64 + lane];
        tot[b] = v;
    }
    finish_rows<B, ADDY>(a, t, lane, tot);
}

template <int BITS, int B, int MODE, int GW>
hipError_t launch_one(const KernelArgs &a, const LaunchShape &ls, hipStream_t stream)
{
    auto kern = dense_sparse_kernel<BITS, B, MODE, GW>;
    static bool attr_set = false; // ask once for more than the default dynamic LDS
    if (!attr_set) {
        if (hipFuncSetAttribute((const void *)kern, hipFuncAttributeMaxDynamicSharedMemorySize,
                                kLdsBudget - (MODE != kSparseAdd ? kTableBytes : 0)) != hipSuccess)
            (void)hipGetLastError(); // not fatal: launches within the default limit still work
        attr_set = true;
    }
    if (ls.waves * 64 > max_threads<BITS, B, GW>()) return hipErrorInvalidConfiguration;
    const dim3 grid((unsigned)(a.tiles * a.split)), block((unsigned)(64 * ls.waves));
    hipLaunchKernelGGL(kern, grid, block, ls.dyn_lds, stream, a);
    return hipGetLastError();
}

template <int BITS, int MODE, int GW>
hipError_t launch_batch(const KernelArgs &a, int batch, const LaunchShape &ls, hipStream_t stream)
{
    switch (batch) {
    case 1: return launch_one<BITS, 1, MODE, GW>(a, ls, stream);
    case 2: return launch_one<BITS, 2, MODE, GW>(a, ls, stream);
    case 3: return launch_one<BITS, 3, MODE, GW>(a, ls, stream);
    case 4: return launch_one<BITS, 4, MODE, GW>(a, ls, stream);
    case 5: return launch_one<BITS, 5, MODE, GW>(a, ls, stream);
    case 6: return launch_one<BITS, 6, MODE, GW>(a, ls, stream);
    case 7: return launch_one<BITS, 7, MODE, GW>(a, ls, stream);
    case 8: return launch_one<BITS, 8, MODE, GW>(a, ls, stream);
    default: return hipErrorInvalidValue;
    }
}

template <int BITS, int MODE>
hipError_t launch_gw(const KernelArgs &a, int batch, const LaunchShape &ls, hipStream_t stream)
{
    switch (ls.gw) {
    case 1: return launch_batch<BITS, MODE, 1>(a, batch, ls, stream);
    case 2: return launch_batch<BITS, MODE, 2>(a, batch, ls, stream);
    case 3: return launch_batch<BITS, MODE, 3>(a, batch, ls, stream);
    case 4: return launch_batch<BITS, MODE, 4>(a, batch, ls, stream);
    default: return hipErrorInvalidValue;
    }
}

} // namespace dev
} // namespace sqllm

#endif
