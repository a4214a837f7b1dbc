// sqllm_pack.hip -- offline packing, the test-only readers, and the launch
// dispatch of the product kernels.
//
// Packed layout (§3.4 "The 3/4-bit storage format": exactly b bits per
// code; the arrangement is this library's): 64-row tiles, 256-column groups,
// the 32b-byte string of each (row, group) cut into 2b pieces of 16 bytes
// that are interleaved over the tile's 64 rows.  Pair p of a group is
// code[2p] | code[2p+1] << b.  4-bit: string byte p = pair p.  3-bit: 8
// units of 12 bytes, 16 pairs each: pair p < 12 = low six bits of unit byte
// p; pair 12+q keeps bits [2k, 2k+2) in the top two bits of unit byte 4k+q.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "sqllm_internal.h"

namespace sqllm {

hipError_t launch_fused2(const KernelArgs &a, int batch, const LaunchShape &ls, hipStream_t stream);
hipError_t launch_gemv2(const KernelArgs &a, int batch, const LaunchShape &ls, hipStream_t stream);
hipError_t launch_group_fused2(const GroupArgs &g, int batch, const LaunchShape &ls, hipStream_t stream);
hipError_t launch_group_gemv2(const GroupArgs &g, int batch, const LaunchShape &ls, hipStream_t stream);
hipError_t launch_fused3(const KernelArgs &a, int batch, const LaunchShape &ls, hipStream_t stream);
hipError_t launch_fused4(const KernelArgs &a, int batch, const LaunchShape &ls, hipStream_t stream);
hipError_t launch_gemv3(const KernelArgs &a, int batch, const LaunchShape &ls, hipStream_t stream);
hipError_t launch_gemv4(const KernelArgs &a, int batch, const LaunchShape &ls, hipStream_t stream);
hipError_t launch_spmv_add(const KernelArgs &a, int batch, const LaunchShape &ls, hipStream_t stream);
hipError_t launch_group_fused3(const GroupArgs &g, int batch, const LaunchShape &ls, hipStream_t stream);
hipError_t launch_group_fused4(const GroupArgs &g, int batch, const LaunchShape &ls, hipStream_t stream);
hipError_t launch_group_gemv3(const GroupArgs &g, int batch, const LaunchShape &ls, hipStream_t stream);
hipError_t launch_group_gemv4(const GroupArgs &g, int batch, const LaunchShape &ls, hipStream_t stream);
hipError_t launch_fused3_compact(const KernelArgs &a, int batch, const LaunchShape &ls, hipStream_t stream);
hipError_t launch_group_fused3_compact(const GroupArgs &g, int batch, const LaunchShape &ls, hipStream_t stream);
#define SQLLM_WIDE(bits)                                                                                              \
    hipError_t launch_fused##bits##_wide(const KernelArgs &, int, const LaunchShape &, hipStream_t);                  \
    hipError_t launch_gemv##bits##_wide(const KernelArgs &, int, const LaunchShape &, hipStream_t);                   \
    hipError_t launch_group_fused##bits##_wide(const GroupArgs &, int, const LaunchShape &, hipStream_t);             \
    hipError_t launch_group_gemv##bits##_wide(const GroupArgs &, int, const LaunchShape &, hipStream_t);
SQLLM_WIDE(2)
SQLLM_WIDE(3)
SQLLM_WIDE(4)
#undef SQLLM_WIDE
hipError_t launch_spmv_add_wide(const KernelArgs &a, int batch, const LaunchShape &ls, hipStream_t stream);

hipError_t launch_dense_sparse(const KernelArgs &a, int bits, int batch, Mode mode, const LaunchShape &ls,
                               hipStream_t stream)
{
    const bool wide = batch > kMaxDotBatch;
    switch (mode) {
    case kFused:
        if (ls.compact) return compact_allowed(bits, batch) ? launch_fused3_compact(a, batch, ls, stream) : hipErrorInvalidValue;
        if (wide)
            return bits == 2   ? launch_fused2_wide(a, batch, ls, stream)
                   : bits == 3 ? launch_fused3_wide(a, batch, ls, stream)
                               : launch_fused4_wide(a, batch, ls, stream);
        return bits == 2 ? launch_fused2(a, batch, ls, stream)
                         : bits == 3 ? launch_fused3(a, batch, ls, stream) : launch_fused4(a, batch, ls, stream);
    case kDenseOnly:
        if (wide)
            return bits == 2   ? launch_gemv2_wide(a, batch, ls, stream)
                   : bits == 3 ? launch_gemv3_wide(a, batch, ls, stream)
                               : launch_gemv4_wide(a, batch, ls, stream);
        return bits == 2 ? launch_gemv2(a, batch, ls, stream)
                         : bits == 3 ? launch_gemv3(a, batch, ls, stream) : launch_gemv4(a, batch, ls, stream);
    case kSparseAdd: return wide ? launch_spmv_add_wide(a, batch, ls, stream) : launch_spmv_add(a, batch, ls, stream);
    }
    return hipErrorInvalidValue;
}

hipError_t launch_dense_sparse_group(const GroupArgs &g, int bits, int batch, Mode mode, const LaunchShape &ls,
                                     hipStream_t stream)
{
    const bool wide = batch > kMaxDotBatch;
    switch (mode) {
    case kFused:
        if (ls.compact) return compact_allowed(bits, batch) ? launch_group_fused3_compact(g, batch, ls, stream) : hipErrorInvalidValue;
        if (wide)
            return bits == 2   ? launch_group_fused2_wide(g, batch, ls, stream)
                   : bits == 3 ? launch_group_fused3_wide(g, batch, ls, stream)
                               : launch_group_fused4_wide(g, batch, ls, stream);
        return bits == 2   ? launch_group_fused2(g, batch, ls, stream)
               : bits == 3 ? launch_group_fused3(g, batch, ls, stream)
                           : launch_group_fused4(g, batch, ls, stream);
    case kDenseOnly:
        if (wide)
            return bits == 2   ? launch_group_gemv2_wide(g, batch, ls, stream)
                   : bits == 3 ? launch_group_gemv3_wide(g, batch, ls, stream)
                               : launch_group_gemv4_wide(g, batch, ls, stream);
        return bits == 2   ? launch_group_gemv2(g, batch, ls, stream)
               : bits == 3 ? launch_group_gemv3(g, batch, ls, stream)
                           : launch_group_gemv4(g, batch, ls, stream);
    case kSparseAdd: break;
    }
    return hipErrorInvalidValue;
}

namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// string byte k of (row, group) -> (dword, shift) inside the 8b dwords
template <int BITS>
__device__ __forceinline__ void put_byte(uint32_t *w, int k, uint32_t v)
{
    w[k >> 2] |= (v & 0xFFu) << (8 * (k & 3));
}

template <int BITS>
__device__ __forceinline__ uint32_t get_byte(const uint32_t *w, int k)
{
    return (w[k >> 2] >> (8 * (k & 3))) & 0xFFu;
}

// the 128 pair values of a group -> its 8b string dwords
template <int BITS>
__device__ __forceinline__ void pairs_to_string(const uint32_t *pair, uint32_t *w)
{
#pragma unroll
    for (int k = 0; k < 8 * BITS; ++k) w[k] = 0;
    if constexpr (BITS == 4) {
#pragma unroll
        for (int p = 0; p < 128; ++p) put_byte<4>(w, p, pair[p]);
    } else if constexpr (BITS == 2) {
#pragma unroll
        for (int p = 0; p < 64; ++p) put_byte<2>(w, p, pair[2 * p] | (pair[2 * p + 1] << 4));
    } else {
#pragma unroll
        for (int u = 0; u < 8; ++u) {
#pragma unroll
            for (int p = 0; p < 12; ++p) put_byte<3>(w, 12 * u + p, pair[16 * u + p]);
#pragma unroll
            for (int q = 0; q < 4; ++q)
#pragma unroll
                for (int k = 0; k < 3; ++k)
                    put_byte<3>(w, 12 * u + 4 * k + q, ((pair[16 * u + 12 + q] >> (2 * k)) & 3u) << 6);
        }
    }
}

template <int BITS>
__device__ __forceinline__ uint32_t string_pair(const uint32_t *w, int p)
{
    if constexpr (BITS == 4) {
        return get_byte<4>(w, p);
    } else if constexpr (BITS == 2) {
        return (get_byte<2>(w, p >> 1) >> (4 * (p & 1))) & 0xFu;
    } else {
        const int u = p >> 4, pu = p & 15;
        if (pu < 12) return get_byte<3>(w, 12 * u + pu) & 0x3Fu;
        uint32_t v = 0;
#pragma unroll
        for (int k = 0; k < 3; ++k) v |= (get_byte<3>(w, 12 * u + 4 * k + pu - 12) >> 6) << (2 * k);
        return v;
    }
}

// One thread per (row, group); thread index -> (tile, group, lane) with the
// lane fastest, so the pieces of 64 rows are written (read) contiguously.
template <int BITS>
__global__ void __launch_bounds__(256) pack_kernel(const uint8_t *__restrict__ codes, int rows, int cols, int groups,
                                                   int64_t total, u32x4 *__restrict__ packed, int *__restrict__ bad)
{
    const int64_t id = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (id >= total) return;
    const int l = (int)(id & 63);
    const int64_t rest = id >> 6;
    const int g = (int)(rest % groups);
    const int64_t t = rest / groups;
    const int64_t r = t * 64 + l;
    uint32_t pair[128];
    uint32_t oor = 0;
#pragma unroll
    for (int p = 0; p < 128; ++p) pair[p] = 0;
    if (r < rows) {
        const u32x4 *src = (const u32x4 *)(codes + r * cols + (int64_t)g * 256);
#pragma unroll
        for (int q = 0; q < 16; ++q) {
            const u32x4 v = src[q];
            const uint32_t word[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
            for (int m = 0; m < 16; m += 2) {
                const uint32_t c0 = (word[m >> 2] >> (8 * (m & 3))) & 0xFFu;
                const uint32_t c1 = (word[(m + 1) >> 2] >> (8 * ((m + 1) & 3))) & 0xFFu;
                oor |= (c0 | c1) >> BITS;
                pair[(q * 16 + m) >> 1] = c0 | (c1 << BITS);
            }
        }
    }
    if (oor) atomicOr(bad, 1);
    uint32_t w[8 * BITS];
    pairs_to_string<BITS>(pair, w);
    u32x4 *dst = packed + ((t * groups + g) * (2 * BITS)) * 64 + l;
#pragma unroll
    for (int q = 0; q < 2 * BITS; ++q) {
        u32x4 v;
        v.x = w[4 * q];
        v.y = w[4 * q + 1];
        v.z = w[4 * q + 2];
        v.w = w[4 * q + 3];
        dst[q * 64] = v;
    }
}

template <int BITS, bool DECODE>
__global__ void __launch_bounds__(256) unpack_kernel(const u32x4 *__restrict__ packed, const uint16_t *__restrict__ lut,
                                                     int rows, int cols, int groups, int64_t total,
                                                     uint8_t *__restrict__ codes, uint16_t *__restrict__ wout)
{
    constexpr uint32_t mask = (1u << BITS) - 1u;
    const int64_t id = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (id >= total) return;
    const int l = (int)(id & 63);
    const int64_t rest = id >> 6;
    const int g = (int)(rest % groups);
    const int64_t t = rest / groups;
    const int64_t r = t * 64 + l;
    if (r >= rows) return;
    uint32_t w[8 * BITS];
    const u32x4 *src = packed + ((t * groups + g) * (2 * BITS)) * 64 + l;
#pragma unroll
    for (int q = 0; q < 2 * BITS; ++q) {
        const u32x4 v = src[q * 64];
        w[4 * q] = v.x;
        w[4 * q + 1] = v.y;
        w[4 * q + 2] = v.z;
        w[4 * q + 3] = v.w;
    }
#pragma unroll
    for (int q = 0; q < 16; ++q) {
        uint32_t out8[4] = {0, 0, 0, 0};
        uint32_t out16[8];
#pragma unroll
        for (int m = 0; m < 16; m += 2) {
            const uint32_t pv = string_pair<BITS>(w, (q * 16 + m) >> 1);
            const uint32_t c0 = pv & mask, c1 = (pv >> BITS) & mask;
            if constexpr (DECODE) {
                out16[m >> 1] = (uint32_t)lut[r * (1 << BITS) + c0] | ((uint32_t)lut[r * (1 << BITS) + c1] << 16);
            } else {
                out8[m >> 2] |= (c0 | (c1 << 8)) << (8 * (m & 3));
            }
        }
        if constexpr (DECODE) {
            u32x4 *dst = (u32x4 *)(wout + r * cols + (int64_t)g * 256 + q * 16);
            u32x4 v0, v1;
            v0.x = out16[0]; v0.y = out16[1]; v0.z = out16[2]; v0.w = out16[3];
            v1.x = out16[4]; v1.y = out16[5]; v1.z = out16[6]; v1.w = out16[7];
            dst[0] = v0;
            dst[1] = v1;
        } else {
            u32x4 v;
            v.x = out8[0]; v.y = out8[1]; v.z = out8[2]; v.w = out8[3];
            *(u32x4 *)(codes + r * cols + (int64_t)g * 256 + q * 16) = v;
        }
    }
}

// Job blockIdx.y: xt[c][b] = x[b][c] for b < batch, 0 up to the padded
// width (CLEAR: xt = 0); one column per thread.
template <bool CLEAR>
__global__ void __launch_bounds__(256) xt_kernel(XtJobs j, int batch, int pad)
{
    const int k = blockIdx.y;
    const int c = blockIdx.x * 256 + threadIdx.x;
    if (k >= j.n || c >= j.cols[k]) return;
    uint16_t *dst = j.xt[k] + (int64_t)c * pad;
    for (int b = 0; b < pad; ++b) dst[b] = !CLEAR && b < batch ? j.x[k][(int64_t)b * j.cols[k] + c] : (uint16_t)0;
}

} // namespace

hipError_t launch_xt_write(const XtJobs &j, int batch, hipStream_t stream)
{
    if (j.n < 1) return hipSuccess;
    hipLaunchKernelGGL(xt_kernel<false>, dim3((unsigned)((j.max_cols + 255) / 256), (unsigned)j.n), dim3(256), 0,
                       stream, j, batch, xt_pad(batch));
    return hipGetLastError();
}

hipError_t launch_xt_clear(const XtJobs &j, int batch, hipStream_t stream)
{
    if (j.n < 1) return hipSuccess;
    hipLaunchKernelGGL(xt_kernel<true>, dim3((unsigned)((j.max_cols + 255) / 256), (unsigned)j.n), dim3(256), 0,
                       stream, j, batch, xt_pad(batch));
    return hipGetLastError();
}

// Reference read stream (test-only): the range's pieces of 1 KiB are cut
// into even contiguous shares, one per wave (the first pieces % waves
// shares one piece longer; lane l reads bytes l*16 .. l*16+15 of each
// piece), D loads in flight, and every word is folded
// into an XOR, stored to the wave's own sink slot (one atomic per wave on a
// shared word would serialise: ~37 ns each, 151 us per launch).  Every step issues D
// loads (indices past the range clamped to its last piece, their words
// masked out), so the compiler's wait counts stay exact.
__global__ void __launch_bounds__(256) stream_read_kernel(const u32x4 *src, int64_t pieces, uint32_t *sink)
{
    constexpr int D = 8;
    const int64_t nwaves = (int64_t)gridDim.x * 4;
    const int64_t wid = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    const int64_t per = pieces / nwaves, rem = pieces - per * nwaves;
    const int64_t p0 = wid * per + min(wid, rem);
    const int64_t p1 = p0 + per + (wid < rem ? 1 : 0);
    uint32_t acc = 0;
    if (p0 < p1) {
        const u32x4 *base = src + lane;
        u32x4 r[D];
#pragma unroll
        for (int k = 0; k < D; ++k) r[k] = __builtin_nontemporal_load(base + min(p0 + k, p1 - 1) * 64);
        for (int64_t j = p0; j < p1; j += D) {
#pragma unroll
            for (int k = 0; k < D; ++k) {
                const uint32_t v = r[k].x ^ r[k].y ^ r[k].z ^ r[k].w;
                acc ^= j + k < p1 ? v : 0u;
                r[k] = __builtin_nontemporal_load(base + min(j + k + D, p1 - 1) * 64);
            }
        }
    }
    // fold the wave's lanes into its slot
    for (int off = 32; off > 0; off >>= 1) acc ^= __shfl_xor(acc, off, 64);
    if (lane == 0) sink[wid] = acc;
}

hipError_t launch_stream_read(const void *src, size_t bytes, uint32_t *sink, hipStream_t stream)
{
    const int64_t pieces = (int64_t)(bytes / 1024);
    hipLaunchKernelGGL(stream_read_kernel, dim3(kStreamReadWaves / 4), dim3(256), 0, stream, (const u32x4 *)src,
                       pieces, sink);
    return hipGetLastError();
}

hipError_t launch_pack(const uint8_t *codes, int rows, int cols, int bits, void *packed, int *bad, hipStream_t stream)
{
    const int groups = cols / 256, tiles = (rows + 63) / 64;
    const int64_t total = (int64_t)tiles * groups * 64;
    const dim3 grid((unsigned)((total + 255) / 256)), block(256);
    if (bits == 2)
        hipLaunchKernelGGL(pack_kernel<2>, grid, block, 0, stream, codes, rows, cols, groups, total, (u32x4 *)packed, bad);
    else if (bits == 3)
        hipLaunchKernelGGL(pack_kernel<3>, grid, block, 0, stream, codes, rows, cols, groups, total, (u32x4 *)packed, bad);
    else
        hipLaunchKernelGGL(pack_kernel<4>, grid, block, 0, stream, codes, rows, cols, groups, total, (u32x4 *)packed, bad);
    return hipGetLastError();
}

hipError_t launch_unpack(const void *packed, const uint16_t *lut, int rows, int cols, int bits, uint8_t *codes,
                         uint16_t *w, hipStream_t stream)
{
    const int groups = cols / 256, tiles = (rows + 63) / 64;
    const int64_t total = (int64_t)tiles * groups * 64;
    const dim3 grid((unsigned)((total + 255) / 256)), block(256);
    const u32x4 *p = (const u32x4 *)packed;
    if (w) {
        if (bits == 2)
            hipLaunchKernelGGL((unpack_kernel<2, true>), grid, block, 0, stream, p, lut, rows, cols, groups, total, codes, w);
        else if (bits == 3)
            hipLaunchKernelGGL((unpack_kernel<3, true>), grid, block, 0, stream, p, lut, rows, cols, groups, total, codes, w);
        else
            hipLaunchKernelGGL((unpack_kernel<4, true>), grid, block, 0, stream, p, lut, rows, cols, groups, total, codes, w);
    } else {
        if (bits == 2)
            hipLaunchKernelGGL((unpack_kernel<2, false>), grid, block, 0, stream, p, lut, rows, cols, groups, total, codes, w);
        else if (bits == 3)
            hipLaunchKernelGGL((unpack_kernel<3, false>), grid, block, 0, stream, p, lut, rows, cols, groups, total, codes, w);
        else
            hipLaunchKernelGGL((unpack_kernel<4, false>), grid, block, 0, stream, p, lut, rows, cols, groups, total, codes, w);
    }
    return hipGetLastError();
}

} // namespace sqllm
