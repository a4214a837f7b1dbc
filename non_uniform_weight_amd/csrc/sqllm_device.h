// sqllm_device.h -- gfx950 device code of the dense-and-sparse LUT GEMV
// y = (D + S) x (SqueezeLLM: Dense-and-Sparse Quantization, summary page,
// §3.4 "Kernel Implementation"; storage per §3.4 "The 3/4-bit storage
// format").  Included by the translation units that instantiate it.
//
// One workgroup owns one row tile (64 rows, one per lane) and a range of its
// 256-column groups.  Every wave does two kinds of work, interleaved:
//
//   dense groups: the layout puts the same 16-byte piece of 64 consecutive
//   rows side by side, so one wave-wide 128-bit load moves 1 KiB of
//   contiguous codes.  Each wave keeps a ring of `ring_depth` groups in
//   flight (codes plus that group's activations) and computes one group
//   while the next ones arrive.  A lookup reads the lane's own copy of its
//   row's *pair* table in LDS: entry e holds the two centroids of code pair e
//   as one half2 at byte (e << 8) | (lane << 2), so a lookup is one
//   conflict-free 32-bit LDS read (the bank is the lane), addressed by one
//   v_perm_b32 straight from a packed byte (4-bit: every pair is a byte;
//   3-bit: 12 of 16 pairs are the low six bits of a byte and the table repeats
//   over the two ignored top bits, the other 4 pairs are gathered from the top
//   bits; the compact 3-bit table instead clears those two bits, one AND per
//   dword, and holds each pair once, which leaves LDS for a wider x).  The products run on the matrix cores (MF, the default): two
//   lookups are a row's 4 consecutive weights, the B operand of one
//   v_mfma_f32_4x4x4f16 step whose A (the same 4 activations of 4 batch
//   columns for every row) is broadcast from the one block of lanes that
//   holds it, so lane = row throughout and no activation passes through
//   LDS.  The dot form (kept for comparison) instead keeps the activation
//   pairs in registers -- lane n of each 16-lane row holds pairs 4n..4n+3
//   (and 64+4n..64+4n+3) of the group -- and v_dot2c_f32_f16 takes its x
//   operand through a DPP row_newbcast:n, which hands lane n's pair to its
//   whole row.
//
//   outlier chunks: the tile's CSR nonzeros are cut into even shares, one per
//   wave of the split (balanced whatever the per-row skew: §3.4 "Kernel
//   Implementation", balanced sparse kernel; Appendix C), 64 per lane-wide
//   chunk.  Within a chunk the rows are non-decreasing: x is gathered, one
//   inclusive prefix sum of the products runs over the wave (DPP row shifts
//   and row broadcasts), and a row's sum is the prefix at its last lane in
//   the chunk less the prefix at the lane before its first, which the row's
//   own lane fetches with two lane permutes (no search for segment starts,
//   no atomics).  When all of x is staged
//   in LDS a chunk follows each dense group; otherwise the chunks come after
//   the dense groups, a round at a time (all of a round's gathers, then its
//   scans), reading x through the cache or, from batch 5 on, from a
//   transposed copy the call writes into the workspace (one load fetches
//   every batch column of a column).
//
// The waves' fp32 row sums are added in a fixed order; the sparse part joins
// the dense part in fp32 before the single rounding (kernel fusion).  A row
// tile's columns may be split over several workgroups: their fp32 sums meet
// in a binary tree of words in the workspace (see finish_rows), one atomic OR
// per level, added in an order that does not depend on which workgroup
// arrives first; the last one rounds and writes y -- no fences or cache
// flushes.

#ifndef SQLLM_DEVICE_H
#define SQLLM_DEVICE_H

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <atomic>
#include <utility>

#include "sqllm_internal.h"

namespace sqllm {
namespace dev {

typedef _Float16 half2_t __attribute__((ext_vector_type(2)));
typedef _Float16 half4_t __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// Zeros read by the ring's placeholder loads: a wave always issues the same
// number of loads per step, so the compiler's wait counts stay exact; a wave
// past its last group reads these 8 KiB (cache resident) instead of codes.
__device__ __attribute__((aligned(16))) uint32_t g_placeholder[8 * 64 * 4];

// Workgroup barrier that orders LDS accesses only: outstanding global loads
// (the ring) stay in flight across it.
__device__ __forceinline__ void lds_barrier()
{
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

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

// (a & mask) | (b & ~mask) as one v_bfi_b32 (written out, the compiler
// turns it back into separate masks).
__device__ __forceinline__ uint32_t bit_insert(uint32_t mask, uint32_t a, uint32_t b)
{
    uint32_t r;
    asm("v_bfi_b32 %0, %1, %2, %3" : "=v"(r) : "v"(mask), "v"(a), "v"(b));
    return r;
}

// Pair-table byte address of pair P (0..127) of a group held in d[].  CT:
// the compact 3-bit table, which takes the address bytes with their top two
// bits cleared.
template <int BITS, int P, bool CT>
__device__ __forceinline__ uint32_t pair_address(const uint32_t *d, uint32_t lane4)
{
    if constexpr (BITS == 4) {
        return __builtin_amdgcn_perm(d[P >> 2], lane4, addr_sel<P & 3>());
    } else if constexpr (BITS == 2) {
        // pair P is nibble P % 2 of string byte P / 2; an odd pair's byte is
        // taken from the dword shifted down by four bits (one shift per
        // dword, shared by its four odd pairs).  The table repeats over the
        // byte's other nibble.
        constexpr int k = (P >> 1) & 3;
        if constexpr ((P & 1) == 0)
            return __builtin_amdgcn_perm(d[P >> 3], lane4, addr_sel<k>());
        else
            return __builtin_amdgcn_perm(d[P >> 3] >> 4, lane4, addr_sel<k>());
    } else {
        constexpr int u = P / 16, pu = P % 16;
        constexpr uint32_t keep = CT ? 0x3F3F3F3Fu : 0xFFFFFFFFu;
        if constexpr (pu < 12) {
            return __builtin_amdgcn_perm(d[3 * u + pu / 4] & keep, lane4, addr_sel<pu % 4>());
        } else {
            // pair 12+q of the unit: bits [2k, 2k+2) are the top bits of unit
            // byte 4k+q.  Byte q of `top` gets them at bits 2k..2k+1 by two
            // bit-field inserts; its bits 6-7 keep other bits, which the table's
            // copies over the top two index bits ignore.
            const uint32_t t01 = bit_insert(0x03030303u, d[3 * u] >> 6, d[3 * u + 1] >> 4);
            const uint32_t top = bit_insert(0x0F0F0F0Fu, t01, d[3 * u + 2] >> 2);
            return __builtin_amdgcn_perm(top & keep, lane4, addr_sel<pu - 12>());
        }
    }
}

// Registers of one group in flight: codes, and the group's activations.
// Dot form: xr[b][0..3] = pairs 4n..4n+3, xr[b][4..7] = pairs 64+4n..64+4n+3
// with n = lane % 16, for batch column b.  Matrix-core form (MF): lane 4k+i
// holds in xq[2h + s] the 8 activations of batch column 4h+i at columns
// 128 s + 8 k .. 128 s + 8 k + 7 of the group.
template <int BITS, int B, bool MF>
struct GroupRegs {
    uint32_t d[Format<BITS>::kDwords];
    uint32_t xr[MF ? 1 : B][8];
    u32x4 xq[MF ? 2 * mf_quads(B) : 1];
};

// Groups a dense wave keeps in flight, sized so the ring stays within 80
// (3-bit), 72 (4-bit, whose table items and lookups need more) or 64 (2-bit,
// whose replicated table stores need more) of the 128
// registers a wave has when 16 waves share a compute unit, less 16 per batch
// quad in the matrix-core form (its accumulators).
constexpr int ring_depth(int bits, int batch, bool mf)
{
    const int per = 8 * bits + (mf ? 8 * mf_quads(batch) : 8 * batch);
    const int d = ((bits == 2 ? 64 : (bits == 3 ? 80 : 72)) - (mf ? 16 * mf_quads(batch) : 0)) / per;
    return d < 1 ? 1 : (d > 3 ? 3 : d);
}

// Loads of group g of tile t into r; g < 0 loads placeholders.
template <int BITS, int B, bool MF>
__device__ __forceinline__ void load_group(GroupRegs<BITS, B, MF> &r, const KernelArgs &a, int t, int g, int lane)
{
    constexpr int NP = Format<BITS>::kPieces;
    const bool real = g >= 0;
    const u32x4 *src = real ? (const u32x4 *)a.packed + ((int64_t)t * a.groups + g) * NP * 64
                            : (const u32x4 *)g_placeholder;
    src += lane;
#pragma unroll
    for (int q = 0; q < NP; ++q) {
        const u32x4 v = __builtin_nontemporal_load(src + q * 64);
        r.d[4 * q + 0] = v.x;
        r.d[4 * q + 1] = v.y;
        r.d[4 * q + 2] = v.z;
        r.d[4 * q + 3] = v.w;
    }
    if constexpr (MF) {
#pragma unroll
        for (int h = 0; h < mf_quads(B); ++h) {
            const int b = 4 * h + (lane & 3); // batch columns past B read placeholders (their sums are dropped)
#pragma unroll
            for (int s = 0; s < 2; ++s) {
                const u32x4 *xs = real && b < B
                                      ? (const u32x4 *)(a.x + (int64_t)b * a.cols + g * 256 + 128 * s + 8 * (lane >> 2))
                                      : (const u32x4 *)g_placeholder + lane;
                r.xq[2 * h + s] = *xs;
            }
        }
        return;
    }
#pragma unroll
    for (int b = 0; b < B; ++b) {
        const u32x4 *xs = real ? (const u32x4 *)((const uint32_t *)a.x + (int64_t)b * (a.cols >> 1) + g * 128)
                               : (const u32x4 *)g_placeholder;
        xs += lane & 15;
        const u32x4 lo = xs[0], hi = xs[16];
        r.xr[b][0] = lo.x;
        r.xr[b][1] = lo.y;
        r.xr[b][2] = lo.z;
        r.xr[b][3] = lo.w;
        r.xr[b][4] = hi.x;
        r.xr[b][5] = hi.y;
        r.xr[b][6] = hi.z;
        r.xr[b][7] = hi.w;
    }
}

// Independent fp32 accumulators per batch column: the products of one
// batch of pairs rotate over acc_chains(B) chains so that no v_dot2c reads an
// accumulator the instruction before it wrote.  The chains are added in a
// fixed order at the end.
constexpr int acc_chains(int batch) { return batch == 1 ? 3 : (batch == 2 ? 2 : 1); }

// The group's math runs in batches of 8 pairs: the table reads of batch
// Q+1 are issued before the products of batch Q, and one wait per batch
// (instead of one per read) covers them.
constexpr int kBatch = 8;

template <int BITS, int B, bool MF, int Q, bool CT>
__device__ __forceinline__ void batch_reads(const GroupRegs<BITS, B, MF> &r, uint32_t lane4, const uint32_t *tab,
                                            uint32_t (&wv)[kBatch])
{
    uint32_t addr[kBatch];
    [&]<int... Ks>(std::integer_sequence<int, Ks...>) {
        ((addr[Ks] = pair_address<BITS, Q * kBatch + Ks, CT>(r.d, lane4)), ...);
    }(std::make_integer_sequence<int, kBatch>{});
#pragma unroll
    for (int k = 0; k < kBatch; ++k) wv[k] = *(const uint32_t *)((const char *)tab + addr[k]);
}

// The products of one batch, v_dot2c_f32_f16 with fp32 accumulation: the
// table entry w of pair P times the activation pair P, which lane n = (P %
// 64) / 4 of each 16-lane row holds (component P % 4 of the group's x
// registers 4h..4h+3, h = P / 64) and a DPP row_newbcast:n operand hands to
// the whole row.  Batch Q (pairs 8Q..8Q+7) reads x registers 4h..4h+3 with
// h = Q / 8 through lanes n0 = 2 (Q % 8) (pairs 8Q..8Q+3) and n0 + 1.
//
// Two hazards need wait states the compiler cannot insert inside asm: a DPP
// instruction must not read a register written by one of the two VALU
// instructions before it, and a register written by a dot instruction may
// be read by another VALU instruction only three instructions later.  The
// products of a batch therefore form one asm block that opens with two
// wait states and closes with three (whatever the compiler places around
// it: it may copy accumulators between blocks), and inside it the chains
// rotate so that each accumulator is written at least three instructions
// before it is read again.  Activation and table registers are only ever
// written by memory loads.
#define SQLLM_DOT(a, x, w, n) "v_dot2c_f32_f16_dpp %[" a "], %[" x "], %[" w "] row_newbcast:%[" n "] row_mask:0xf bank_mask:0xf\n"

template <int B, int N0>
struct BatchDots;

template <int N0>
struct BatchDots<1, N0> { // chains k % 3
    static __device__ __forceinline__ void run(const uint32_t *x, const uint32_t *w, float *acc)
    {
        asm volatile("s_nop 1\n" SQLLM_DOT("a0", "x0", "w0", "n0") SQLLM_DOT("a1", "x1", "w1", "n0")
                         SQLLM_DOT("a2", "x2", "w2", "n0") SQLLM_DOT("a0", "x3", "w3", "n0")
                             SQLLM_DOT("a1", "x0", "w4", "n1") SQLLM_DOT("a2", "x1", "w5", "n1")
                                 SQLLM_DOT("a0", "x2", "w6", "n1") SQLLM_DOT("a1", "x3", "w7", "n1") "s_nop 2\n"
                     : [a0] "+v"(acc[0]), [a1] "+v"(acc[1]), [a2] "+v"(acc[2])
                     : [x0] "v"(x[0]), [x1] "v"(x[1]), [x2] "v"(x[2]), [x3] "v"(x[3]), [w0] "v"(w[0]),
                       [w1] "v"(w[1]), [w2] "v"(w[2]), [w3] "v"(w[3]), [w4] "v"(w[4]), [w5] "v"(w[5]),
                       [w6] "v"(w[6]), [w7] "v"(w[7]), [n0] "n"(N0), [n1] "n"(N0 + 1));
    }
};

template <int N0>
struct BatchDots<2, N0> { // acc[b * 2 + k % 2]; x[b * 4 + c]
    static __device__ __forceinline__ void run(const uint32_t *x, const uint32_t *w, float *acc)
    {
        asm volatile("s_nop 1\n" SQLLM_DOT("a00", "x00", "w0", "n0") SQLLM_DOT("a10", "x10", "w0", "n0")
                         SQLLM_DOT("a01", "x01", "w1", "n0") SQLLM_DOT("a11", "x11", "w1", "n0")
                             SQLLM_DOT("a00", "x02", "w2", "n0") SQLLM_DOT("a10", "x12", "w2", "n0")
                                 SQLLM_DOT("a01", "x03", "w3", "n0") SQLLM_DOT("a11", "x13", "w3", "n0")
                                     SQLLM_DOT("a00", "x00", "w4", "n1") SQLLM_DOT("a10", "x10", "w4", "n1")
                                         SQLLM_DOT("a01", "x01", "w5", "n1") SQLLM_DOT("a11", "x11", "w5", "n1")
                                             SQLLM_DOT("a00", "x02", "w6", "n1") SQLLM_DOT("a10", "x12", "w6", "n1")
                                                 SQLLM_DOT("a01", "x03", "w7", "n1")
                                                     SQLLM_DOT("a11", "x13", "w7", "n1") "s_nop 2\n"
                     : [a00] "+v"(acc[0]), [a01] "+v"(acc[1]), [a10] "+v"(acc[2]), [a11] "+v"(acc[3])
                     : [x00] "v"(x[0]), [x01] "v"(x[1]), [x02] "v"(x[2]), [x03] "v"(x[3]), [x10] "v"(x[4]),
                       [x11] "v"(x[5]), [x12] "v"(x[6]), [x13] "v"(x[7]), [w0] "v"(w[0]), [w1] "v"(w[1]),
                       [w2] "v"(w[2]), [w3] "v"(w[3]), [w4] "v"(w[4]), [w5] "v"(w[5]), [w6] "v"(w[6]),
                       [w7] "v"(w[7]), [n0] "n"(N0), [n1] "n"(N0 + 1));
    }
};

// Batch columns 3 and up: one chain each; a block per pair (the columns'
// products are B >= 3 instructions apart).
#define SQLLM_DOTS3(n) SQLLM_DOT("a0", "x0", "w", n) SQLLM_DOT("a1", "x1", "w", n) SQLLM_DOT("a2", "x2", "w", n)
#define SQLLM_PAIR_OPERANDS(w_)                                                                                    \
    [w] "v"(w_), [n] "n"(N)

template <int B, int N>
struct PairDots;

template <int N>
struct PairDots<3, N> {
    static __device__ __forceinline__ void run(const uint32_t *x, uint32_t w, float *acc)
    {
        asm volatile("s_nop 1\n" SQLLM_DOTS3("n") "s_nop 2\n"
                     : [a0] "+v"(acc[0]), [a1] "+v"(acc[1]), [a2] "+v"(acc[2])
                     : [x0] "v"(x[0]), [x1] "v"(x[1]), [x2] "v"(x[2]), SQLLM_PAIR_OPERANDS(w));
    }
};
template <int N>
struct PairDots<4, N> {
    static __device__ __forceinline__ void run(const uint32_t *x, uint32_t w, float *acc)
    {
        asm volatile("s_nop 1\n" SQLLM_DOTS3("n") SQLLM_DOT("a3", "x3", "w", "n") "s_nop 2\n"
                     : [a0] "+v"(acc[0]), [a1] "+v"(acc[1]), [a2] "+v"(acc[2]), [a3] "+v"(acc[3])
                     : [x0] "v"(x[0]), [x1] "v"(x[1]), [x2] "v"(x[2]), [x3] "v"(x[3]), SQLLM_PAIR_OPERANDS(w));
    }
};
template <int N>
struct PairDots<5, N> {
    static __device__ __forceinline__ void run(const uint32_t *x, uint32_t w, float *acc)
    {
        asm volatile("s_nop 1\n" SQLLM_DOTS3("n") SQLLM_DOT("a3", "x3", "w", "n") SQLLM_DOT("a4", "x4", "w", "n") "s_nop 2\n"
                     : [a0] "+v"(acc[0]), [a1] "+v"(acc[1]), [a2] "+v"(acc[2]), [a3] "+v"(acc[3]),
                       [a4] "+v"(acc[4])
                     : [x0] "v"(x[0]), [x1] "v"(x[1]), [x2] "v"(x[2]), [x3] "v"(x[3]), [x4] "v"(x[4]),
                       SQLLM_PAIR_OPERANDS(w));
    }
};
template <int N>
struct PairDots<6, N> {
    static __device__ __forceinline__ void run(const uint32_t *x, uint32_t w, float *acc)
    {
        asm volatile("s_nop 1\n" SQLLM_DOTS3("n") SQLLM_DOT("a3", "x3", "w", "n") SQLLM_DOT("a4", "x4", "w", "n")
                         SQLLM_DOT("a5", "x5", "w", "n") "s_nop 2\n"
                     : [a0] "+v"(acc[0]), [a1] "+v"(acc[1]), [a2] "+v"(acc[2]), [a3] "+v"(acc[3]),
                       [a4] "+v"(acc[4]), [a5] "+v"(acc[5])
                     : [x0] "v"(x[0]), [x1] "v"(x[1]), [x2] "v"(x[2]), [x3] "v"(x[3]), [x4] "v"(x[4]),
                       [x5] "v"(x[5]), SQLLM_PAIR_OPERANDS(w));
    }
};
template <int N>
struct PairDots<7, N> {
    static __device__ __forceinline__ void run(const uint32_t *x, uint32_t w, float *acc)
    {
        asm volatile("s_nop 1\n" SQLLM_DOTS3("n") SQLLM_DOT("a3", "x3", "w", "n") SQLLM_DOT("a4", "x4", "w", "n")
                         SQLLM_DOT("a5", "x5", "w", "n") SQLLM_DOT("a6", "x6", "w", "n") "s_nop 2\n"
                     : [a0] "+v"(acc[0]), [a1] "+v"(acc[1]), [a2] "+v"(acc[2]), [a3] "+v"(acc[3]),
                       [a4] "+v"(acc[4]), [a5] "+v"(acc[5]), [a6] "+v"(acc[6])
                     : [x0] "v"(x[0]), [x1] "v"(x[1]), [x2] "v"(x[2]), [x3] "v"(x[3]), [x4] "v"(x[4]),
                       [x5] "v"(x[5]), [x6] "v"(x[6]), SQLLM_PAIR_OPERANDS(w));
    }
};
template <int N>
struct PairDots<8, N> {
    static __device__ __forceinline__ void run(const uint32_t *x, uint32_t w, float *acc)
    {
        asm volatile("s_nop 1\n" SQLLM_DOTS3("n") SQLLM_DOT("a3", "x3", "w", "n") SQLLM_DOT("a4", "x4", "w", "n")
                         SQLLM_DOT("a5", "x5", "w", "n") SQLLM_DOT("a6", "x6", "w", "n")
                             SQLLM_DOT("a7", "x7", "w", "n") "s_nop 2\n"
                     : [a0] "+v"(acc[0]), [a1] "+v"(acc[1]), [a2] "+v"(acc[2]), [a3] "+v"(acc[3]),
                       [a4] "+v"(acc[4]), [a5] "+v"(acc[5]), [a6] "+v"(acc[6]), [a7] "+v"(acc[7])
                     : [x0] "v"(x[0]), [x1] "v"(x[1]), [x2] "v"(x[2]), [x3] "v"(x[3]), [x4] "v"(x[4]),
                       [x5] "v"(x[5]), [x6] "v"(x[6]), [x7] "v"(x[7]), SQLLM_PAIR_OPERANDS(w));
    }
};

// acc[b * acc_chains(B) + chain]
template <int BITS, int B, int Q>
__device__ __forceinline__ void batch_macs(const GroupRegs<BITS, B, false> &r, const uint32_t (&wv)[kBatch], float *acc)
{
    constexpr int h = Q / 8, n0 = 2 * (Q % 8);
    if constexpr (B <= 2) {
        uint32_t x[4 * B];
#pragma unroll
        for (int b = 0; b < B; ++b)
#pragma unroll
            for (int c = 0; c < 4; ++c) x[4 * b + c] = r.xr[b][4 * h + c];
        BatchDots<B, n0>::run(x, wv, acc);
    } else {
        [&]<int... Ks>(std::integer_sequence<int, Ks...>) {
            (
                [&] {
                    uint32_t x[B];
#pragma unroll
                    for (int b = 0; b < B; ++b) x[b] = r.xr[b][4 * h + Ks % 4];
                    PairDots<B, n0 + Ks / 4>::run(x, wv[Ks], acc);
                }(),
                ...);
        }(std::make_integer_sequence<int, kBatch>{});
    }
}

// All 128 pairs (256 codes) of one group.
template <int BITS, int B, bool CT>
__device__ __forceinline__ void mac_group(const GroupRegs<BITS, B, false> &r, uint32_t lane4, const uint32_t *tab,
                                          float *acc)
{
    constexpr int NQ = 128 / kBatch;
    uint32_t wv[2][kBatch];
    batch_reads<BITS, B, false, 0, CT>(r, lane4, tab, wv[0]);
    [&]<int... Qs>(std::integer_sequence<int, Qs...>) {
        (
            [&] {
                if constexpr (Qs + 1 < NQ) batch_reads<BITS, B, false, Qs + 1, CT>(r, lane4, tab, wv[(Qs + 1) & 1]);
                // one wait for the whole batch: the empty statement needs all
                // eight table reads of batch Qs
                const uint32_t(&cur)[kBatch] = wv[Qs & 1];
                asm volatile("" ::"v"(cur[0]), "v"(cur[1]), "v"(cur[2]), "v"(cur[3]), "v"(cur[4]), "v"(cur[5]),
                             "v"(cur[6]), "v"(cur[7]));
                batch_macs<BITS, B, Qs>(r, cur, acc);
            }(),
            ...);
    }(std::make_integer_sequence<int, NQ>{});
}

// Matrix-core form: v_mfma_f32_4x4x4f16 in its 16-block shape.  Block q of
// the instruction is lanes 4q..4q+3: lane 4q+i gives row i of the block's A
// (4 x 4), lane 4q+j gives column j of its B (4 x 4), and register i of lane
// 4q+j receives D[i][j].  With CBSZ = 4 every block takes the A of block
// ABID instead of its own.  Here B is the lane's own row (lane = row of the
// tile: two table entries, 4 consecutive weights) and A the 4 activations of
// batch columns 4h..4h+3 at those columns, broadcast from the block that
// holds them: register i of lane r ends with row r's sum for batch column
// 4h+i.  No activation passes through LDS; the 16 blocks each hold a
// different 8 columns of x, so one 16-byte register per 128 columns and
// batch quad serves every step.
// Accumulator chains per batch quad: two while one or two quads alternate
// (consecutive matrix steps then never wait on each other's results), one
// from three quads on (the quads alternate; it saves registers).
constexpr int mf_chains(int batch) { return mf_quads(batch) >= 3 ? 1 : 2; }

// Step m (columns 4m .. 4m + 3 of the group) of every batch quad; cw holds
// the table entries of the step's batch of 8 pairs.
template <int BITS, int B, int M>
__device__ __forceinline__ void mf_step(const GroupRegs<BITS, B, true> &r, const uint32_t (&cw)[kBatch],
                                        f32x4 (&macc)[mf_quads(B)][2])
{
    constexpr int S = M % 4, sx = M / 32, blk = (M % 32) / 2, part = M % 2;
    const half4_t bv = __builtin_bit_cast(half4_t, u32x2{cw[2 * S], cw[2 * S + 1]});
#pragma unroll
    for (int h = 0; h < mf_quads(B); ++h) {
        const u32x4 xq = r.xq[2 * h + sx];
        const half4_t av = __builtin_bit_cast(half4_t, part ? u32x2{xq.z, xq.w} : u32x2{xq.x, xq.y});
        macc[h][mf_chains(B) == 2 ? (S & 1) : 0] =
            __builtin_amdgcn_mfma_f32_4x4x4f16(av, bv, macc[h][mf_chains(B) == 2 ? (S & 1) : 0], 4, blk, 0);
    }
}

template <int BITS, int B, bool CT>
__device__ __forceinline__ void mac_group(const GroupRegs<BITS, B, true> &r, uint32_t lane4, const uint32_t *tab,
                                          f32x4 (&macc)[mf_quads(B)][2])
{
    constexpr int NQ = 128 / kBatch; // 16 batches of 8 pairs (16 columns, 4 steps of 4)
    uint32_t wv[2][kBatch];
    batch_reads<BITS, B, true, 0, CT>(r, lane4, tab, wv[0]);
    [&]<int... Qs>(std::integer_sequence<int, Qs...>) {
        (
            [&] {
                if constexpr (Qs + 1 < NQ) batch_reads<BITS, B, true, Qs + 1, CT>(r, lane4, tab, wv[(Qs + 1) & 1]);
                const uint32_t(&cw)[kBatch] = wv[Qs & 1];
                mf_step<BITS, B, 4 * Qs + 0>(r, cw, macc);
                mf_step<BITS, B, 4 * Qs + 1>(r, cw, macc);
                mf_step<BITS, B, 4 * Qs + 2>(r, cw, macc);
                mf_step<BITS, B, 4 * Qs + 3>(r, cw, macc);
            }(),
            ...);
    }(std::make_integer_sequence<int, NQ>{});
}

// Pair table of the tile (256 entries per lane; 64 when compact).  Work item
// (lane l, low code h): lo = LUT[row][h]; for every high code c, entry
// h | c << b (3-bit, full table: also with both ignored top bits set every
// way) = lo | LUT[row][c] << 16.
// A thread's items idx = threadIdx.x + k * blockDim.x (k < N) all belong to
// lane idx % 64, so they share one load of the row's table.  The loads are
// issued apart from the stores so that they go out ahead of the code loads.
template <int BITS, int N>
struct TableItems {
    uint32_t lw[Format<BITS>::kEntries / 2];
    uint32_t lo[N];
};

template <int BITS, int N>
__device__ __forceinline__ void table_items_load(TableItems<BITS, N> &it, const uint16_t *__restrict__ lut,
                                                 int idx0, int stride, int row0, int rows)
{
    constexpr int E = Format<BITS>::kEntries;
    const int r = min(row0 + (idx0 & 63), rows - 1);
    if constexpr (E == 4) { // 8-byte table rows
        const u32x2 v = *(const u32x2 *)(lut + (int64_t)r * E);
        it.lw[0] = v.x;
        it.lw[1] = v.y;
    } else {
        const u32x4 *lrow = (const u32x4 *)(lut + (int64_t)r * E);
#pragma unroll
        for (int q = 0; q < E / 8; ++q) {
            const u32x4 v = lrow[q];
            it.lw[4 * q + 0] = v.x;
            it.lw[4 * q + 1] = v.y;
            it.lw[4 * q + 2] = v.z;
            it.lw[4 * q + 3] = v.w;
        }
    }
#pragma unroll
    for (int k = 0; k < N; ++k) { // items past the table load a valid entry and are not stored
        const int h = min((idx0 + k * stride) >> 6, E - 1);
        it.lo[k] = lut[(int64_t)r * E + h];
    }
}

template <int BITS, int N, bool CT>
__device__ __forceinline__ void table_items_store(const TableItems<BITS, N> &it, uint32_t *tab, int idx0, int stride)
{
    constexpr int E = Format<BITS>::kEntries;
    const int l = idx0 & 63;
#pragma unroll
    for (int k = 0; k < N; ++k) {
        const int h = (idx0 + k * stride) >> 6;
        if (h >= E) break;
#pragma unroll
        for (int c = 0; c < E; ++c) {
            const uint32_t hi = (c & 1) ? (it.lw[c >> 1] & 0xFFFF0000u) : (it.lw[c >> 1] << 16);
            const uint32_t v = it.lo[k] | hi;
            if constexpr (BITS == 4) {
                tab[(h | (c << 4)) * 64 + l] = v;
            } else if constexpr (BITS == 2) {
#pragma unroll
                for (int j = 0; j < 16; ++j) tab[(h | (c << 2) | (j << 4)) * 64 + l] = v;
            } else if constexpr (CT) {
                tab[(h | (c << 3)) * 64 + l] = v;
            } else {
#pragma unroll
                for (int j = 0; j < 4; ++j) tab[(h | (c << 3) | (j << 6)) * 64 + l] = v;
            }
        }
    }
}

// Chunks of 64 nonzeros a wave loads per round (two registers per chunk:
// column and value), the first round held through the dense steps.  Fewer
// above batch 8, and at 2 bits and batch 1, where 4 made the matrix-core
// group kernel spill 8 registers (2: the 2-bit stream 5% faster).
constexpr int round_chunks(int bits, int batch)
{
    return bits == 3 && batch == 1 ? 8 : (batch > 8 || (bits == 2 && batch == 1) ? 2 : 4);
}

// Loads of nonzeros [base, base + 64 * R): column and raw fp16 value of one
// nonzero per lane and chunk, each zero-extended in a register of its own (so
// that nothing waits for them before they are used).  Lanes past v1 load
// nonzero v1 - 1 (any valid index would do; their products are dropped), so
// a round always issues the same number of loads and the waits stay exact.
template <int R>
struct SparseRound {
    uint32_t col[R];
    uint32_t val[R];
};

template <int R>
__device__ __forceinline__ void sparse_round_load(SparseRound<R> &sr, const KernelArgs &a, int base, int v1, int lane)
{
#pragma unroll
    for (int k = 0; k < R; ++k) {
        const int ic = max(min(base + k * 64 + lane, v1 - 1), 0);
        sr.col[k] = a.col[ic];
        sr.val[k] = a.val[ic];
    }
}

__device__ __forceinline__ int lane_read(int src_lane, int v) { return __builtin_amdgcn_ds_bpermute(src_lane << 2, v); }
__device__ __forceinline__ float lane_read(int src_lane, float v)
{
    return __int_as_float(__builtin_amdgcn_ds_bpermute(src_lane << 2, __float_as_int(v)));
}

// Value of v from lane p - N of the same 16-lane row (0 for the row's first
// N lanes), and the last value of the previous row(s) (row_bcast: lane 15 of
// each row to rows 1 and 3, lane 31 to rows 2 and 3; 0 elsewhere).
template <int N>
__device__ __forceinline__ float row_shr(float v)
{
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x110 + N, 0xF, 0xF, true));
}
__device__ __forceinline__ float row_bcast15(float v)
{
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x142, 0xA, 0xF, false));
}
__device__ __forceinline__ float row_bcast31(float v)
{
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x143, 0xC, 0xF, false));
}

// Adds S x of the chunk of nonzeros [cb, min(cb + 64, v1)) (this lane's:
// column colv, fp16 value valv; lanes past v1 contribute nothing) into the
// row lanes' acc.  rp_lo / rp_hi: row pointers of this lane's row and the
// next one (lane = row of the tile).  x from LDS (XL: staged [B][cols] fp16
// at xl) or global memory.  acc[b * NC] is batch column b's first chain.
//
// The chunk's rows are non-decreasing, so each row's products are a run of
// lanes.  An inclusive prefix sum over the wave (DPP row shifts, then row
// broadcasts) gives every run's sum as the difference of two prefix values,
// which each row lane fetches from the run's last lane and the lane before
// its first.
// The activations of this lane's nonzero (column colv) for every batch column.
template <int B, bool XL>
__device__ __forceinline__ void sparse_gather(uint32_t colv, const KernelArgs &a, const uint16_t *xl, uint16_t (&xv)[B])
{
#pragma unroll
    for (int b = 0; b < B; ++b) {
        const int64_t xi = (int64_t)b * a.cols + (int)colv;
        xv[b] = XL ? xl[xi] : a.x[xi];
    }
}

// The same from the transposed copy: one load, one cache line per lane.
template <int B>
__device__ __forceinline__ void sparse_gather_t(uint32_t colv, const uint16_t *xt, uint16_t (&xv)[B])
{
    constexpr int P = xt_pad(B);
    uint32_t w[P / 2];
    if constexpr (P == 2) {
        w[0] = *(const uint32_t *)(xt + (int64_t)colv * 2);
    } else if constexpr (P == 4) {
        const u32x2 v = *(const u32x2 *)(xt + (int64_t)colv * 4);
        w[0] = v.x;
        w[1] = v.y;
    } else if constexpr (P == 8) {
        const u32x4 v = *(const u32x4 *)(xt + (int64_t)colv * 8);
        w[0] = v.x;
        w[1] = v.y;
        w[2] = v.z;
        w[3] = v.w;
    } else {
        const u32x4 *p = (const u32x4 *)(xt + (int64_t)colv * 16);
        const u32x4 v0 = p[0], v1 = p[1];
        w[0] = v0.x;
        w[1] = v0.y;
        w[2] = v0.z;
        w[3] = v0.w;
        w[4] = v1.x;
        w[5] = v1.y;
        w[6] = v1.z;
        w[7] = v1.w;
    }
#pragma unroll
    for (int b = 0; b < B; ++b) xv[b] = (uint16_t)(w[b >> 1] >> (16 * (b & 1)));
}

template <int B, int NC>
__device__ __forceinline__ void sparse_scan(uint32_t valv, const uint16_t (&xv)[B], int cb, int v1, int lane, int rp_lo,
                                            int rp_hi, float *acc)
{
    const float vv = cb + lane < v1 ? f16_to_f32((uint16_t)valv) : 0.f;
    float pre[B];
#pragma unroll
    for (int b = 0; b < B; ++b) {
        float v = vv * f16_to_f32(xv[b]);
        v += row_shr<1>(v);
        v += row_shr<2>(v);
        v += row_shr<4>(v);
        v += row_shr<8>(v);
        v += row_bcast15(v); // rows 1 and 3 (0 elsewhere)
        v += row_bcast31(v); // rows 2 and 3 (0 elsewhere)
        pre[b] = v;
    }
    // lane r: row r's nonzeros in this chunk are chunk lanes [first, last]
    const int hi = min(min(rp_hi, cb + 64), v1);
    const int first = max(rp_lo, cb) - cb, last = hi - 1 - cb;
    const bool present = first <= last;
    const int e_hi = present ? last : 0, e_lo = present && first > 0 ? first - 1 : 0;
#pragma unroll
    for (int b = 0; b < B; ++b) {
        const float top = lane_read(e_hi, pre[b]);
        const float below = lane_read(e_lo, pre[b]);
        if (present) acc[b * NC] += first > 0 ? top - below : top;
    }
}

template <int B, int NC, bool XL>
__device__ __forceinline__ void sparse_chunk(uint32_t colv, uint32_t valv, int cb, int v1, const KernelArgs &a, int lane,
                                             int rp_lo, int rp_hi, const uint16_t *xl, float *acc)
{
    uint16_t xv[B];
    sparse_gather<B, XL>(colv, a, xl, xv);
    sparse_scan<B, NC>(valv, xv, cb, v1, lane, rp_lo, rp_hi, acc);
}

// Issue the first ring of code loads only after the pair table is built:
// behind a deep queue of streaming code loads the table's own loads return
// late and hold back every group's math.
constexpr bool kRingAfterTable = true;

// Quads (16 bytes) of x each thread stages in LDS from registers loaded in
// the prologue; the rest of a wider x is copied in a loop before the table
// barrier.
constexpr int kStageQuads = 4;

// Round and store (or hand over) this workgroup's fp32 row sums.  With the
// row tile split over several workgroups (this one is leaf s), the partial
// sums meet in a binary tree of 64-bit words in the workspace, one word per
// pairing and (tile, batch column, row): at a level of m nodes, nodes 2j and
// 2j+1 share word j, each setting its half with one atomic OR (the fp32 bits
// inverted, so that an empty half reads 0; -0.0 and +0.0 stay distinct); an
// odd last node passes up unpaired.  The one that finds the other half
// already there adds left + right, clears the word and goes on to the next
// level; the last one rounds once and stores y.  Which workgroup arrives
// first does not change any sum, so repeated launches give identical bits,
// and every word is zero again when the launch has finished.
// Without helpers the tree spans the split's leaves, words from t * stride
// (stride = split - 1).  With e > 0 helpers (an outlier plan; stride =
// kMaxSplit - 1) the owners' leaves [0, split) and the helpers' [split,
// split + e) first form a tree each, (split - 1) and (e - 1) words, and the
// two roots meet in one more word: helpers hold no code stream and finish
// early, so an owner that arrives last climbs its own tree and one word.
template <int B>
__device__ __forceinline__ bool climb(const KernelArgs &a, int t, int stride, int b, int lane, float &v, int i, int m,
                                      int base)
{
    while (m > 1) {
        if ((m & 1) && i == m - 1) { // unpaired: passes up as it is
            i >>= 1;
            base += m >> 1;
            m = (m + 1) >> 1;
            continue;
        }
        unsigned long long *w = a.slots + (((int64_t)t * stride + base + (i >> 1)) * B + b) * 64 + lane;
        const uint32_t enc = ~__float_as_uint(v);
        const unsigned long long mine = (i & 1) ? (unsigned long long)enc << 32 : (unsigned long long)enc;
        const unsigned long long old = __hip_atomic_fetch_or(w, mine, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        const uint32_t other = (i & 1) ? (uint32_t)old : (uint32_t)(old >> 32);
        if (other == 0) return false; // the partner has not arrived: it goes on
        const float o = __uint_as_float(~other);
        v = (i & 1) ? o + v : v + o; // left + right
        __hip_atomic_store(w, 0ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        i >>= 1;
        base += m >> 1;
        m = (m + 1) >> 1;
    }
    return true;
}

template <int B, bool ADDY>
__device__ __forceinline__ void finish_rows(const KernelArgs &a, int t, int s, int lane, const float *tot, int split,
                                            int e, int stride)
{
    const int row = t * 64 + lane;
#pragma unroll
    for (int b = 0; b < B; ++b) {
        float v = tot[b];
        bool last;
        if (e == 0)
            last = climb<B>(a, t, stride, b, lane, v, s, split, 0);
        else if (s < split)
            last = climb<B>(a, t, stride, b, lane, v, s, split, 0) &&
                   climb<B>(a, t, stride, b, lane, v, 0, 2, split + e - 2);
        else
            last = climb<B>(a, t, stride, b, lane, v, s - split, e, split - 1) &&
                   climb<B>(a, t, stride, b, lane, v, 1, 2, split + e - 2);
        if (last && row < a.rows) {
            if constexpr (ADDY) v += f16_to_f32(a.y[(int64_t)b * a.ldy + row]);
            a.y[(int64_t)b * a.ldy + row] = f32_to_f16_rne(v);
        }
    }
}

// ---------------------------------------------------------------------------
// The kernel.  MODE: kFused y = (D+S)x; kDenseOnly y = Dx; kSparseAdd y += Sx.
// Grid: tiles * split workgroups; workgroup (tile t, split s) owns column
// groups [s*gps, min((s+1)*gps, groups)) and share s of the tile's nonzeros.
// Every wave does both kinds of work: dense groups gb + w + j*W, and one of
// the split * W even shares of the tile's nonzeros, a chunk after each dense
// group (the rest after the last one).
// LDS: the pair table (static, dense modes; it must stay the only static
// array so that it starts at LDS address 0) and, when a.x_lds, all of x for
// the outlier gathers (dynamic, [B][cols] fp16).
//
// Order of work: row pointers, table rows and x to stage go out first, then
// the first ring of code loads, then the first round of nonzeros.  Every dense step issues one group of loads
// (placeholders past the wave's last group), so the wait before each group's
// math lets exactly D-1 groups stay in flight.
// A helper workgroup of an outlier plan: share s of tile t's nonzeros (of
// count * W even shares, as the tile's owners cut them), nothing else -- no
// pair table, no code loads, whose queue it would otherwise wait behind --
// then the wave reduction and leaf s of the tile's combine.
// red: LDS for the reduction (W * B * 64 floats); xs: LDS for x when staged.
template <int B, bool ADDY>
__device__ __forceinline__ void helper_body(const KernelArgs &a, int t, int s, int count, float *red, uint32_t *xs)
{
    constexpr int NC = 1;
    constexpr int R = B <= 2 ? 8 : (B <= 8 ? 4 : 2); // chunks per round: their gathers stay in registers
    const int nt = blockDim.x;
    const int W = nt >> 6;
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    const int row0 = t * 64;
    const int rp_lo = a.row_ptr[min(row0 + lane, a.rows)];
    const int rp_hi = a.row_ptr[min(row0 + lane + 1, a.rows)];
    const int nz0 = __builtin_amdgcn_readfirstlane(rp_lo);
    const int nz1 = __builtin_amdgcn_readlane(rp_hi, 63);
    const uint32_t len = (uint32_t)(nz1 - nz0);
    const uint32_t parts = (uint32_t)(count * W), part = (uint32_t)(w * count + s);
    const uint32_t per = len / parts, extra = len - per * parts;
    const int v0 = nz0 + (int)(part * per + min(part, extra));
    const int v1 = v0 + (int)(per + (part < extra ? 1u : 0u));
    if (a.x_lds) { // uniform: all of x into LDS
        const int nxq = B * (a.cols >> 3);
        for (int i = threadIdx.x; i < nxq; i += nt) ((u32x4 *)xs)[i] = ((const u32x4 *)a.x)[i];
        lds_barrier();
    }
    const uint16_t *xl = (const uint16_t *)xs;
    float acc[B];
#pragma unroll
    for (int b = 0; b < B; ++b) acc[b] = 0.f;
    SparseRound<R> cv;
    for (int base = v0; base < v1; base += 64 * R) {
        sparse_round_load(cv, a, base, v1, lane);
        uint16_t xg[R][B];
#pragma unroll
        for (int k = 0; k < R; ++k)
            if (base + 64 * k < v1) {
                if (a.x_lds)
                    sparse_gather<B, true>(cv.col[k], a, xl, xg[k]);
                else if (B >= kXtBatch && a.xt)
                    sparse_gather_t<B>(cv.col[k], a.xt, xg[k]);
                else
                    sparse_gather<B, false>(cv.col[k], a, xl, xg[k]);
            }
#pragma unroll
        for (int k = 0; k < R; ++k)
            if (base + 64 * k < v1) sparse_scan<B, NC>(cv.val[k], xg[k], base + 64 * k, v1, lane, rp_lo, rp_hi, acc);
    }
#pragma unroll
    for (int b = 0; b < B; ++b) red[(w * B + b) * 64 + lane] = acc[b];
    lds_barrier();
    if (w != 0) return;
    float tot[B];
#pragma unroll
    for (int b = 0; b < B; ++b) {
        float v = 0.f;
        for (int k = 0; k < W; ++k) v += red[(k * B + b) * 64 + lane];
        tot[b] = v;
    }
    finish_rows<B, ADDY>(a, t, s, lane, tot, a.split, count - a.split, kMaxSplit - 1);
}

// Every argument (and the workgroup size) into registers at once: one round
// of scalar loads at the start instead of one per first use.
__device__ __forceinline__ void load_args_now(const KernelArgs &a)
{
    asm volatile("" ::"s"(a.packed), "s"(a.lut), "s"(a.row_ptr), "s"(a.col), "s"(a.val), "s"(a.x), "s"(a.y),
                 "s"(a.slots), "s"(a.rows), "s"(a.ldy), "s"(a.cols), "s"(a.tiles), "s"(a.groups), "s"(a.split), "s"(a.gps),
                 "s"(a.x_lds), "s"(a.xt), "s"(a.sparse_naive), "s"(a.plan), "s"(a.helpers), "s"(blockDim.x));
}

template <int BITS, int B, int MODE, bool MF, bool CT>
__device__ __forceinline__ void product_body(const KernelArgs &a, int bid)
{
    load_args_now(a);
    constexpr bool DENSE = MODE != kSparseAdd;
    constexpr bool SPARSE = MODE != kDenseOnly;
    constexpr bool ADDY = MODE == kSparseAdd;
    static_assert(!MF || DENSE, "matrix-core form: dense modes");
    constexpr int E = Format<BITS>::kEntries;
    constexpr int D = ring_depth(BITS, B, MF);
    constexpr int ITEMS = DENSE && E >= 8 ? (64 * E) / 512 : 1; // table items per thread with 8 waves
    static_assert(!CT || (compact_allowed(BITS, B) && MF && MODE == kFused), "compact table: 3-bit fused, matrix cores");
    __shared__ __align__(16) uint32_t tab[DENSE ? dense_lds_bytes(B, CT) / 4 : kMaxWaves * B * 64];
    extern __shared__ __align__(16) uint32_t dyn[];

    const int nt = blockDim.x;
    const int W = nt >> 6;
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    // Workgroups [0, helpers) of a planned launch are helpers: helper h takes
    // leaf split + e of tile t's combine (plan entry (t << 4) | e) and only
    // outliers; the rest own (tile, column range) pairs as without a plan.
    // count: the tile's partial sums (its owners and helpers).
    typedef const __attribute__((address_space(4))) int32_t *const_i32_ptr; // read-only: scalar loads
    const bool helper = bid < a.helpers;
    int t, s;
    if (helper) {
        const int e = ((const_i32_ptr)a.plan)[1 + a.tiles + bid];
        t = e >> 4;
        s = a.split + (e & 15);
    } else {
        t = (bid - a.helpers) / a.split;
        s = bid - a.helpers - t * a.split;
    }
    const int count = a.helpers > 0 ? a.split + ((const_i32_ptr)a.plan)[1 + t] : a.split;
    if constexpr (SPARSE) {
        if (helper) { // uniform over the workgroup
            helper_body<B, ADDY>(a, t, s, count, (float *)tab, dyn);
            return;
        }
    }
    const int row0 = t * 64;
    const uint32_t lane4 = (uint32_t)lane << 2;

    constexpr int NC = MF ? 1 : acc_chains(B);
    float acc[B * NC]; // dense chains (dot form); outliers add into chain 0
#pragma unroll
    for (int k = 0; k < B * NC; ++k) acc[k] = 0.f;
    constexpr int NX = MF ? mf_quads(B) : 1;
    f32x4 macc[NX][2]; // matrix-core form: [batch quad][chain] (chain 1 unused from three quads on)
#pragma unroll
    for (int h = 0; h < NX; ++h) macc[h][0] = macc[h][1] = f32x4{0.f, 0.f, 0.f, 0.f};
    uint32_t *xstage = dyn; // dynamic LDS: x staged for the outlier gathers

    // -- 1. the pair-table items beyond ITEMS per thread (workgroups of fewer
    //       than 8 waves only)
    if constexpr (DENSE) {
        for (int idx = threadIdx.x + ITEMS * nt; idx < 64 * E; idx += nt) {
            TableItems<BITS, 1> it2;
            table_items_load<BITS, 1>(it2, a.lut, idx, nt, row0, a.rows);
            table_items_store<BITS, 1, CT>(it2, tab, idx, nt);
        }
    }

    // -- 2. small loads first: this thread's table rows (ahead of every other
    //       load: the table is what the first group's math waits for), the
    //       tile's row pointers and quads of x to stage
    TableItems<BITS, ITEMS> items; // loaded by every thread (no branch), stored by those that own items
    if constexpr (DENSE) {
        table_items_load<BITS, ITEMS>(items, a.lut, threadIdx.x, nt, row0, a.rows);
        asm volatile("" ::: "memory"); // the loads may not sink below this point
    }
    int rp_lo = 0, rp_hi = 0;
    if constexpr (SPARSE) {
        rp_lo = a.row_ptr[min(row0 + lane, a.rows)];
        rp_hi = a.row_ptr[min(row0 + lane + 1, a.rows)];
    }
    const int nxq = (SPARSE && a.x_lds) ? B * (a.cols >> 3) : 0; // 16-byte quads of x to stage
    u32x4 xq[SPARSE ? kStageQuads : 1];
    if constexpr (SPARSE) {
#pragma unroll
        for (int k = 0; k < kStageQuads; ++k) // past the end: a valid quad, not stored
            xq[k] = ((const u32x4 *)a.x)[min((int)threadIdx.x + k * nt, max(nxq - 1, 0))];
    }

    // -- 3. the first ring of code loads (here, or once the table is built:
    //       a queue of streaming code loads delays the table's loads)
    const int gb = s * a.gps;
    const int ge = min(gb + a.gps, a.groups);
    const int cnt = DENSE && !helper ? max(0, (ge - gb - w + W - 1) / W) : 0; // this wave's groups
    GroupRegs<BITS, B, MF> ring[DENSE ? D : 1];
    auto issue_ring = [&]() {
        if constexpr (DENSE) {
#pragma unroll
            for (int k = 0; k < D; ++k) load_group<BITS, B, MF>(ring[k], a, t, k < cnt ? gb + w + k * W : -1, lane);
        }
    };
    auto dense_math = [&](const GroupRegs<BITS, B, MF> &r) {
        if constexpr (DENSE && MF)
            mac_group<BITS, B, CT>(r, lane4, tab, macc);
        else if constexpr (DENSE)
            mac_group<BITS, B, CT>(r, lane4, tab, acc);
    };
    if constexpr (!kRingAfterTable) issue_ring();

    // -- 4. this wave's share of the nonzeros and its first round of loads
    int nz0 = 0, v0 = 0, v1 = 0;
    constexpr int R = round_chunks(BITS, B);
    SparseRound<R> cv;
    if constexpr (SPARSE) {
        // the tile's ends, as uniform (scalar) loads: waiting for them does
        // not wait for the vector loads in flight
        const const_i32_ptr rptr = (const_i32_ptr)a.row_ptr;
        nz0 = rptr[row0];
        const int nz1 = rptr[min(row0 + 64, a.rows)];
        // share part of `parts` even shares: the first len % parts get one more
        const uint32_t len = (uint32_t)(nz1 - nz0);
        const uint32_t parts = (uint32_t)(count * W), part = (uint32_t)(w * count + s);
        const uint32_t per = len / parts, extra = len - per * parts;
        v0 = nz0 + (int)(part * per + min(part, extra));
        v1 = v0 + (int)(per + (part < extra ? 1u : 0u));
        if (a.sparse_naive) v1 = v0; // the naive form below takes every nonzero
        sparse_round_load(cv, a, v0, v1, lane);
    }

    // -- 5. store the pair table and the staged x, then a barrier that
    //       orders LDS only: the ring stays in flight across it
    if constexpr (DENSE) {
        if ((int)threadIdx.x < 64 * E) table_items_store<BITS, ITEMS, CT>(items, tab, threadIdx.x, nt);
    }
    if constexpr (SPARSE) {
#pragma unroll
        for (int k = 0; k < kStageQuads; ++k)
            if ((int)threadIdx.x + k * nt < nxq) ((u32x4 *)xstage)[threadIdx.x + k * nt] = xq[k];
        // the rest kStageQuads quads per thread at a time: all of a batch's
        // loads go out before its stores wait for them
        for (int i0 = threadIdx.x + kStageQuads * nt; i0 < nxq; i0 += kStageQuads * nt) {
            u32x4 v[kStageQuads];
#pragma unroll
            for (int k = 0; k < kStageQuads; ++k) v[k] = ((const u32x4 *)a.x)[min(i0 + k * nt, nxq - 1)];
#pragma unroll
            for (int k = 0; k < kStageQuads; ++k)
                if (i0 + k * nt < nxq) ((u32x4 *)xstage)[i0 + k * nt] = v[k];
        }
    }
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
    if constexpr (kRingAfterTable) issue_ring();

    // -- 6. dense steps: a main loop in which every step refills the ring,
    //       then the last (fewer than 2D) groups, each of those followed by
    //       one chunk of the first round of nonzeros
    const uint16_t *xl = (const uint16_t *)xstage;
    const int r0end = min(v1, v0 + 64 * R);
    auto chunk = [&](auto kc) { // chunk K of the first round, if the share has it
        constexpr int K = decltype(kc)::value;
        if constexpr (SPARSE && K < R) {
            const int cbk = v0 + 64 * K;
            if (cbk < r0end) {
                if (a.x_lds)
                    sparse_chunk<B, NC, true>(cv.col[K], cv.val[K], cbk, v1, a, lane, rp_lo, rp_hi, xl, acc);
                else
                    sparse_chunk<B, NC, false>(cv.col[K], cv.val[K], cbk, v1, a, lane, rp_lo, rp_hi, xl, acc);
            }
        }
    };
    int done = 0; // chunks of the first round taken
    if constexpr (DENSE) {
        int j0 = 0;
        for (; j0 + 2 * D <= cnt; j0 += D) {
#pragma unroll
            for (int k = 0; k < D; ++k) {
                dense_math(ring[k]);
                load_group<BITS, B, MF>(ring[k], a, t, gb + w + (j0 + k + D) * W, lane);
            }
        }
        [&]<int... Ks>(std::integer_sequence<int, Ks...>) {
            (
                [&] {
                    constexpr int k = Ks;
                    const int j = j0 + k;
                    if (j < cnt) {
                        dense_math(ring[k]);
                        if (j + D < cnt) load_group<BITS, B, MF>(ring[k], a, t, gb + w + (j + D) * W, lane);
                        if (a.x_lds) {
                            chunk(std::integral_constant<int, k>{});
                            done = k + 1;
                        }
                    }
                }(),
                ...);
            (
                [&] {
                    constexpr int k = Ks;
                    if (j0 + D + k < cnt) {
                        dense_math(ring[k]);
                        if (a.x_lds) {
                            chunk(std::integral_constant<int, D + k>{});
                            done = D + k + 1;
                        }
                    }
                }(),
                ...);
        }(std::make_integer_sequence<int, D>{});
    }

    // -- 7. the rest of the nonzeros
    if constexpr (SPARSE) {
        // the ablation's naive form (one thread per row, as an unbalanced CSR
        // kernel does): wave 0 of the tile's first workgroup, lane = row
        if (a.sparse_naive && s == 0 && w == 0) {
            for (int i = rp_lo; i < rp_hi; ++i) {
                const float vv = f16_to_f32(a.val[i]);
                const int col = a.col[i];
#pragma unroll
                for (int b = 0; b < B; ++b) {
                    const int64_t xi = (int64_t)b * a.cols + col;
                    acc[b * NC] += vv * f16_to_f32(a.x_lds ? xl[xi] : a.x[xi]);
                }
            }
        }
        // the rest a round at a time: every gather of the round, then the
        // scans, so that a round waits for memory once rather than per chunk
        auto finish_round = [&](int base, int kfirst) {
            uint16_t xg[R][B];
#pragma unroll
            for (int k = 0; k < R; ++k)
                if (k >= kfirst && base + 64 * k < v1) {
                    if (a.x_lds)
                        sparse_gather<B, true>(cv.col[k], a, xl, xg[k]);
                    else if (B >= kXtBatch && a.xt)
                        sparse_gather_t<B>(cv.col[k], a.xt, xg[k]);
                    else
                        sparse_gather<B, false>(cv.col[k], a, xl, xg[k]);
                }
#pragma unroll
            for (int k = 0; k < R; ++k)
                if (k >= kfirst && base + 64 * k < v1)
                    sparse_scan<B, NC>(cv.val[k], xg[k], base + 64 * k, v1, lane, rp_lo, rp_hi, acc);
        };
        finish_round(v0, done);
        for (int base = v0 + 64 * R; base < v1; base += 64 * R) {
            sparse_round_load(cv, a, base, v1, lane);
            finish_round(base, 0);
        }
    }
    lds_barrier(); // pair table no longer needed

    // -- 8. reduce the waves (fixed order), then round and store / hand over
    float *red = (float *)tab;
    if constexpr (MF) {
        // register i of the batch quad h: batch column 4h+i of this lane's row
#pragma unroll
        for (int b = 0; b < B; ++b) {
            if constexpr (mf_chains(B) == 2)
                red[(w * B + b) * 64 + lane] = acc[b] + macc[b / 4][0][b % 4] + macc[b / 4][1][b % 4];
            else
                red[(w * B + b) * 64 + lane] = acc[b] + macc[b / 4][0][b % 4];
        }
    } else {
#pragma unroll
        for (int b = 0; b < B; ++b) {
            float v = acc[b * NC];
#pragma unroll
            for (int c = 1; c < NC; ++c) v += acc[b * NC + c];
            red[(w * B + b) * 64 + lane] = v;
        }
    }
    lds_barrier();
    if (w != 0) return;
    float tot[B];
#pragma unroll
    for (int b = 0; b < B; ++b) {
        float v = 0.f;
        for (int k = 0; k < W; ++k) v += red[(k * B + b) * 64 + lane];
        tot[b] = v;
    }
    finish_rows<B, ADDY>(a, t, s, lane, tot, a.split, count - a.split, a.helpers > 0 ? kMaxSplit - 1 : count - 1);
}

template <int BITS, int B, int MODE, bool MF, bool CT>
__global__ void __launch_bounds__(kMaxWaves * 64) dense_sparse_kernel(KernelArgs a)
{
    product_body<BITS, B, MODE, MF, CT>(a, blockIdx.x);
}

// Several independent products in one launch: the workgroups of row y of the
// grid run product y (those past its tiles x split workgroups exit at once).
// The hardware starts workgroups in grid order as soon as a compute unit has
// room, so one product's start-up (table rows, first code latency) and tail
// (reductions) overlap the other products' code streams.  The product index
// is blockIdx.y, so its arguments come in one round of scalar loads.
template <int BITS, int B, int MODE, bool MF, bool CT>
__global__ void __launch_bounds__(kMaxWaves * 64) dense_sparse_group_kernel(GroupArgs g)
{
    const KernelArgs &a = g.item[blockIdx.y];
    load_args_now(a);
    if ((int)blockIdx.x >= a.tiles * a.split + a.helpers) return;
    product_body<BITS, B, MODE, MF, CT>(a, blockIdx.x);
}

// Ask once per kernel and device for more than the default dynamic LDS (the
// attribute belongs to the device current at the call).  Not fatal when
// refused: launches within the default limit still work, larger ones report
// the launch error.
inline void raise_lds_limit(const void *kern, std::atomic<uint64_t> &done, int bytes)
{
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) {
        (void)hipGetLastError();
        return;
    }
    const uint64_t bit = 1ull << (dev & 63);
    if (done.load(std::memory_order_relaxed) & bit) return;
    if (hipFuncSetAttribute(kern, hipFuncAttributeMaxDynamicSharedMemorySize, bytes) != hipSuccess)
        (void)hipGetLastError();
    done.fetch_or(bit, std::memory_order_relaxed);
}

template <int BITS, int B, int MODE, bool MF, bool CT>
hipError_t launch_one(const KernelArgs &a, const LaunchShape &ls, hipStream_t stream)
{
    auto kern = dense_sparse_kernel<BITS, B, MODE, MF, CT>;
    static std::atomic<uint64_t> attr_devices{0};
    raise_lds_limit((const void *)kern, attr_devices, kLdsBudget - (int)static_lds_bytes(MODE != kSparseAdd, B, CT));
    if (ls.waves < 1 || ls.waves > kMaxWaves) return hipErrorInvalidConfiguration;
    const dim3 grid((unsigned)(a.tiles * a.split + a.helpers)), block((unsigned)(64 * ls.waves));
    hipLaunchKernelGGL(kern, grid, block, ls.dyn_lds, stream, a);
    return hipGetLastError();
}

template <int BITS, int B, int MODE, bool MF, bool CT>
hipError_t launch_group_one(const GroupArgs &g, const LaunchShape &ls, hipStream_t stream)
{
    auto kern = dense_sparse_group_kernel<BITS, B, MODE, MF, CT>;
    static std::atomic<uint64_t> attr_devices{0};
    raise_lds_limit((const void *)kern, attr_devices, kLdsBudget - (int)static_lds_bytes(true, B, CT));
    if (ls.waves < 1 || ls.waves > kMaxWaves || g.n < 1 || g.n > kMaxGroup) return hipErrorInvalidConfiguration;
    const dim3 grid((unsigned)g.wgs, (unsigned)g.n), block((unsigned)(64 * ls.waves));
    hipLaunchKernelGGL(kern, grid, block, ls.dyn_lds, stream, g);
    return hipGetLastError();
}

// The dense modes in the matrix-core form when the shape asks for it (and
// always above kMaxDotBatch, where the dot form is not built); the dot form
// and the outlier-only mode otherwise.  CT: the compact-table kernels (the
// fused matrix-core form only).
template <int BITS, int B, int MODE, bool CT>
hipError_t launch_group_form(const GroupArgs &g, const LaunchShape &ls, hipStream_t stream)
{
    if constexpr (CT) {
        if constexpr (compact_allowed(BITS, B) && MODE == kFused) return launch_group_one<BITS, B, MODE, true, true>(g, ls, stream);
        return hipErrorInvalidValue;
    } else {
        if constexpr (MODE != kSparseAdd)
            if (ls.mf || B > kMaxDotBatch) return launch_group_one<BITS, B, MODE, true, false>(g, ls, stream);
        if constexpr (MODE == kSparseAdd || B <= kMaxDotBatch)
            return launch_group_one<BITS, B, MODE, false, false>(g, ls, stream);
        return hipErrorInvalidValue;
    }
}

template <int BITS, int B, int MODE, bool CT>
hipError_t launch_form(const KernelArgs &a, const LaunchShape &ls, hipStream_t stream)
{
    if constexpr (CT) {
        if constexpr (compact_allowed(BITS, B) && MODE == kFused) return launch_one<BITS, B, MODE, true, true>(a, ls, stream);
        return hipErrorInvalidValue;
    } else {
        if constexpr (MODE != kSparseAdd)
            if (ls.mf || B > kMaxDotBatch) return launch_one<BITS, B, MODE, true, false>(a, ls, stream);
        if constexpr (MODE == kSparseAdd || B <= kMaxDotBatch) return launch_one<BITS, B, MODE, false, false>(a, ls, stream);
        return hipErrorInvalidValue;
    }
}

// Batches LO..HI of one (bits, mode).  The batch-1..8 kernels, the
// batch-9..16 ones and the compact-table ones are instantiated in separate
// translation units: sharing one unit changes the compiler's code for the
// small batches (measured 6% slower at batch 1).
template <int BITS, int MODE, int LO, int HI, bool CT = false>
hipError_t launch_group_batch(const GroupArgs &g, int batch, const LaunchShape &ls, hipStream_t stream)
{
    hipError_t r = hipErrorInvalidValue;
    [&]<int... Ks>(std::integer_sequence<int, Ks...>) {
        ((batch == LO + Ks ? (void)(r = launch_group_form<BITS, LO + Ks, MODE, CT>(g, ls, stream)) : void()), ...);
    }(std::make_integer_sequence<int, HI - LO + 1>{});
    return r;
}

template <int BITS, int MODE, int LO, int HI, bool CT = false>
hipError_t launch_batch(const KernelArgs &a, int batch, const LaunchShape &ls, hipStream_t stream)
{
    hipError_t r = hipErrorInvalidValue;
    [&]<int... Ks>(std::integer_sequence<int, Ks...>) {
        ((batch == LO + Ks ? (void)(r = launch_form<BITS, LO + Ks, MODE, CT>(a, ls, stream)) : void()), ...);
    }(std::make_integer_sequence<int, HI - LO + 1>{});
    return r;
}

} // namespace dev
} // namespace sqllm

#undef SQLLM_DOT
#undef SQLLM_DOTS3
#undef SQLLM_PAIR_OPERANDS

#endif
