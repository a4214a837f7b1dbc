// sqllm_internal.h -- declarations shared by the C-ABI layer and the kernels
// (plain C++, no HIP types except the runtime's status and stream handles).
#ifndef SQLLM_INTERNAL_H
#define SQLLM_INTERNAL_H

#include <stdint.h>

#include <hip/hip_runtime_api.h>

namespace sqllm {

constexpr int kTileRows = 64;     // rows per tile = lanes per wave
constexpr int kGroupCols = 256;   // codes per group
constexpr int kMaxBatch = 16;
constexpr int kMaxDotBatch = 8;   // the v_dot2c form is built up to this batch; above it only the matrix cores
constexpr int kMaxWaves = 16;     // waves per workgroup
constexpr int kMaxSplit = 16;     // workgroups sharing one row tile (the owners and any helpers)
constexpr int kMaxHelpers = 8;    // helpers one row tile may get from an outlier plan
constexpr int kTableBytes = 256 * 64 * 4;           // pair table: 256 entries x 64 lanes x half2
// The compact 3-bit pair table: the two top bits of a pair's address byte
// are masked (one AND per dword of codes), so the table holds the 64 pairs
// once (16 KB) instead of four times.  A fused launch at batch 2..8 takes it
// when that is what lets x be staged in LDS for the outlier gathers (x of
// 22016x8192 at batch 4 beside two tables per compute unit, of 8192x8192 at
// batch 8 beside one); otherwise the AND costs more than it saves.
constexpr bool compact_allowed(int bits, int batch) { return bits == 3 && batch >= 2 && batch <= kMaxDotBatch; }
constexpr int table_bytes(bool compact) { return compact ? 64 * 64 * 4 : kTableBytes; }
// Static LDS of a dense-mode workgroup: the pair table, which the wave
// reduction (up to kMaxWaves x batch x 64 floats) reuses once the dense part
// is done, so at least that.
constexpr int dense_lds_bytes(int batch, bool compact)
{
    return table_bytes(compact) > kMaxWaves * batch * 64 * 4 ? table_bytes(compact) : kMaxWaves * batch * 64 * 4;
}
constexpr int kLdsBudget = 160 * 1024;              // LDS per compute unit on gfx950
constexpr int kSparseShare = 512; // outlier nonzeros per wave the outlier-only kernel aims for
constexpr int kDefaultWaves = 8;  // waves per workgroup: two workgroups share a compute unit

enum Mode { kFused = 0, kDenseOnly = 1, kSparseAdd = 2 };

struct KernelArgs {
    const void *packed;       // packed codes (16-byte aligned)
    const uint16_t *lut;      // fp16 [rows][2^bits]
    const int32_t *row_ptr;   // [rows + 1]
    const uint16_t *col;      // [nnz]
    const uint16_t *val;      // fp16 [nnz]
    const uint16_t *x;        // fp16 [batch][cols]
    uint16_t *y;              // fp16 [batch][rows]
    unsigned long long *slots;  // workspace: split - 1 combine words per (tile, batch, row)
    int rows, cols, tiles, groups;
    int ldy;                  // y's batch stride: rows, or more for a row slice of a larger product
    int split;                // workgroups per row tile
    int gps;                  // column groups per workgroup (the last one may have fewer)
    int x_lds;                // 1: all of x staged in LDS for the outlier gathers
    const uint16_t *xt;       // else, batch >= kXtBatch: x transposed, [cols][xt_pad(batch)] fp16 (or null)
    int sparse_naive;         // 1 (ablation): one lane per row walks its own nonzeros, no balancing
    const int32_t *plan;      // with helpers > 0: per-tile helper counts at plan[1 + t], then the helpers
    int helpers;              // workgroups that only take shares of a heavy tile's nonzeros (grid's first)
};

// Independent products run by one launch (same bits and batch).
constexpr int kMaxGroup = 8;
struct GroupArgs {
    int n;                        // products (grid rows)
    int wgs;                      // grid columns: the most workgroups of any product
    KernelArgs item[kMaxGroup];
};

// Matrix-core form of the dense part: batch columns in quads of 4.
constexpr int mf_quads(int batch) { return (batch + 3) / 4; }

// One launch configuration, chosen on the host.
struct LaunchShape {
    int waves;                // waves per workgroup
    size_t dyn_lds;           // dynamic LDS bytes (staged x)
    int mf;                   // 1: dense part on the matrix cores, 0: dot form (batch <= kMaxDotBatch)
    int compact;              // 1: the compact 3-bit pair table (fused, matrix cores, batch 2..8)
};

hipError_t launch_dense_sparse(const KernelArgs &a, int bits, int batch, Mode mode, const LaunchShape &ls,
                               hipStream_t stream);
hipError_t launch_dense_sparse_group(const GroupArgs &g, int bits, int batch, Mode mode, const LaunchShape &ls,
                                     hipStream_t stream);
// Rank selection over 16-bit keys: bin and rank within the bin of ranks r0,
// r1 (fp16 order keys), or of the high then low key halves (fp32).
struct SelectOut {
    uint32_t bin[2];
    uint32_t pad0[2];
    int64_t rest[2];
    uint32_t bin2[2];
    uint32_t pad1[2];
    int64_t rest2[2];
};
hipError_t launch_rank_select(const void *src, bool fp32, int64_t n, int64_t r0, int64_t r1, uint32_t *bins,
                              SelectOut *out, hipStream_t stream);
hipError_t launch_outlier_count(const uint16_t *w, const float *sens, int rows, int cols, uint16_t t_min,
                                uint16_t t_max, float t_s, int32_t *counts, unsigned long long *total,
                                hipStream_t stream);
hipError_t launch_outlier_extract(const uint16_t *w, const float *sens, int rows, int cols, uint16_t t_min,
                                  uint16_t t_max, float t_s, int32_t *counts, int32_t *row_ptr, uint16_t *col_idx,
                                  uint16_t *val, int64_t capacity, uint16_t *dense, float *sens_dense, int *overflow,
                                  hipStream_t stream);
hipError_t launch_kmeans(const uint16_t *dense, const float *sens, int rows, int cols, int bits, int iters,
                         uint8_t *codes, uint16_t *lut, hipStream_t stream);
hipError_t launch_pack(const uint8_t *codes, int rows, int cols, int bits, void *packed, int *bad, hipStream_t stream);
hipError_t launch_unpack(const void *packed, const uint16_t *lut, int rows, int cols, int bits, uint8_t *codes,
                         uint16_t *w, hipStream_t stream);

// Dynamic LDS of a workgroup that stages x for the outlier gathers: every
// column of every batch column.
inline size_t staged_x_bytes(int64_t cols, int batch) { return (size_t)cols * batch * 2; }

// x transposed for the outlier gathers from batch kXtBatch on, when the
// products reading one x carry at least kXtMinNnz nonzeros: all batch
// columns of a column in one 16-byte word (two above batch 8; padded with
// zeros).  Below that the two extra launches (write, clear) cost more than
// the gathers save.
constexpr int kXtBatch = 5;
constexpr int64_t kXtMinNnz = 400000;
constexpr int xt_pad(int batch) { return batch <= 2 ? 2 : (batch <= 4 ? 4 : (batch <= 8 ? 8 : 16)); }
inline size_t xt_bytes(int64_t cols, int batch)
{
    return batch < kXtBatch ? 0 : ((size_t)cols * xt_pad(batch) * 2 + 255) / 256 * 256;
}
// Transposed copies of up to kMaxGroup activations: written before the
// product launch and cleared after it (the workspace is zero between calls).
struct XtJobs {
    int n;
    int max_cols;
    const uint16_t *x[kMaxGroup];
    uint16_t *xt[kMaxGroup];
    int cols[kMaxGroup];
};
constexpr int kStreamReadWaves = 4096; // waves of the reference read stream: one sink slot each
hipError_t launch_stream_read(const void *src, size_t bytes, uint32_t *sink, hipStream_t stream);
hipError_t launch_xt_write(const XtJobs &j, int batch, hipStream_t stream);
hipError_t launch_xt_clear(const XtJobs &j, int batch, hipStream_t stream);

// Static LDS of a kernel: the pair table (dense modes) or the wave
// reduction area (outlier-only mode).
inline size_t static_lds_bytes(bool dense, int batch, bool compact)
{
    return dense ? (size_t)dense_lds_bytes(batch, compact) : (size_t)kMaxWaves * batch * 64 * 4;
}

} // namespace sqllm

#endif
