// sqllm_api.cpp -- the C ABI declared in include/sqllm.h: argument checks
// (all done on the host before any HIP call), the split heuristic, and the
// kernel launches on the caller's stream.
#include "sqllm.h"

#include <stdint.h>
#include <stdlib.h>

#include "sqllm_internal.h"

using namespace sqllm;

namespace {

// Tuning knobs (environment, read once): SQLLM_WAVES_3 / SQLLM_WAVES_4 set
// the waves per workgroup of the dense kernels, SQLLM_TARGET_WGS the
// workgroup count the column split aims for, SQLLM_SPLIT forces a split.
struct Tuning {
    int waves3 = 4, waves4 = 8, waves_sparse = 4;
    int target_wgs = 1024;
    int force_split = 0;
    Tuning()
    {
        auto get = [](const char *name, int lo, int hi, int dflt) {
            const char *v = getenv(name);
            if (!v || !*v) return dflt;
            long x = strtol(v, nullptr, 10);
            return (x < lo || x > hi) ? dflt : (int)x;
        };
        waves3 = get("SQLLM_WAVES_3", 1, kMaxWaves, waves3);
        waves4 = get("SQLLM_WAVES_4", 1, kMaxWaves, waves4);
        target_wgs = get("SQLLM_TARGET_WGS", 1, 1 << 20, target_wgs);
        force_split = get("SQLLM_SPLIT", 1, kSplitCap, 0);
    }
};

Tuning &tuning_state()
{
    static Tuning t;
    return t;
}

const Tuning &tuning() { return tuning_state(); }

bool aligned(const void *p, uintptr_t a) { return ((uintptr_t)p & (a - 1)) == 0; }

int64_t tiles_of(int64_t rows) { return (rows + kTileRows - 1) / kTileRows; }

sqllm_status check_shape(int64_t rows, int64_t cols)
{
    if (rows < 1 || cols < kGroupCols || cols % kGroupCols != 0) return SQLLM_ERR_SHAPE;
    if (rows > (int64_t)1 << 30 || cols > (int64_t)1 << 30) return SQLLM_ERR_SHAPE;
    return SQLLM_OK;
}

// Workspace layout: fp32 partial sums from the start, one arrival counter per
// row tile in the LAST 4 * tiles bytes.  Counters of calls with different
// tile counts overlap only each other (all zero between calls) and never the
// partial sums of any call the workspace is large enough for.
size_t workspace_need(int64_t rows, int batch)
{
    const int64_t tiles = tiles_of(rows);
    return (size_t)tiles * 4 + (size_t)tiles * kSplitCap * (size_t)batch * kTileRows * sizeof(float);
}

// Column split: enough workgroups to fill the chip, at least one 256-column
// group per wave.
void choose_split_dense(int64_t tiles, int64_t groups, int waves, int *split, int *gps)
{
    int64_t s = tuning().force_split;
    if (s <= 0) {
        s = (tuning().target_wgs + tiles - 1) / tiles;
        int64_t cap = groups / waves;
        if (cap < 1) cap = 1;
        if (s > cap) s = cap;
    }
    if (s > kSplitCap) s = kSplitCap;
    if (s > groups) s = groups;
    if (s < 1) s = 1;
    int64_t g = (groups + s - 1) / s;
    s = (groups + g - 1) / g; // no empty splits
    *split = (int)s;
    *gps = (int)g;
}

// Outlier-only split: about 2048 nonzeros per workgroup on average.
int choose_split_sparse(int64_t tiles, int64_t nnz)
{
    int64_t s = tuning().force_split;
    if (s <= 0) {
        const int64_t per_tile = (nnz + tiles - 1) / tiles;
        s = (per_tile + 2047) / 2048;
    }
    if (s > kSplitCap) s = kSplitCap;
    if (s < 1) s = 1;
    return (int)s;
}

sqllm_status common_checks(int64_t rows, int64_t cols, const uint16_t *x, int batch, const uint16_t *y)
{
    if (!x || !y) return SQLLM_ERR_NULL;
    sqllm_status st = check_shape(rows, cols);
    if (st != SQLLM_OK) return st;
    if (batch < 1 || batch > kMaxBatch) return SQLLM_ERR_BATCH;
    if (!aligned(x, 4) || !aligned(y, 4)) return SQLLM_ERR_ALIGN;
    return SQLLM_OK;
}

sqllm_status sparse_checks(const int32_t *row_ptr, const uint16_t *col_idx, const uint16_t *val, int64_t nnz,
                           int64_t cols)
{
    if (nnz < 0 || nnz > INT32_MAX) return SQLLM_ERR_SHAPE;
    if (nnz > 0) {
        if (!row_ptr || !col_idx || !val) return SQLLM_ERR_NULL;
        if (cols > 65536) return SQLLM_ERR_SHAPE;
        if (!aligned(row_ptr, 4) || !aligned(col_idx, 2) || !aligned(val, 2)) return SQLLM_ERR_ALIGN;
    }
    return SQLLM_OK;
}

sqllm_status workspace_checks(int split, int64_t rows, int batch, void *ws, size_t ws_bytes)
{
    if (split <= 1) return SQLLM_OK;
    if (!ws || !aligned(ws, 256) || ws_bytes % 4 != 0 || ws_bytes < workspace_need(rows, batch))
        return SQLLM_ERR_WORKSPACE;
    return SQLLM_OK;
}

void attach_workspace(KernelArgs &a, void *ws, size_t ws_bytes)
{
    a.part = (float *)ws;
    a.counters = ws ? (uint32_t *)((char *)ws + ws_bytes) - a.tiles : nullptr;
}

} // namespace

extern "C" {

const char *sqllm_status_string(sqllm_status s)
{
    switch (s) {
    case SQLLM_OK: return "SQLLM_OK";
    case SQLLM_ERR_NULL: return "SQLLM_ERR_NULL: required pointer is NULL";
    case SQLLM_ERR_BITS: return "SQLLM_ERR_BITS: bits must be 3 or 4";
    case SQLLM_ERR_SHAPE: return "SQLLM_ERR_SHAPE: rows/cols/nnz out of range";
    case SQLLM_ERR_BATCH: return "SQLLM_ERR_BATCH: batch must be in [1, 8]";
    case SQLLM_ERR_ALIGN: return "SQLLM_ERR_ALIGN: pointer not aligned as required";
    case SQLLM_ERR_CODE_RANGE: return "SQLLM_ERR_CODE_RANGE: a code is >= 2^bits";
    case SQLLM_ERR_HIP: return "SQLLM_ERR_HIP: HIP runtime or launch failure";
    case SQLLM_ERR_WORKSPACE: return "SQLLM_ERR_WORKSPACE: workspace missing, misaligned or too small";
    }
    return "SQLLM_ERR_UNKNOWN";
}

size_t sqllm_packed_bytes(int64_t rows, int64_t cols, int bits)
{
    if ((bits != 3 && bits != 4) || check_shape(rows, cols) != SQLLM_OK) return 0;
    return (size_t)(tiles_of(rows) * kTileRows * cols * bits / 8);
}

size_t sqllm_workspace_bytes(int64_t rows, int64_t cols, int batch)
{
    if (check_shape(rows, cols) != SQLLM_OK || batch < 1 || batch > kMaxBatch) return 0;
    return workspace_need(rows, batch);
}

sqllm_status sqllm_pack(const uint8_t *codes, int64_t rows, int64_t cols, int bits, void *packed, hipStream_t stream)
{
    if (!codes || !packed) return SQLLM_ERR_NULL;
    if (bits != 3 && bits != 4) return SQLLM_ERR_BITS;
    sqllm_status st = check_shape(rows, cols);
    if (st != SQLLM_OK) return st;
    if (!aligned(codes, 16) || !aligned(packed, 16)) return SQLLM_ERR_ALIGN;
    int *bad = nullptr;
    if (hipMalloc((void **)&bad, sizeof(int)) != hipSuccess) return SQLLM_ERR_HIP;
    int host_bad = 0;
    bool ok = hipMemsetAsync(bad, 0, sizeof(int), stream) == hipSuccess &&
              launch_pack(codes, (int)rows, (int)cols, bits, packed, bad, stream) == hipSuccess &&
              hipMemcpyAsync(&host_bad, bad, sizeof(int), hipMemcpyDeviceToHost, stream) == hipSuccess &&
              hipStreamSynchronize(stream) == hipSuccess;
    (void)hipFree(bad);
    if (!ok) return SQLLM_ERR_HIP;
    return host_bad ? SQLLM_ERR_CODE_RANGE : SQLLM_OK;
}

sqllm_status sqllm_gemv(const void *packed, const uint16_t *lut, int bits, int64_t rows, int64_t cols,
                        const uint16_t *x, int batch, uint16_t *y, void *workspace, size_t workspace_bytes,
                        hipStream_t stream)
{
    return sqllm_dense_sparse_gemv(packed, lut, bits, nullptr, nullptr, nullptr, 0, rows, cols, x, batch, y,
                                   workspace, workspace_bytes, stream);
}

sqllm_status sqllm_dense_sparse_gemv(const void *packed, const uint16_t *lut, int bits, const int32_t *row_ptr,
                                     const uint16_t *col_idx, const uint16_t *val, int64_t nnz, int64_t rows,
                                     int64_t cols, const uint16_t *x, int batch, uint16_t *y, void *workspace,
                                     size_t workspace_bytes, hipStream_t stream)
{
    if (!packed || !lut) return SQLLM_ERR_NULL;
    sqllm_status st = common_checks(rows, cols, x, batch, y);
    if (st != SQLLM_OK) return st;
    if (bits != 3 && bits != 4) return SQLLM_ERR_BITS;
    st = sparse_checks(row_ptr, col_idx, val, nnz, cols);
    if (st != SQLLM_OK) return st;
    if (!aligned(packed, 16) || !aligned(lut, 16)) return SQLLM_ERR_ALIGN;

    KernelArgs a{};
    a.packed = packed;
    a.lut = lut;
    a.row_ptr = row_ptr;
    a.col = col_idx;
    a.val = val;
    a.x = x;
    a.y = y;
    a.rows = (int)rows;
    a.cols = (int)cols;
    a.tiles = (int)tiles_of(rows);
    a.groups = (int)(cols / kGroupCols);
    const int waves = bits == 3 ? tuning().waves3 : tuning().waves4;
    choose_split_dense(a.tiles, a.groups, waves, &a.split, &a.gps);
    st = workspace_checks(a.split, rows, batch, workspace, workspace_bytes);
    if (st != SQLLM_OK) return st;
    attach_workspace(a, workspace, workspace_bytes);
    const bool sparse = nnz > 0;
    if (launch_dense_sparse(a, bits, batch, true, sparse, false, waves, stream) != hipSuccess) return SQLLM_ERR_HIP;
    return SQLLM_OK;
}

sqllm_status sqllm_spmv_add(const int32_t *row_ptr, const uint16_t *col_idx, const uint16_t *val, int64_t nnz,
                            int64_t rows, int64_t cols, const uint16_t *x, int batch, uint16_t *y, void *workspace,
                            size_t workspace_bytes, hipStream_t stream)
{
    sqllm_status st = common_checks(rows, cols, x, batch, y);
    if (st != SQLLM_OK) return st;
    st = sparse_checks(row_ptr, col_idx, val, nnz, cols);
    if (st != SQLLM_OK) return st;
    if (nnz == 0) return SQLLM_OK;

    KernelArgs a{};
    a.row_ptr = row_ptr;
    a.col = col_idx;
    a.val = val;
    a.x = x;
    a.y = y;
    a.rows = (int)rows;
    a.cols = (int)cols;
    a.tiles = (int)tiles_of(rows);
    a.groups = (int)(cols / kGroupCols);
    a.split = choose_split_sparse(a.tiles, nnz);
    a.gps = 0;
    st = workspace_checks(a.split, rows, batch, workspace, workspace_bytes);
    if (st != SQLLM_OK) return st;
    attach_workspace(a, workspace, workspace_bytes);
    if (launch_dense_sparse(a, 3, batch, false, true, true, tuning().waves_sparse, stream) != hipSuccess)
        return SQLLM_ERR_HIP;
    return SQLLM_OK;
}

sqllm_status sqllm_test_tuning(int waves3, int waves4, int target_wgs, int split)
{
    const Tuning dflt;
    if (waves3 > kMaxWaves || waves4 > kMaxWaves || split > kSplitCap) return SQLLM_ERR_SHAPE;
    Tuning &t = tuning_state();
    t.waves3 = waves3 > 0 ? waves3 : dflt.waves3;
    t.waves4 = waves4 > 0 ? waves4 : dflt.waves4;
    t.target_wgs = target_wgs > 0 ? target_wgs : dflt.target_wgs;
    t.force_split = split > 0 ? split : dflt.force_split;
    return SQLLM_OK;
}

sqllm_status sqllm_test_unpack(const void *packed, int64_t rows, int64_t cols, int bits, uint8_t *codes,
                               hipStream_t stream)
{
    if (!packed || !codes) return SQLLM_ERR_NULL;
    if (bits != 3 && bits != 4) return SQLLM_ERR_BITS;
    sqllm_status st = check_shape(rows, cols);
    if (st != SQLLM_OK) return st;
    if (!aligned(packed, 16) || !aligned(codes, 16)) return SQLLM_ERR_ALIGN;
    return launch_unpack(packed, nullptr, (int)rows, (int)cols, bits, codes, nullptr, stream) == hipSuccess
               ? SQLLM_OK
               : SQLLM_ERR_HIP;
}

sqllm_status sqllm_test_decode(const void *packed, const uint16_t *lut, int64_t rows, int64_t cols, int bits,
                               uint16_t *w, hipStream_t stream)
{
    if (!packed || !lut || !w) return SQLLM_ERR_NULL;
    if (bits != 3 && bits != 4) return SQLLM_ERR_BITS;
    sqllm_status st = check_shape(rows, cols);
    if (st != SQLLM_OK) return st;
    if (!aligned(packed, 16) || !aligned(w, 16) || !aligned(lut, 2)) return SQLLM_ERR_ALIGN;
    return launch_unpack(packed, lut, (int)rows, (int)cols, bits, nullptr, w, stream) == hipSuccess ? SQLLM_OK
                                                                                                    : SQLLM_ERR_HIP;
}

} // extern "C"
