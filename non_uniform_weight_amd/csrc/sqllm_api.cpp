// sqllm_api.cpp -- the C ABI declared in include/sqllm.h: argument checks
// (all done on the host before any HIP call), the choice of launch shape,
// and the kernel launches on the caller's stream.
#include "sqllm.h"

#include <stdint.h>
#include <stdlib.h>

#include <algorithm>

#include "sqllm_internal.h"

using namespace sqllm;

namespace {

// Launch-shape knobs for tests and ablations only (sqllm_test_tuning); every
// ordinary call uses the built-in defaults, and no environment variable
// changes a launch.  Every value gives the same result within the stated
// tolerance.
struct Tuning {
    int target_wgs = 256;   // workgroups the column split aims for (one per compute unit)
    int min_gps = 8;        // fewest column groups per workgroup (pair-table build amortisation)
    int force_split = 0;    // 0: choose; else workgroups per row tile
    int force_waves = 0;    // 0: choose; else waves per workgroup
    int sparse_naive = 0;   // ablation: 1 = outliers one lane per row, unbalanced
    int dot_only = 0;       // ablation: 1 = dense part in the v_dot2c form instead of the matrix cores
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

// Combine words of a call whose row tiles are split over `split`
// workgroups: split - 1 eight-byte words per (tile, batch column, row of
// tile) (none at split 1).
size_t words_need(int64_t rows, int batch, int split)
{
    return split > 1 ? (size_t)tiles_of(rows) * (size_t)(split - 1) * (size_t)batch * kTileRows * 8 : 0;
}

// The workspace one product may need: the words of the largest split, then
// (from batch kXtBatch) x transposed for the outlier gathers, always at that
// offset (a call's words, and those of a row slice, stay below it).
size_t workspace_need(int64_t rows, int64_t cols, int batch)
{
    return words_need(rows, batch, kMaxSplit) + xt_bytes(cols, batch);
}

// Outliers at batch >= kXtBatch whose x is not staged in LDS gather from a
// transposed copy in the workspace (when the workspace has room for it):
// one load per nonzero instead of one per batch column.
bool wants_xt(const KernelArgs &a, int batch, int64_t nnz) { return batch >= kXtBatch && nnz > 0 && !a.x_lds; }

int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

// Column split and waves for the dense modes: at most target_wgs workgroups
// (one per compute unit; a few more leave a tail in which some units run two
// workgroups: 11008x4096 at split 2, 344 workgroups, measured 10.8 us against
// 8.3 at split 1), one split more only when fewer than 60% of the units would
// be busy, and at least min_gps groups per workgroup.
// total_tiles: row tiles of every product sharing the launch.
void choose_split(KernelArgs &a, int64_t total_tiles)
{
    const int64_t G = a.groups;
    int64_t s = tuning().force_split;
    if (s <= 0) {
        const int64_t t = tuning().target_wgs;
        s = t / total_tiles;
        if (s < 1) s = 1;
        if (total_tiles * s * 5 < t * 3) ++s;
        int64_t cap = G / tuning().min_gps;
        if (cap < 1) cap = 1;
        if (s > cap) s = cap;
    }
    if (s > G) s = G;
    if (s > kMaxSplit) s = kMaxSplit;
    if (s < 1) s = 1;
    const int gps = (int)ceil_div(G, s);
    a.split = (int)ceil_div(G, gps); // no empty splits
    a.gps = gps;
}

// More workgroups than units: 8 waves, two workgroups per unit.  One
// workgroup per unit: 8 waves up to 16 column groups (two groups per wave,
// so that a wave's ring of loads overlaps: 8192x8192 at 16 groups per
// workgroup measured 7% faster than 16 waves of one group), 12 waves up to
// 32 groups (13824x5120 at 20 groups: 9.7 us against 10.2 at 10 waves and
// 10.6 at 16), 16 beyond.
int choose_waves(int64_t workgroups, int gps)
{
    if (tuning().force_waves) return tuning().force_waves;
    if (workgroups > tuning().target_wgs || gps <= 16) return kDefaultWaves;
    return gps <= 32 ? 12 : kMaxWaves;
}

// A group launch of more tiles than compute units but at most two per unit
// runs two 8-wave workgroups per unit, and at split 1 some units get two
// whole tiles while others get one.  Leading products then go to split 2
// while the launch stays within two workgroups per unit: their half tiles
// are dispatched first and take one slot of every unit, the whole tiles the
// other (q, k, v of 8192x8192, 384 tiles: q at split 2 gives 512
// workgroups, 19.6 us against 21.1 at split 1; splitting the last product
// instead, or (gate, up) at 688 tiles in any mix, measured slower).
// Returns the launch's workgroup count.
int64_t fill_two_slots(GroupArgs &g, int64_t wgs, void *const *own_ws, const size_t *own_bytes, int batch)
{
    const int64_t t = tuning().target_wgs;
    if (tuning().force_split || tuning().force_waves || wgs <= t || wgs >= 2 * t) return wgs;
    for (int k = 0; k < g.n; ++k)
        if (g.item[k].split != 1 || g.item[k].helpers > 0) return wgs;
    for (int k = 0; k < g.n; ++k) {
        KernelArgs &a = g.item[k];
        if (wgs + a.tiles > 2 * t || a.groups < 2 * tuning().min_gps) break;
        if (!own_ws[k] || own_bytes[k] < words_need(a.rows, batch, 2)) break;
        a.gps = (int)ceil_div(a.groups, 2);
        a.split = (int)ceil_div(a.groups, a.gps);
        wgs += (int64_t)a.tiles * (a.split - 1);
        if ((int64_t)a.tiles * a.split > g.wgs) g.wgs = a.tiles * a.split;
    }
    return wgs;
}

// The same for one product of more tiles than compute units but fewer than
// twice as many: it runs as two row slices in one group launch, the first h
// tiles at split 2 and the rest whole, h chosen so that the launch has two
// workgroups per unit (22016x8192, 344 tiles: 168 tiles at split 2 and 176
// whole, where at split 1 the 88 units that run two whole tiles end long
// after the others).  The slices share x, the outliers' arrays, the
// transposed x and the workspace (only the first slice uses its words).
// False when the launch shape is forced or the workspace lacks the words.
bool slice_for_two_slots(const KernelArgs &a, int bits, int batch, void *ws, size_t ws_bytes, GroupArgs &g)
{
    const int64_t t = tuning().target_wgs;
    if (tuning().force_split || tuning().force_waves || a.split != 1 || a.tiles <= t || a.tiles >= 2 * t) return false;
    const int h = (int)(2 * t - a.tiles);
    if (a.groups < 2 * tuning().min_gps) return false;
    if (!ws || !aligned(ws, 256) || ws_bytes < words_need((int64_t)h * kTileRows, batch, 2)) return false;
    const int64_t r0 = (int64_t)h * kTileRows;
    KernelArgs lo = a, hi = a;
    lo.rows = (int)r0;
    lo.tiles = h;
    lo.gps = (int)ceil_div(a.groups, 2);
    lo.split = (int)ceil_div(a.groups, lo.gps);
    hi.rows = a.rows - (int)r0;
    hi.tiles = a.tiles - h;
    hi.packed = (const char *)a.packed + r0 * a.cols * bits / 8; // tile-major codes: whole tiles precede
    hi.lut = a.lut + r0 * (1 << bits);
    if (a.row_ptr) hi.row_ptr = a.row_ptr + r0; // absolute offsets into col / val
    hi.y = a.y + r0;                            // ldy stays the whole product's row count
    hi.slots = nullptr;
    g = GroupArgs{};
    g.n = 2;
    g.item[0] = lo;
    g.item[1] = hi;
    g.wgs = lo.tiles * lo.split > hi.tiles ? lo.tiles * lo.split : hi.tiles;
    return true;
}

// Dense part on the matrix cores: one 4x4x4 step covers 4 columns of 4
// batch columns where the dot form spends one v_dot2c per pair and batch
// column (measured faster at every batch, 1 included).
int use_mf(int batch) { return tuning().dot_only && batch <= kMaxDotBatch ? 0 : 1; }

// Stage x in LDS for the outlier gathers when it fits beside the pair table
// (in half of the LDS when the launch has more workgroups than units, so
// that two share a unit).  The compact 3-bit table is taken (for the whole
// launch) only when some product's x fits beside it and not beside the full
// table; a launch of products that all fit, or none, keeps the full table.
// a[0..n): the launch's products (all fused when nnz > 0).
void choose_x_lds(KernelArgs *a, int n, int bits, int batch, int64_t nnz, int64_t workgroups, LaunchShape &ls)
{
    const size_t budget = workgroups > tuning().target_wgs ? kLdsBudget / 2 : kLdsBudget;
    const size_t full = static_lds_bytes(true, batch, false), compact = static_lds_bytes(true, batch, true);
    ls.compact = 0;
    for (int k = 0; k < n; ++k) {
        a[k].x_lds = 0;
        const size_t staged = staged_x_bytes(a[k].cols, batch);
        if (nnz > 0 && ls.mf && compact_allowed(bits, batch) && full + staged > budget && compact + staged <= budget)
            ls.compact = 1;
    }
    if (nnz <= 0) return;
    const size_t table = ls.compact ? compact : full;
    for (int k = 0; k < n; ++k) {
        const size_t staged = staged_x_bytes(a[k].cols, batch);
        if (table + staged <= budget) {
            a[k].x_lds = 1;
            if (staged > ls.dyn_lds) ls.dyn_lds = staged;
        }
    }
}

void choose_dense(KernelArgs &a, int bits, int batch, int64_t nnz, LaunchShape &ls)
{
    choose_split(a, a.tiles);
    ls.mf = use_mf(batch);
    ls.waves = choose_waves((int64_t)a.tiles * a.split, a.gps);
    ls.dyn_lds = 0;
    choose_x_lds(&a, 1, bits, batch, nnz, (int64_t)a.tiles * a.split, ls);
}

// Outlier-only kernel: about kSparseShare nonzeros per wave; x staged in LDS
// when it fits.
void choose_sparse(KernelArgs &a, int batch, int64_t nnz, LaunchShape &ls)
{
    const int waves = tuning().force_waves ? tuning().force_waves : kDefaultWaves;
    int64_t s = tuning().force_split;
    if (s <= 0) {
        const int64_t per_tile = ceil_div(nnz, a.tiles);
        s = ceil_div(per_tile, (int64_t)waves * kSparseShare);
    }
    if (s > kMaxSplit) s = kMaxSplit;
    if (s < 1) s = 1;
    a.split = (int)s;
    a.gps = 0;
    ls.waves = waves;
    const size_t staged = staged_x_bytes(a.cols, batch);
    a.x_lds = static_lds_bytes(false, batch, false) + staged <= (size_t)kLdsBudget;
    ls.dyn_lds = a.x_lds ? staged : 0;
}

sqllm_status common_checks(int64_t rows, int64_t cols, const uint16_t *x, int batch, const uint16_t *y)
{
    if (!x || !y) return SQLLM_ERR_NULL;
    sqllm_status st = check_shape(rows, cols);
    if (st != SQLLM_OK) return st;
    if (batch < 1 || batch > kMaxBatch) return SQLLM_ERR_BATCH;
    if (!aligned(x, 16) || !aligned(y, 4)) return SQLLM_ERR_ALIGN;
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
    if (!ws || !aligned(ws, 256) || ws_bytes < words_need(rows, batch, split)) return SQLLM_ERR_WORKSPACE;
    return SQLLM_OK;
}

// Sets a.xt when the outliers want a transposed x, the products reading
// that x carry at least kXtMinNnz nonzeros (nnz_x) and the workspace holds
// it; products with the same x share one copy.  The copy is written before
// the product launch and cleared after it, so the workspace is all zero
// again between calls (any later call may use those bytes as its words).
void plan_xt(KernelArgs &a, int batch, int64_t nnz, int64_t nnz_x, void *ws, size_t ws_bytes, XtJobs &jobs)
{
    a.xt = nullptr;
    if (!wants_xt(a, batch, nnz) || nnz_x < kXtMinNnz || !ws || !aligned(ws, 256) ||
        ws_bytes < workspace_need(a.rows, a.cols, batch))
        return;
    for (int k = 0; k < jobs.n; ++k)
        if (jobs.x[k] == a.x && jobs.cols[k] == a.cols) {
            a.xt = jobs.xt[k];
            return;
        }
    uint16_t *xt = (uint16_t *)((char *)ws + words_need(a.rows, batch, kMaxSplit));
    jobs.x[jobs.n] = a.x;
    jobs.xt[jobs.n] = xt;
    jobs.cols[jobs.n] = a.cols;
    if (a.cols > jobs.max_cols) jobs.max_cols = a.cols;
    ++jobs.n;
    a.xt = xt;
}

KernelArgs base_args(int64_t rows, int64_t cols, const uint16_t *x, uint16_t *y, void *ws)
{
    KernelArgs a{};
    a.x = x;
    a.y = y;
    a.slots = (unsigned long long *)ws;
    a.rows = (int)rows;
    a.ldy = (int)rows;
    a.cols = (int)cols;
    a.tiles = (int)tiles_of(rows);
    a.groups = (int)(cols / kGroupCols);
    a.sparse_naive = tuning().sparse_naive;
    return a;
}

// Everything the single call decides before launching: the launch shape,
// the transposed x, and the row slices of a product of 257..511 tiles.
sqllm_status plan_single(KernelArgs &a, int bits, int batch, int64_t nnz, void *ws, size_t ws_bytes, LaunchShape &ls,
                         XtJobs &jobs, GroupArgs &g, bool &sliced)
{
    choose_dense(a, bits, batch, nnz, ls);
    sqllm_status st = workspace_checks(a.split, a.rows, batch, ws, ws_bytes);
    if (st != SQLLM_OK) return st;
    plan_xt(a, batch, nnz, nnz, ws, ws_bytes, jobs);
    sliced = slice_for_two_slots(a, bits, batch, ws, ws_bytes, g);
    if (sliced) ls.waves = choose_waves((int64_t)g.item[0].tiles * g.item[0].split + g.item[1].tiles, g.item[0].gps);
    return SQLLM_OK;
}

// One launch of a group call: the products with outliers (fused) or those
// without.  g.n = 0 when there are none; which[k] is the item index of
// g.item[k].
sqllm_status plan_group_pass(const sqllm_product *items, int n, int bits, int batch, bool fused, void *workspace,
                             size_t workspace_bytes, GroupArgs &g, LaunchShape &ls, XtJobs &jobs, int *which)
{
    g = GroupArgs{};
    ls = LaunchShape{};
    jobs = XtJobs{};
    int64_t total_tiles = 0;
    for (int i = 0; i < n; ++i)
        if ((items[i].nnz > 0) == fused) total_tiles += tiles_of(items[i].rows);
    if (total_tiles == 0) return SQLLM_OK;
    size_t ws_off = 0;
    int64_t wgs = 0;
    void *own_ws[kMaxGroup];   // each product's workspace region (slots, then transposed x) or null
    size_t own_bytes[kMaxGroup];
    int64_t own_nnz[kMaxGroup];
    for (int i = 0; i < n; ++i) {
        const sqllm_product &p = items[i];
        const size_t need = workspace_need(p.rows, p.cols, batch); // every product has its own region
        if ((p.nnz > 0) != fused) {
            ws_off += need;
            continue;
        }
        void *mine = workspace ? (void *)((char *)workspace + ws_off) : nullptr;
        const size_t left = workspace && workspace_bytes > ws_off ? workspace_bytes - ws_off : 0;
        KernelArgs a = base_args(p.rows, p.cols, p.x, p.y, mine);
        ws_off += need;
        a.packed = p.packed;
        a.lut = p.lut;
        a.row_ptr = p.row_ptr;
        a.col = p.col_idx;
        a.val = p.val;
        choose_split(a, total_tiles);
        if (fused && p.plan_helpers > 0) {
            // an outlier plan: helpers first in the grid, the owners of a tile
            // at most kMaxSplit - kMaxHelpers, every tile's combine sized for
            // kMaxSplit partial sums
            if (a.split > kMaxSplit - kMaxHelpers) {
                a.gps = (int)ceil_div(a.groups, kMaxSplit - kMaxHelpers);
                a.split = (int)ceil_div(a.groups, a.gps);
            }
            a.plan = p.plan;
            a.helpers = (int)p.plan_helpers;
            if (!workspace || left < words_need(p.rows, batch, kMaxSplit)) return SQLLM_ERR_WORKSPACE;
        }
        if (a.split > 1 && (!workspace || left < words_need(p.rows, batch, a.split))) return SQLLM_ERR_WORKSPACE;
        own_ws[g.n] = mine;
        own_bytes[g.n] = left < need ? left : need;
        own_nnz[g.n] = p.nnz;
        which[g.n] = i;
        g.item[g.n] = a;
        const int64_t mine_wgs = (int64_t)a.tiles * a.split + a.helpers;
        if (mine_wgs > g.wgs) g.wgs = (int)mine_wgs;
        wgs += mine_wgs;
        ++g.n;
    }
    if (wgs > INT32_MAX) return SQLLM_ERR_SHAPE;
    wgs = fill_two_slots(g, wgs, own_ws, own_bytes, batch);
    ls.mf = use_mf(batch);
    int max_gps = 1;
    for (int k = 0; k < g.n; ++k)
        if (g.item[k].gps > max_gps) max_gps = g.item[k].gps;
    ls.waves = choose_waves(wgs, max_gps);
    // products that share x (as q, k and v do) share one transposed copy
    choose_x_lds(g.item, g.n, bits, batch, fused ? 1 : 0, wgs, ls);
    for (int k = 0; k < g.n; ++k) {
        int64_t nnz_x = 0; // nonzeros of this launch's products that gather from the same x
        for (int j = 0; j < g.n; ++j)
            if (g.item[j].x == g.item[k].x && g.item[j].cols == g.item[k].cols && !g.item[j].x_lds)
                nnz_x += own_nnz[j];
        plan_xt(g.item[k], batch, fused ? 1 : 0, nnz_x, own_ws[k], own_bytes[k], jobs);
    }
    return SQLLM_OK;
}

} // namespace

extern "C" {

const char *sqllm_status_string(sqllm_status s)
{
    switch (s) {
    case SQLLM_OK: return "SQLLM_OK";
    case SQLLM_ERR_NULL: return "SQLLM_ERR_NULL: required pointer is NULL";
    case SQLLM_ERR_BITS: return "SQLLM_ERR_BITS: bits must be 2, 3 or 4";
    case SQLLM_ERR_SHAPE: return "SQLLM_ERR_SHAPE: rows/cols/nnz out of range";
    case SQLLM_ERR_BATCH: return "SQLLM_ERR_BATCH: batch must be in [1, 16]";
    case SQLLM_ERR_ALIGN: return "SQLLM_ERR_ALIGN: pointer not aligned as required";
    case SQLLM_ERR_CODE_RANGE: return "SQLLM_ERR_CODE_RANGE: a code is >= 2^bits";
    case SQLLM_ERR_HIP: return "SQLLM_ERR_HIP: HIP runtime or launch failure";
    case SQLLM_ERR_WORKSPACE: return "SQLLM_ERR_WORKSPACE: workspace missing, misaligned or too small";
    case SQLLM_ERR_CAPACITY: return "SQLLM_ERR_CAPACITY: more outliers than the CSR buffers hold";
    case SQLLM_ERR_SCRATCH: return "SQLLM_ERR_SCRATCH: the launch needs more than the fixed 16 MiB scratch";
    }
    return "SQLLM_ERR_UNKNOWN";
}

size_t sqllm_packed_bytes(int64_t rows, int64_t cols, int bits)
{
    if ((bits < 2 || bits > 4) || check_shape(rows, cols) != SQLLM_OK) return 0;
    return (size_t)(tiles_of(rows) * kTileRows * cols * bits / 8);
}

size_t sqllm_workspace_bytes(int64_t rows, int64_t cols, int batch)
{
    if (check_shape(rows, cols) != SQLLM_OK || batch < 1 || batch > kMaxBatch) return 0;
    return workspace_need(rows, cols, batch);
}

sqllm_status sqllm_pack(const uint8_t *codes, int64_t rows, int64_t cols, int bits, void *packed, void *workspace,
                        size_t workspace_bytes, hipStream_t stream)
{
    if (!codes || !packed || !workspace) return SQLLM_ERR_NULL;
    if (bits < 2 || bits > 4) return SQLLM_ERR_BITS;
    sqllm_status st = check_shape(rows, cols);
    if (st != SQLLM_OK) return st;
    if (!aligned(codes, 16) || !aligned(packed, 16)) return SQLLM_ERR_ALIGN;
    if (!aligned(workspace, 4) || workspace_bytes < 4) return SQLLM_ERR_WORKSPACE;
    int *bad = (int *)workspace; // the caller's: the library allocates nothing
    int host_bad = 0;
    const bool ok = hipMemsetAsync(bad, 0, sizeof(int), stream) == hipSuccess &&
                    launch_pack(codes, (int)rows, (int)cols, bits, packed, bad, stream) == hipSuccess &&
                    hipMemcpyAsync(&host_bad, bad, sizeof(int), hipMemcpyDeviceToHost, stream) == hipSuccess &&
                    hipStreamSynchronize(stream) == hipSuccess;
    if (!ok) return SQLLM_ERR_HIP;
    if (host_bad) { // leave the caller's word zero again (it may be a hot-call workspace)
        if (hipMemsetAsync(bad, 0, sizeof(int), stream) != hipSuccess || hipStreamSynchronize(stream) != hipSuccess)
            return SQLLM_ERR_HIP;
        return SQLLM_ERR_CODE_RANGE;
    }
    return SQLLM_OK;
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
    if (bits < 2 || bits > 4) return SQLLM_ERR_BITS;
    st = sparse_checks(row_ptr, col_idx, val, nnz, cols);
    if (st != SQLLM_OK) return st;
    if (!aligned(packed, 16) || !aligned(lut, 16)) return SQLLM_ERR_ALIGN;

    KernelArgs a = base_args(rows, cols, x, y, workspace);
    a.packed = packed;
    a.lut = lut;
    a.row_ptr = row_ptr;
    a.col = col_idx;
    a.val = val;
    LaunchShape ls{};
    XtJobs jobs{};
    GroupArgs g;
    bool sliced = false;
    st = plan_single(a, bits, batch, nnz, workspace, workspace_bytes, ls, jobs, g, sliced);
    if (st != SQLLM_OK) return st;
    const Mode mode = nnz > 0 ? kFused : kDenseOnly;
    if (launch_xt_write(jobs, batch, stream) != hipSuccess ||
        (sliced ? launch_dense_sparse_group(g, bits, batch, mode, ls, stream)
                : launch_dense_sparse(a, bits, batch, mode, ls, stream)) != hipSuccess ||
        launch_xt_clear(jobs, batch, stream) != hipSuccess)
        return SQLLM_ERR_HIP;
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

    KernelArgs a = base_args(rows, cols, x, y, workspace);
    a.row_ptr = row_ptr;
    a.col = col_idx;
    a.val = val;
    LaunchShape ls{};
    choose_sparse(a, batch, nnz, ls);
    st = workspace_checks(a.split, rows, batch, workspace, workspace_bytes);
    if (st != SQLLM_OK) return st;
    XtJobs jobs{};
    plan_xt(a, batch, nnz, nnz, workspace, workspace_bytes, jobs);
    if (launch_xt_write(jobs, batch, stream) != hipSuccess ||
        launch_dense_sparse(a, 3, batch, kSparseAdd, ls, stream) != hipSuccess ||
        launch_xt_clear(jobs, batch, stream) != hipSuccess)
        return SQLLM_ERR_HIP;
    return SQLLM_OK;
}

size_t sqllm_group_workspace_bytes(const sqllm_product *items, int n, int batch)
{
    if (!items || n < 1 || n > kMaxGroup || batch < 1 || batch > kMaxBatch) return 0;
    size_t total = 0;
    for (int i = 0; i < n; ++i) {
        if (check_shape(items[i].rows, items[i].cols) != SQLLM_OK) return 0;
        total += workspace_need(items[i].rows, items[i].cols, batch);
    }
    return total;
}

sqllm_status sqllm_test_stream_read(const void *src, size_t bytes, uint32_t *sink, hipStream_t stream)
{
    if (!src || !sink) return SQLLM_ERR_NULL;
    if (bytes == 0 || bytes % 1024 != 0) return SQLLM_ERR_SHAPE;
    if (!aligned(src, 16) || !aligned(sink, 4)) return SQLLM_ERR_ALIGN;
    return launch_stream_read(src, bytes, sink, stream) == hipSuccess ? SQLLM_OK : SQLLM_ERR_HIP;
}

size_t sqllm_outlier_plan_len(int64_t rows)
{
    if (rows < 1 || rows > (int64_t)1 << 30) return 0;
    const int64_t tiles = tiles_of(rows);
    return (size_t)(1 + tiles + kMaxHelpers * tiles);
}

size_t sqllm_outlier_plan(const int32_t *row_ptr, int64_t rows, int32_t *plan, size_t plan_len)
{
    const size_t cap = sqllm_outlier_plan_len(rows);
    if (!row_ptr || !plan || cap == 0 || plan_len < cap || row_ptr[0] != 0) return 0;
    for (int64_t r = 0; r < rows; ++r)
        if (row_ptr[r + 1] < row_ptr[r]) return 0;
    const int64_t tiles = tiles_of(rows);
    const int64_t nnz = row_ptr[rows];
    // q: twice the average tile's nonzeros; a tile above it gets a helper per
    // further q (so that no workgroup's share exceeds about q), at most 8
    const int64_t q = 2 * ceil_div(nnz, tiles);
    int64_t h = 0;
    for (int64_t t = 0; t < tiles; ++t) {
        const int64_t n_t = row_ptr[std::min((t + 1) * kTileRows, rows)] - row_ptr[t * kTileRows];
        int64_t e = (q > 0 && n_t > q) ? ceil_div(n_t, q) - 1 : 0;
        if (e > kMaxHelpers) e = kMaxHelpers;
        plan[1 + t] = (int32_t)e;
        h += e;
    }
    plan[0] = (int32_t)h;
    int64_t k = 1 + tiles;
    for (int64_t t = 0; t < tiles; ++t)
        for (int32_t e = 0; e < plan[1 + t]; ++e) plan[k++] = (int32_t)((t << 4) | e);
    return (size_t)k;
}

sqllm_status sqllm_dense_sparse_gemv_group(const sqllm_product *items, int n, int bits, int batch, void *workspace,
                                           size_t workspace_bytes, hipStream_t stream)
{
    if (!items) return SQLLM_ERR_NULL;
    if (n < 1 || n > kMaxGroup) return SQLLM_ERR_SHAPE;
    if (bits < 2 || bits > 4) return SQLLM_ERR_BITS;
    if (batch < 1 || batch > kMaxBatch) return SQLLM_ERR_BATCH;
    // every product's arguments first, as for the single call
    for (int i = 0; i < n; ++i) {
        const sqllm_product &p = items[i];
        if (!p.packed || !p.lut) return SQLLM_ERR_NULL;
        sqllm_status st = common_checks(p.rows, p.cols, p.x, batch, p.y);
        if (st != SQLLM_OK) return st;
        st = sparse_checks(p.row_ptr, p.col_idx, p.val, p.nnz, p.cols);
        if (st != SQLLM_OK) return st;
        if (!aligned(p.packed, 16) || !aligned(p.lut, 16)) return SQLLM_ERR_ALIGN;
        if (p.plan_helpers < 0 || p.plan_helpers > (int64_t)kMaxHelpers * tiles_of(p.rows)) return SQLLM_ERR_SHAPE;
        if (p.plan_helpers > 0 && !p.plan) return SQLLM_ERR_NULL;
        if (p.plan_helpers > 0 && !aligned(p.plan, 4)) return SQLLM_ERR_ALIGN;
    }
    if (workspace && !aligned(workspace, 256)) return SQLLM_ERR_WORKSPACE;
    // products with outliers run in one launch, those without in another
    for (int pass = 0; pass < 2; ++pass) {
        const bool fused = pass == 0;
        GroupArgs g;
        LaunchShape ls;
        XtJobs jobs;
        int which[kMaxGroup];
        sqllm_status st = plan_group_pass(items, n, bits, batch, fused, workspace, workspace_bytes, g, ls, jobs, which);
        if (st != SQLLM_OK) return st;
        if (g.n == 0) continue;
        // one product: the single-product kernel (its arguments come without
        // the table lookup, measured 0.2-0.4 us faster per launch)
        const Mode mode = fused ? kFused : kDenseOnly;
        if (launch_xt_write(jobs, batch, stream) != hipSuccess ||
            (g.n == 1 ? launch_dense_sparse(g.item[0], bits, batch, mode, ls, stream)
                      : launch_dense_sparse_group(g, bits, batch, mode, ls, stream)) != hipSuccess ||
            launch_xt_clear(jobs, batch, stream) != hipSuccess)
            return SQLLM_ERR_HIP;
    }
    return SQLLM_OK;
}

// ---- offline split and k-means

namespace {
constexpr size_t kBinsBytes = 65536 * 4;
constexpr size_t kMiscBytes = 256; // rank selection (64 B), total, overflow flag

sqllm_status quantize_shape(const void *w, int64_t rows, int64_t cols)
{
    if (!w) return SQLLM_ERR_NULL;
    if (rows < 1 || cols < 1 || cols > 65536 || rows > INT32_MAX / cols) return SQLLM_ERR_SHAPE;
    if (!aligned(w, 2)) return SQLLM_ERR_ALIGN;
    return SQLLM_OK;
}
} // namespace

size_t sqllm_quantize_workspace_bytes(int64_t rows, int64_t cols)
{
    if (rows < 1 || cols < 1 || cols > 65536 || rows > INT32_MAX / cols) return 0;
    return kBinsBytes + kMiscBytes + (size_t)rows * 4;
}

namespace {
// IEEE total order key back to the bit pattern (binary16 / binary32).
uint16_t f16_from_key(uint32_t k) { return (uint16_t)((k & 0x8000u) ? (k & 0x7FFFu) : (~k & 0xFFFFu)); }
uint32_t f32_from_key(uint32_t k) { return (k & 0x80000000u) ? (k & 0x7FFFFFFFu) : ~k; }

int64_t rank_of(int64_t n, int ppm) // floor(n * ppm / 1e6) without overflow
{
    return (n / 1000000) * ppm + ((n % 1000000) * ppm) / 1000000;
}
} // namespace

sqllm_status sqllm_outlier_thresholds(const uint16_t *w, const float *sens, int64_t rows, int64_t cols, int tail_ppm,
                                      int top_ppm, void *workspace, size_t workspace_bytes, uint16_t *t_min,
                                      uint16_t *t_max, float *t_s, int64_t *nnz, hipStream_t stream)
{
    sqllm_status st = quantize_shape(w, rows, cols);
    if (st != SQLLM_OK) return st;
    if (!t_min || !t_max || !nnz || (sens && !t_s)) return SQLLM_ERR_NULL;
    if (tail_ppm < 0 || tail_ppm >= 500000) return SQLLM_ERR_SHAPE;
    if (sens && (top_ppm < 0 || top_ppm >= 1000000)) return SQLLM_ERR_SHAPE;
    if (sens && !aligned(sens, 4)) return SQLLM_ERR_ALIGN;
    if (!workspace || !aligned(workspace, 256) || workspace_bytes < sqllm_quantize_workspace_bytes(rows, cols))
        return SQLLM_ERR_WORKSPACE;
    const int64_t n = rows * cols;
    const int64_t tail = rank_of(n, tail_ppm);
    uint32_t *bins = (uint32_t *)workspace;
    SelectOut *sel = (SelectOut *)((char *)workspace + kBinsBytes);
    unsigned long long *total = (unsigned long long *)((char *)workspace + kBinsBytes + 64);
    int32_t *counts = (int32_t *)((char *)workspace + kBinsBytes + kMiscBytes);
    SelectOut hw{}, hs{};
    if (launch_rank_select(w, false, n, tail, n - 1 - tail, bins, sel, stream) != hipSuccess ||
        hipMemcpyAsync(&hw, sel, sizeof(hw), hipMemcpyDeviceToHost, stream) != hipSuccess)
        return SQLLM_ERR_HIP;
    if (sens) {
        const int64_t r = n - 1 - rank_of(n, top_ppm); // one rank: the fp32 passes select a single value
        if (launch_rank_select(sens, true, n, r, r, bins, sel, stream) != hipSuccess ||
            hipMemcpyAsync(&hs, sel, sizeof(hs), hipMemcpyDeviceToHost, stream) != hipSuccess)
            return SQLLM_ERR_HIP;
    }
    if (hipStreamSynchronize(stream) != hipSuccess) return SQLLM_ERR_HIP;
    const uint16_t lo = f16_from_key(hw.bin[0]), hi = f16_from_key(hw.bin[1]);
    float ts = __builtin_inff();
    if (sens) {
        const uint32_t bits = f32_from_key((hs.bin[0] << 16) | hs.bin2[0]);
        __builtin_memcpy(&ts, &bits, 4);
    }
    unsigned long long ht = 0;
    if (hipMemsetAsync(total, 0, sizeof(*total), stream) != hipSuccess ||
        launch_outlier_count(w, sens, (int)rows, (int)cols, lo, hi, ts, counts, total, stream) != hipSuccess ||
        hipMemcpyAsync(&ht, total, sizeof(ht), hipMemcpyDeviceToHost, stream) != hipSuccess ||
        hipStreamSynchronize(stream) != hipSuccess)
        return SQLLM_ERR_HIP;
    *t_min = lo;
    *t_max = hi;
    if (t_s) *t_s = ts;
    *nnz = (int64_t)ht;
    return SQLLM_OK;
}

sqllm_status sqllm_outlier_extract(const uint16_t *w, const float *sens, int64_t rows, int64_t cols, uint16_t t_min,
                                   uint16_t t_max, float t_s, int32_t *row_ptr, uint16_t *col_idx, uint16_t *val,
                                   int64_t nnz_capacity, uint16_t *dense, float *sens_dense, void *workspace,
                                   size_t workspace_bytes, hipStream_t stream)
{
    sqllm_status st = quantize_shape(w, rows, cols);
    if (st != SQLLM_OK) return st;
    if (!row_ptr || !dense || (nnz_capacity > 0 && (!col_idx || !val)) || (sens_dense && !sens))
        return SQLLM_ERR_NULL;
    if (nnz_capacity < 0) return SQLLM_ERR_SHAPE;
    if (!aligned(row_ptr, 4) || !aligned(dense, 2) || (sens && !aligned(sens, 4)) ||
        (sens_dense && !aligned(sens_dense, 4)))
        return SQLLM_ERR_ALIGN;
    if (!workspace || !aligned(workspace, 256) || workspace_bytes < sqllm_quantize_workspace_bytes(rows, cols))
        return SQLLM_ERR_WORKSPACE;
    int *overflow = (int *)((char *)workspace + kBinsBytes + 128);
    int32_t *counts = (int32_t *)((char *)workspace + kBinsBytes + kMiscBytes);
    int hov = 0;
    if (hipMemsetAsync(overflow, 0, sizeof(int), stream) != hipSuccess ||
        launch_outlier_extract(w, sens, (int)rows, (int)cols, t_min, t_max, t_s, counts, row_ptr, col_idx, val,
                               nnz_capacity, dense, sens_dense, overflow, stream) != hipSuccess ||
        hipMemcpyAsync(&hov, overflow, sizeof(int), hipMemcpyDeviceToHost, stream) != hipSuccess ||
        hipStreamSynchronize(stream) != hipSuccess)
        return SQLLM_ERR_HIP;
    return hov ? SQLLM_ERR_CAPACITY : SQLLM_OK;
}

sqllm_status sqllm_kmeans_lut(const uint16_t *dense, const float *sens, int64_t rows, int64_t cols, int bits, int iters,
                              uint8_t *codes, uint16_t *lut, hipStream_t stream)
{
    sqllm_status st = quantize_shape(dense, rows, cols);
    if (st != SQLLM_OK) return st;
    if (!codes || !lut) return SQLLM_ERR_NULL;
    if (bits < 2 || bits > 4) return SQLLM_ERR_BITS;
    if (iters < 0 || iters > 1000) return SQLLM_ERR_SHAPE;
    if (!aligned(lut, 2) || (sens && !aligned(sens, 4))) return SQLLM_ERR_ALIGN;
    if (launch_kmeans(dense, sens, (int)rows, (int)cols, bits, iters, codes, lut, stream) != hipSuccess)
        return SQLLM_ERR_HIP;
    return SQLLM_OK;
}

sqllm_status sqllm_test_tuning(int target_wgs, int min_gps, int split, int waves, int sparse_naive, int dot_only)
{
    const Tuning dflt;
    if (split > kMaxSplit || waves > kMaxWaves || sparse_naive < 0 || sparse_naive > 1 || dot_only < 0 ||
        dot_only > 1)
        return SQLLM_ERR_SHAPE;
    Tuning &t = tuning_state();
    t.target_wgs = target_wgs > 0 ? target_wgs : dflt.target_wgs;
    t.min_gps = min_gps > 0 ? min_gps : dflt.min_gps;
    t.force_split = split > 0 ? split : dflt.force_split;
    t.force_waves = waves > 0 ? waves : dflt.force_waves;
    t.sparse_naive = sparse_naive;
    t.dot_only = dot_only;
    return SQLLM_OK;
}

sqllm_status sqllm_test_launch_plan(int mode, int n, const int64_t *rows, const int64_t *cols, const int64_t *nnz,
                                    int batch, size_t workspace_bytes, int *plan)
{
    if (!rows || !cols || !nnz || !plan) return SQLLM_ERR_NULL;
    if (mode < 0 || mode > 2 || n < 1 || n > kMaxGroup || (mode == 0 && n != 1)) return SQLLM_ERR_SHAPE;
    if (batch < 1 || batch > kMaxBatch) return SQLLM_ERR_BATCH;
    for (int i = 0; i < n; ++i) {
        const sqllm_status st = check_shape(rows[i], cols[i]);
        if (st != SQLLM_OK) return st;
        if (nnz[i] < 0 || nnz[i] >= ((int64_t)1 << 31)) return SQLLM_ERR_SHAPE;
        if (mode == 2 && cols[i] != cols[0]) return SQLLM_ERR_SHAPE;
    }
    // stand-ins for device addresses: aligned, distinct, never dereferenced (nothing is launched)
    const uintptr_t base = (uintptr_t)1 << 40, stride = (uintptr_t)1 << 36;
    auto fake = [&](int i, int k) { return (void *)(base + (uintptr_t)(i * 8 + k) * stride); };
    void *ws = workspace_bytes ? (void *)(base / 2) : nullptr;
    if (mode == 0) {
        KernelArgs a = base_args(rows[0], cols[0], (const uint16_t *)fake(0, 0), (uint16_t *)fake(0, 1), ws);
        a.packed = fake(0, 2);
        a.lut = (const uint16_t *)fake(0, 3);
        if (nnz[0] > 0) {
            a.row_ptr = (const int32_t *)fake(0, 4);
            a.col = (const uint16_t *)fake(0, 5);
            a.val = (const uint16_t *)fake(0, 6);
        }
        LaunchShape ls{};
        XtJobs jobs{};
        GroupArgs g;
        bool sliced = false;
        const sqllm_status st = plan_single(a, 3, batch, nnz[0], ws, workspace_bytes, ls, jobs, g, sliced);
        if (st != SQLLM_OK) return st;
        plan[0] = sliced ? g.item[0].split : a.split;
        plan[1] = sliced ? g.item[0].gps : a.gps;
        plan[2] = ls.waves;
        plan[3] = a.xt ? 1 : (a.x_lds ? 2 : 0);
        plan[4] = sliced ? g.item[0].tiles : 0;
        plan[5] = ls.mf | (ls.compact << 1);
        return SQLLM_OK;
    }
    sqllm_product items[kMaxGroup] = {}; // no outlier plans
    for (int i = 0; i < n; ++i) {
        sqllm_product &p = items[i];
        p.packed = fake(i, 2);
        p.lut = (const uint16_t *)fake(i, 3);
        p.row_ptr = nnz[i] > 0 ? (const int32_t *)fake(i, 4) : nullptr;
        p.col_idx = nnz[i] > 0 ? (const uint16_t *)fake(i, 5) : nullptr;
        p.val = nnz[i] > 0 ? (const uint16_t *)fake(i, 6) : nullptr;
        p.nnz = nnz[i];
        p.rows = rows[i];
        p.cols = cols[i];
        p.x = (const uint16_t *)fake(mode == 2 ? 0 : i, 0);
        p.y = (uint16_t *)fake(i, 1);
    }
    int mf = use_mf(batch), compact = 0;
    for (int pass = 0; pass < 2; ++pass) {
        GroupArgs g;
        LaunchShape ls;
        XtJobs jobs;
        int which[kMaxGroup];
        const sqllm_status st = plan_group_pass(items, n, 3, batch, pass == 0, ws, workspace_bytes, g, ls, jobs, which);
        if (st != SQLLM_OK) return st;
        for (int k = 0; k < g.n; ++k) {
            int *q = plan + 5 * which[k];
            q[0] = g.item[k].split;
            q[1] = g.item[k].gps;
            q[2] = ls.waves;
            q[3] = g.item[k].xt ? 1 : (g.item[k].x_lds ? 2 : 0);
            q[4] = 0;
        }
        if (g.n) mf = ls.mf;
        if (g.n && ls.compact) compact = 1;
    }
    plan[5 * n] = mf | (compact << 1);
    return SQLLM_OK;
}

sqllm_status sqllm_test_unpack(const void *packed, int64_t rows, int64_t cols, int bits, uint8_t *codes,
                               hipStream_t stream)
{
    if (!packed || !codes) return SQLLM_ERR_NULL;
    if (bits < 2 || bits > 4) return SQLLM_ERR_BITS;
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
    if (bits < 2 || bits > 4) return SQLLM_ERR_BITS;
    sqllm_status st = check_shape(rows, cols);
    if (st != SQLLM_OK) return st;
    if (!aligned(packed, 16) || !aligned(w, 16) || !aligned(lut, 2)) return SQLLM_ERR_ALIGN;
    return launch_unpack(packed, lut, (int)rows, (int)cols, bits, nullptr, w, stream) == hipSuccess ? SQLLM_OK
                                                                                                    : SQLLM_ERR_HIP;
}

} // extern "C"
