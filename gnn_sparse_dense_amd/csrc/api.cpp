// C ABI of the CSR SpMM library: plan construction (validation, descriptors,
// narrowing, row split), the rule router and the per-call launches.
#include <algorithm>
#include <chrono>
#include <climits>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <new>
#include <vector>

#include "alloc.h"
#include "plan.h"

#define SPMM_API extern "C" __attribute__((visibility("default")))

namespace gspmm {
int64_t colscan_blocks(int64_t nnz);
}

using namespace gspmm;

namespace {

thread_local int t_status = SPMM_OK;
thread_local char t_msg[512] = "";

int fail(int status, const char *fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(t_msg, sizeof(t_msg), fmt, ap);
    va_end(ap);
    t_status = status;
    return status;
}

int succeed() {
    t_status = SPMM_OK;
    t_msg[0] = '\0';
    return SPMM_OK;
}

int fail_oom(const char *context);

int fail_hip(hipError_t e, const char *what) {
    (void)hipGetLastError();
    if (e == hipErrorOutOfMemory) return fail_oom(what);
    return fail(SPMM_E_HIP, "%s: %s", what, hipGetErrorString(e));
}

bool is_device_ptr(const void *p) {
    if (p == nullptr) return false;
    hipPointerAttribute_t attr;
    std::memset(&attr, 0, sizeof(attr));
    const hipError_t e = hipPointerGetAttributes(&attr, p);
    if (e != hipSuccess) {
        (void)hipGetLastError();
        return false;
    }
    return attr.type == hipMemoryTypeDevice || attr.type == hipMemoryTypeManaged;
}

// A failed device allocation as a status: OOM names the buffer and, when the
// memory limit refused it, the limit.
int fail_oom(const char *context) {
    const OomInfo o = last_oom();
    if (o.simulated)
        return fail(SPMM_E_OOM, "%s: device allocation of %s (%lld bytes) exceeds the memory limit of %lld bytes",
                    context, o.what, (long long)o.bytes, (long long)o.limit);
    return fail(SPMM_E_OOM, "%s: device allocation of %s (%lld bytes) failed", context, o.what, (long long)o.bytes);
}

template <typename T>
int dev_alloc(T **p, int64_t count, const char *what) {
    *p = nullptr;
    if (count <= 0) return SPMM_OK;
    if (dmalloc(p, (size_t)count * sizeof(T), what) != hipSuccess) return fail_oom("out of device memory");
    return SPMM_OK;
}

template <typename T>
void dev_free(T *&p) {
    dfree(p);
    p = nullptr;
}

void free_split(spmm_plan *p) {
    dev_free(p->heavy_rows);
    dev_free(p->seg_first);
    dev_free(p->seg_begin);
    dev_free(p->seg_end);
    dev_free(p->partial);
    dev_free(p->part_arg);
    dev_free(p->seg_order);
    p->split = false;
    p->n_heavy = p->n_seg = 0;
    p->n_light = p->M;
}

void free_tiles(spmm_plan *p) {
    dev_free(p->tiles);
    p->tile_cap = p->tile_words = 0;
}

void free_mfma(spmm_plan *p) {
    dev_free(p->mfma_tiles);
    dev_free(p->mfma_tiles_lo);
    dev_free(p->mfma_tile_exp);
    dev_free(p->mfma_rowptr);
    dev_free(p->mfma_col);
    dev_free(p->mfma_val);
    p->mfma_rnnz = 0;
}

void free_pairs(spmm_plan *p) {
    dev_free(p->pair_prow);
    dev_free(p->pair_col);
    dev_free(p->pair_val);
    p->pair_nvec = 0;
    p->pair_unsorted = false;
}

void free_merge(spmm_plan *p) {
    dev_free(p->merge_seg_row);
    dev_free(p->merge_seg_entry);
    dev_free(p->merge_carry_row);
    dev_free(p->merge_carry_arg);
    dev_free(p->merge_carry);
    p->merge_nseg = 0;
}

void free_window_runs(spmm_plan *p) {
    dev_free(p->win_lo);
    dev_free(p->win_in);
}

// Per-row run lengths (entries below / inside the row's window) for the
// sorted-row window kernel; only for plans whose rows are all sorted.
int build_window_runs(spmm_plan *p) {
    if (!p->rows_sorted || p->win_lo || p->M == 0) return SPMM_OK;
    int st;
    if ((st = dev_alloc(&p->win_lo, p->M, "window runs")) || (st = dev_alloc(&p->win_in, p->M, "window runs"))) {
        free_window_runs(p);
        return st;
    }
    hipError_t e = launch_window_runs(p->rowptr, p->col, p->M, p->win_lo, p->win_in, nullptr);
    if (e == hipSuccess) e = hipDeviceSynchronize();
    if (e != hipSuccess) {
        free_window_runs(p);
        return fail_hip(e, "window runs");
    }
    return SPMM_OK;
}

void free_plan(spmm_plan *p) {
    if (!p) return;
    free_window_runs(p);
    free_merge(p);
    free_split(p);
    free_tiles(p);
    free_mfma(p);
    free_pairs(p);
    dev_free(p->rowptr);
    dev_free(p->col);
    dev_free(p->val);
    delete p;
}

// Every device buffer a plan may own (null when not built).
std::vector<const void *> plan_buffers(const spmm_plan *p) {
    return {p->rowptr, p->col, p->val, p->heavy_rows, p->seg_first, p->seg_begin, p->seg_end, p->seg_order,
            p->partial, p->part_arg, p->tiles, p->win_lo, p->win_in, p->mfma_tiles, p->mfma_tiles_lo,
            p->mfma_tile_exp, p->mfma_rowptr, p->mfma_col, p->mfma_val, p->pair_prow, p->pair_col, p->pair_val,
            p->merge_seg_row, p->merge_seg_entry, p->merge_carry_row, p->merge_carry_arg, p->merge_carry};
}

// Device bytes a plan holds.
int64_t plan_bytes(const spmm_plan *p) {
    int64_t b = 0;
    for (const void *q : plan_buffers(p)) b += dbytes(q);
    return b;
}

// Budget of one call on plan p (or on no plan).
struct PlanScope {
    CallScope scope;
    explicit PlanScope(const spmm_plan *p) : scope(p ? plan_bytes(p) : 0, p ? p->mem_limit : 0) {}
};

// Bumps the plan's generation when a call changed the set of its device
// buffers: kernels captured before then hold addresses that may be freed.
struct GenerationGuard {
    spmm_plan *p;
    std::vector<const void *> before;
    explicit GenerationGuard(spmm_plan *plan) : p(plan), before(plan_buffers(plan)) {}
    ~GenerationGuard() {
        if (plan_buffers(p) != before) ++p->generation;
    }
};

// Restores the caller's current device on scope exit.
struct DeviceGuard {
    int prev = -1;
    explicit DeviceGuard(int dev) {
        if (hipGetDevice(&prev) == hipSuccess && prev != dev) (void)hipSetDevice(dev);
        else prev = -1;
    }
    ~DeviceGuard() {
        if (prev >= 0) (void)hipSetDevice(prev);
    }
};

// Default split parameters.  ParamSpMM's split granularity SG (section 5.1,
// eq. 3) is the mean non-empty row length rounded up to a multiple of the
// wave width; with wave64 and GNN-typical degrees that is 64.  Threshold T =
// max(2 SG, 128): rows a few times longer than the mean leave the light-row
// waves, where they hold up the other rows of their wave.  Piece length L =
// max(SG, 512): pieces stay long enough that the partial rows are a small
// share of the traffic.  (Power-law: T = L = 512 3.84 ms, T = 128 / L = 512
// 3.77 ms, with the pieces in first-column order.)  The split itself is
// switched on only for graphs with hubs, rows longer than H = max(SG, 512)
// (and a degree CV above 1): a low-degree graph with a few rows of a hundred
// or so entries keeps its row tiles, which the split would turn off.
//
// Rows of more than kMaxWholeRow entries are split in every mode, and no
// piece is longer: a wave then walks at most 64 x 2^24 entries, so its 32-bit
// entry counters never come near 2^31 (and no single wave is left with a row
// of hundreds of millions of entries).
constexpr int64_t kMaxWholeRow = int64_t(1) << 24;

void auto_split_params(const spmm_plan *p, int64_t *T, int64_t *L, int64_t *H) {
    const int64_t nonempty = p->M - p->n_empty;
    const double dhat = nonempty > 0 ? (double)p->nnz / (double)nonempty : 0.0;
    const int64_t sg = (int64_t)std::ceil(dhat / 64.0) * 64;
    *T = std::min(p->opt_T >= 0 ? p->opt_T : std::max<int64_t>(2 * sg, 128), kMaxWholeRow);
    *L = std::min(p->opt_L > 0 ? p->opt_L : std::max<int64_t>(sg, 512), kMaxWholeRow);
    *H = p->opt_T >= 0 ? p->opt_T : std::max<int64_t>(sg, 512);
}

int build_split(spmm_plan *p) {
    free_split(p);
    int64_t T, L, H;
    auto_split_params(p, &T, &L, &H);
    const bool chosen =
        p->opt_split == 1 || (p->opt_split == -1 && p->dmax > H && p->cv_deg > 1.0);
    const bool enabled = chosen || p->dmax > kMaxWholeRow;
    if (enabled && !chosen) T = kMaxWholeRow;      // only the over-long rows
    p->T = T;
    p->L = L;
    if (!enabled || p->M == 0) return SPMM_OK;

    const int64_t nblocks = (p->M + kRowsPerScanBlock - 1) / kRowsPerScanBlock;
    PartCount *d_counts = nullptr;
    int st = dev_alloc(&d_counts, nblocks, "split counts");
    if (st) return st;
    hipError_t e = launch_part_count(p->rowptr, p->M, T, L, d_counts, nblocks, nullptr);
    std::vector<PartCount> counts((size_t)nblocks);
    if (e == hipSuccess)
        e = hipMemcpy(counts.data(), d_counts, sizeof(PartCount) * nblocks, hipMemcpyDeviceToHost);
    if (e != hipSuccess) {
        dev_free(d_counts);
        return fail_hip(e, "row split count");
    }
    PartCount run{0, 0, 0};
    for (auto &c : counts) {            // exclusive scan in block order
        const PartCount here = c;
        c = run;
        run.n_heavy += here.n_heavy;
        run.n_seg += here.n_seg;
        run.n_light += here.n_light;
    }
    if (run.n_heavy == 0) {
        dev_free(d_counts);
        return SPMM_OK;
    }
    if (run.n_seg >= INT_MAX || run.n_seg * (int64_t)kPartialWidth < 0) {
        dev_free(d_counts);
        return fail(SPMM_E_UNSUPPORTED, "row split would create %lld pieces", (long long)run.n_seg);
    }
    p->n_heavy = run.n_heavy;
    p->n_seg = run.n_seg;
    p->n_light = run.n_light;
    if ((st = dev_alloc(&p->heavy_rows, p->n_heavy, "heavy rows")) ||
        (st = dev_alloc(&p->seg_first, p->n_heavy + 1, "piece index")) ||
        (st = dev_alloc(&p->seg_begin, p->n_seg, "piece begin")) ||
        (st = dev_alloc(&p->seg_end, p->n_seg, "piece end")) ||
        (st = dev_alloc(&p->partial, p->n_seg * kPartialWidth, "partial sums")) ||
        (st = dev_alloc(&p->part_arg, p->n_seg * kPartialWidth, "partial argmax"))) {
        dev_free(d_counts);
        free_split(p);
        return st;
    }
    e = hipMemcpy(d_counts, counts.data(), sizeof(PartCount) * nblocks, hipMemcpyHostToDevice);
    if (e == hipSuccess)
        e = launch_part_write(p->rowptr, p->M, T, L, d_counts, p->heavy_rows, p->seg_first,
                              p->seg_begin, p->seg_end, nullptr, nblocks, nullptr);
    const int nseg32 = (int)p->n_seg;
    if (e == hipSuccess)
        e = hipMemcpy(p->seg_first + p->n_heavy, &nseg32, sizeof(int), hipMemcpyHostToDevice);
    if (e == hipSuccess) e = hipDeviceSynchronize();
    dev_free(d_counts);
    if (e != hipSuccess) {
        free_split(p);
        return fail_hip(e, "row split write");
    }
    p->split = true;
    // run the pieces of all heavy rows in the order of their first column:
    // pieces in flight together then gather from nearby B rows (same bits)
    if (p->opt_piece_order) {
        if ((st = dev_alloc(&p->seg_order, p->n_seg, "piece order"))) {
            free_split(p);
            return st;
        }
        e = build_piece_order(p->col, p->seg_begin, p->n_seg, p->seg_order);
        if (e != hipSuccess) {
            free_split(p);
            return fail_hip(e, "piece order");
        }
    }
    return SPMM_OK;
}

// Row-tile records for low, even degrees (RA-SpMM's sparse-uniform regime):
// a record holds 8 row ends plus up to `cap` indexes (and values), with cap
// sized to cover the mean tile plus four standard deviations of its entry
// count.  Built when the mean degree is at most 16 and the degree CV at most
// 1, and the graph is not split.
int build_tiles_as(spmm_plan *p, int cap, bool compact) {
    free_tiles(p);
    const int idx_words = compact ? cap / 2 : cap;
    const int rs = (compact ? 3 : kTileRows) + idx_words + (p->val ? cap : 0);
    const int64_t ntiles = (p->M + kTileRows - 1) / kTileRows;
    const int64_t nblocks = tile_build_blocks(p->M);
    int64_t *d_ovf = nullptr;
    int st = dev_alloc(&d_ovf, nblocks, "tile overflow counts");
    if (!st) st = dev_alloc(&p->tiles, ntiles * rs, "row tiles");
    if (st) {
        dev_free(d_ovf);
        return st;
    }
    std::vector<int64_t> ovf((size_t)nblocks);
    hipError_t e = hipMemset(p->tiles, 0, sizeof(int) * ntiles * rs);
    if (e == hipSuccess)
        e = launch_tile_build(p->rowptr, p->col, p->val, p->M, cap, rs, compact, p->tiles, d_ovf, nblocks, nullptr);
    if (e == hipSuccess) e = hipMemcpy(ovf.data(), d_ovf, sizeof(int64_t) * nblocks, hipMemcpyDeviceToHost);
    dev_free(d_ovf);
    if (e != hipSuccess) {
        free_tiles(p);
        return fail_hip(e, "row tile build");
    }
    p->tile_cap = cap;
    p->tile_words = rs;
    p->tile_compact = compact;
    p->tile_overflow = 0;
    for (int64_t n : ovf) p->tile_overflow += n;
    return SPMM_OK;
}

// Row-tile records for low, even degrees (RA-SpMM's sparse-uniform regime):
// a record holds 8 row bounds plus up to `cap` indexes (and values), with cap
// sized to cover the mean tile plus four standard deviations of its entry
// count.  Built when the mean degree is at most 16, the degree CV at most 1
// and the graph is not split.  Compact records (16-bit offsets from a tile
// base) are kept when at most 5% of tiles overflow them; otherwise wide ones.
int build_tiles(spmm_plan *p) {
    free_tiles(p);
    const double mt = kTileRows * p->mean_deg;
    const double sd = std::sqrt((double)kTileRows) * p->cv_deg * p->mean_deg;
    int cap = (int)std::ceil((mt + 4.0 * sd + 4.0) / 8.0) * 8;
    cap = std::max(8, cap);
    const bool fits = cap <= kTileMaxCap;
    cap = std::min(cap, kTileMaxCap);
    const bool enabled =
        p->opt_tiles >= 1 ||
        (p->opt_tiles == -1 && !p->split && p->mean_deg <= 16.0 && p->cv_deg <= 1.0 && fits);
    if (!enabled || p->M == 0 || p->split) return SPMM_OK;
    const int64_t ntiles = (p->M + kTileRows - 1) / kTileRows;
    int st = build_tiles_as(p, cap, p->opt_tiles != 2);
    if (st) return st;
    if (p->tile_compact && p->tile_overflow * 20 > ntiles) st = build_tiles_as(p, cap, false);
    return st;
}

// fp16 community tiles and the residual CSR (built when SPMM_OPT_MFMA is set).
int build_mfma(spmm_plan *p, bool split) {
    free_mfma(p);
    if (p->M + 1 > INT_MAX) return fail(SPMM_E_UNSUPPORTED, "fp16 tiles need M + 1 below 2^31");
    const int64_t ntiles = (p->M + kWinRows - 1) / kWinRows;
    int *d_flag = nullptr;
    int st;
    if ((st = dev_alloc(&p->mfma_tiles, ntiles * 8 * kMfmaKSteps * 64, "fp16 community tiles")) ||
        (split && (st = dev_alloc(&p->mfma_tiles_lo, ntiles * 8 * kMfmaKSteps * 64, "fp16 low halves"))) ||
        (split && (st = dev_alloc(&p->mfma_tile_exp, ntiles, "tile exponents"))) ||
        (st = dev_alloc(&p->mfma_rowptr, p->M + 1, "residual rowptr")) || (st = dev_alloc(&d_flag, 1, "range flag"))) {
        free_mfma(p);
        dev_free(d_flag);
        return st;
    }
    hipError_t e = mfma_build_tiles(p->rowptr, p->col, p->val, p->M, p->mfma_tiles, p->mfma_tiles_lo,
                                    p->mfma_tile_exp, ntiles, p->mfma_rowptr, d_flag,
                                    nullptr);
    int flag = 0, rnnz = 0;
    if (e == hipSuccess) e = hipMemcpy(&flag, d_flag, sizeof(int), hipMemcpyDeviceToHost);
    if (e == hipSuccess) e = hipMemcpy(&rnnz, p->mfma_rowptr + p->M, sizeof(int), hipMemcpyDeviceToHost);
    dev_free(d_flag);
    if (e != hipSuccess) {
        free_mfma(p);
        return fail_hip(e, "fp16 tile build");
    }
    if (flag) {
        free_mfma(p);
        return fail(SPMM_E_UNSUPPORTED, split ? "an in-block sum of weights is not finite"
                                               : "an in-block sum of weights is outside the fp16 range (or not finite)");
    }
    p->mfma_rnnz = rnnz;
    if ((st = dev_alloc(&p->mfma_col, rnnz, "residual col")) ||
        (p->val && (st = dev_alloc(&p->mfma_val, rnnz, "residual val")))) {
        free_mfma(p);
        return st;
    }
    e = mfma_write_residual(p->rowptr, p->col, p->val, p->M, p->mfma_rowptr, p->mfma_col, p->mfma_val, nullptr);
    if (e != hipSuccess) {
        free_mfma(p);
        return fail_hip(e, "residual CSR build");
    }
    return SPMM_OK;
}

// V = 2 panels (built when SPMM_OPT_VBLOCK is set).
int build_pairs(spmm_plan *p) {
    free_pairs(p);
    if (p->K >= (int64_t(1) << 30)) return fail(SPMM_E_UNSUPPORTED, "V = 2 panels need K below 2^30");
    const int64_t npanels = (p->M + 1) / 2;
    int st = dev_alloc(&p->pair_prow, npanels + 1, "panel rowptr");
    if (st) return st;
    PairOutput out;
    const hipError_t e = pair_build(p->rowptr, p->col, p->val, p->M, p->K, p->nnz, p->rows_sorted, p->pair_prow, &out);
    if (e != hipSuccess) {
        free_pairs(p);
        return fail_hip(e, "V = 2 panel build");
    }
    p->pair_col = out.pcol;
    p->pair_val = out.pval;
    p->pair_nvec = out.nvec;
    p->pair_unsorted = out.unsorted != 0;
    return SPMM_OK;
}

// Automatic V = 2 panels (SPMM_OPT_VBLOCK = -1): for a plan that is not split
// and whose rows are all stored with ascending columns, count the panels'
// nonzero vectors with one merge pass, and build the panels when their
// padding share 1 - nnz / (2 vectors) is at most kPairMaxPadding.  There each
// gather of a B row serves 1.4 or more entries on average, and the build (two
// merge passes and a scan, no sort) repays itself within a few hundred
// products (kNN line graph: 1.5x faster products).
int auto_pairs(spmm_plan *p) {
    if (p->opt_vblock != -1 || p->pair_prow || p->split || !p->rows_sorted || p->M < 2 || p->nnz == 0 ||
        p->K >= (int64_t(1) << 30))
        return SPMM_OK;
    int64_t vectors = 0;
    const hipError_t e = pair_count_sorted(p->rowptr, p->col, p->M, &vectors);
    if (e != hipSuccess) return fail_hip(e, "V = 2 panel count");
    const double padding = vectors > 0 ? 1.0 - (double)p->nnz / (2.0 * (double)vectors) : 1.0;
    if (padding > kPairMaxPadding) return SPMM_OK;
    return build_pairs(p);
}

// Merge-path segments (built when SPMM_OPT_BALANCE is 1).
int build_merge(spmm_plan *p) {
    free_merge(p);
    if (p->M + p->nnz >= INT_MAX) return fail(SPMM_E_UNSUPPORTED, "merge path needs M + nnz below 2^31");
    const int64_t nseg = (p->M + p->nnz + kMergeItems - 1) / kMergeItems;
    int st;
    if ((st = dev_alloc(&p->merge_seg_row, nseg + 1, "merge rows")) ||
        (st = dev_alloc(&p->merge_seg_entry, nseg + 1, "merge entries")) ||
        (st = dev_alloc(&p->merge_carry_row, nseg, "merge carry rows")) ||
        (st = dev_alloc(&p->merge_carry, nseg * kPartialWidth, "merge carries")) ||
        (st = dev_alloc(&p->merge_carry_arg, nseg * kPartialWidth, "merge carry argmax"))) {
        free_merge(p);
        return st;
    }
    const hipError_t e = merge_build(p->rowptr, p->M, p->nnz, nseg, p->merge_seg_row, p->merge_seg_entry);
    if (e != hipSuccess) {
        free_merge(p);
        return fail_hip(e, "merge path build");
    }
    p->merge_nseg = nseg;
    return SPMM_OK;
}

double pair_padding(const spmm_plan *p) {
    return p->pair_nvec > 0 ? 1.0 - (double)p->nnz / (2.0 * (double)p->pair_nvec) : 0.0;
}

int pow2_ceil(int64_t x) {
    int g = 1;
    while (g < x && g < 64) g <<= 1;
    return g;
}

bool aligned(const void *p, size_t a) { return ((uintptr_t)p % a) == 0; }

// Rule router (first matching rule per decision; forced options override):
//  * vector width: 4 floats for any N >= 4 (16-byte accesses at element
//    alignment, a row's last vector moved back to end at column N); float1
//    where a row spans only a few float4 lanes and gathers, not DRAM, bound
//    the product, and on small graphs below 128 floats; below 4 floats 2
//    (aligned, N = 2) or 1;
//  * lanes per row: one pass of the row's group spans the W = N / vec vector
//    columns (several rows per wave when W < 64; coarsening F = 2 when
//    W > 64), following ParamSpMM's thread-coarsening analysis (section 3.3)
//    with the MAC-job gap kept at zero wherever N allows;
//  * low mean degree (< 8, RA-SpMM's sparse-uniform regime): half the lanes
//    and F = 2, doubling the rows per wave so more rows' gathers are in
//    flight per wave; widths that leave a quarter of the covering lane group
//    idle take the same shape below mean degree 16;
//  * small graphs (fewer than two waves per CU at 16 rows per wave):
//    launch-bound, so as many waves as possible: no coarsening, and 8 lanes
//    per row (more column slices) up to 32 vectors;
//  * skewed degrees (CV > 1, RA-SpMM's sparse-skewed / extreme-skew regime),
//    where neighbours carry no locality, with a B of 128 floats or more in a
//    multiple of 32 floats: 64-column slices (128-column slices from 512
//    floats), so each pass over the graph touches a part of B that stays in
//    the Infinity Cache longer; at other widths one slice of the covering
//    lane group;
//  * the LDS window kernels for community structure above 32 floats; V = 2
//    panels where the plan built them;
//  * fp16 matrix-core tiles only when the caller enabled them (they follow
//    the looser fp16 contract) and the run is a sum or mean with 16-byte
//    aligned float4 access;
//  * XCD remap in chunks of 256 blocks (rows sharing B rows meet in one L2,
//    all XCDs sweep one region together): measured neutral or better on
//    every regime, and better than chunks of 64 or 1024.
// The thresholds come from rocprofv3-timed sweeps over seven graphs and 25
// widths (the router sweep of the benchmark).
Route route_for(const spmm_plan *p, int64_t N, int reduce, const void *B, const void *C, const void *argmax) {
    Route r;
    const bool a16 = aligned(B, 16) && aligned(C, 16) && (!argmax || aligned(argmax, 16));
    const bool a8 = aligned(B, 8) && aligned(C, 8) && (!argmax || aligned(argmax, 16));
    const bool a4 = aligned(B, 4) && aligned(C, 4) && (!argmax || aligned(argmax, 8));
    const bool skewed = p->cv_deg > 1.0;
    const bool small = p->M * 4 < (int64_t)p->num_cus * 2 * 64;
    // whole float4 vectors: 16-byte aligned rows
    const bool whole4 = N % 4 == 0 && a16;
    // float4 lanes also where rows are only 4-byte aligned or N is not a
    // multiple of 4 (the last vector of a row ends at column N): one 16-byte
    // access per lane instead of two or four narrower ones (road graph, 33
    // floats: 0.094 vs 0.198 ms in float1 lanes; 602 floats: 1.38 vs 1.60 ms
    // in float2 lanes)
    const bool ragged4 = N >= 4 && a4;
    int vec = (whole4 || ragged4) ? 4 : (N % 2 == 0 && a8) ? 2 : 1;
    // Float1 lanes instead where a row spans only a few float4 lanes and the
    // rate of gathers, not DRAM, bounds the product: rows of at most 8
    // floats at mean degree 16 and above, whose B rows stay in cache
    // (community graph, 8 floats: 0.071 vs 0.095 ms; 7 floats: 0.072 vs
    // 0.095 ms), at most 16 floats on split skewed graphs, where a wave's
    // rows then number fewer and end closer together (power-law graph, 16
    // floats: 1.09 vs 1.34 ms; mixed graph, 8 floats: 0.317 vs 0.372 ms),
    // and below 128 floats on launch-bound small graphs, where float1 lanes
    // give more waves (2,000-node graph, 16 floats: 8.1 vs 8.5 us)
    // (not when the caller forced the window kernels on: they need float4)
    if (vec == 4 && p->opt_window != 1 &&
        ((N <= 8 && p->mean_deg >= 16.0) || (N <= 16 && p->split) || (small && N < 128)))
        vec = 1;
    if (p->opt_vec == 4 && (whole4 || ragged4)) vec = 4;
    else if (p->opt_vec == 2 && N % 2 == 0 && a8) vec = 2;
    else if (p->opt_vec == 1) vec = 1;
    const int64_t W = (N + vec - 1) / vec;
    int G = std::max(4, pow2_ceil(W));
    int F = W > G ? 2 : 1;
    const bool pow2 = (W & (W - 1)) == 0;
    // widths that are a multiple of 8 vectors but not a power of two (96,
    // 160, 192 floats): rounding G up to a power of two leaves lanes idle
    const bool odd8 = !skewed && W % 8 == 0 && !pow2 && W < 64;
    // other widths of 17 to 63 vectors that leave a quarter or more of their
    // power-of-two lane group idle (66, 130, 140 floats): at mean degree below
    // 16, half the group, coarsened, so that a row's second vector slot takes
    // the remainder and each wave holds twice the rows (diffusion graph, 66
    // floats: 0.292 vs 0.328 ms; 130 floats: 0.505 vs 0.556 ms); at higher or
    // skewed degrees the whole group stays faster (community graph, 130
    // floats: 0.539 vs 0.570 ms)
    int pc = 1;
    while (pc < W) pc <<= 1;
    const bool ragged = !pow2 && W > 16 && W < 64 && 4 * W <= 3 * pc && p->mean_deg < 16.0 && !skewed;
    if (skewed && W >= 32 && W % 8 == 0) {
        // skewed graphs: column slices of 32 lanes from 64 to 128 vectors, of
        // 16 lanes otherwise (each pass over the graph touches a part of every
        // B row, which keeps more of B in the Infinity Cache); measured at
        // widths of a multiple of 32 floats: at other widths a nearly empty
        // last slice costs a whole pass (power-law graph, 130 floats: one
        // 64-lane slice 4.92 ms, three 16-lane slices 6.01 ms)
        G = (W >= 64 && W <= 128) ? 32 : 16;
        F = 1;
    } else if (small) {
        // launch-bound: as many waves as possible, so no coarsening, and 8
        // lanes per row (more column slices) up to 128 columns
        F = 1;
        if (W <= 32) G = 8;
    } else if (odd8) {
        // low degree: row tiles of 8 lanes x 2 vectors, in 64-column slices;
        // else half the lanes, coarsened, in one slice
        G = p->mean_deg < 8.0 ? 8 : G / 2;
        F = 2;
    } else if (ragged) {
        G = (int)pc / 2;
        F = 2;
    } else if (p->mean_deg < 8.0 && G >= 16 && W <= G) {
        G /= 2;
        F = 2;
    } else if (p->mean_deg >= 8.0 && W > 64 && W % 64 == 0) {
        // wide features at higher degree: 64-lane slices without coarsening
        F = 1;
    }
    if (p->opt_lanes) G = p->opt_lanes;
    if (p->opt_coarsen) F = p->opt_coarsen;
    r.vec = vec;
    r.lanes = G;
    r.coarsen = F;
    r.slices = (int)((W + (int64_t)G * F - 1) / ((int64_t)G * F));
    r.xcd_remap = p->opt_xcd >= 0 ? p->opt_xcd : 1;
    r.nt_store = p->opt_nt >= 0 ? p->opt_nt : 0;
    r.split = p->split;
    r.tiled = p->tiles != nullptr && !p->split && (G == 4 || G == 8);
    r.compact = r.tiled && p->tile_compact;
    // community structure with features of more than 32 floats: stage B's
    // row blocks in LDS (community graph, 33 floats: 0.114 vs 0.184 ms in
    // 16-lane rows; at 32 floats and below 8-lane rows are as fast or
    // faster).  One dispatch holds at most 2^32 / kWinBlock row blocks,
    // about 10^9 rows; larger graphs take the row kernels.
    const bool win_grid = (p->M + kWinRows - 1) / kWinRows <= (int64_t)(UINT32_MAX / kWinBlock);
    r.window = !p->split && vec == 4 && p->opt_lanes == 0 && p->opt_coarsen == 0 && win_grid &&
               (p->opt_window == 1 || (p->opt_window == -1 && p->win_frac >= 0.5 && N > 32));
    // fp16 community tiles, when the caller asked for them
    r.mfma = p->opt_mfma > 0 && p->mfma_tiles != nullptr && reduce != SPMM_MAX && N % 4 == 0 && a16;
    // merge-path balancing, when the caller chose it
    r.merge = !r.mfma && p->opt_balance == 1 && p->merge_seg_row != nullptr;
    if (r.merge) {
        const bool al2 = N % 2 == 0 && a8;
        // skewed graphs: 64-column slices (each pass over the graph touches a
        // quarter of a 256-byte B row), as for the row kernels; float4 lanes
        // at any width from 256 floats (whole4 or ragged4)
        r.vec = p->cv_deg > 1.0 ? 1 : (N >= 256 && (whole4 || ragged4)) ? 4 : (N >= 128 && al2) ? 2 : 1;
        r.lanes = 64;
        r.coarsen = 1;
        const int64_t w = std::min<int64_t>(N, kPartialWidth);
        r.slices = (int)((w + 64 * r.vec - 1) / (64 * r.vec));
        r.tiled = r.compact = r.window = r.split = r.pairs = false;
        return r;
    }
    // V = 2 panels, when built: by padding share (ParamSpMM's PR for V), or forced
    // (with community structure as well, the window kernel's 64-column
    // slices beat the panels from 512 columns, and above 256 columns when the
    // width is not a power of two: kNN line graph 0.976 vs 1.036 ms at 512
    // columns, 0.633 vs 0.924 ms at 300)
    // The panels have float4 and float1 forms only: a float2 width of 128
    // floats or more keeps the float2 row kernel (kNN line graph, 130 floats:
    // 0.745 vs 0.789 ms; 602 floats: 2.51 vs 3.36 ms).
    r.pairs = !r.mfma && p->pair_prow != nullptr && p->opt_vblock != 0 &&
              (reduce != SPMM_MAX || !p->pair_unsorted) &&
              (p->opt_vblock == 2 ||
               (!p->split && pair_padding(p) <= kPairMaxPadding && !(vec == 2 && N >= 128) &&
                !(r.window && (W >= 128 || (W > 64 && (W & (W - 1)) != 0)))));
    if (r.pairs) {
        r.vec = vec == 4 ? 4 : 1;
        const int64_t Wp = (N + r.vec - 1) / r.vec;
        // at most 32 lanes: two 128-column slices beat one of 256 (kNN line
        // graph, 256 columns: 0.497 vs 0.519 ms); a width that is not a power
        // of two takes its largest power-of-two factor, so that no lane idles
        // (kNN, 96 and 160 columns: 8 lanes; 192: 16)
        int lanes = std::min(32, std::max(4, pow2_ceil(Wp)));
        const int64_t factor = Wp & -Wp;
        if ((Wp & (Wp - 1)) != 0 && factor >= 4) lanes = (int)std::min<int64_t>(32, factor);
        // other widths past 32 vectors that are not a power of two: 64 lanes,
        // the fewest slices (kNN line graph, 130 floats: 0.358 vs 0.444 ms at
        // 32 lanes; 1026 floats: 2.84 vs 3.20 ms)
        else if ((Wp & (Wp - 1)) != 0 && Wp > 32) lanes = 64;
        r.lanes = p->opt_lanes ? p->opt_lanes : lanes;
        r.coarsen = 1;
        r.slices = (int)((Wp + r.lanes - 1) / r.lanes);
        r.tiled = r.compact = r.window = r.split = false;
        // panels of neighbouring rows: the plain block order keeps a panel's
        // neighbours in flight together (kNN line graph, N = 16..512: as fast
        // or faster than the XCD remap)
        r.xcd_remap = p->opt_xcd >= 0 ? p->opt_xcd : 0;
        return r;
    }
    if (r.window || r.mfma) {
        r.vec = 4;
        r.lanes = kWinCols / 4;
        r.coarsen = 1;
        r.slices = (int)((N + kWinCols - 1) / kWinCols);
        r.tiled = false;
        r.compact = false;
        r.window = !r.mfma;
        r.window_sorted = r.window && p->rows_sorted && p->win_lo != nullptr;
        r.split = r.split && !r.mfma;
    }
    return r;
}

// Launch the row kernel over tasks [0, ntasks), one task group per wave, in
// several dispatches when one grid would exceed the 2^32 work-item limit of a
// dispatch dimension.
hipError_t launch_rows(RowKernelFn fn, RowArgs a, int rows_per_wave, int slices, hipStream_t s) {
    const int64_t per_block = (int64_t)rows_per_wave * kWaves;
    const int64_t max_blocks = (int64_t)(UINT32_MAX / kBlock);
    const int64_t end = a.ntasks;
    for (int64_t base = 0; base < end; base += max_blocks * per_block) {
        const int64_t n = std::min(end - base, max_blocks * per_block);
        a.task_base = base;
        a.ntasks = base + n;
        void *args[] = {&a};
        const dim3 grid((unsigned)((n + per_block - 1) / per_block), (unsigned)slices);
        const hipError_t e =
            hipLaunchKernel(reinterpret_cast<const void *>(fn), grid, dim3(kBlock), args, 0, s);
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

}  // namespace

SPMM_API int spmm_last_error(char *buf, int64_t cap) {
    if (buf && cap > 0) {
        std::strncpy(buf, t_msg, (size_t)cap - 1);
        buf[cap - 1] = '\0';
    }
    return t_status;
}

SPMM_API int spmm_set_mem_limit(int64_t bytes) {
    if (bytes < 0) return fail(SPMM_E_INVALID_ARG, "memory limit must be >= 0 (0: none)");
    set_thread_limit(bytes);
    return succeed();
}

SPMM_API int spmm_mem_stats(struct spmm_mem_stats *out) {
    if (!out) return fail(SPMM_E_INVALID_ARG, "output is NULL");
    out->in_use = dbytes_in_use();
    out->last_call_peak = last_call_peak();
    out->last_call_allocs = last_call_allocs();
    out->thread_limit = thread_limit();
    return succeed();
}

SPMM_API spmm_plan_t spmm_plan_create(const int64_t *rowptr, const int64_t *col, const float *val,
                                      int64_t M, int64_t K) {
    const auto t0 = std::chrono::steady_clock::now();
    PlanScope budget(nullptr);
    if (M < 0 || K < 0) {
        fail(SPMM_E_INVALID_ARG, "negative size (M=%lld, K=%lld)", (long long)M, (long long)K);
        return nullptr;
    }
    if (M >= INT_MAX || K >= INT_MAX) {
        fail(SPMM_E_UNSUPPORTED, "M and K must be below 2^31 - 1");
        return nullptr;
    }
    if (!rowptr) {
        fail(SPMM_E_INVALID_ARG, "rowptr is NULL");
        return nullptr;
    }
    if (!is_device_ptr(rowptr)) {
        fail(SPMM_E_INVALID_ARG, "rowptr is not device memory");
        return nullptr;
    }
    hipError_t e = hipDeviceSynchronize();   // inputs may still be in flight on other streams
    if (e != hipSuccess) {
        fail_hip(e, "synchronise before plan creation");
        return nullptr;
    }
    int64_t ends[2] = {0, 0};
    e = hipMemcpy(&ends[0], rowptr, sizeof(int64_t), hipMemcpyDeviceToHost);
    if (e == hipSuccess) e = hipMemcpy(&ends[1], rowptr + M, sizeof(int64_t), hipMemcpyDeviceToHost);
    if (e != hipSuccess) {
        fail_hip(e, "read rowptr[0] and rowptr[M]");
        return nullptr;
    }
    if (ends[0] != 0) {
        fail(SPMM_E_BAD_CSR, "invalid CSR: first bad row 0 (rowptr[0] = %lld, expected 0)",
             (long long)ends[0]);
        return nullptr;
    }
    const int64_t nnz = ends[1];
    if (nnz < 0) {
        fail(SPMM_E_BAD_CSR, "invalid CSR: rowptr[M] = %lld is negative", (long long)nnz);
        return nullptr;
    }
    if (nnz >= INT_MAX) {
        fail(SPMM_E_UNSUPPORTED, "nnz = %lld must be below 2^31 - 1", (long long)nnz);
        return nullptr;
    }
    if (nnz > 0 && K == 0) {
        fail(SPMM_E_BAD_CSR, "invalid CSR: %lld entries with K = 0", (long long)nnz);
        return nullptr;
    }
    if (nnz > 0 && !is_device_ptr(col)) {
        fail(SPMM_E_INVALID_ARG, "col is NULL or not device memory");
        return nullptr;
    }
    if (val && nnz > 0 && !is_device_ptr(val)) {
        fail(SPMM_E_INVALID_ARG, "val is not device memory");
        return nullptr;
    }

    spmm_plan *p = new (std::nothrow) spmm_plan();
    if (!p) {
        fail(SPMM_E_OOM, "host allocation of the plan failed");
        return nullptr;
    }
    (void)hipGetDevice(&p->device);
    int cus = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, p->device) == hipSuccess && cus > 0)
        p->num_cus = cus;
    p->M = M;
    p->K = K;
    p->nnz = nnz;
    p->n_light = M;

    int st;
    if ((st = dev_alloc(&p->rowptr, M + 1, "rowptr")) || (st = dev_alloc(&p->col, nnz, "col")) ||
        (val && (st = dev_alloc(&p->val, nnz, "val")))) {
        free_plan(p);
        return nullptr;
    }

    // rowptr: validation, descriptors, int32 copy
    const int64_t rblocks = (M + kRowsPerScanBlock - 1) / kRowsPerScanBlock;
    RowScanOut *d_rows = nullptr;
    if ((st = dev_alloc(&d_rows, std::max<int64_t>(rblocks, 1), "row scan"))) {
        free_plan(p);
        return nullptr;
    }
    if (M == 0) e = hipMemset(p->rowptr, 0, sizeof(int));
    else e = launch_rowscan(rowptr, M, p->rowptr, d_rows, rblocks, nullptr);
    std::vector<RowScanOut> rs((size_t)rblocks);
    if (e == hipSuccess && rblocks > 0)
        e = hipMemcpy(rs.data(), d_rows, sizeof(RowScanOut) * rblocks, hipMemcpyDeviceToHost);
    dev_free(d_rows);
    if (e != hipSuccess) {
        fail_hip(e, "row scan");
        free_plan(p);
        return nullptr;
    }
    int64_t bad_row = INT64_MAX, sum_deg = 0, sum_deg2 = 0, dmax = 0, n_empty = 0;
    for (const auto &r : rs) {
        bad_row = std::min(bad_row, r.bad_row);
        sum_deg += r.sum_deg;
        sum_deg2 += r.sum_deg2;
        dmax = std::max(dmax, r.dmax);
        n_empty += r.n_empty;
    }
    if (bad_row != INT64_MAX) {
        fail(SPMM_E_BAD_CSR, "invalid CSR: first bad row %lld (rowptr decreases)", (long long)bad_row);
        free_plan(p);
        return nullptr;
    }

    // col: range check, int32 copy
    if (nnz > 0) {
        const int64_t cblocks = colscan_blocks(nnz);
        int64_t *d_bad = nullptr;
        if ((st = dev_alloc(&d_bad, cblocks, "col scan"))) {
            free_plan(p);
            return nullptr;
        }
        e = launch_colscan(col, nnz, K, p->col, d_bad, cblocks, nullptr);
        std::vector<int64_t> bad((size_t)cblocks);
        if (e == hipSuccess)
            e = hipMemcpy(bad.data(), d_bad, sizeof(int64_t) * cblocks, hipMemcpyDeviceToHost);
        dev_free(d_bad);
        if (e != hipSuccess) {
            fail_hip(e, "column scan");
            free_plan(p);
            return nullptr;
        }
        const int64_t bad_pos = *std::min_element(bad.begin(), bad.end());
        if (bad_pos != INT64_MAX) {
            // locate the row owning entry bad_pos (error path only)
            std::vector<int64_t> h_rowptr((size_t)M + 1);
            int64_t row = -1;
            if (hipMemcpy(h_rowptr.data(), rowptr, sizeof(int64_t) * (M + 1), hipMemcpyDeviceToHost) ==
                hipSuccess)
                row = (int64_t)(std::upper_bound(h_rowptr.begin(), h_rowptr.end(), bad_pos) -
                                h_rowptr.begin()) - 1;
            fail(SPMM_E_BAD_CSR, "invalid CSR: first bad row %lld (entry %lld has a column outside [0, %lld))",
                 (long long)row, (long long)bad_pos, (long long)K);
            free_plan(p);
            return nullptr;
        }
        if (val) {
            e = hipMemcpy(p->val, val, sizeof(float) * nnz, hipMemcpyDeviceToDevice);
            if (e != hipSuccess) {
                fail_hip(e, "copy val");
                free_plan(p);
                return nullptr;
            }
        }
    }

    // share of entries inside their row's aligned kWinRows block
    if (nnz > 0) {
        const int64_t wblocks = (M + kRowsPerScanBlock - 1) / kRowsPerScanBlock;
        int64_t *d_w = nullptr;
        if ((st = dev_alloc(&d_w, 2 * wblocks, "window scan"))) {
            free_plan(p);
            return nullptr;
        }
        e = launch_window_scan(p->rowptr, p->col, M, d_w, wblocks, nullptr);
        std::vector<int64_t> wc((size_t)(2 * wblocks));
        if (e == hipSuccess) e = hipMemcpy(wc.data(), d_w, sizeof(int64_t) * 2 * wblocks, hipMemcpyDeviceToHost);
        dev_free(d_w);
        if (e != hipSuccess) {
            fail_hip(e, "window scan");
            free_plan(p);
            return nullptr;
        }
        int64_t inside = 0, unsorted = 0;
        for (int64_t b = 0; b < wblocks; ++b) {
            inside += wc[2 * b];
            unsorted += wc[2 * b + 1];
        }
        p->win_frac = (double)inside / (double)nnz;
        p->rows_sorted = unsorted == 0;
        if (p->win_frac >= 0.5 && (st = build_window_runs(p))) {
            free_plan(p);
            return nullptr;
        }
    }

    // descriptors (RA-SpMM: M, mean degree, coefficient of variation)
    p->dmax = dmax;
    p->n_empty = n_empty;
    p->sum_deg2 = sum_deg2;
    p->mean_deg = M > 0 ? (double)sum_deg / (double)M : 0.0;
    if (M > 0 && sum_deg > 0) {
        const __int128 num = (__int128)M * (__int128)sum_deg2 - (__int128)sum_deg * (__int128)sum_deg;
        const double var = (double)num / ((double)M * (double)M);
        p->cv_deg = std::sqrt(std::max(var, 0.0)) / p->mean_deg;
    }

    if ((st = build_split(p)) || (st = build_tiles(p)) || (st = auto_pairs(p))) {
        free_plan(p);
        return nullptr;
    }
    e = hipDeviceSynchronize();
    if (e != hipSuccess) {
        fail_hip(e, "plan creation");
        free_plan(p);
        return nullptr;
    }
    p->plan_ms = std::chrono::duration<double, std::milli>(std::chrono::steady_clock::now() - t0).count();
    succeed();
    return p;
}

SPMM_API int spmm_plan_destroy(spmm_plan_t plan) {
    if (!plan) return succeed();
    DeviceGuard dg(plan->device);
    free_plan(plan);
    return succeed();
}

SPMM_API int spmm_plan_set_option(spmm_plan_t p, int option, int64_t value) {
    if (!p) return fail(SPMM_E_INVALID_ARG, "plan is NULL");
    DeviceGuard dg(p->device);
    PlanScope budget(p);
    GenerationGuard gen(p);
    const int64_t prev_T = p->opt_T, prev_L = p->opt_L, prev_split = p->opt_split;
    const int prev_order = p->opt_piece_order;
    switch (option) {
        case SPMM_OPT_SPLIT_T:
            if (value < -1) return fail(SPMM_E_INVALID_ARG, "split threshold must be >= -1");
            p->opt_T = value;
            break;
        case SPMM_OPT_SPLIT_L:
            if (value == 0 || value < -1) return fail(SPMM_E_INVALID_ARG, "piece length must be > 0 or -1");
            p->opt_L = value;
            break;
        case SPMM_OPT_SPLIT_MODE:
            if (value < -1 || value > 1) return fail(SPMM_E_INVALID_ARG, "split mode must be -1, 0 or 1");
            p->opt_split = value;
            break;
        case SPMM_OPT_TILES: {
            if (value < -1 || value > 2) return fail(SPMM_E_INVALID_ARG, "tiles must be -1, 0, 1 or 2");
            p->opt_tiles = value;
            const hipError_t e = hipDeviceSynchronize();
            if (e != hipSuccess) return fail_hip(e, "synchronise before rebuilding the tiles");
            const int st = build_tiles(p);
            if (st) return st;
            return succeed();
        }
        case SPMM_OPT_WINDOW: {
            if (value < -1 || value > 1) return fail(SPMM_E_INVALID_ARG, "window must be -1, 0 or 1");
            const hipError_t e = hipDeviceSynchronize();
            if (e != hipSuccess) return fail_hip(e, "synchronise before changing the window runs");
            // the per-row runs serve only the window kernel: off frees them,
            // on (or automatic with community structure) builds them
            p->opt_window = 0;
            if (value == 0) {
                free_window_runs(p);
                return succeed();
            }
            if (value == 1 || p->win_frac >= 0.5) {
                const int st = build_window_runs(p);
                if (st) return st;
            }
            p->opt_window = value;
            return succeed();
        }
        case SPMM_OPT_LANES:
            if (!(value == 0 || value == 4 || value == 8 || value == 16 || value == 32 || value == 64))
                return fail(SPMM_E_INVALID_ARG, "lanes per row must be 0, 4, 8, 16, 32 or 64");
            p->opt_lanes = (int)value;
            return succeed();
        case SPMM_OPT_COARSEN:
            if (value < 0 || value > 2) return fail(SPMM_E_INVALID_ARG, "coarsening must be 0, 1 or 2");
            p->opt_coarsen = (int)value;
            return succeed();
        case SPMM_OPT_VEC:
            if (!(value == 0 || value == 1 || value == 2 || value == 4))
                return fail(SPMM_E_INVALID_ARG, "vector width must be 0, 1, 2 or 4");
            p->opt_vec = (int)value;
            return succeed();
        case SPMM_OPT_XCD_REMAP:
            if (value < -1 || value > 1) return fail(SPMM_E_INVALID_ARG, "XCD remap must be -1, 0 or 1");
            p->opt_xcd = (int)value;
            return succeed();
        case SPMM_OPT_PIECE_ORDER:
            if (value < 0 || value > 1) return fail(SPMM_E_INVALID_ARG, "piece order must be 0 or 1");
            p->opt_piece_order = (int)value;
            break;
        case SPMM_OPT_MEM_LIMIT:
            if (value < 0) return fail(SPMM_E_INVALID_ARG, "memory limit must be >= 0 (0: none)");
            p->mem_limit = value;
            return succeed();
        case SPMM_OPT_SPLIT_FUSED:
            if (value < 0 || value > 1) return fail(SPMM_E_INVALID_ARG, "split fused must be 0 or 1");
            p->opt_split_fused = (int)value;
            return succeed();
        case SPMM_OPT_NT_STORE:
            if (value < -1 || value > 1) return fail(SPMM_E_INVALID_ARG, "nt store must be -1, 0 or 1");
            p->opt_nt = (int)value;
            return succeed();
        case SPMM_OPT_BALANCE: {
            if (value < 0 || value > 1) return fail(SPMM_E_INVALID_ARG, "balance must be 0 or 1");
            const hipError_t e = hipDeviceSynchronize();
            if (e != hipSuccess) return fail_hip(e, "synchronise before changing the balancing");
            p->opt_balance = 0;
            if (value == 0) {
                free_merge(p);
                return succeed();
            }
            if (!p->merge_seg_row) {
                const int st = build_merge(p);
                if (st) return st;
            }
            p->opt_balance = 1;
            return succeed();
        }
        case SPMM_OPT_VBLOCK: {
            if (value < -1 || value > 2) return fail(SPMM_E_INVALID_ARG, "vblock must be -1, 0, 1 or 2");
            const hipError_t e = hipDeviceSynchronize();
            if (e != hipSuccess) return fail_hip(e, "synchronise before changing the V = 2 panels");
            p->opt_vblock = 0;
            if (value == 0) {
                free_pairs(p);
                return succeed();
            }
            if (value == -1) {
                p->opt_vblock = -1;
                const int st = auto_pairs(p);
                if (st) {
                    p->opt_vblock = 0;
                    return st;
                }
                return succeed();
            }
            if (!p->pair_prow) {
                const int st = build_pairs(p);
                if (st) return st;
            }
            p->opt_vblock = (int)value;
            return succeed();
        }
        case SPMM_OPT_MFMA: {
            if (value < 0 || value > 2) return fail(SPMM_E_INVALID_ARG, "mfma must be 0, 1 or 2");
            const hipError_t e = hipDeviceSynchronize();
            if (e != hipSuccess) return fail_hip(e, "synchronise before changing the fp16 tiles");
            p->opt_mfma = 0;
            if (value == 0) {
                free_mfma(p);
                return succeed();
            }
            if (!p->mfma_tiles || (p->mfma_tiles_lo != nullptr) != (value == 2)) {
                const int st = build_mfma(p, value == 2);
                if (st) return st;
            }
            p->opt_mfma = (int)value;
            return succeed();
        }

        default:
            return fail(SPMM_E_INVALID_ARG, "unknown option %d", option);
    }
    const hipError_t e = hipDeviceSynchronize();
    if (e != hipSuccess) return fail_hip(e, "synchronise before rebuilding the split");
    int st = build_split(p);
    if (!st) st = build_tiles(p);
    if (st) {
        // keep the plan usable: back to the previous split parameters (the
        // memory they held was just freed), keeping the first error
        const int keep = t_status;
        char msg[sizeof(t_msg)];
        std::memcpy(msg, t_msg, sizeof(msg));
        p->opt_T = prev_T;
        p->opt_L = prev_L;
        p->opt_split = prev_split;
        p->opt_piece_order = prev_order;
        BudgetPause restore_what_the_plan_held;
        if (build_split(p) == SPMM_OK) (void)build_tiles(p);
        t_status = keep;
        std::memcpy(t_msg, msg, sizeof(msg));
        return st;
    }
    return succeed();
}

SPMM_API int spmm_plan_info(spmm_plan_t p, struct spmm_plan_info *out) {
    if (!p || !out) return fail(SPMM_E_INVALID_ARG, "plan or output is NULL");
    struct spmm_plan_info info;
    std::memset(&info, 0, sizeof(info));
    info.M = p->M;
    info.K = p->K;
    info.nnz = p->nnz;
    info.dmax = p->dmax;
    info.n_empty = p->n_empty;
    info.mean_deg = p->mean_deg;
    info.cv_deg = p->cv_deg;
    info.split_T = p->T;
    info.split_L = p->L;
    info.n_heavy = p->split ? p->n_heavy : 0;
    info.n_seg = p->split ? p->n_seg : 0;
    info.split_ratio = p->M > 0 ? (double)(p->split ? p->n_light + p->n_seg : p->M) / (double)p->M : 1.0;
    info.has_val = p->val != nullptr;
    info.index_bits = 32;
    info.plan_ms = p->plan_ms;
    info.route_N = p->route_N;
    info.route_lanes = p->route.lanes;
    info.route_vec = p->route.vec;
    info.route_coarsen = p->route.coarsen;
    info.route_rows_per_wave = 64 / p->route.lanes;
    info.route_slices = p->route.slices;
    info.route_xcd_remap = p->route.xcd_remap;
    info.route_nt_store = p->route.nt_store;
    info.route_split = p->route.split ? 1 : 0;
    info.tiles = p->tiles ? (p->tile_compact ? 2 : 1) : 0;
    info.tile_overflow = p->tile_overflow;
    info.tile_cap = p->tile_cap;
    info.route_tiled = p->route.tiled ? 1 : 0;
    info.route_window = p->route.window ? (p->route.window_sorted ? 2 : 1) : 0;
    info.win_frac = p->win_frac;
    info.mfma_resid_nnz = p->mfma_tiles ? p->mfma_rnnz : 0;
    info.mfma_tiles = p->mfma_tiles ? (p->mfma_tiles_lo ? 2 : 1) : 0;
    info.route_mfma = p->route.mfma ? 1 : 0;
    info.pair_vectors = p->pair_prow ? p->pair_nvec : 0;
    info.pair_padding = p->pair_prow ? pair_padding(p) : 0.0;
    info.pairs_built = p->pair_prow ? (p->pair_unsorted ? 2 : 1) : 0;
    info.route_pairs = p->route.pairs ? 1 : 0;
    info.merge_segments = p->merge_seg_row ? p->merge_nseg : 0;
    info.route_merge = p->route.merge ? 1 : 0;
    info.piece_order = p->seg_order != nullptr ? 1 : 0;
    info.generation = p->generation;
    info.device_bytes = plan_bytes(p);
    info.mem_limit = p->mem_limit;
    info.route_fused_split = p->route.fused_split ? 1 : 0;

    *out = info;
    return succeed();
}

SPMM_API int spmm_plan_route(spmm_plan_t p, int64_t N, int reduce) {
    if (!p) return fail(SPMM_E_INVALID_ARG, "plan is NULL");
    if (N <= 0) return fail(SPMM_E_INVALID_ARG, "N must be positive");
    if (reduce < SPMM_SUM || reduce > SPMM_MAX) return fail(SPMM_E_INVALID_ARG, "unknown reduce %d", reduce);
    static const float dummy[4] __attribute__((aligned(16))) = {0, 0, 0, 0};
    p->route = route_for(p, N, reduce, dummy, dummy, nullptr);
    p->route_N = N;
    return succeed();
}

SPMM_API int spmm_plan_partition(spmm_plan_t p, int64_t *seg_row, int64_t *seg_begin, int64_t *seg_end,
                                 int64_t seg_cap, int64_t *light, int64_t light_cap, int64_t *counts) {
    if (!p || !counts) return fail(SPMM_E_INVALID_ARG, "plan or counts is NULL");
    if (seg_cap < 0 || light_cap < 0) return fail(SPMM_E_INVALID_ARG, "negative capacity");
    if ((seg_cap > 0 && (!seg_row || !seg_begin || !seg_end)) || (light_cap > 0 && !light))
        return fail(SPMM_E_INVALID_ARG, "output array is NULL");
    DeviceGuard dg(p->device);
    const int64_t nh = p->split ? p->n_heavy : 0;
    const int64_t ns = p->split ? p->n_seg : 0;
    const int64_t nl = p->split ? p->n_light : p->M;
    counts[0] = nh;
    counts[1] = ns;
    counts[2] = nl;
    hipError_t e = hipSuccess;
    if (ns > 0 && seg_cap > 0) {
        std::vector<int> hr((size_t)nh), sf((size_t)nh + 1), sb((size_t)ns), se((size_t)ns);
        e = hipMemcpy(hr.data(), p->heavy_rows, sizeof(int) * nh, hipMemcpyDeviceToHost);
        if (e == hipSuccess) e = hipMemcpy(sf.data(), p->seg_first, sizeof(int) * (nh + 1), hipMemcpyDeviceToHost);
        if (e == hipSuccess) e = hipMemcpy(sb.data(), p->seg_begin, sizeof(int) * ns, hipMemcpyDeviceToHost);
        if (e == hipSuccess) e = hipMemcpy(se.data(), p->seg_end, sizeof(int) * ns, hipMemcpyDeviceToHost);
        if (e != hipSuccess) return fail_hip(e, "copy row split");
        for (int64_t h = 0; h < nh; ++h)
            for (int64_t s = sf[h]; s < sf[h + 1] && s < seg_cap; ++s) seg_row[s] = hr[h];
        for (int64_t s = 0; s < ns && s < seg_cap; ++s) {
            seg_begin[s] = sb[s];
            seg_end[s] = se[s];
        }
    }
    if (light_cap > 0) {
        if (p->split) {
            std::vector<int> rp((size_t)p->M + 1);
            e = hipMemcpy(rp.data(), p->rowptr, sizeof(int) * (p->M + 1), hipMemcpyDeviceToHost);
            if (e != hipSuccess) return fail_hip(e, "copy rowptr");
            int64_t n = 0;
            for (int64_t i = 0; i < p->M && n < light_cap; ++i)
                if (rp[i + 1] - rp[i] <= p->T) light[n++] = i;
        } else {
            for (int64_t i = 0; i < nl && i < light_cap; ++i) light[i] = i;
        }
    }
    return succeed();
}

SPMM_API int spmm_run(spmm_plan_t p, const float *B, float *C, int64_t *argmax, int64_t N, int reduce,
                      void *stream) {
    if (!p) return fail(SPMM_E_INVALID_ARG, "plan is NULL");
    if (N <= 0) return fail(SPMM_E_INVALID_ARG, "N must be positive (got %lld)", (long long)N);
    if (reduce < SPMM_SUM || reduce > SPMM_MAX) return fail(SPMM_E_INVALID_ARG, "unknown reduce %d", reduce);
    if (argmax && reduce != SPMM_MAX) return fail(SPMM_E_INVALID_ARG, "argmax is only produced by SPMM_MAX");
    if (N >= INT_MAX) return fail(SPMM_E_UNSUPPORTED, "N must be below 2^31 - 1");
    if (p->M == 0) return succeed();
    if (!is_device_ptr(C)) return fail(SPMM_E_INVALID_ARG, "C is NULL or not device memory");
    if (p->K > 0 && !is_device_ptr(B)) return fail(SPMM_E_INVALID_ARG, "B is NULL or not device memory");
    if (argmax && !is_device_ptr(argmax)) return fail(SPMM_E_INVALID_ARG, "argmax is not device memory");
    {
        const uintptr_t b0 = (uintptr_t)B, b1 = b0 + (uintptr_t)(p->K * N) * sizeof(float);
        const uintptr_t c0 = (uintptr_t)C, c1 = c0 + (uintptr_t)(p->M * N) * sizeof(float);
        const uintptr_t a0 = (uintptr_t)argmax, a1 = a0 + (uintptr_t)(p->M * N) * sizeof(int64_t);
        if (B && b0 < c1 && c0 < b1) return fail(SPMM_E_INVALID_ARG, "B overlaps C");
        if (B && argmax && b0 < a1 && a0 < b1) return fail(SPMM_E_INVALID_ARG, "B overlaps argmax");
        if (argmax && c0 < a1 && a0 < c1) return fail(SPMM_E_INVALID_ARG, "C overlaps argmax");
    }
    DeviceGuard dg(p->device);
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    const bool is_max = reduce == SPMM_MAX;
    const bool has_val = p->val != nullptr;

    Route r = route_for(p, N, reduce, B, C, argmax);
    if (r.mfma) {
        p->route = r;
        p->route_N = N;
        MfmaArgs ma;
        ma.atiles = p->mfma_tiles;
        ma.atiles_lo = p->mfma_tiles_lo;
        ma.tile_exp = p->mfma_tile_exp;
        ma.rowptr = p->rowptr;
        ma.rrowptr = p->mfma_rowptr;
        ma.rcol = p->mfma_col;
        ma.rval = p->mfma_val;
        ma.B = B;
        ma.C = C;
        ma.M = p->M;
        ma.K = p->K;
        ma.N = N;
        ma.nslices = r.slices;
        ma.mean = reduce == SPMM_MEAN;
        ma.xcd_remap = r.xcd_remap;
        const hipError_t e = launch_mfma(ma, has_val, s);
        if (e != hipSuccess) return fail_hip(e, "fp16 tile kernel launch");
        return succeed();
    }
    if (r.merge) {
        MergeKernelFn mf = merge_kernel(r.vec, has_val, is_max);
        if (!mf) return fail(SPMM_E_UNSUPPORTED, "no merge kernel for vec=%d", r.vec);
        p->route = r;
        p->route_N = N;
        MergeArgs ma;
        std::memset(&ma, 0, sizeof(ma));
        ma.rowptr = p->rowptr;
        ma.col = p->col;
        ma.val = p->val;
        ma.seg_row = p->merge_seg_row;
        ma.seg_entry = p->merge_seg_entry;
        ma.B = B;
        ma.C = C;
        ma.argmax = argmax;
        ma.carry = p->merge_carry;
        ma.carry_arg = p->merge_carry_arg;
        ma.carry_row = p->merge_carry_row;
        ma.M = p->M;
        ma.N = N;
        ma.nseg = p->merge_nseg;
        ma.mean = reduce == SPMM_MEAN;
        for (int64_t p0 = 0; p0 < N; p0 += kPartialWidth) {
            // a last pass narrower than one vector starts earlier (as for the
            // split's passes; the overlap is recomputed with the same bits)
            ma.c_end = std::min<int64_t>(N, p0 + kPartialWidth);
            ma.c_begin = std::min(p0, std::max<int64_t>(0, ma.c_end - r.vec));
            const hipError_t e = launch_merge(mf, ma, r.vec, is_max, s);
            if (e != hipSuccess) return fail_hip(e, "merge kernel launch");
        }
        return succeed();
    }
    if (r.pairs) {
        PairKernelFn pf = pair_kernel(r.lanes, r.vec, has_val, is_max);
        if (!pf) return fail(SPMM_E_UNSUPPORTED, "no panel kernel for lanes=%d vec=%d", r.lanes, r.vec);
        if (r.slices > 65535) return fail(SPMM_E_UNSUPPORTED, "N = %lld needs too many column slices", (long long)N);
        p->route = r;
        p->route_N = N;
        PairArgs pa;
        std::memset(&pa, 0, sizeof(pa));
        pa.prow = p->pair_prow;
        pa.pcol = p->pair_col;
        pa.pval = p->pair_val;
        pa.rowptr = p->rowptr;
        pa.B = B;
        pa.C = C;
        pa.argmax = argmax;
        pa.M = p->M;
        pa.N = N;
        pa.npanels = (p->M + 1) / 2;
        pa.mean = reduce == SPMM_MEAN;
        pa.xcd_remap = r.xcd_remap;
        const hipError_t e = launch_pairs(pf, pa, r.lanes, r.slices, s);
        if (e != hipSuccess) return fail_hip(e, "panel kernel launch");
        return succeed();
    }
    // 4-lane float4 row tiles at mean degree 8 and above: entries in batches
    // of 4, not 8 (fewer idle slots in a row's last batch: rows of exactly 10
    // entries fill 10 of 12 slots instead of 10 of 16; diffusion graph, 16
    // floats, mean: 0.0732 vs 0.0752 ms; at mean degree 3 the batches of 8
    // stay faster, road graph 16 floats: 0.0400 vs 0.0420 ms)
    const bool batch4 = r.tiled && r.lanes == 4 && r.vec == 4 && r.coarsen == 1 && !is_max && p->mean_deg >= 8.0;
    RowKernelKey key{r.lanes, r.vec, r.coarsen, has_val, is_max, false, r.tiled, r.compact, batch4};
    RowKernelFn fn = row_kernel(key);
    if (!fn) return fail(SPMM_E_UNSUPPORTED, "no kernel for lanes=%d vec=%d coarsen=%d", r.lanes, r.vec, r.coarsen);
    if (r.slices > 65535) return fail(SPMM_E_UNSUPPORTED, "N = %lld needs too many column slices", (long long)N);
    p->route = r;
    p->route_N = N;

    RowArgs a;
    std::memset(&a, 0, sizeof(a));
    a.rowptr = p->rowptr;
    a.col = p->col;
    a.val = p->val;
    a.tiles = p->tiles;
    a.tile_cap = p->tile_cap;
    a.tile_words = p->tile_words;
    a.B = B;
    a.out = C;
    a.argmax = argmax;
    a.ldo = N;
    a.N = N;
    a.K = p->K;
    a.c_begin = 0;
    a.c_end = N;
    a.ntasks = p->M;
    a.skip_above = p->split ? (int)std::min<int64_t>(p->T, INT_MAX) : INT_MAX;
    a.mean = reduce == SPMM_MEAN;
    a.xcd_remap = r.xcd_remap;
    a.nt_store = r.nt_store;
    a.win_lo = p->win_lo;
    a.win_in = p->win_in;
    // arguments of the piece kernel for columns [w0, w1)
    auto piece_args = [&](int64_t w0, int64_t w1) {
        RowArgs pa;
        std::memset(&pa, 0, sizeof(pa));
        pa.seg_begin = p->seg_begin;
        pa.seg_end = p->seg_end;
        pa.col = p->col;
        pa.val = p->val;
        pa.B = B;
        pa.out = p->partial;
        pa.part_arg = p->part_arg;
        pa.ldo = kPartialWidth;
        pa.N = N;
        pa.K = p->K;
        pa.c_begin = w0;
        pa.c_end = w1;
        pa.ntasks = p->n_seg;
        pa.xcd_remap = 0;
        pa.nt_store = 0;
        pa.task_perm = p->seg_order;
        return pa;
    };
    const bool split = p->split && p->n_seg > 0;
    // a split product of one column pass: light rows and pieces in one dispatch
    const bool fused = split && p->opt_split_fused != 0 && !r.window && !r.tiled && N <= kPartialWidth &&
                       split_fused_available(r.lanes, r.vec, r.coarsen);
    hipError_t e = hipSuccess;
    bool fused_done = false;
    if (fused) {
        e = launch_split_fused(r.lanes, has_val, is_max, a, piece_args(0, N), r.slices, s, &fused_done);
        if (e != hipSuccess) return fail_hip(e, "split kernel launch");
    }
    if (!fused_done) {
        e = r.window ? launch_window(a, has_val, is_max, r.window_sorted, s) : launch_rows(fn, a, 64 / r.lanes, r.slices, s);
        if (e != hipSuccess) return fail_hip(e, "row kernel launch");
    }
    p->route.fused_split = fused_done;

    if (split) {
        for (int64_t p0 = 0; p0 < N; p0 += kPartialWidth) {
            const int64_t w1 = std::min<int64_t>(N, p0 + kPartialWidth);
            // a last pass narrower than one vector starts earlier, so that its
            // vectors stay inside the pass (the overlap is recomputed with the
            // same bits)
            const int64_t w0 = std::min(p0, std::max<int64_t>(0, w1 - r.vec));
            const int64_t Wv = (w1 - w0 + r.vec - 1) / r.vec;
            const int F = Wv > 64 ? 2 : 1;
            const int slices = (int)((Wv + 64 * F - 1) / (64 * F));
            if (!fused_done) {
                RowKernelFn pf = row_kernel(RowKernelKey{64, r.vec, F, has_val, is_max, true, false, false, false});
                if (!pf) return fail(SPMM_E_UNSUPPORTED, "no piece kernel for vec=%d", r.vec);
                e = launch_rows(pf, piece_args(w0, w1), 1, slices, s);
                if (e != hipSuccess) return fail_hip(e, "piece kernel launch");
            }
            CombineArgs ca;
            ca.heavy_rows = p->heavy_rows;
            ca.seg_first = p->seg_first;
            ca.rowptr = p->rowptr;
            ca.partial = p->partial;
            ca.part_arg = p->part_arg;
            ca.C = C;
            ca.argmax = argmax;
            ca.N = N;
            ca.c_begin = w0;
            ca.c_end = w1;
            ca.n_heavy = p->n_heavy;
            ca.mean = reduce == SPMM_MEAN;
            e = launch_combine(ca, is_max, s);
            if (e != hipSuccess) return fail_hip(e, "combine launch");
        }
    }
    return succeed();
}

SPMM_API int spmm_plan_features(spmm_plan_t p, int64_t V, struct spmm_features *out) {
    if (!p || !out) return fail(SPMM_E_INVALID_ARG, "plan or output is NULL");
    if (V < 1 || V > 64) return fail(SPMM_E_INVALID_ARG, "V must be in [1, 64]");
    DeviceGuard dg(p->device);
    PlanScope budget(p);
    struct spmm_features f;
    std::memset(&f, 0, sizeof(f));
    f.n = p->M;
    f.nnz = p->nnz;
    f.dmax = p->dmax;
    f.V = V;
    f.n_nonempty = p->M - p->n_empty;
    f.delta = p->M > 0 ? (double)f.n_nonempty / (double)p->M : 0.0;
    f.mean_deg = p->mean_deg;
    f.cv_deg = p->cv_deg;
    if (f.n_nonempty > 0) {
        // empty rows add nothing to the degree sums: the same exact fold as the plan's CV
        const int64_t n = f.n_nonempty;
        f.mean_deg_nonempty = (double)p->nnz / (double)n;
        const __int128 num = (__int128)n * (__int128)p->sum_deg2 - (__int128)p->nnz * (__int128)p->nnz;
        const double var = (double)num / ((double)n * (double)n);
        f.cv_deg_nonempty = f.mean_deg_nonempty > 0 ? std::sqrt(std::max(var, 0.0)) / f.mean_deg_nonempty : 0.0;
    }
    f.density = (p->M > 0 && p->K > 0) ? (double)p->nnz / ((double)p->M * (double)p->K) : 0.0;
    f.split_ratio = p->M > 0 ? (double)(p->split ? p->n_light + p->n_seg : p->M) / (double)p->M : 1.0;
    f.win_frac = p->win_frac;
    hipError_t e = hipDeviceSynchronize();
    int64_t bw_sum = 0, bw_max = 0, rows = 0, distinct = 0, vectors = 0;
    if (e == hipSuccess)
        e = pattern_features(p->rowptr, p->col, p->M, p->K, p->nnz, V, &bw_sum, &bw_max, &rows, &distinct, &vectors);
    if (e != hipSuccess) return fail_hip(e, "feature pass");
    f.mean_bandwidth = rows > 0 ? (double)bw_sum / (double)rows : 0.0;
    f.max_bandwidth = bw_max;
    f.nnz_distinct = distinct;
    f.nnz_vectors = vectors;
    f.padding_ratio = vectors > 0 ? 1.0 - (double)distinct / ((double)vectors * (double)V) : 0.0;
    *out = f;
    return succeed();
}

SPMM_API int spmm_plan_reorder(spmm_plan_t p, int method, int64_t *perm) {
    if (!p) return fail(SPMM_E_INVALID_ARG, "plan is NULL");
    if (method != SPMM_REORDER_RCM) return fail(SPMM_E_INVALID_ARG, "unknown reordering method %d", method);
    if (p->M != p->K) return fail(SPMM_E_INVALID_ARG, "reordering needs a square matrix (M = %lld, K = %lld)",
                                  (long long)p->M, (long long)p->K);
    if (p->M == 0) return succeed();
    if (!is_device_ptr(perm)) return fail(SPMM_E_INVALID_ARG, "perm is NULL or not device memory");
    DeviceGuard dg(p->device);
    PlanScope budget(p);
    hipError_t e = hipDeviceSynchronize();
    int64_t levels = 0;
    if (e == hipSuccess) e = rcm_order(p->rowptr, p->col, p->M, p->nnz, perm, &levels);
    if (e != hipSuccess) return fail_hip(e, "reordering");
    return succeed();
}

SPMM_API spmm_plan_t spmm_plan_permute(spmm_plan_t p, const int64_t *perm) {
    if (!p) {
        fail(SPMM_E_INVALID_ARG, "plan is NULL");
        return nullptr;
    }
    if (p->M != p->K) {
        fail(SPMM_E_INVALID_ARG, "permuting needs a square matrix");
        return nullptr;
    }
    if (p->M > 0 && !is_device_ptr(perm)) {
        fail(SPMM_E_INVALID_ARG, "perm is NULL or not device memory");
        return nullptr;
    }
    DeviceGuard dg(p->device);
    PlanScope budget(p);
    int64_t *rp = nullptr, *cl = nullptr;
    float *vl = nullptr;
    if (dev_alloc(&rp, p->M + 1, "permuted rowptr") || dev_alloc(&cl, p->nnz, "permuted col") ||
        (p->val && dev_alloc(&vl, p->nnz, "permuted val"))) {
        dev_free(rp);
        dev_free(cl);
        dev_free(vl);
        return nullptr;
    }
    bool bad = false;
    hipError_t e = hipDeviceSynchronize();
    if (e == hipSuccess && p->M > 0) e = permute_csr(p->rowptr, p->col, p->val, p->M, p->nnz, perm, rp, cl, vl, &bad);
    else if (e == hipSuccess) e = hipMemset(rp, 0, sizeof(int64_t));
    spmm_plan_t t = nullptr;
    if (e != hipSuccess) fail_hip(e, "permute");
    else if (bad) fail(SPMM_E_INVALID_ARG, "perm is not a permutation of [0, %lld)", (long long)p->M);
    else t = spmm_plan_create(rp, cl, vl, p->M, p->K);
    dev_free(rp);
    dev_free(cl);
    dev_free(vl);
    return t;
}

// Argument checks shared by the edge-list entry points.
static int check_coo_args(const int64_t *row, const int64_t *col, const float *val, int64_t E, int64_t M, int64_t K,
                   const int64_t *rowptr_out, const int64_t *col_out, const float *val_out) {
    if (E < 0 || M < 0 || K < 0) return fail(SPMM_E_INVALID_ARG, "negative size");
    if (E >= INT_MAX || M >= INT_MAX || K >= INT_MAX)
        return fail(SPMM_E_UNSUPPORTED, "E, M and K must be below 2^31 - 1");
    if (!is_device_ptr(rowptr_out)) return fail(SPMM_E_INVALID_ARG, "rowptr_out is NULL or not device memory");
    if (E > 0) {
        if (!is_device_ptr(row) || !is_device_ptr(col))
            return fail(SPMM_E_INVALID_ARG, "row / col are NULL or not device memory");
        if (!is_device_ptr(col_out)) return fail(SPMM_E_INVALID_ARG, "col_out is NULL or not device memory");
        if (val && !is_device_ptr(val)) return fail(SPMM_E_INVALID_ARG, "val is not device memory");
        if (val && !is_device_ptr(val_out)) return fail(SPMM_E_INVALID_ARG, "val_out is NULL or not device memory");
    }
    return SPMM_OK;
}

SPMM_API int spmm_coo_to_csr(const int64_t *row, const int64_t *col, const float *val, int64_t E, int64_t M,
                             int64_t K, int64_t *rowptr_out, int64_t *col_out, float *val_out) {
    if (const int st = check_coo_args(row, col, val, E, M, K, rowptr_out, col_out, val_out)) return st;
    hipError_t e = hipDeviceSynchronize();
    if (e != hipSuccess) return fail_hip(e, "synchronise before the edge-list sort");
    PlanScope budget(nullptr);
    int64_t bad = -1;
    e = coo_to_csr(row, col, val, E, M, K, rowptr_out, col_out, val ? val_out : nullptr, &bad, nullptr);
    if (e != hipSuccess) return fail_hip(e, "edge-list sort");
    if (bad >= 0) return fail(SPMM_E_BAD_CSR, "edge %lld has a row outside [0, %lld) or a column outside [0, %lld)",
                              (long long)bad, (long long)M, (long long)K);
    return succeed();
}

SPMM_API int spmm_coo_to_csr_noalloc(const int64_t *row, const int64_t *col, const float *val, int64_t E,
                                     int64_t M, int64_t K, int64_t *rowptr_out, int64_t *col_out,
                                     float *val_out) {
    if (const int st = check_coo_args(row, col, val, E, M, K, rowptr_out, col_out, val_out)) return st;
    if (E > kNoAllocMaxEdges)
        return fail(SPMM_E_UNSUPPORTED, "the allocation-free edge-list sort takes at most %lld edges (got %lld)",
                    (long long)kNoAllocMaxEdges, (long long)E);
    hipError_t e = hipDeviceSynchronize();
    if (e != hipSuccess) return fail_hip(e, "synchronise before the edge-list sort");
    int64_t bad = -1;
    int too_large = 0;
    e = coo_to_csr_noalloc(row, col, val, E, M, K, rowptr_out, col_out, val ? val_out : nullptr, &bad, &too_large);
    if (e != hipSuccess) return fail_hip(e, "edge-list sort");
    if (too_large)
        return fail(SPMM_E_UNSUPPORTED, "the edge-list sort of %lld edges does not fit the %lld-byte workspace",
                    (long long)E, (long long)kNoAllocScratchBytes);
    if (bad >= 0) return fail(SPMM_E_BAD_CSR, "edge %lld has a row outside [0, %lld) or a column outside [0, %lld)",
                              (long long)bad, (long long)M, (long long)K);
    return succeed();
}

SPMM_API spmm_plan_t spmm_plan_transpose(spmm_plan_t p, int scale) {
    if (!p) {
        fail(SPMM_E_INVALID_ARG, "plan is NULL");
        return nullptr;
    }
    if (scale != 0 && scale != 1) {
        fail(SPMM_E_INVALID_ARG, "scale must be 0 or 1");
        return nullptr;
    }
    DeviceGuard dg(p->device);
    PlanScope budget(p);
    int64_t *rp = nullptr, *cl = nullptr;
    float *vl = nullptr;
    const bool want_val = p->val != nullptr || scale == 1;
    int st;
    if ((st = dev_alloc(&rp, p->K + 1, "transposed rowptr")) || (st = dev_alloc(&cl, p->nnz, "transposed col")) ||
        (want_val && (st = dev_alloc(&vl, p->nnz, "transposed val")))) {
        dev_free(rp);
        dev_free(cl);
        dev_free(vl);
        return nullptr;
    }
    hipError_t e = hipDeviceSynchronize();
    if (e == hipSuccess)
        e = transpose_csr(p->rowptr, p->col, p->val, p->M, p->K, p->nnz, scale == 1, rp, cl, vl, nullptr);
    spmm_plan_t t = nullptr;
    if (e != hipSuccess) fail_hip(e, "transpose");
    else t = spmm_plan_create(rp, cl, vl, p->K, p->M);
    dev_free(rp);
    dev_free(cl);
    dev_free(vl);
    return t;
}

SPMM_API int spmm_max_backward(spmm_plan_t pt, const int64_t *argmax, const float *dC, float *dB, int64_t N,
                               void *stream) {
    if (!pt) return fail(SPMM_E_INVALID_ARG, "plan is NULL");
    if (N <= 0) return fail(SPMM_E_INVALID_ARG, "N must be positive");
    if (N >= INT_MAX) return fail(SPMM_E_UNSUPPORTED, "N must be below 2^31 - 1");
    if (pt->val) return fail(SPMM_E_UNSUPPORTED, "max backward needs the transpose of an unweighted adjacency");
    if (pt->M == 0) return succeed();
    if (!is_device_ptr(dB)) return fail(SPMM_E_INVALID_ARG, "dB is NULL or not device memory");
    if (pt->K > 0 && (!is_device_ptr(argmax) || !is_device_ptr(dC)))
        return fail(SPMM_E_INVALID_ARG, "argmax / dC are NULL or not device memory");
    DeviceGuard dg(pt->device);
    MaxGradArgs a;
    a.rowptr_t = pt->rowptr;
    a.col_t = pt->col;
    a.argmax = argmax;
    a.dC = dC;
    a.dB = dB;
    a.rows = pt->M;
    a.N = N;
    const hipError_t e = launch_maxgrad(a, reinterpret_cast<hipStream_t>(stream));
    if (e != hipSuccess) return fail_hip(e, "max backward launch");
    return succeed();
}
