// Vectorized blocking with V = 2 (ParamSpMM section 3.1 and PCSR, section
// 4.2): rows 2g and 2g+1 form a panel whose entries are grouped into nonzero
// vectors, one per column present in either row, so one gather of B's row
// serves both rows.  ParamSpMM limits V to {1, 2}; V = 2 pays when the rows of
// a panel share columns (a low padding ratio, eq. 2).
//
// Panel format (built once, on request):
//   prow  int32 [npanels + 1]  vector range of each panel
//   pcol  uint32 [nvec]         column | (row 2g absent) << 30 | (row 2g+1 absent) << 31
//   pval  fp32 [nvec][2]        the two rows' values (0 where absent; weighted only)
// A column stored k times in one row and m times in the other gives
// max(k, m) vectors, the i-th pairing the rows' i-th occurrences, so every
// stored entry is used exactly once.  Vectors run in ascending column order
// (occurrences in stored order): for rows stored with ascending columns this
// is the stored order, and the kernel below reproduces the row kernel's bits.
//
// Kernel: the row kernel's mapping with a panel in place of a row (G lanes
// per panel, 64/G panels per wave, vectors staged in LDS, predicated batches);
// each vector's B slice is loaded once and folded into both rows'
// accumulators (skipping absent slots), so the absent half of a vector costs
// no arithmetic and no rounding.
#include <hipcub/hipcub.hpp>

#include <climits>
#include <vector>

#include "alloc.h"
#include "row_kernel_impl.h"

namespace gspmm {

namespace {

constexpr unsigned kAbsent0 = 1u << 30;
constexpr unsigned kAbsent1 = 1u << 31;
constexpr unsigned kColMask = kAbsent0 - 1u;

// Key of entry p of row r: panel, column, then the row's half of the panel.
__global__ __launch_bounds__(kBlock) void pair_keys_kernel(const int *__restrict__ rowptr, const int *__restrict__ col,
                                                           int64_t M, int64_t K, uint64_t *__restrict__ keys,
                                                           int *__restrict__ pos) {
    const int lane = threadIdx.x & 63;
    const int64_t stride = (int64_t)gridDim.x * kWaves;
    for (int64_t row = (int64_t)blockIdx.x * kWaves + (threadIdx.x >> 6); row < M; row += stride) {
        const uint64_t base = (uint64_t)(row >> 1) * (uint64_t)K;
        const uint64_t half = (uint64_t)(row & 1);
        for (int64_t p = (int64_t)rowptr[row] + lane; p < rowptr[row + 1]; p += 64) {
            keys[p] = ((base + (uint64_t)col[p]) << 1) | half;
            pos[p] = (int)p;
        }
    }
}

// One thread per panel walks the panel's sorted entries (they occupy
// [rowptr[2g], rowptr[min(2g+2, M)]) of the sorted arrays).  count: vectors
// per panel (and whether the panel's rows are stored with ascending columns);
// write: the vectors themselves.
template <bool WRITE>
__global__ __launch_bounds__(kBlock) void pair_walk_kernel(const int *__restrict__ rowptr,
                                                           const int *__restrict__ col,
                                                           const float *__restrict__ val, int64_t M, int64_t K,
                                                           const uint64_t *__restrict__ skeys,
                                                           const int *__restrict__ spos, int *__restrict__ count,
                                                           int *__restrict__ unsorted, const int *__restrict__ prow,
                                                           unsigned *__restrict__ pcol, float *__restrict__ pval) {
    const int64_t npanels = (M + 1) / 2;
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t g = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; g < npanels; g += stride) {
        const int s = rowptr[2 * g];
        const int e = rowptr[min(2 * g + 2, M)];
        const uint64_t pbase = (uint64_t)g * (uint64_t)K;
        int out = WRITE ? prow[g] : 0;
        int nvec = 0;
        for (int i = s; i < e;) {
            const uint64_t kh = skeys[i] >> 1;
            int j = i;
            while (j < e && skeys[j] == (kh << 1)) ++j;
            int k = j;
            while (k < e && (skeys[k] >> 1) == kh) ++k;
            const int n0 = j - i, n1 = k - j;
            const int nv = max(n0, n1);
            if constexpr (WRITE) {
                const unsigned c = (unsigned)(kh - pbase);
                for (int r = 0; r < nv; ++r) {
                    const int v = out + r;
                    pcol[v] = c | (r >= n0 ? kAbsent0 : 0u) | (r >= n1 ? kAbsent1 : 0u);
                    if (pval) {
                        pval[2 * (int64_t)v] = r < n0 ? val[spos[i + r]] : 0.0f;
                        pval[2 * (int64_t)v + 1] = r < n1 ? val[spos[j + r]] : 0.0f;
                    }
                }
                out += nv;
            }
            nvec += nv;
            i = k;
        }
        if constexpr (!WRITE) {
            count[g] = nvec;
            bool bad = false;
            for (int64_t r = 2 * g; r < min(2 * g + 2, M); ++r)
                for (int p = rowptr[r] + 1; p < rowptr[r + 1]; ++p) bad = bad || col[p] < col[p - 1];
            if (bad) *unsorted = 1;   // every writer stores the same value
        }
    }
}

// Folds vectors [lo, hi) of the staged list into both rows' accumulators.
template <int VEC, bool HAS_VAL, bool IS_MAX>
__device__ __forceinline__ void consume_pair(const unsigned *cp, const float *vp, int lo, int hi,
                                             const float *__restrict__ Bp, int64_t N, int colf, bool ok,
                                             float (&acc)[2][VEC], int (&arg)[2][VEC]) {
    constexpr int U = VEC == 4 ? 4 : 8;
    for (int k = lo; k < hi; k += U) {
        unsigned cw[U];
        float w[U][2];
        bool vld[U];
        float bv[U][VEC];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            vld[u] = k + u < hi;
            const int kk = vld[u] ? k + u : lo;
            cw[u] = cp[kk];
            w[u][0] = HAS_VAL ? vp[2 * kk] : 1.0f;
            w[u][1] = HAS_VAL ? vp[2 * kk + 1] : 1.0f;
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
#pragma unroll
            for (int e = 0; e < VEC; ++e) bv[u][e] = 0.0f;
            if (vld[u] && ok) load_vec<VEC>(Bp + elem_off(cw[u] & kColMask, N, colf), bv[u]);
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            if (!vld[u]) continue;
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                if (cw[u] & (h ? kAbsent1 : kAbsent0)) continue;
#pragma unroll
                for (int e = 0; e < VEC; ++e) {
                    if constexpr (IS_MAX) {
                        const float t = HAS_VAL ? w[u][h] * bv[u][e] : bv[u][e];
                        if (arg[h][e] < 0 || t > acc[h][e]) {
                            acc[h][e] = t;
                            arg[h][e] = (int)(cw[u] & kColMask);
                        }
                    } else {
                        acc[h][e] = HAS_VAL ? __builtin_fmaf(w[u][h], bv[u][e], acc[h][e]) : acc[h][e] + bv[u][e];
                    }
                }
            }
        }
    }
}

template <int G, int VEC, bool HAS_VAL, bool IS_MAX>
__global__ __launch_bounds__(kBlock) void pair_kernel_t(PairArgs a) {
    static_assert(G >= 4 && G <= 64 && (64 % G) == 0, "lanes per panel");
    constexpr int R = 64 / G;          // panels per wave
    constexpr int SL = G * VEC;        // columns per slice
    constexpr int NT = kChunk / 64;
    __shared__ unsigned s_col[kWaves][kChunk];
    __shared__ float s_val[kWaves][HAS_VAL ? 2 * kChunk : 1];

    const int lane = threadIdx.x & 63;
    const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);   // uniform per wave
    const int64_t gx = gridDim.x;
    int64_t lin = (int64_t)blockIdx.y * gx + blockIdx.x;
    if (a.xcd_remap) lin = xcd_remap_block(lin, gx * (int64_t)gridDim.y);
    const int64_t bx = lin % gx, by = lin / gx;
    const int64_t task0 = a.task_base + (bx * kWaves + wv) * R;
    if (task0 >= a.npanels) return;                     // uniform per wave
    const int g = lane % G;
    const int sub = lane / G;
    const int64_t c0 = by * SL + (int64_t)g * VEC;
    const bool ok = c0 < a.N;
    // a vector that would run past column N ends there instead (the launch
    // guarantees N >= VEC); it writes only the columns past its neighbour's
    const int colf = (int)(VEC > 1 && c0 > a.N - VEC ? a.N - VEC : c0);
    const int skip = (int)(c0 - colf);

    const int64_t v = task0 + sub;
    const bool live = v < a.npanels;
    int beg = 0, end = 0;
    if (live) {
        beg = a.prow[v];
        end = a.prow[v + 1];
    }
    const int deg = end - beg;
    const int beg0 = __builtin_amdgcn_readfirstlane(beg);   // lane 0's panel is task0 < npanels
    int off = 0, total = 0;
#pragma unroll
    for (int s = 0; s < R; ++s) {
        const int ds = __builtin_amdgcn_readlane(deg, s * G);
        off += (s < sub) ? ds : 0;
        total += ds;
    }

    float acc[2][VEC];
    int arg[2][VEC];
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int e = 0; e < VEC; ++e) {
            acc[h][e] = IS_MAX ? -INFINITY : 0.0f;
            arg[h][e] = -1;
        }

    for (int64_t cb64 = 0; cb64 < total; cb64 += kChunk) {   // 64-bit: total may lie within kChunk of 2^31
        const int cb = (int)cb64;
        const int cn = min(kChunk, total - cb);
        const int nt = (cn + 63) >> 6;
        unsigned cr[NT];
        float vr[NT][2];
#pragma unroll
        for (int t = 0; t < NT; ++t) {
            if (t < nt) {
                const int p = beg0 + cb + min(t * 64 + lane, cn - 1);
                cr[t] = a.pcol[p];
                if constexpr (HAS_VAL) {
                    const f32x2 w2 = *reinterpret_cast<const f32x2 *>(a.pval + 2 * (int64_t)p);
                    vr[t][0] = w2.x;
                    vr[t][1] = w2.y;
                }
            }
        }
#pragma unroll
        for (int t = 0; t < NT; ++t) {
            if (t < nt) {
                s_col[wv][t * 64 + lane] = cr[t];
                if constexpr (HAS_VAL) {
                    s_val[wv][2 * (t * 64 + lane)] = vr[t][0];
                    s_val[wv][2 * (t * 64 + lane) + 1] = vr[t][1];
                }
            }
        }
        wave_lds_sync();
        const int lo = max(off, cb) - cb;
        const int hi = min(off + deg, cb + cn) - cb;
        consume_pair<VEC, HAS_VAL, IS_MAX>(s_col[wv], s_val[wv], lo, hi, a.B, a.N, colf, ok, acc, arg);
        wave_lds_sync();
    }

    if (!live || !ok) return;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        const int64_t row = 2 * v + h;
        if (row >= a.M) break;
        const int d = a.rowptr[row + 1] - a.rowptr[row];
        float res[VEC];
        int ar[VEC];
#pragma unroll
        for (int e = 0; e < VEC; ++e) {
            if constexpr (IS_MAX) {
                res[e] = d > 0 ? acc[h][e] : 0.0f;
                ar[e] = d > 0 ? arg[h][e] : -1;
            } else {
                res[e] = acc[h][e];
            }
        }
        if constexpr (!IS_MAX) mean_divide<VEC>(a.mean != 0, d, res);
        store_vec<VEC>(a.C + row * a.N + colf, res, false, skip);
        if constexpr (IS_MAX)
            if (a.argmax) store_arg64<VEC>(a.argmax + row * a.N + colf, ar, skip);
    }
}

template <int G, int VEC>
PairKernelFn pick_pair(bool has_val, bool is_max) {
    if (is_max) return has_val ? pair_kernel_t<G, VEC, true, true> : pair_kernel_t<G, VEC, false, true>;
    return has_val ? pair_kernel_t<G, VEC, true, false> : pair_kernel_t<G, VEC, false, false>;
}

template <int VEC>
PairKernelFn pick_pair_vec(int lanes, bool has_val, bool is_max) {
    switch (lanes) {
        case 4: return pick_pair<4, VEC>(has_val, is_max);
        case 8: return pick_pair<8, VEC>(has_val, is_max);
        case 16: return pick_pair<16, VEC>(has_val, is_max);
        case 32: return pick_pair<32, VEC>(has_val, is_max);
        case 64: return pick_pair<64, VEC>(has_val, is_max);
        default: return nullptr;
    }
}

int64_t walk_grid(int64_t n) { return std::max<int64_t>(1, std::min<int64_t>((n + kBlock - 1) / kBlock, 1 << 16)); }

}  // namespace

namespace {

constexpr int kCountBlocks = 1024;

// Nonzero vectors of the V = 2 panels of a plan whose rows are all stored with
// ascending columns: one thread per panel merges its two sorted rows (equal
// columns pair one occurrence of each), so no sort is needed.  One partial
// count per block, folded on the host.
__global__ __launch_bounds__(kBlock) void pair_count_sorted_kernel(const int *__restrict__ rowptr,
                                                                   const int *__restrict__ col, int64_t M,
                                                                   int64_t *__restrict__ partial) {
    const int64_t npanels = (M + 1) / 2;
    const int64_t stride = (int64_t)gridDim.x * kBlock;
    int64_t n = 0;
    for (int64_t g = (int64_t)blockIdx.x * kBlock + threadIdx.x; g < npanels; g += stride) {
        int i = rowptr[2 * g];
        const int ie = rowptr[2 * g + 1];
        int j = ie;
        const int je = rowptr[min(2 * g + 2, M)];
        while (i < ie && j < je) {
            const int a = col[i], b = col[j];
            i += a <= b;
            j += b <= a;
            ++n;
        }
        n += (ie - i) + (je - j);
    }
    __shared__ int64_t sh[kBlock];
    sh[threadIdx.x] = n;
    __syncthreads();
    for (int o = kBlock / 2; o > 0; o >>= 1) {
        if (threadIdx.x < o) sh[threadIdx.x] += sh[threadIdx.x + o];
        __syncthreads();
    }
    if (threadIdx.x == 0) partial[blockIdx.x] = sh[0];
}

// Panels of a plan whose rows are all stored with ascending columns, by a
// merge of each panel's two rows (the same vectors, in the same order, as the
// sort-based walk): count writes vectors per panel, write the vectors.
template <bool WRITE>
__global__ __launch_bounds__(kBlock) void pair_merge_kernel(const int *__restrict__ rowptr,
                                                            const int *__restrict__ col,
                                                            const float *__restrict__ val, int64_t M,
                                                            int *__restrict__ count, const int *__restrict__ prow,
                                                            unsigned *__restrict__ pcol, float *__restrict__ pval) {
    const int64_t npanels = (M + 1) / 2;
    const int64_t stride = (int64_t)gridDim.x * kBlock;
    for (int64_t g = (int64_t)blockIdx.x * kBlock + threadIdx.x; g < npanels; g += stride) {
        int i = rowptr[2 * g];
        const int ie = rowptr[2 * g + 1];
        int j = ie;
        const int je = rowptr[min(2 * g + 2, M)];
        int v = WRITE ? prow[g] : 0;
        while (i < ie || j < je) {
            const int a = i < ie ? col[i] : INT_MAX;
            const int b = j < je ? col[j] : INT_MAX;
            const bool t0 = i < ie && a <= b;        // row 2g takes part
            const bool t1 = j < je && b <= a;        // row 2g+1 takes part
            if constexpr (WRITE) {
                pcol[v] = (unsigned)(t0 ? a : b) | (t0 ? 0u : kAbsent0) | (t1 ? 0u : kAbsent1);
                if (pval) {
                    pval[2 * (int64_t)v] = t0 ? val[i] : 0.0f;
                    pval[2 * (int64_t)v + 1] = t1 ? val[j] : 0.0f;
                }
            }
            i += t0;
            j += t1;
            ++v;
        }
        if constexpr (!WRITE) count[g] = v;
    }
}

}  // namespace

hipError_t pair_count_sorted(const int *rowptr, const int *col, int64_t M, int64_t *vectors) {
    *vectors = 0;
    const int64_t npanels = (M + 1) / 2;
    if (npanels == 0) return hipSuccess;
    const int64_t nb = std::max<int64_t>(1, std::min<int64_t>((npanels + kBlock - 1) / kBlock, kCountBlocks));
    int64_t *partial = nullptr;
    hipError_t e = dmalloc(&partial, sizeof(int64_t) * (size_t)nb, "panel count records");
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(pair_count_sorted_kernel, dim3((unsigned)nb), dim3(kBlock), 0, nullptr, rowptr, col, M,
                       partial);
    std::vector<int64_t> h((size_t)nb);
    e = hipGetLastError();
    if (e == hipSuccess) e = hipMemcpy(h.data(), partial, sizeof(int64_t) * (size_t)nb, hipMemcpyDeviceToHost);
    dfree(partial);
    if (e != hipSuccess) return e;
    for (int64_t x : h) *vectors += x;
    return hipSuccess;
}

// Panels of a plan whose rows are all sorted: per-panel merge counts, their
// exclusive scan, then the merge again writing the vectors.
hipError_t pair_build_sorted(const int *rowptr, const int *col, const float *val, int64_t M, int *prow,
                             PairOutput *out) {
    const int64_t npanels = (M + 1) / 2;
    int *cnt = nullptr;
    void *scan_tmp = nullptr;
    size_t scan_bytes = 0;
    hipError_t e = dmalloc(&cnt, sizeof(int) * (size_t)(npanels + 1), "panel counts");
    if (e == hipSuccess) e = hipMemset(cnt + npanels, 0, sizeof(int));
    if (e == hipSuccess && npanels > 0) {
        hipLaunchKernelGGL(pair_merge_kernel<false>, dim3((unsigned)walk_grid(npanels)), dim3(kBlock), 0, nullptr,
                           rowptr, col, val, M, cnt, nullptr, nullptr, nullptr);
        e = hipGetLastError();
    }
    if (e == hipSuccess) e = hipcub::DeviceScan::ExclusiveSum(nullptr, scan_bytes, cnt, prow, (int)(npanels + 1));
    if (e == hipSuccess) e = dmalloc(&scan_tmp, scan_bytes > 0 ? scan_bytes : 1, "panel scan storage");
    if (e == hipSuccess) e = hipcub::DeviceScan::ExclusiveSum(scan_tmp, scan_bytes, cnt, prow, (int)(npanels + 1));
    int nvec = 0;
    if (e == hipSuccess) e = hipMemcpy(&nvec, prow + npanels, sizeof(int), hipMemcpyDeviceToHost);
    if (e == hipSuccess && nvec > 0) {
        e = dmalloc(&out->pcol, sizeof(unsigned) * (size_t)nvec, "panel columns");
        if (e == hipSuccess && val) e = dmalloc(&out->pval, sizeof(float) * 2 * (size_t)nvec, "panel values");
        if (e == hipSuccess) {
            hipLaunchKernelGGL(pair_merge_kernel<true>, dim3((unsigned)walk_grid(npanels)), dim3(kBlock), 0,
                               nullptr, rowptr, col, val, M, nullptr, prow, out->pcol, out->pval);
            e = hipGetLastError();
        }
        if (e == hipSuccess) e = hipDeviceSynchronize();
        if (e != hipSuccess) {
            dfree(out->pcol);
            dfree(out->pval);
            out->pcol = nullptr;
            out->pval = nullptr;
        }
    }
    out->nvec = nvec;
    dfree(cnt);
    dfree(scan_tmp);
    return e;
}

hipError_t pair_build(const int *rowptr, const int *col, const float *val, int64_t M, int64_t K, int64_t nnz,
                      bool rows_sorted, int *prow, PairOutput *out) {
    out->nvec = 0;
    out->unsorted = 0;
    out->pcol = nullptr;
    out->pval = nullptr;
    if (rows_sorted) return pair_build_sorted(rowptr, col, val, M, prow, out);
    const int64_t npanels = (M + 1) / 2;
    uint64_t *ka = nullptr, *kb = nullptr;
    int *pa = nullptr, *pb = nullptr, *cnt = nullptr, *flag = nullptr;
    void *tmp = nullptr;
    size_t tmp_bytes = 0;
    hipError_t e = dmalloc(&cnt, sizeof(int) * (size_t)(npanels + 1), "panel counts");
    if (e == hipSuccess) e = dmalloc(&flag, sizeof(int), "panel flag");
    if (e == hipSuccess) e = hipMemset(flag, 0, sizeof(int));
    if (e == hipSuccess) e = hipMemset(cnt + npanels, 0, sizeof(int));
    const int64_t n = std::max<int64_t>(nnz, 1);
    if (e == hipSuccess) e = dmalloc(&ka, sizeof(uint64_t) * n, "panel sort keys");
    if (e == hipSuccess) e = dmalloc(&kb, sizeof(uint64_t) * n, "panel sort keys (alternate)");
    if (e == hipSuccess) e = dmalloc(&pa, sizeof(int) * n, "panel sort positions");
    if (e == hipSuccess) e = dmalloc(&pb, sizeof(int) * n, "panel sort positions (alternate)");
    hipcub::DoubleBuffer<uint64_t> keys(ka, kb);
    hipcub::DoubleBuffer<int> pos(pa, pb);
    if (e == hipSuccess && nnz > 0) {
        const int64_t gw = std::max<int64_t>(1, std::min<int64_t>((M + kWaves - 1) / kWaves, 1 << 20));
        hipLaunchKernelGGL(pair_keys_kernel, dim3((unsigned)gw), dim3(kBlock), 0, nullptr, rowptr, col, M, K, ka, pa);
        e = hipGetLastError();
        const uint64_t kmax = (((uint64_t)((M - 1) >> 1) * (uint64_t)K + (uint64_t)(K - 1)) << 1) | 1u;
        int end_bit = 1;
        while (end_bit < 64 && (kmax >> end_bit) != 0) ++end_bit;
        if (e == hipSuccess) e = hipcub::DeviceRadixSort::SortPairs(nullptr, tmp_bytes, keys, pos, (int)nnz, 0, end_bit);
        if (e == hipSuccess) e = dmalloc(&tmp, tmp_bytes > 0 ? tmp_bytes : 1, "panel sort storage");
        if (e == hipSuccess) e = hipcub::DeviceRadixSort::SortPairs(tmp, tmp_bytes, keys, pos, (int)nnz, 0, end_bit);
    }
    if (e == hipSuccess && npanels > 0) {
        hipLaunchKernelGGL(pair_walk_kernel<false>, dim3((unsigned)walk_grid(npanels)), dim3(kBlock), 0, nullptr,
                           rowptr, col, val, M, K, keys.Current(), pos.Current(), cnt, flag, nullptr, nullptr,
                           nullptr);
        e = hipGetLastError();
    }
    size_t scan_bytes = 0;
    void *scan_tmp = nullptr;
    if (e == hipSuccess) e = hipcub::DeviceScan::ExclusiveSum(nullptr, scan_bytes, cnt, prow, (int)(npanels + 1));
    if (e == hipSuccess) e = dmalloc(&scan_tmp, scan_bytes > 0 ? scan_bytes : 1, "panel scan storage");
    if (e == hipSuccess) e = hipcub::DeviceScan::ExclusiveSum(scan_tmp, scan_bytes, cnt, prow, (int)(npanels + 1));
    int nvec = 0, unsorted = 0;
    if (e == hipSuccess) e = hipMemcpy(&nvec, prow + npanels, sizeof(int), hipMemcpyDeviceToHost);
    if (e == hipSuccess) e = hipMemcpy(&unsorted, flag, sizeof(int), hipMemcpyDeviceToHost);
    if (e == hipSuccess && nvec > 0) {
        e = dmalloc(&out->pcol, sizeof(unsigned) * (size_t)nvec, "panel columns");
        if (e == hipSuccess && val) e = dmalloc(&out->pval, sizeof(float) * 2 * (size_t)nvec, "panel values");
        if (e == hipSuccess) {
            hipLaunchKernelGGL(pair_walk_kernel<true>, dim3((unsigned)walk_grid(npanels)), dim3(kBlock), 0, nullptr,
                               rowptr, col, val, M, K, keys.Current(), pos.Current(), nullptr, nullptr, prow,
                               out->pcol, out->pval);
            e = hipGetLastError();
        }
        if (e == hipSuccess) e = hipDeviceSynchronize();
        if (e != hipSuccess) {
            if (out->pcol) dfree(out->pcol);
            if (out->pval) dfree(out->pval);
            out->pcol = nullptr;
            out->pval = nullptr;
        }
    }
    out->nvec = nvec;
    out->unsorted = unsorted;
    for (void *q : {(void *)ka, (void *)kb, (void *)pa, (void *)pb, (void *)cnt, (void *)flag, tmp, scan_tmp})
        if (q) dfree(q);
    return e;
}

PairKernelFn pair_kernel(int lanes, int vec, bool has_val, bool is_max) {
    if (vec == 4) return pick_pair_vec<4>(lanes, has_val, is_max);
    if (vec == 1) return pick_pair_vec<1>(lanes, has_val, is_max);
    return nullptr;
}

hipError_t launch_pairs(PairKernelFn fn, PairArgs a, int lanes, int slices, hipStream_t s) {
    const int64_t per_block = (int64_t)(64 / lanes) * kWaves;
    const int64_t max_blocks = (int64_t)(UINT32_MAX / kBlock);
    const int64_t end = a.npanels;
    for (int64_t base = 0; base < end; base += max_blocks * per_block) {
        const int64_t n = std::min(end - base, max_blocks * per_block);
        a.task_base = base;
        a.npanels = base + n;
        void *args[] = {&a};
        const dim3 grid((unsigned)((n + per_block - 1) / per_block), (unsigned)slices);
        const hipError_t e = hipLaunchKernel(reinterpret_cast<const void *>(fn), grid, dim3(kBlock), args, 0, s);
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

}  // namespace gspmm
