// Merge-path balancing, the alternative to the row split (RA-SpMM, related
// work on load balancing: merge-based sparse computation partitions the work
// along a virtual merge path over the CSR stream).  The CSR is read as the
// merge of two sorted lists, the M row ends rowptr[1..M] and the nnz entry
// indices; each wave takes one segment of kMergeItems consecutive items of
// that merge, so every wave does the same amount of work (entries plus row
// ends) whatever the degree distribution.
//
// Plan time: the (row, entry) coordinate where each segment starts, by binary
// search on the merge path's diagonals.
// Run time, one wave per segment, all 64 lanes on the columns (VEC floats
// each): the segment's entries and the ends of the rows it finishes are
// staged in LDS; entries are gathered in predicated batches that run across
// row boundaries, so a batch's loads are in flight together however short
// the rows are; a row that ends inside the segment is written when its end
// item is reached, complete if it also started in the segment, else as a raw
// partial; the row still open at the segment's end leaves its partial in a
// carry slot.  A fix-up folds each carried row's pieces in segment order
// (sum: ((c0 + c1) + ...) + tail; max: strict '>', so the earlier piece wins
// ties), then applies the mean's division.  No atomics: results are bitwise
// reproducible; rows inside one segment sum in stored order with one
// accumulator, as in the row kernels.
#include <climits>

#include "row_kernel_impl.h"

namespace gspmm {

namespace {

constexpr int kMergeNT = kMergeItems / 64;

__global__ void merge_coords_kernel(const int *__restrict__ rowptr, int64_t M, int64_t nnz, int64_t nseg,
                                    int *__restrict__ seg_row, int *__restrict__ seg_entry) {
    const int64_t total = M + nnz;
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t w = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; w <= nseg; w += stride) {
        const int64_t d = min(w * kMergeItems, total);
        int64_t lo = max(d - nnz, (int64_t)0), hi = min(d, M);
        while (lo < hi) {   // rows whose end item lies among the first d items
            const int64_t piv = (lo + hi) >> 1;
            if (rowptr[piv + 1] <= d - piv - 1) lo = piv + 1;
            else hi = piv;
        }
        seg_row[w] = (int)lo;
        seg_entry[w] = (int)(d - lo);
    }
}

template <int VEC, bool IS_MAX>
__device__ __forceinline__ void merge_emit(const MergeArgs &a, int64_t row, int deg, bool complete, int colf,
                                           int skip, bool ok, const float (&acc)[VEC], const int (&arg)[VEC]) {
    if (!ok) return;
    float res[VEC];
    int ar[VEC];
#pragma unroll
    for (int e = 0; e < VEC; ++e) {
        if constexpr (IS_MAX) {
            res[e] = (complete && deg == 0) ? 0.0f : acc[e];
            ar[e] = (complete && deg == 0) ? -1 : arg[e];
        } else {
            res[e] = acc[e];
        }
    }
    if constexpr (!IS_MAX) mean_divide<VEC>(a.mean != 0, complete ? deg : 0, res);
    store_vec<VEC>(a.C + row * a.N + colf, res, false, skip);
    if constexpr (IS_MAX)
        if (a.argmax) store_arg64<VEC>(a.argmax + row * a.N + colf, ar, skip);
}

template <int VEC, bool HAS_VAL, bool IS_MAX>
__global__ __launch_bounds__(kBlock) void merge_kernel_t(MergeArgs a) {
    constexpr int U = VEC == 4 ? 4 : 8;
    __shared__ int s_col[kWaves][kMergeItems];
    __shared__ int s_val[kWaves][HAS_VAL ? kMergeItems : 1];
    __shared__ int s_end[kWaves][kMergeItems];
    const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
    const int64_t w = (int64_t)blockIdx.x * kWaves + wv;
    if (w >= a.nseg) return;                            // uniform per wave
    const int64_t c = a.c_begin + (int64_t)blockIdx.y * 64 * VEC + (int64_t)lane * VEC;
    const bool ok = c < a.c_end;
    // a vector that would run past the pass's last column ends there instead
    // (the pass is at least VEC wide) and writes only its own columns
    const int colf = (int)(VEC > 1 && c > a.c_end - VEC ? a.c_end - VEC : c);
    const int skip = (int)(c - colf);

    const int i0 = a.seg_row[w], p0 = a.seg_entry[w];
    const int i1 = a.seg_row[w + 1], p1 = a.seg_entry[w + 1];
    const int ne = p1 - p0, nr = i1 - i0;               // entries, row ends (each <= kMergeItems)
#pragma unroll
    for (int t = 0; t < kMergeNT; ++t) {
        const int q = t * 64 + lane;
        if (q < ne) {
            s_col[wv][q] = a.col[p0 + q];
            if constexpr (HAS_VAL) s_val[wv][q] = __float_as_int(a.val[p0 + q]);
        }
        if (q < nr) s_end[wv][q] = a.rowptr[i0 + 1 + q];
    }
    const int start0 = i0 < a.M ? a.rowptr[i0] : p0;
    const bool carried_in = p0 > start0;                // row i0 began in an earlier segment
    wave_lds_sync();

    float acc[VEC];
    int arg[VEC];
#pragma unroll
    for (int e = 0; e < VEC; ++e) {
        acc[e] = IS_MAX ? -INFINITY : 0.0f;
        arg[e] = -1;
    }
    int i = i0;
    int row_start = start0;
    int end_i = nr > 0 ? s_end[wv][0] : INT_MAX;        // end of row i if it ends in this segment
    bool touched = false;
    auto finish_row = [&]() {
        merge_emit<VEC, IS_MAX>(a, i, end_i - row_start, !(i == i0 && carried_in), colf, skip, ok, acc, arg);
#pragma unroll
        for (int e = 0; e < VEC; ++e) {
            acc[e] = IS_MAX ? -INFINITY : 0.0f;
            arg[e] = -1;
        }
        touched = false;
        row_start = end_i;
        ++i;
        end_i = (i - i0) < nr ? s_end[wv][i - i0] : INT_MAX;
    };

    for (int k = 0; k < ne; k += U) {
        int cidx[U];
        float wgt[U];
        bool vld[U];
        float bv[U][VEC];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            vld[u] = k + u < ne;
            const int kk = vld[u] ? k + u : 0;
            cidx[u] = s_col[wv][kk];
            wgt[u] = HAS_VAL ? __int_as_float(s_val[wv][kk]) : 1.0f;
#pragma unroll
            for (int e = 0; e < VEC; ++e) bv[u][e] = 0.0f;
            if (vld[u] && ok) load_vec<VEC>(a.B + elem_off(cidx[u], a.N, colf), bv[u]);
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            if (!vld[u]) continue;
            const int p = p0 + k + u;
            while (p >= end_i) finish_row();
#pragma unroll
            for (int e = 0; e < VEC; ++e) {
                if constexpr (IS_MAX) {
                    const float t = HAS_VAL ? wgt[u] * bv[u][e] : bv[u][e];
                    if (arg[e] < 0 || t > acc[e]) {
                        acc[e] = t;
                        arg[e] = cidx[u];
                    }
                } else {
                    acc[e] = HAS_VAL ? __builtin_fmaf(wgt[u], bv[u][e], acc[e]) : acc[e] + bv[u][e];
                }
            }
            touched = true;
        }
    }
    while (i < i1) finish_row();                        // rows (or empty rows) ending after the last entry

    // the row still open at the segment's end: its partial goes to the carry slot
    const bool carry = i1 < a.M && touched;
    if (lane == 0) a.carry_row[w] = carry ? i1 : -1;
    if (carry && ok) {
        const int64_t off = w * kPartialWidth + (colf - a.c_begin);
        store_vec<VEC>(a.carry + off, acc, false, skip);
        if constexpr (IS_MAX) store_arg32<VEC>(a.carry_arg + off, arg, skip);
    }
}

// One block per segment w, one thread per column of the pass: a segment that
// starts a chain of carries for row r folds the chain and the raw tail left
// in C by the segment where r ends.
template <bool IS_MAX>
__global__ __launch_bounds__(kPartialWidth) void merge_fixup_kernel(MergeArgs a) {
    const int64_t w = blockIdx.x;
    const int r = a.carry_row[w];
    if (r < 0 || (w > 0 && a.carry_row[w - 1] == r)) return;   // uniform per block
    const int64_t c = a.c_begin + threadIdx.x;
    if (c >= a.c_end) return;
    float total = a.carry[w * kPartialWidth + threadIdx.x];
    int targ = IS_MAX ? a.carry_arg[w * kPartialWidth + threadIdx.x] : 0;
    int64_t w2 = w + 1;
    for (; w2 < a.nseg && a.carry_row[w2] == r; ++w2) {
        const float x = a.carry[w2 * kPartialWidth + threadIdx.x];
        if constexpr (IS_MAX) {
            const int xa = a.carry_arg[w2 * kPartialWidth + threadIdx.x];
            if (targ < 0 || (xa >= 0 && x > total)) {
                total = x;
                targ = xa;
            }
        } else {
            total = total + x;
        }
    }
    float *cp = a.C + (int64_t)r * a.N + c;
    const float tail = *cp;
    const int deg = a.rowptr[r + 1] - a.rowptr[r];
    if constexpr (IS_MAX) {
        const int64_t tail_arg = a.argmax ? a.argmax[(int64_t)r * a.N + c] : -1;
        if (targ < 0 || (tail_arg >= 0 && tail > total)) {
            total = tail;
            targ = (int)tail_arg;
        }
        *cp = total;
        if (a.argmax) a.argmax[(int64_t)r * a.N + c] = targ;
    } else {
        float res[1] = {total + tail};
        mean_divide<1>(a.mean != 0, deg, res);
        *cp = res[0];
    }
}

template <int VEC>
MergeKernelFn pick_merge(bool has_val, bool is_max) {
    if (is_max) return has_val ? merge_kernel_t<VEC, true, true> : merge_kernel_t<VEC, false, true>;
    return has_val ? merge_kernel_t<VEC, true, false> : merge_kernel_t<VEC, false, false>;
}

}  // namespace

hipError_t merge_build(const int *rowptr, int64_t M, int64_t nnz, int64_t nseg, int *seg_row, int *seg_entry) {
    const int64_t n = nseg + 1;
    const int64_t grid = std::max<int64_t>(1, std::min<int64_t>((n + kBlock - 1) / kBlock, 1 << 16));
    hipLaunchKernelGGL(merge_coords_kernel, dim3((unsigned)grid), dim3(kBlock), 0, nullptr, rowptr, M, nnz, nseg,
                       seg_row, seg_entry);
    hipError_t e = hipGetLastError();
    if (e == hipSuccess) e = hipDeviceSynchronize();
    return e;
}

MergeKernelFn merge_kernel(int vec, bool has_val, bool is_max) {
    if (vec == 4) return pick_merge<4>(has_val, is_max);
    if (vec == 2) return pick_merge<2>(has_val, is_max);
    if (vec == 1) return pick_merge<1>(has_val, is_max);
    return nullptr;
}

hipError_t launch_merge(MergeKernelFn fn, const MergeArgs &a, int vec, bool is_max, hipStream_t s) {
    const int64_t width = a.c_end - a.c_begin;
    const int slices = (int)((width + 64 * vec - 1) / (64 * vec));
    const int64_t blocks = (a.nseg + kWaves - 1) / kWaves;
    if (blocks > (int64_t)(UINT32_MAX / kBlock) || a.nseg > (int64_t)UINT32_MAX)
        return hipErrorInvalidConfiguration;
    MergeArgs args = a;
    void *kargs[] = {&args};
    hipError_t e = hipLaunchKernel(reinterpret_cast<const void *>(fn), dim3((unsigned)blocks, (unsigned)slices),
                                   dim3(kBlock), kargs, 0, s);
    if (e != hipSuccess) return e;
    if (is_max)
        hipLaunchKernelGGL(merge_fixup_kernel<true>, dim3((unsigned)a.nseg), dim3(kPartialWidth), 0, s, args);
    else
        hipLaunchKernelGGL(merge_fixup_kernel<false>, dim3((unsigned)a.nseg), dim3(kPartialWidth), 0, s, args);
    return hipGetLastError();
}

}  // namespace gspmm
