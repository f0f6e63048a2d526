// Matrix-core path for community-structured graphs (RA-SpMM, "Kernel
// families": a dense tile path for community blocks, which gains by cutting
// memory traffic rather than by reaching the matrix cores' peak).
//
// Plan time: for every aligned block of kWinRows rows, the entries whose
// column lies in the same block become one dense kWinRows x kWinRows fp16
// tile (duplicates summed in fp32 in stored order, rounded once), stored in
// the operand order of v_mfma_f32_32x32x16_f16; all other entries form a
// residual CSR in stored order.
//
// Run time: one 1024-thread workgroup per (block, kWinCols-column slice).
//   1. B's kWinRows x kWinCols slice is read once from HBM, rounded to fp16 and
//      stored transposed in LDS, so each lane's 8 consecutive k values of the
//      B operand are one 16-byte LDS read.
//   2. Wave w computes the 32 x 32 output tile (row group w % 8, column group
//      w / 8) over kMfmaKSteps k-steps; its A operand streams from the
//      fragment-ordered tile in HBM, four k-steps ahead.
//   3. The accumulators go to an fp32 C tile in LDS (over the B^T bytes), and
//      the row walk of the CSR kernels adds the residual entries in stored
//      order, 16 lanes x float4 per row, then divides for the mean and writes C.
// No atomics: results are bitwise reproducible.
#include <hipcub/hipcub.hpp>

#include "row_kernel_impl.h"

namespace gspmm {

typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

namespace {

constexpr int kTileUnits = 8 * kMfmaKSteps * 64;   // 16-byte units per tile
static_assert(kWinRows == 256 && kWinCols == 64 && kWinBlock == 1024,
              "the tile kernel assumes 256-row blocks, 64-column slices and 16 waves");

int64_t wave_grid(int64_t M) { return std::max<int64_t>(1, std::min<int64_t>((M + kWaves - 1) / kWaves, 1 << 20)); }

// One wave per row.  Lane l owns tile columns 4l .. 4l+3 and adds the row's
// in-block weights to them in stored order; the sums are rounded to fp16 and
// stored at their operand positions.  Also counts the row's residual entries.
__global__ __launch_bounds__(kBlock) void mfma_tile_build_kernel(const int *__restrict__ rowptr,
                                                                 const int *__restrict__ col,
                                                                 const float *__restrict__ val, int64_t M,
                                                                 uint4 *__restrict__ atiles, int *__restrict__ rcount,
                                                                 int *__restrict__ range_flag) {
    const int lane = threadIdx.x & 63;
    const int64_t stride = (int64_t)gridDim.x * kWaves;
    for (int64_t row = (int64_t)blockIdx.x * kWaves + (threadIdx.x >> 6); row < M; row += stride) {
        const int64_t w0 = (row / kWinRows) * kWinRows;
        const int beg = rowptr[row], end = rowptr[row + 1];
        float s0 = 0.0f, s1 = 0.0f, s2 = 0.0f, s3 = 0.0f;
        int nres = 0;
        for (int cb = beg; cb < end; cb += 64) {
            const int p = cb + lane;
            const bool has = p < end;
            const int c = has ? col[p] : 0;
            const float w = has ? (val ? val[p] : 1.0f) : 0.0f;
            const int64_t wr = (int64_t)c - w0;
            const bool inw = has && wr >= 0 && wr < kWinRows;
            nres += (has && !inw) ? 1 : 0;
            const int n = min(64, end - cb);
            for (int j = 0; j < n; ++j) {
                const int wj = __shfl(inw ? (int)wr : -1, j);
                const float aj = __shfl(w, j);
                if (wj >= 0 && (wj >> 2) == lane) {
                    const int e = wj & 3;
                    if (e == 0) s0 += aj;
                    else if (e == 1) s1 += aj;
                    else if (e == 2) s2 += aj;
                    else s3 += aj;
                }
            }
        }
#pragma unroll
        for (int o = 32; o > 0; o >>= 1) nres += __shfl_xor(nres, o);

        const int r = (int)(row - w0);
        const int k = 4 * lane;
        const int rg = r >> 5, ks = k >> 4, hh = (k >> 3) & 1, j = k & 7;
        const int lf = (r & 31) + 32 * hh;
        const int64_t tile = row / kWinRows;
        _Float16 *dst = reinterpret_cast<_Float16 *>(atiles + tile * kTileUnits + (rg * kMfmaKSteps + ks) * 64 + lf) + j;
        const f16x4 h = {(_Float16)s0, (_Float16)s1, (_Float16)s2, (_Float16)s3};
        *reinterpret_cast<f16x4 *>(dst) = h;
        // fp32 values at or above 65520 round to infinity in fp16 (NaN fails the test too)
        const bool bad = !(fabsf(s0) < 65520.0f) || !(fabsf(s1) < 65520.0f) || !(fabsf(s2) < 65520.0f) ||
                         !(fabsf(s3) < 65520.0f);
        if (bad) *range_flag = 1;   // every writer stores the same value
        if (lane == 0) rcount[row] = nres;
    }
}

// One wave per row: the row's residual entries, compacted in stored order.
__global__ __launch_bounds__(kBlock) void mfma_residual_kernel(const int *__restrict__ rowptr,
                                                               const int *__restrict__ col,
                                                               const float *__restrict__ val, int64_t M,
                                                               const int *__restrict__ rrowptr, int *__restrict__ rcol,
                                                               float *__restrict__ rval) {
    const int lane = threadIdx.x & 63;
    const uint64_t below = (1ull << lane) - 1ull;
    const int64_t stride = (int64_t)gridDim.x * kWaves;
    for (int64_t row = (int64_t)blockIdx.x * kWaves + (threadIdx.x >> 6); row < M; row += stride) {
        const int64_t w0 = (row / kWinRows) * kWinRows;
        const int beg = rowptr[row], end = rowptr[row + 1];
        int out = rrowptr[row];
        for (int cb = beg; cb < end; cb += 64) {
            const int p = cb + lane;
            const bool has = p < end;
            const int c = has ? col[p] : 0;
            const int64_t wr = (int64_t)c - w0;
            const bool res = has && !(wr >= 0 && wr < kWinRows);
            const uint64_t m = __ballot(res);
            if (res) {
                const int q = out + __popcll(m & below);
                rcol[q] = c;
                if (rval) rval[q] = val[p];
            }
            out += __popcll(m);
        }
    }
}

// Rows task0 .. task0 + 3 of one wave: start from the tile result in LDS, add
// the residual entries in stored order, write C.
template <bool HAS_VAL>
__device__ __forceinline__ void residual_rows(const MfmaArgs &a, int64_t task0, int lane, int *s_col, int *s_val,
                                              const int (&colf)[1], const bool (&ok)[1], const float *s_tile,
                                              int64_t w0) {
    constexpr int G = kWinCols / 4, R = 64 / G, CH = kWinChunk, NT = CH / 64;
    const int sub = lane / G, g = lane % G;
    const int64_t v = task0 + sub;
    const bool live = v < a.M;
    int beg = 0, end = 0;
    if (live) {
        beg = a.rrowptr[v];
        end = a.rrowptr[v + 1];
    }
    const int deg = end - beg;
    const int beg0 = __builtin_amdgcn_readfirstlane(beg);   // lane 0 holds row task0 < M
    int off = 0, total = 0;
#pragma unroll
    for (int s = 0; s < R; ++s) {
        const int ds = __builtin_amdgcn_readlane(deg, s * G);
        off += (s < sub) ? ds : 0;
        total += ds;
    }

    float acc[1][4];
    int arg[1][4];
    {
        f32x4 t = {0.0f, 0.0f, 0.0f, 0.0f};
        if (live) t = reinterpret_cast<const f32x4 *>(s_tile)[(v - w0) * (kWinCols / 4) + g];
        acc[0][0] = t.x;
        acc[0][1] = t.y;
        acc[0][2] = t.z;
        acc[0][3] = t.w;
#pragma unroll
        for (int e = 0; e < 4; ++e) arg[0][e] = -1;
    }

    for (int cb = 0; cb < total; cb += CH) {
        const int cn = min(CH, total - cb);
        const int nt = (cn + 63) >> 6;
        int cr[NT];
        int vr[NT];
#pragma unroll
        for (int t = 0; t < NT; ++t) {
            if (t < nt) {
                const int p = beg0 + cb + min(t * 64 + lane, cn - 1);
                cr[t] = a.rcol[p];
                if constexpr (HAS_VAL) vr[t] = __float_as_int(a.rval[p]);
            }
        }
#pragma unroll
        for (int t = 0; t < NT; ++t) {
            if (t < nt) {
                s_col[t * 64 + lane] = cr[t];
                if constexpr (HAS_VAL) s_val[t * 64 + lane] = vr[t];
            }
        }
        wave_lds_sync();
        const int lo = max(off, cb) - cb;
        const int hi = min(off + deg, cb + cn) - cb;
        consume<1, 4, HAS_VAL, false, false, 4>(s_col, s_val, lo, hi, a.B, a.N, colf, ok, acc, arg);
        wave_lds_sync();
    }

    if (live && ok[0]) {
        const int dfull = a.mean ? a.rowptr[v + 1] - a.rowptr[v] : 0;
        float res[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) res[e] = dfull > 0 ? acc[0][e] / (float)dfull : acc[0][e];
        store_vec<4>(a.C + v * a.N + colf[0], res, false);
    }
}

template <bool HAS_VAL>
__global__ __launch_bounds__(kWinBlock) void mfma_tile_kernel_t(MfmaArgs a, int64_t block_base, int64_t nblocks) {
    constexpr int WW = kWinBlock / 64;   // 16 waves: 8 row groups x 2 column groups of 32
    constexpr int R = 64 / (kWinCols / 4);
    __shared__ __align__(16) float s_tile[kWinRows * kWinCols];   // fp16 B^T, then the fp32 C tile
    __shared__ int s_col[WW][kWinChunk];
    __shared__ int s_val[WW][HAS_VAL ? kWinChunk : 1];
    static_assert(kWinCols * kMfmaBtPitch * 2 <= (int)sizeof(float) * kWinRows * kWinCols, "B^T fits the C tile");

    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    int64_t lin = blockIdx.x;
    if (a.xcd_remap) lin = xcd_remap_block(lin, (int64_t)gridDim.x);
    lin += block_base;
    if (lin >= nblocks) return;   // never taken: the grid covers [block_base, nblocks) exactly
    const int64_t tile = lin / a.nslices, slice = lin % a.nslices;
    const int64_t w0 = tile * kWinRows, c0 = slice * kWinCols;
    const int rg = wv & 7, cg = wv >> 3;

    const uint4 *ap = a.atiles + tile * kTileUnits + (int64_t)rg * kMfmaKSteps * 64 + lane;
    uint4 ar[4];
#pragma unroll
    for (int s = 0; s < 4; ++s) ar[s] = ap[s * 64];

    _Float16 *sbt = reinterpret_cast<_Float16 *>(s_tile);
    {
        // thread (q, o): rows 4o .. 4o+3 of column quad q, stored as 4 columns of B^T
        const int q = tid & 15, o = tid >> 4;
        const int64_t cc = c0 + 4 * q;
        f32x4 v[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int64_t br = w0 + 4 * o + r;
            v[r] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
            if (br < a.K && cc < a.N) v[r] = *reinterpret_cast<const f32x4 *>(a.B + br * a.N + cc);
        }
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const f16x4 h = {(_Float16)v[0][e], (_Float16)v[1][e], (_Float16)v[2][e], (_Float16)v[3][e]};
            *reinterpret_cast<f16x4 *>(sbt + (4 * q + e) * kMfmaBtPitch + 4 * o) = h;
        }
    }
    __syncthreads();

    f32x16 acc = {};
    const _Float16 *bp = sbt + (cg * 32 + (lane & 31)) * kMfmaBtPitch + 8 * (lane >> 5);
#pragma unroll
    for (int ks = 0; ks < kMfmaKSteps; ++ks) {
        const uint4 au = ar[ks & 3];
        if (ks + 4 < kMfmaKSteps) ar[ks & 3] = ap[(ks + 4) * 64];
        const f16x8 av = __builtin_bit_cast(f16x8, au);
        const f16x8 bv = *reinterpret_cast<const f16x8 *>(bp + ks * 16);
        acc = __builtin_amdgcn_mfma_f32_32x32x16_f16(av, bv, acc, 0, 0, 0);
    }
    __syncthreads();   // all waves are done with B^T
#pragma unroll
    for (int r = 0; r < 16; ++r)
        s_tile[(rg * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3)) * kWinCols + cg * 32 + (lane & 31)] = acc[r];
    __syncthreads();

    const int g = lane % (kWinCols / 4);
    int colf[1];
    bool ok[1];
    colf[0] = (int)(c0 + 4 * g);
    ok[0] = c0 + 4 * g < a.N;
    for (int pass = 0; pass < kWinRows / (WW * R); ++pass) {
        const int64_t task0 = w0 + (int64_t)(pass * WW + wv) * R;
        if (task0 < a.M) residual_rows<HAS_VAL>(a, task0, lane, s_col[wv], s_val[wv], colf, ok, s_tile, w0);
    }
}

}  // namespace

hipError_t mfma_build_tiles(const int *rowptr, const int *col, const float *val, int64_t M, uint4 *atiles,
                            int64_t ntiles, int *rrowptr, int *range_flag, hipStream_t s) {
    hipError_t e = hipSuccess;
    if (ntiles > 0 && (e = hipMemsetAsync(atiles, 0, (size_t)ntiles * kTileUnits * sizeof(uint4), s)) != hipSuccess)
        return e;
    if ((e = hipMemsetAsync(range_flag, 0, sizeof(int), s)) != hipSuccess) return e;
    int *cnt = nullptr;
    void *tmp = nullptr;
    size_t tmp_bytes = 0;
    if ((e = hipMalloc(&cnt, sizeof(int) * (size_t)(M + 1))) != hipSuccess) return e;
    e = hipMemsetAsync(cnt + M, 0, sizeof(int), s);
    if (e == hipSuccess && M > 0) {
        hipLaunchKernelGGL(mfma_tile_build_kernel, dim3((unsigned)wave_grid(M)), dim3(kBlock), 0, s, rowptr, col, val,
                           M, atiles, cnt, range_flag);
        e = hipGetLastError();
    }
    if (e == hipSuccess) e = hipcub::DeviceScan::ExclusiveSum(nullptr, tmp_bytes, cnt, rrowptr, (int)(M + 1), s);
    if (e == hipSuccess) e = hipMalloc(&tmp, tmp_bytes > 0 ? tmp_bytes : 1);
    if (e == hipSuccess) e = hipcub::DeviceScan::ExclusiveSum(tmp, tmp_bytes, cnt, rrowptr, (int)(M + 1), s);
    if (e == hipSuccess) e = hipStreamSynchronize(s);
    if (tmp) (void)hipFree(tmp);
    (void)hipFree(cnt);
    return e;
}

hipError_t mfma_write_residual(const int *rowptr, const int *col, const float *val, int64_t M, const int *rrowptr,
                               int *rcol, float *rval, hipStream_t s) {
    if (M == 0) return hipSuccess;
    hipLaunchKernelGGL(mfma_residual_kernel, dim3((unsigned)wave_grid(M)), dim3(kBlock), 0, s, rowptr, col, val, M,
                       rrowptr, rcol, rval);
    hipError_t e = hipGetLastError();
    if (e == hipSuccess) e = hipStreamSynchronize(s);
    return e;
}

hipError_t launch_mfma(const MfmaArgs &a, bool has_val, hipStream_t s) {
    const int64_t ntiles = (a.M + kWinRows - 1) / kWinRows;
    const int64_t nb = ntiles * a.nslices;
    const int64_t max_blocks = (int64_t)(UINT32_MAX / kWinBlock);
    for (int64_t base = 0; base < nb; base += max_blocks) {
        const int64_t n = std::min(nb - base, max_blocks);
        if (has_val)
            hipLaunchKernelGGL(mfma_tile_kernel_t<true>, dim3((unsigned)n), dim3(kWinBlock), 0, s, a, base, base + n);
        else
            hipLaunchKernelGGL(mfma_tile_kernel_t<false>, dim3((unsigned)n), dim3(kWinBlock), 0, s, a, base, base + n);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

}  // namespace gspmm
