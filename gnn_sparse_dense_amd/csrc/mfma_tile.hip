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

#include "alloc.h"
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
// mode 0: fp16 tiles; mode 1: only the largest |sum| of every tile (split
// tiles, first pass); mode 2: split tiles, sums scaled by 2^tile_exp[t] and
// stored as an fp16 high half (atiles) plus an fp16 low half (atiles_lo).
__global__ __launch_bounds__(kBlock) void mfma_tile_build_kernel(const int *__restrict__ rowptr,
                                                                 const int *__restrict__ col,
                                                                 const float *__restrict__ val, int64_t M,
                                                                 uint4 *__restrict__ atiles, int *__restrict__ rcount,
                                                                 int *__restrict__ range_flag, int mode,
                                                                 unsigned *__restrict__ tile_max,
                                                                 const int *__restrict__ tile_exp,
                                                                 uint4 *__restrict__ atiles_lo) {
    const int lane = threadIdx.x & 63;
    const int64_t stride = (int64_t)gridDim.x * kWaves;
    for (int64_t row = (int64_t)blockIdx.x * kWaves + (threadIdx.x >> 6); row < M; row += stride) {
        const int64_t w0 = (row / kWinRows) * kWinRows;
        const int beg = rowptr[row], end = rowptr[row + 1];
        float s0 = 0.0f, s1 = 0.0f, s2 = 0.0f, s3 = 0.0f;
        int nres = 0;
        for (int64_t cb = beg; cb < end; cb += 64) {
            const int64_t p = cb + lane;
            const bool has = p < end;
            const int c = has ? col[p] : 0;
            const float w = has ? (val ? val[p] : 1.0f) : 0.0f;
            const int64_t wr = (int64_t)c - w0;
            const bool inw = has && wr >= 0 && wr < kWinRows;
            nres += (has && !inw) ? 1 : 0;
            const int n = (int)min((int64_t)64, end - cb);
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
        const int64_t tile = row / kWinRows;
        if (mode == 1) {
            float m = fmaxf(fmaxf(fabsf(s0), fabsf(s1)), fmaxf(fabsf(s2), fabsf(s3)));
            if (!(m <= 3.0e38f)) *range_flag = 1;   // not finite
#pragma unroll
            for (int o = 32; o > 0; o >>= 1) m = fmaxf(m, __shfl_xor(m, o));
            if (lane == 0 && m > 0.0f) atomicMax(tile_max + tile, __float_as_uint(m));   // non-negative: int order
            continue;
        }

        const int r = (int)(row - w0);
        const int k = 4 * lane;
        const int rg = r >> 5, ks = k >> 4, hh = (k >> 3) & 1, j = k & 7;
        const int lf = (r & 31) + 32 * hh;
        const int64_t unit = tile * kTileUnits + (rg * kMfmaKSteps + ks) * 64 + lf;
        _Float16 *dst = reinterpret_cast<_Float16 *>(atiles + unit) + j;
        if (mode == 2) {
            const int ex = tile_exp[tile];
            const float x0 = ldexpf(s0, ex), x1 = ldexpf(s1, ex), x2 = ldexpf(s2, ex), x3 = ldexpf(s3, ex);
            const f16x4 h = {(_Float16)x0, (_Float16)x1, (_Float16)x2, (_Float16)x3};
            const f16x4 l = {(_Float16)(x0 - (float)h[0]), (_Float16)(x1 - (float)h[1]), (_Float16)(x2 - (float)h[2]),
                             (_Float16)(x3 - (float)h[3])};
            *reinterpret_cast<f16x4 *>(dst) = h;
            *reinterpret_cast<f16x4 *>(reinterpret_cast<_Float16 *>(atiles_lo + unit) + j) = l;
        } else {
            const f16x4 h = {(_Float16)s0, (_Float16)s1, (_Float16)s2, (_Float16)s3};
            *reinterpret_cast<f16x4 *>(dst) = h;
            // fp32 values at or above 65520 round to infinity in fp16 (NaN fails the test too)
            const bool bad = !(fabsf(s0) < 65520.0f) || !(fabsf(s1) < 65520.0f) || !(fabsf(s2) < 65520.0f) ||
                             !(fabsf(s3) < 65520.0f);
            if (bad) *range_flag = 1;   // every writer stores the same value
        }
        if (lane == 0) rcount[row] = nres;
    }
}

// Split tiles: the power of two that brings a tile's largest |sum| just
// below 2^15, so the low halves stay normal fp16 numbers.
__global__ void tile_exp_kernel(const unsigned *__restrict__ tile_max, int64_t ntiles, int *__restrict__ tile_exp) {
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; t < ntiles; t += stride) {
        const float m = __uint_as_float(tile_max[t]);
        int e = 0;
        if (m > 0.0f) (void)frexpf(m, &e);   // m < 2^e
        tile_exp[t] = m > 0.0f ? 15 - e : 0;
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
        for (int64_t cb = beg; cb < end; cb += 64) {
            const int64_t p = cb + lane;
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

    for (int64_t cb64 = 0; cb64 < total; cb64 += CH) {   // 64-bit: total may lie within CH of 2^31
        const int cb = (int)cb64;
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
        for (int e = 0; e < 4; ++e) res[e] = acc[0][e];
        mean_divide<4>(a.mean != 0, dfull, res);
        store_vec<4>(a.C + v * a.N + colf[0], res, false);
    }
}

// B^T in LDS, two layouts.  Split tiles (three products per k-step: the
// operand reads bind) store 16-byte chunk j (8 k values) of column c at half
// bt_off(c, j): rows of kWinRows halves, chunk index XOR-swizzled by
// h(c) = (c ^ c >> 2) & 15, so that both accesses spread over all 64 banks:
// the MFMA operand read (16 consecutive columns per 256-byte pass, one chunk
// each: t -> t ^ t >> 2 is invertible on 4 bits, so h takes 16 values) and
// the transposing store (16 column quads q of one k range, 8-byte halves of
// two chunks: c = 4q + e gives h = q ^ ((q & 3) << 2) ^ e, again 16 values).
// fp16 tiles (one product per k-step: the staging of B binds) keep rows of
// kMfmaBtPitch = kWinRows + 8 halves (a 16-byte skew per row), written by
// the staging map that reads 256 contiguous bytes of a B row per 16 lanes.
// Measured on the community graph (N = 512, flushed): the swizzle takes split
// tiles from 1.121 to 1.044 ms; on fp16 tiles it cost 0.858 -> 0.966 ms.
__device__ __forceinline__ int bt_off(int c, int j) { return c * kWinRows + 8 * (j ^ ((c ^ (c >> 2)) & 15)); }

// LDS of one workgroup: B^T (fp16; high and low halves for split tiles) while
// the products run, then the fp32 C tile and the residual walk's staging.
constexpr int kBtBytes = kWinCols * kMfmaBtPitch * 2;
constexpr int kTileBytes = kWinRows * kWinCols * 4;
constexpr int kStageBytes = (kWinBlock / 64) * kWinChunk * 4;
constexpr int kMfmaLds = kTileBytes + 2 * kStageBytes;
static_assert(2 * kBtBytes <= kMfmaLds, "both B^T halves fit");

// Two workgroups (32 waves) per CU: at most 64 VGPRs.
template <bool HAS_VAL, bool SPLIT>
__global__ __launch_bounds__(kWinBlock) __attribute__((amdgpu_waves_per_eu(8, 8))) void mfma_tile_kernel_t(
    MfmaArgs a, int64_t block_base, int64_t nblocks) {
    constexpr int WW = kWinBlock / 64;   // 16 waves: 8 row groups x 2 column groups of 32
    constexpr int R = 64 / (kWinCols / 4);
    constexpr int AH = SPLIT ? 2 : 4;    // k-steps of A in flight
    __shared__ __align__(16) unsigned char smem[kMfmaLds];
    // per-wave maxima of the B slice: in the staging area, idle until the residual walk
    float *s_red = reinterpret_cast<float *>(smem + kMfmaLds) - WW;
    static_assert(2 * kBtBytes + (int)sizeof(float) * WW <= kMfmaLds, "scratch clear of B^T");
    float *s_tile = reinterpret_cast<float *>(smem);
    int *s_col = reinterpret_cast<int *>(smem + kTileBytes);
    int *s_val = reinterpret_cast<int *>(smem + kTileBytes + kStageBytes);
    _Float16 *sbt = reinterpret_cast<_Float16 *>(smem);
    _Float16 *sbt_lo = reinterpret_cast<_Float16 *>(smem + kBtBytes);

    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    int64_t lin = blockIdx.x;
    if (a.xcd_remap) lin = xcd_remap_block(lin, (int64_t)gridDim.x);
    lin += block_base;
    if (lin >= nblocks) return;   // never taken: the grid covers [block_base, nblocks) exactly
    const int64_t tile = lin / a.nslices, slice = lin % a.nslices;
    const int64_t w0 = tile * kWinRows, c0 = slice * kWinCols;
    const int rg = wv & 7, cg = wv >> 3;

    const int64_t aoff = tile * kTileUnits + (int64_t)rg * kMfmaKSteps * 64 + lane;
    const uint4 *ap = a.atiles + aoff;
    const uint4 *apl = SPLIT ? a.atiles_lo + aoff : nullptr;
    uint4 ar[AH], arl[AH];
#pragma unroll
    for (int s = 0; s < AH; ++s) {
        ar[s] = ap[s * 64];
        if constexpr (SPLIT) arl[s] = apl[s * 64];
    }

    int bexp = 0;
    {
        // thread (q, o): rows 4o .. 4o+3 of column quad q, stored as 4 columns of B^T.
        // Split tiles: lanes 0-7 take quads 0-7 of an even o, lanes 8-15 the
        // same quads of o + 1, so that each 16-lane group stores two whole
        // chunks per column quad (bank-conflict free with the swizzle); every
        // 16 lanes of one o still read one contiguous 256-byte stretch of a
        // B row.  fp16 tiles: lanes 0-15 take quads 0-15 of one o.
        const int q = SPLIT ? (tid & 7) | (((tid >> 4) & 1) << 3) : tid & 15;
        const int o = SPLIT ? ((tid >> 3) & 1) | ((tid >> 5) << 1) : tid >> 4;
        const int64_t cc = c0 + 4 * q;
        f32x4 v[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int64_t br = w0 + 4 * o + r;
            v[r] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
            if (br < a.K && cc < a.N) v[r] = *reinterpret_cast<const f32x4 *>(a.B + br * a.N + cc);
        }
        if constexpr (SPLIT) {
            // the slice's largest |b| sets a power of two that keeps the low halves normal
            float m = 0.0f;
#pragma unroll
            for (int r = 0; r < 4; ++r)
                m = fmaxf(m, fmaxf(fmaxf(fabsf(v[r].x), fabsf(v[r].y)), fmaxf(fabsf(v[r].z), fabsf(v[r].w))));
#pragma unroll
            for (int off = 32; off > 0; off >>= 1) m = fmaxf(m, __shfl_xor(m, off));
            if (lane == 0) s_red[wv] = m;
            __syncthreads();
            m = 0.0f;
#pragma unroll
            for (int w = 0; w < WW; ++w) m = fmaxf(m, s_red[w]);
            int e = 0;
            if (m > 0.0f && m <= 3.0e38f) (void)frexpf(m, &e);
            bexp = (m > 0.0f && m <= 3.0e38f) ? 15 - e : 0;
        }
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            if constexpr (SPLIT) {
                f16x4 h, l;
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const float x = ldexpf(v[r][e], bexp);
                    h[r] = (_Float16)x;
                    l[r] = (_Float16)(x - (float)h[r]);
                }
                *reinterpret_cast<f16x4 *>(sbt + bt_off(4 * q + e, o >> 1) + 4 * (o & 1)) = h;
                *reinterpret_cast<f16x4 *>(sbt_lo + bt_off(4 * q + e, o >> 1) + 4 * (o & 1)) = l;
            } else {
                const f16x4 h = {(_Float16)v[0][e], (_Float16)v[1][e], (_Float16)v[2][e], (_Float16)v[3][e]};
                *reinterpret_cast<f16x4 *>(sbt + (4 * q + e) * kMfmaBtPitch + 4 * o) = h;
            }
        }
    }
    __syncthreads();

    f32x16 acc = {};
    const int bcol = cg * 32 + (lane & 31);
    const int boff = bcol * kMfmaBtPitch + 8 * (lane >> 5);   // fp16 tiles
#pragma unroll
    for (int ks = 0; ks < kMfmaKSteps; ++ks) {
        const uint4 au = ar[ks % AH];
        if (ks + AH < kMfmaKSteps) ar[ks % AH] = ap[(ks + AH) * 64];
        const f16x8 av = __builtin_bit_cast(f16x8, au);
        const f16x8 bv = *reinterpret_cast<const f16x8 *>(
            sbt + (SPLIT ? bt_off(bcol, 2 * ks + (lane >> 5)) : boff + ks * 16));
        acc = __builtin_amdgcn_mfma_f32_32x32x16_f16(av, bv, acc, 0, 0, 0);
        if constexpr (SPLIT) {
            const uint4 aul = arl[ks % AH];
            if (ks + AH < kMfmaKSteps) arl[ks % AH] = apl[(ks + AH) * 64];
            const f16x8 avl = __builtin_bit_cast(f16x8, aul);
            const f16x8 bvl = *reinterpret_cast<const f16x8 *>(sbt_lo + bt_off(bcol, 2 * ks + (lane >> 5)));
            acc = __builtin_amdgcn_mfma_f32_32x32x16_f16(av, bvl, acc, 0, 0, 0);
            acc = __builtin_amdgcn_mfma_f32_32x32x16_f16(avl, bv, acc, 0, 0, 0);
        }
    }
    const int unscale = SPLIT ? -(a.tile_exp[tile] + bexp) : 0;
    __syncthreads();   // all waves are done with B^T
#pragma unroll
    for (int r = 0; r < 16; ++r)
        s_tile[(rg * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3)) * kWinCols + cg * 32 + (lane & 31)] =
            SPLIT ? ldexpf(acc[r], unscale) : acc[r];
    __syncthreads();

    const int g = lane % (kWinCols / 4);
    int colf[1];
    bool ok[1];
    colf[0] = (int)(c0 + 4 * g);
    ok[0] = c0 + 4 * g < a.N;
    for (int pass = 0; pass < kWinRows / (WW * R); ++pass) {
        const int64_t task0 = w0 + (int64_t)(pass * WW + wv) * R;
        if (task0 < a.M)
            residual_rows<HAS_VAL>(a, task0, lane, s_col + wv * kWinChunk, s_val + wv * kWinChunk, colf, ok, s_tile,
                                   w0);
    }
}

}  // namespace

hipError_t mfma_build_tiles(const int *rowptr, const int *col, const float *val, int64_t M, uint4 *atiles,
                            uint4 *atiles_lo, int *tile_exp, int64_t ntiles, int *rrowptr, int *range_flag,
                            hipStream_t s) {
    hipError_t e = hipSuccess;
    const size_t tile_bytes = (size_t)ntiles * kTileUnits * sizeof(uint4);
    if (ntiles > 0 && (e = hipMemsetAsync(atiles, 0, tile_bytes, s)) != hipSuccess) return e;
    if (ntiles > 0 && atiles_lo && (e = hipMemsetAsync(atiles_lo, 0, tile_bytes, s)) != hipSuccess) return e;
    if ((e = hipMemsetAsync(range_flag, 0, sizeof(int), s)) != hipSuccess) return e;
    int *cnt = nullptr;
    unsigned *tmax = nullptr;
    void *tmp = nullptr;
    size_t tmp_bytes = 0;
    if ((e = dmalloc(&cnt, sizeof(int) * (size_t)(M + 1), "tile entry counts")) != hipSuccess) return e;
    e = hipMemsetAsync(cnt + M, 0, sizeof(int), s);
    if (e == hipSuccess && atiles_lo && ntiles > 0) {
        e = dmalloc(&tmax, sizeof(unsigned) * (size_t)ntiles, "tile maxima");
        if (e == hipSuccess) e = hipMemsetAsync(tmax, 0, sizeof(unsigned) * (size_t)ntiles, s);
        if (e == hipSuccess) {
            hipLaunchKernelGGL(mfma_tile_build_kernel, dim3((unsigned)wave_grid(M)), dim3(kBlock), 0, s, rowptr, col,
                               val, M, atiles, cnt, range_flag, 1, tmax, nullptr, nullptr);
            e = hipGetLastError();
        }
        if (e == hipSuccess) {
            const int64_t g = std::max<int64_t>(1, std::min<int64_t>((ntiles + kBlock - 1) / kBlock, 1 << 16));
            hipLaunchKernelGGL(tile_exp_kernel, dim3((unsigned)g), dim3(kBlock), 0, s, tmax, ntiles, tile_exp);
            e = hipGetLastError();
        }
    }
    if (e == hipSuccess && M > 0) {
        hipLaunchKernelGGL(mfma_tile_build_kernel, dim3((unsigned)wave_grid(M)), dim3(kBlock), 0, s, rowptr, col, val,
                           M, atiles, cnt, range_flag, atiles_lo ? 2 : 0, nullptr, tile_exp, atiles_lo);
        e = hipGetLastError();
    }
    if (e == hipSuccess) e = hipcub::DeviceScan::ExclusiveSum(nullptr, tmp_bytes, cnt, rrowptr, (int)(M + 1), s);
    if (e == hipSuccess) e = dmalloc(&tmp, tmp_bytes > 0 ? tmp_bytes : 1, "residual scan storage");
    if (e == hipSuccess) e = hipcub::DeviceScan::ExclusiveSum(tmp, tmp_bytes, cnt, rrowptr, (int)(M + 1), s);
    if (e == hipSuccess) e = hipStreamSynchronize(s);
    if (tmp) dfree(tmp);
    if (tmax) dfree(tmax);
    dfree(cnt);
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
        void (*kern)(MfmaArgs, int64_t, int64_t) =
            a.atiles_lo ? (has_val ? mfma_tile_kernel_t<true, true> : mfma_tile_kernel_t<false, true>)
                        : (has_val ? mfma_tile_kernel_t<true, false> : mfma_tile_kernel_t<false, false>);
        hipLaunchKernelGGL(kern, dim3((unsigned)n), dim3(kWinBlock), 0, s, a, base, base + n);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

}  // namespace gspmm
