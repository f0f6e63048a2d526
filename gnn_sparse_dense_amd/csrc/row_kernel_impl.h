// Row kernel of the CSR SpMM: G lanes per output row, 64/G rows per wave64.
//
// Mapping (ParamSpMM section 2, Algorithm 1: a worker owns a segment of one C
// row and walks that row's entries; graph-spmm card, "Method": every feature
// column of a row belongs to one lane, which keeps that output's running value
// in its own register, and waves never exchange partial results, so there are
// no atomic updates):
//   * lane g of a row's group owns columns c0 + (f*G + g)*VEC .. +VEC-1 for
//     f < F (F = coarsening factor, ParamSpMM section 3.3 / GE-SpMM section
//     III-C "coarse-grained warp merging"), so for each entry the group's B
//     access is one contiguous, coalesced run of G*VEC floats per f;
//   * the wave's entries (all of its rows together) are staged kChunk at a
//     time in LDS with coalesced loads and then read back by every lane of the
//     owning group (GE-SpMM section III-B "coalesced row caching");
//   * several rows per wave when G < 64 serve narrow N and low degree
//     (DualGCN section 3.3, sparse path: a warp handles a subset of rows);
//   * each lane walks its row's entries in stored order with one accumulator
//     per output (fused multiply-add for sum/mean, strict '>' for max), so
//     every variant produces the same bits for a given row.
// Piece mode runs the same loop over pieces of split rows and writes partial
// results (plus int32 partial argmax) for the ordered combine.
#pragma once

#include <climits>
#include <cmath>

#include "spmm_internal.h"

namespace gspmm {

typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef int i32x2 __attribute__((ext_vector_type(2)));
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef long long i64x2 __attribute__((ext_vector_type(2)));
// The same vectors at their element alignment: a row of B or C starts at a
// multiple of 4 bytes only when N is not a multiple of 4 (or the caller's
// pointer is offset), and global loads and stores of 2 or 4 dwords need dword
// alignment only, so such rows still take one 8- or 16-byte access per lane.
typedef float f32x2a __attribute__((ext_vector_type(2), aligned(4)));
typedef float f32x4a __attribute__((ext_vector_type(4), aligned(4)));
typedef int i32x2a __attribute__((ext_vector_type(2), aligned(4)));
typedef int i32x4a __attribute__((ext_vector_type(4), aligned(4)));
typedef long long i64x2a __attribute__((ext_vector_type(2), aligned(8)));

// Block id permutation for the 8 XCDs.  The hardware hands consecutive block
// ids to the XCDs round-robin, each XCD with its own L2.  Within every run of
// kXcds * kXcdChunk hardware blocks, this gives XCD x the kXcdChunk
// consecutive logical blocks x*kXcdChunk ..: rows that share B rows (banded
// or community graphs) then meet in one L2, while all XCDs still sweep the
// same region of B and C together (one moving window in DRAM rather than
// eight).  A tail shorter than a full run is split into 8 contiguous ranges.
__device__ __forceinline__ int64_t xcd_remap_block(int64_t b, int64_t nb) {
    constexpr int64_t S = (int64_t)kXcds * kXcdChunk;
    const int64_t full = (nb / S) * S;
    if (b >= full) {
        const int64_t rb = b - full, rn = nb - full;
        const int64_t per = rn / kXcds, rem = rn % kXcds;
        const int64_t x = rb % kXcds, j = rb / kXcds;
        return full + (x < rem ? x * (per + 1) + j : rem * (per + 1) + (x - rem) * per + j);
    }
    const int64_t base = (b / S) * S, r = b - base;
    return base + (r % kXcds) * kXcdChunk + r / kXcds;
}

// Element offset of row r, column c of a row-major matrix with n columns,
// for 0 <= r, c, n < 2^31: one 32 x 32 -> 64-bit multiply-add rather than a
// full 64-bit product (three quarter-rate multiplies per gather).
__device__ __forceinline__ int64_t elem_off(int r, int64_t n, int c) {
    return (int64_t)((uint64_t)(uint32_t)r * (uint32_t)n + (uint32_t)c);
}

// Orders this wave's LDS writes before its later LDS reads (and reads before
// the next overwrite).  A wave's LDS operations execute in program order, so
// only compiler reordering has to be prevented.
__device__ __forceinline__ void wave_lds_sync() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

template <int VEC>
__device__ __forceinline__ void load_vec(const float *p, float (&x)[VEC]) {
    if constexpr (VEC == 4) {
        const f32x4 v = *reinterpret_cast<const f32x4a *>(p);
        x[0] = v.x; x[1] = v.y; x[2] = v.z; x[3] = v.w;
    } else if constexpr (VEC == 2) {
        const f32x2 v = *reinterpret_cast<const f32x2a *>(p);
        x[0] = v.x; x[1] = v.y;
    } else {
        x[0] = *p;
    }
}

// Stores of one lane's vector.  skip > 0 marks a row's last vector moved back
// to end at the launch's last column (lane_columns): it writes only its
// elements skip .. VEC-1, the columns no other lane writes.  The wave-wide
// test comes first, so that waves without such a lane (every wave when N is
// a multiple of VEC) take one scalar branch; it also keeps the window
// kernels within their 64 registers.
template <int VEC>
__device__ __forceinline__ void store_vec(float *p, const float (&x)[VEC], bool nt, int skip = 0) {
    if (VEC > 1 && __builtin_amdgcn_ballot_w64(skip > 0) != 0 && skip > 0) {
#pragma unroll
        for (int e = 1; e < VEC; ++e)
            if (e >= skip) p[e] = x[e];   // at most 3 elements per row: plain stores
    } else if constexpr (VEC == 4) {
        const f32x4a v = {x[0], x[1], x[2], x[3]};
        if (nt) __builtin_nontemporal_store(v, reinterpret_cast<f32x4a *>(p));
        else *reinterpret_cast<f32x4a *>(p) = v;
    } else if constexpr (VEC == 2) {
        const f32x2a v = {x[0], x[1]};
        if (nt) __builtin_nontemporal_store(v, reinterpret_cast<f32x2a *>(p));
        else *reinterpret_cast<f32x2a *>(p) = v;
    } else {
        if (nt) __builtin_nontemporal_store(x[0], p);
        else *p = x[0];
    }
}

template <int VEC>
__device__ __forceinline__ void store_arg64(int64_t *p, const int (&x)[VEC], int skip = 0) {
    if (VEC > 1 && __builtin_amdgcn_ballot_w64(skip > 0) != 0 && skip > 0) {
#pragma unroll
        for (int e = 1; e < VEC; ++e)
            if (e >= skip) p[e] = x[e];
    } else if constexpr (VEC == 4) {
        reinterpret_cast<i64x2a *>(p)[0] = i64x2a{x[0], x[1]};
        reinterpret_cast<i64x2a *>(p)[1] = i64x2a{x[2], x[3]};
    } else if constexpr (VEC == 2) {
        *reinterpret_cast<i64x2a *>(p) = i64x2a{x[0], x[1]};
    } else {
        *p = x[0];
    }
}

template <int VEC>
__device__ __forceinline__ void store_arg32(int *p, const int (&x)[VEC], int skip = 0) {
    if (VEC > 1 && __builtin_amdgcn_ballot_w64(skip > 0) != 0 && skip > 0) {
#pragma unroll
        for (int e = 1; e < VEC; ++e)
            if (e >= skip) p[e] = x[e];
    } else if constexpr (VEC == 4) *reinterpret_cast<i32x4a *>(p) = i32x4a{x[0], x[1], x[2], x[3]};
    else if constexpr (VEC == 2) *reinterpret_cast<i32x2a *>(p) = i32x2a{x[0], x[1]};
    else *p = x[0];
}

// Gathers and reduces entries [lo, hi) of the staged index list cp (values vp,
// as fp32 bit patterns) into this lane's accumulators.  Batches of U entries:
// all loads of a batch are issued before the first use, and a short row (or
// the tail of a long one) is one predicated batch rather than one round trip
// per entry.  Entries are folded in stored order with one accumulator per
// output: fused multiply-add (plain add when unweighted) or strict '>'.
// WIN: entries whose column lies in [w0, w0 + kWinRows) read B from the
// block's LDS copy sB (kWinCols columns per row, lane quad g) instead of HBM.
// IDX16: the index list holds 16-bit offsets from `base` (compact row tiles).
template <int F, int VEC, bool HAS_VAL, bool IS_MAX, bool WIN = false, int UB = 0, bool IDX16 = false>
__device__ __forceinline__ void consume(const void *cpv, const int *vp, int lo, int hi, const float *__restrict__ Bp,
                                        int64_t N, const int (&colf)[F], const bool (&ok)[F],
                                        float (&acc)[F][VEC], int (&arg)[F][VEC],
                                        const f32x4 *sB = nullptr, int64_t w0 = 0, int g = 0, int base = 0) {
    const int *cp = static_cast<const int *>(cpv);
    const unsigned short *cp16 = static_cast<const unsigned short *>(cpv);
    constexpr int U = UB ? UB : ((F * VEC <= 4) ? 8 : 4);
    for (int k = lo; k < hi; k += U) {
        int cidx[U];
        float w[U];
        bool vld[U];
        float bv[U][F][VEC];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            vld[u] = k + u < hi;
            const int kk = vld[u] ? k + u : lo;
            cidx[u] = IDX16 ? base + (int)cp16[kk] : cp[kk];
            w[u] = HAS_VAL ? __int_as_float(vp[kk]) : 1.0f;
        }
#pragma unroll
        for (int u = 0; u < U; ++u)
#pragma unroll
            for (int f = 0; f < F; ++f) {
#pragma unroll
                for (int e = 0; e < VEC; ++e) bv[u][f][e] = 0.0f;
                if constexpr (WIN) {
                    static_assert(F == 1 && VEC == 4, "window path: one float4 per lane");
                    const int64_t wr = (int64_t)cidx[u] - w0;
                    if (vld[u] && ok[f]) {
                        if (wr >= 0 && wr < kWinRows) {
                            const f32x4 t = sB[wr * (kWinCols / 4) + g];
                            bv[u][f][0] = t.x; bv[u][f][1] = t.y; bv[u][f][2] = t.z; bv[u][f][3] = t.w;
                        } else {
                            load_vec<VEC>(Bp + elem_off(cidx[u], N, colf[f]), bv[u][f]);
                        }
                    }
                } else {
                    if (vld[u] && ok[f]) load_vec<VEC>(Bp + elem_off(cidx[u], N, colf[f]), bv[u][f]);
                }
            }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            if (!vld[u]) continue;
#pragma unroll
            for (int f = 0; f < F; ++f)
#pragma unroll
                for (int e = 0; e < VEC; ++e) {
                    if constexpr (IS_MAX) {
                        const float t = HAS_VAL ? w[u] * bv[u][f][e] : bv[u][f][e];
                        if (arg[f][e] < 0 || t > acc[f][e]) {
                            acc[f][e] = t;
                            arg[f][e] = cidx[u];
                        }
                    } else {
                        acc[f][e] = HAS_VAL ? __builtin_fmaf(w[u], bv[u][f][e], acc[f][e]) : acc[f][e] + bv[u][f][e];
                    }
                }
        }
    }
}

template <int F, int VEC, bool IS_MAX>
__device__ __forceinline__ void init_acc(float (&acc)[F][VEC], int (&arg)[F][VEC]) {
#pragma unroll
    for (int f = 0; f < F; ++f)
#pragma unroll
        for (int e = 0; e < VEC; ++e) {
            acc[f][e] = IS_MAX ? -INFINITY : 0.0f;
            arg[f][e] = -1;
        }
}

// The mean's division by the row degree (one IEEE fp32 division per output;
// empty rows keep their 0).  The mean flag is uniform, and the branch on it
// must stay a branch: the compiler would otherwise run the division sequence
// (about 15 instructions per element) for every sum as well and select.
template <int VEC>
__device__ __forceinline__ void mean_divide(bool mean, int deg, float (&res)[VEC]) {
    if (mean) {
        asm volatile("" ::: "memory");   // nothing to hoist out of this branch
#pragma unroll
        for (int e = 0; e < VEC; ++e) res[e] = deg > 0 ? res[e] / (float)deg : res[e];
    }
}

// Epilogue of one output row (or piece): mean division, empty-row values,
// argmax as int64 column ids (int32 in piece mode).
template <int F, int VEC, bool IS_MAX, bool PIECES>
__device__ __forceinline__ void store_out(const RowArgs &a, int64_t orow, int deg, const int (&colf)[F],
                                          const bool (&ok)[F], const float (&acc)[F][VEC],
                                          const int (&arg)[F][VEC]) {
    float *orow_p = a.out + orow * a.ldo;
#pragma unroll
    for (int f = 0; f < F; ++f) {
        if (!ok[f]) continue;
        const int64_t cc = (int64_t)colf[f] - a.c_begin;
        // lanes own columns c_begin + k*VEC ..; a vector moved back to end at
        // c_end starts off that grid, and its first elements are a neighbour's
        const int skip = (VEC - ((colf[f] - (int)a.c_begin) & (VEC - 1))) & (VEC - 1);   // VEC a power of two
        float res[VEC];
        int ar[VEC];
#pragma unroll
        for (int e = 0; e < VEC; ++e) {
            if constexpr (IS_MAX) {
                res[e] = deg > 0 ? acc[f][e] : 0.0f;
                ar[e] = deg > 0 ? arg[f][e] : -1;
            } else {
                res[e] = acc[f][e];
            }
        }
        if constexpr (!IS_MAX && !PIECES) mean_divide<VEC>(a.mean != 0, deg, res);
        store_vec<VEC>(orow_p + cc, res, a.nt_store != 0, skip);
        if constexpr (IS_MAX) {
            if constexpr (PIECES) store_arg32<VEC>(a.part_arg + orow * a.ldo + cc, ar, skip);
            else if (a.argmax) store_arg64<VEC>(a.argmax + orow * a.ldo + cc, ar, skip);
        }
    }
}

// Column ownership of lane g within its row group for the slice starting at c0.
// When the launch's width is not a multiple of VEC, the one vector that would
// run past c_end is moved back to end there: it reads the last VEC columns,
// the lower ones of which its neighbour lane also reads, and writes only the
// columns past its neighbour's (store_out), so every access stays inside the
// row (the launch guarantees c_end - c_begin >= VEC) and no two lanes write
// the same element.
template <int G, int VEC, int F>
__device__ __forceinline__ void lane_columns(const RowArgs &a, int64_t c0, int g, int (&colf)[F], bool (&ok)[F]) {
#pragma unroll
    for (int f = 0; f < F; ++f) {
        const int64_t c = c0 + (int64_t)(f * G + g) * VEC;
        ok[f] = c < a.c_end;
        const int64_t last = a.c_end - VEC;   // first column of the last whole vector
        colf[f] = (int)(VEC > 1 && c > last ? last : c);
    }
}

// Rows (or pieces) task0 .. task0 + 64/G - 1 of one wave from the CSR arrays:
// row bounds, then the wave's index chunk staged in LDS, then the gathers.
template <int G, int VEC, int F, bool HAS_VAL, bool IS_MAX, bool PIECES, int CH = kChunk, bool WIN = false>
__device__ __forceinline__ void row_task(const RowArgs &a, int64_t task0, int lane, int *s_col, int *s_val,
                                         const int (&colf)[F], const bool (&ok)[F],
                                         const f32x4 *sB = nullptr, int64_t w0 = 0) {
    constexpr int R = 64 / G;
    constexpr int NT = CH / 64;        // staging loads per lane per chunk
    const int sub = lane / G;
    int64_t v = task0 + sub;
    bool live = v < a.ntasks;
    if constexpr (PIECES)
        if (live && a.task_perm) v = a.task_perm[v];   // the piece this task computes
    int beg = 0, end = 0;
    if (live) {
        if constexpr (PIECES) {
            beg = a.seg_begin[v];
            end = a.seg_end[v];
        } else {
            beg = a.rowptr[v];
            end = a.rowptr[v + 1];
        }
    }
    int deg = end - beg;
    if (!PIECES && deg > a.skip_above) {   // split row: its pieces produce the output
        deg = 0;
        live = false;
    }

    // Position of this group's entries in the wave's concatenated entry list.
    const int beg0 = __builtin_amdgcn_readfirstlane(beg);
    int off = 0, total = 0;
    bool contiguous = true;
#pragma unroll
    for (int s = 0; s < R; ++s) {
        const int ds = __builtin_amdgcn_readlane(deg, s * G);
        const int bs = __builtin_amdgcn_readlane(beg, s * G);
        off += (s < sub) ? ds : 0;
        contiguous = contiguous && (ds == 0 || bs == beg0 + total);
        total += ds;
    }

    float acc[F][VEC];
    int arg[F][VEC];
    init_acc<F, VEC, IS_MAX>(acc, arg);

    for (int cb = 0; cb < total; cb += CH) {
        const int cn = min(CH, total - cb);
        const int nt = (cn + 63) >> 6;
        int cr[NT];
        int vr[NT];
#pragma unroll
        for (int t = 0; t < NT; ++t) {
            if (t < nt) {
                const int q = cb + min(t * 64 + lane, cn - 1);
                int p;
                if (contiguous) {
                    p = beg0 + q;
                } else {
                    p = 0;
                    int o = 0;
#pragma unroll
                    for (int s = 0; s < R; ++s) {
                        const int ds = __builtin_amdgcn_readlane(deg, s * G);
                        const int bs = __builtin_amdgcn_readlane(beg, s * G);
                        p = (q >= o && q < o + ds) ? bs + (q - o) : p;
                        o += ds;
                    }
                }
                cr[t] = a.col[p];
                if constexpr (HAS_VAL) vr[t] = __float_as_int(a.val[p]);
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
        // window blocks read most of B from LDS: shorter batches keep the
        // 1024-thread block within 64 VGPRs (two blocks per CU)
        consume<F, VEC, HAS_VAL, IS_MAX, WIN, WIN ? 4 : 0>(s_col, s_val, lo, hi, a.B, a.N, colf, ok, acc, arg,
                                                          sB, w0, lane % G);
        wave_lds_sync();
    }

    if (live) store_out<F, VEC, IS_MAX, PIECES>(a, v, deg, colf, ok, acc, arg);
}

// lin -> (lin mod d, lin div d) for a linear block id: nothing to divide for
// d = 1, a 32-bit division while the grid has fewer than 2^32 blocks (a
// 64-bit one costs about 80 scalar instructions per wave).
__device__ __forceinline__ void split_block_id(int64_t lin, int64_t d, int64_t *rem, int64_t *quo) {
    if (d == 1) {
        *rem = 0;
        *quo = lin;
    } else if ((int64_t)gridDim.x * gridDim.y <= (int64_t)UINT32_MAX) {
        const uint32_t l = (uint32_t)lin, q = l / (uint32_t)d;
        *quo = q;
        *rem = l - q * (uint32_t)d;
    } else {
        *quo = lin / d;
        *rem = lin - *quo * d;
    }
}

// Block -> (first wave task, column slice), optionally XCD-aware.
__device__ __forceinline__ void block_coords(const RowArgs &a, int64_t *bx, int64_t *by) {
    const int64_t gx = gridDim.x;
    int64_t lin = (int64_t)blockIdx.y * gx + blockIdx.x;
    if (a.xcd_remap) lin = xcd_remap_block(lin, gx * (int64_t)gridDim.y);
    if (gridDim.y == 1) {            // one column slice: lin is the task group
        *bx = lin;
        *by = 0;
        return;
    }
    split_block_id(lin, gx, bx, by);
}

template <int G, int VEC, int F, bool HAS_VAL, bool IS_MAX, bool PIECES>
__global__ __launch_bounds__(kBlock) void row_kernel_t(RowArgs a) {
    static_assert(G >= 4 && G <= 64 && (64 % G) == 0, "lanes per row");
    constexpr int R = 64 / G;          // rows (or pieces) per wave
    constexpr int SL = G * VEC * F;    // columns per slice
    __shared__ int s_col[kWaves][kChunk];
    __shared__ int s_val[kWaves][HAS_VAL ? kChunk : 1];

    const int lane = threadIdx.x & 63;
    const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);   // uniform per wave
    int64_t bx, by;
    block_coords(a, &bx, &by);
    const int64_t task0 = a.task_base + (bx * kWaves + wv) * R;
    if (task0 >= a.ntasks) return;                     // uniform per wave
    int colf[F];
    bool ok[F];
    lane_columns<G, VEC, F>(a, a.c_begin + by * SL, lane % G, colf, ok);
    row_task<G, VEC, F, HAS_VAL, IS_MAX, PIECES>(a, task0, lane, s_col[wv], s_val[wv], colf, ok);
}

// Row-tile kernel for low-degree graphs.  The plan stores every kTileRows-row
// tile as one fixed-size record holding the tile's row bounds and indexes
// (and values), so a wave reads its 64/G / kTileRows records with one
// coalesced pass and has bounds and indexes together: its gathers start one
// memory latency after launch instead of two (bounds, then indexes).
//   wide record:    kTileRows int32 cumulative row ends (-1 in the last word
//                   marks an overflow tile), tile_cap int32 column ids;
//   compact record: int32 base column (-1 marks an overflow tile), kTileRows
//                   uint8 cumulative row ends in two words, tile_cap uint16
//                   offsets from the base;
// then, when weighted, tile_cap fp32 values.  Overflow tiles (more entries
// than tile_cap, or a column span beyond 16 bits) go through the CSR path.
// UB: entries per batch (0: the consume loop's default).
template <int G, int VEC, int F, bool HAS_VAL, bool IS_MAX, bool COMPACT, int UB = 0>
__global__ __launch_bounds__(kBlock) void tile_kernel_t(RowArgs a) {
    static_assert(G == 4 || G == 8, "a wave holds one or two row tiles");
    constexpr int R = 64 / G;
    constexpr int TPW = R / kTileRows;       // tiles per wave
    constexpr int SL = G * VEC * F;
    constexpr int NL = kTileLdsWords / 64;   // record loads per lane
    constexpr int HDR = COMPACT ? 3 : kTileRows;
    __shared__ int s_rec[kWaves][kTileLdsWords];
    __shared__ int s_col[kWaves][kChunk];
    __shared__ int s_val[kWaves][HAS_VAL ? kChunk : 1];

    const int lane = threadIdx.x & 63;
    const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);   // uniform per wave
    const int sub = lane / G;
    int64_t bx, by;
    block_coords(a, &bx, &by);
    const int64_t tile0 = a.task_base / kTileRows + (bx * kWaves + wv) * TPW;
    const int64_t row0 = tile0 * kTileRows;
    if (row0 >= a.ntasks) return;                      // uniform per wave
    int colf[F];
    bool ok[F];
    lane_columns<G, VEC, F>(a, a.c_begin + by * SL, lane % G, colf, ok);

    const int rs = a.tile_words;
    const int64_t ntiles = (a.ntasks + kTileRows - 1) / kTileRows;
    const int nwords = (int)min((int64_t)TPW, ntiles - tile0) * rs;
    const int *rec = a.tiles + tile0 * rs;
    int r[NL];
#pragma unroll
    for (int i = 0; i < NL; ++i)
        if (i * 64 < nwords) r[i] = rec[min(i * 64 + lane, nwords - 1)];
#pragma unroll
    for (int i = 0; i < NL; ++i)
        if (i * 64 < nwords) s_rec[wv][i * 64 + lane] = r[i];
    wave_lds_sync();

    bool overflow = false;
#pragma unroll
    for (int t = 0; t < TPW; ++t)
        if (t * rs < nwords) overflow = overflow || s_rec[wv][t * rs + (COMPACT ? 0 : kTileRows - 1)] < 0;
    if (overflow) {                                     // uniform: CSR path for these rows
        row_task<G, VEC, F, HAS_VAL, IS_MAX, false>(a, row0, lane, s_col[wv], s_val[wv], colf, ok);
        return;
    }

    const int t = sub / kTileRows;
    const int j = sub - t * kTileRows;
    const int64_t orow = row0 + sub;
    const bool live = orow < a.ntasks;
    const int *hdr = s_rec[wv] + t * rs;
    int b = 0, e = 0, base = 0;
    if constexpr (COMPACT) {
        base = hdr[0];
        e = (hdr[1 + (j >> 2)] >> (8 * (j & 3))) & 255;
        if (j) b = (hdr[1 + ((j - 1) >> 2)] >> (8 * ((j - 1) & 3))) & 255;
    } else {
        e = hdr[j];
        if (j) b = hdr[j - 1];
    }
    const int deg = live ? e - b : 0;
    const int idx_words = COMPACT ? a.tile_cap / 2 : a.tile_cap;
    const int *vp = hdr + HDR + idx_words + b;
    float acc[F][VEC];
    int arg[F][VEC];
    init_acc<F, VEC, IS_MAX>(acc, arg);
    if constexpr (COMPACT) {
        const unsigned short *cp16 = reinterpret_cast<const unsigned short *>(hdr + HDR) + b;
        consume<F, VEC, HAS_VAL, IS_MAX, false, UB, true>(cp16, vp, 0, deg, a.B, a.N, colf, ok, acc, arg, nullptr,
                                                        0, 0, base);
    } else {
        consume<F, VEC, HAS_VAL, IS_MAX, false, UB>(hdr + HDR + b, vp, 0, deg, a.B, a.N, colf, ok, acc, arg);
    }
    if (live) store_out<F, VEC, IS_MAX, false>(a, orow, deg, colf, ok, acc, arg);
}

// Window kernels for graphs whose neighbours mostly fall in their own aligned
// block of kWinRows rows (community / locality structure, RA-SpMM's
// community regime).  A 1024-thread block owns one such block of rows and one
// kWinCols-wide column slice: it first copies B's rows of that block (the
// window, 64 KB) into LDS, then its 16 waves walk the block's rows four at a
// time (16 lanes x float4 per row), reading entries inside the window from
// LDS.  Every B row of the window is then read from HBM once per slice
// instead of once per referencing row.  Both kernels fold each row's entries
// in stored order with one accumulator, so every result bit is the row
// kernel's.

// Block -> (first row of the window, first column of the slice).  Consecutive
// linear ids walk the slices of one row block, so the block's indexes stay in
// one L2 while its slices run.
__device__ __forceinline__ void window_coords(const RowArgs &a, int64_t *w0, int64_t *c0) {
    const int64_t gx = gridDim.x;
    int64_t lin = (int64_t)blockIdx.y * gx + blockIdx.x;
    if (a.xcd_remap) lin = xcd_remap_block(lin, gx * (int64_t)gridDim.y);
    int64_t tile, slice;
    split_block_id(lin, gridDim.y, &slice, &tile);
    *w0 = tile * kWinRows;
    *c0 = slice * kWinCols;
}

// The window: B rows w0 .. w0 + kWinRows - 1, columns c0 .. c0 + kWinCols - 1,
// zero past the edges of B.  Slot q holds the vector that lane q of a row
// reads: when N is not a multiple of 4, the vector that would run past column
// N ends there instead (as in lane_columns; N >= 4).
__device__ __forceinline__ void load_window(const RowArgs &a, f32x4 *s_B, int64_t w0, int64_t c0) {
    constexpr int Q = kWinCols / 4;                 // float4 per window row
    for (int i = threadIdx.x; i < kWinRows * Q; i += kWinBlock) {
        const int r = i / Q, q = i - (i / Q) * Q;
        const int64_t brow = w0 + r, bcol = c0 + q * 4;
        f32x4 v = {0.0f, 0.0f, 0.0f, 0.0f};
        if (brow < a.K && bcol < a.N) {
            const int64_t bc = bcol > a.N - 4 ? a.N - 4 : bcol;
            v = *reinterpret_cast<const f32x4a *>(a.B + brow * a.N + bc);
        }
        s_B[i] = v;
    }
    __syncthreads();
}

// Any column order: each entry picks LDS or HBM by its own column.
template <bool HAS_VAL, bool IS_MAX>
__global__ __launch_bounds__(kWinBlock) void window_kernel_t(RowArgs a) {
    constexpr int G = kWinCols / 4, VEC = 4, F = 1, R = 64 / G;   // one float4 per lane
    constexpr int WW = kWinBlock / 64;              // waves per block
    __shared__ f32x4 s_B[kWinRows * (kWinCols / 4)];
    __shared__ int s_col[WW][kWinChunk];
    __shared__ int s_val[WW][HAS_VAL ? kWinChunk : 1];

    const int lane = threadIdx.x & 63;
    const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);   // uniform per wave
    int64_t w0, c0;
    window_coords(a, &w0, &c0);
    load_window(a, s_B, w0, c0);

    int colf[F];
    bool ok[F];
    lane_columns<G, VEC, F>(a, c0, lane % G, colf, ok);
    for (int pass = 0; pass < kWinRows / (WW * R); ++pass) {
        const int64_t task0 = w0 + (int64_t)(pass * WW + wv) * R;
        if (task0 < a.ntasks)
            row_task<G, VEC, F, HAS_VAL, IS_MAX, false, kWinChunk, true>(a, task0, lane, s_col[wv], s_val[wv],
                                                                       colf, ok, s_B, w0);
    }
}

// Staged entry of the sorted-row window kernel: a key, and the value's bits
// beside it when the graph is weighted, so one LDS read returns both.  The
// key of an entry outside the window is its column; inside the window it is
// the bitwise complement of the window row's byte offset (a negative
// number), worked out once per entry at staging time, where one instruction
// serves 64 entries, rather than in the fold loop, where it serves four.
constexpr int kWinRowBytes = kWinCols * 4;
template <bool HAS_VAL> struct WinEntry { typedef int type; };
template <> struct WinEntry<true> { typedef i32x2 type; };
__device__ __forceinline__ int ent_key(int e) { return e; }
__device__ __forceinline__ int ent_key(i32x2 e) { return e.x; }
__device__ __forceinline__ float ent_val(int) { return 1.0f; }
__device__ __forceinline__ float ent_val(i32x2 e) { return __int_as_float(e.y); }
__device__ __forceinline__ int win_key(int c, int wlo) {
    const int r = c - wlo;
    return (unsigned)r < (unsigned)kWinRows ? ~(r * kWinRowBytes) : c;
}

// Folds one B vector (entry column c, weight w) into the accumulators.
template <bool HAS_VAL, bool IS_MAX>
__device__ __forceinline__ void win_fold(float (&acc)[1][4], int (&arg)[1][4], const f32x4 &b, float w, int c) {
    const float b4[4] = {b.x, b.y, b.z, b.w};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        if constexpr (IS_MAX) {
            const float t = HAS_VAL ? w * b4[e] : b4[e];
            if (arg[0][e] < 0 || t > acc[0][e]) {
                acc[0][e] = t;
                arg[0][e] = c;
            }
        } else {
            acc[0][e] = HAS_VAL ? __builtin_fmaf(w, b4[e], acc[0][e]) : acc[0][e] + b4[e];
        }
    }
}

// Staged entries [lo, hi) of one row, all outside the window (keys are
// columns): predicated batches of U gathers from HBM, as in the row kernel.
template <bool HAS_VAL, bool IS_MAX, int U, typename E>
__device__ __forceinline__ void win_hbm_run(const E *se, int lo, int hi, const RowArgs &a, int colf, bool ok,
                                            float (&acc)[1][4], int (&arg)[1][4]) {
    for (int k = lo; k < hi; k += U) {
        E ent[U];
        f32x4 b[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            ent[u] = se[k + u < hi ? k + u : lo];
            b[u] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
            if (k + u < hi && ok) b[u] = *reinterpret_cast<const f32x4a *>(a.B + elem_off(ent_key(ent[u]), a.N, colf));
        }
#pragma unroll
        for (int u = 0; u < U; ++u)
            if (k + u < hi) win_fold<HAS_VAL, IS_MAX>(acc, arg, b[u], ent_val(ent[u]), ent_key(ent[u]));
    }
}

// B vector of an inside-window key for the lane whose float4 sits at byte
// g16 of each window row: g16 + ~key = (g16 - 1) - key.
__device__ __forceinline__ f32x4 win_vec(const f32x4 *sB, int g16m1, int key) {
    return *reinterpret_cast<const f32x4 *>(reinterpret_cast<const char *>(sB) + (g16m1 - key));
}

// Staged entries [lo, hi) of one row, all inside the window: B from LDS, in
// full batches of four, then one predicated batch for the last one to three
// (lanes past the end re-read entry lo, inside the window too).
template <bool HAS_VAL, bool IS_MAX, typename E>
__device__ __forceinline__ void win_lds_run(const E *se, int lo, int hi, const f32x4 *sB, int g16m1, int wlo,
                                            float (&acc)[1][4], int (&arg)[1][4]) {
    constexpr int U = 4;
    int k = lo;
    for (; k + U <= hi; k += U) {
        E ent[U];
        f32x4 b[U];
#pragma unroll
        for (int u = 0; u < U; ++u) ent[u] = se[k + u];
#pragma unroll
        for (int u = 0; u < U; ++u) b[u] = win_vec(sB, g16m1, ent_key(ent[u]));
#pragma unroll
        for (int u = 0; u < U; ++u)
            win_fold<HAS_VAL, IS_MAX>(acc, arg, b[u], ent_val(ent[u]),
                                      IS_MAX ? wlo + (~ent_key(ent[u])) / kWinRowBytes : 0);
    }
    if (k < hi) {
        E ent[U - 1];
        f32x4 b[U - 1];
#pragma unroll
        for (int u = 0; u < U - 1; ++u) ent[u] = se[k + u < hi ? k + u : lo];
#pragma unroll
        for (int u = 0; u < U - 1; ++u) b[u] = win_vec(sB, g16m1, ent_key(ent[u]));
#pragma unroll
        for (int u = 0; u < U - 1; ++u)
            if (k + u < hi)
                win_fold<HAS_VAL, IS_MAX>(acc, arg, b[u], ent_val(ent[u]),
                                          IS_MAX ? wlo + (~ent_key(ent[u])) / kWinRowBytes : 0);
    }
}

// Rows with non-decreasing columns (checked when the plan is built).  Within
// any stretch of such a row the entries fall in three runs: columns below
// the window, inside it, above it.  Folding the runs one after the other
// keeps the stored order, while the HBM gathers of the outer runs no longer
// hold up the LDS batches of the inner run, and the inner run needs no
// per-entry choice between LDS and HBM.  Run lengths per row come from the
// plan (win_lo, win_in), read beside the row bounds.
template <bool HAS_VAL, bool IS_MAX>
__global__ __launch_bounds__(kWinBlock) __attribute__((amdgpu_waves_per_eu(8, 8)))
void window_sorted_kernel_t(RowArgs a) {
    constexpr int G = kWinCols / 4, R = 64 / G;     // 16 lanes x float4 per row, 4 rows per wave
    constexpr int WW = kWinBlock / 64;
    constexpr int NT = kWinChunk / 64;
    typedef typename WinEntry<HAS_VAL>::type E;
    __shared__ f32x4 s_B[kWinRows * (kWinCols / 4)];
    __shared__ E s_e[WW][kWinChunk];

    const int lane = threadIdx.x & 63;
    const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);   // uniform per wave
    const int sub = lane / G, g = lane % G;
    int64_t w0, c0;
    window_coords(a, &w0, &c0);
    load_window(a, s_B, w0, c0);
    const int wlo = (int)w0;
    const int g16m1 = g * 16 - 1;
    const bool ok = c0 + g * 4 < a.c_end;
    const int colf = (int)(c0 + g * 4 > a.c_end - 4 ? a.c_end - 4 : c0 + g * 4);   // as in lane_columns
    E *se = s_e[wv];

    for (int pass = 0; pass < kWinRows / (WW * R); ++pass) {
        const int64_t task0 = w0 + (int64_t)(pass * WW + wv) * R;
        if (task0 >= a.ntasks) continue;            // uniform per wave
        const int64_t v = task0 + sub;
        bool live = v < a.ntasks;
        int beg = 0, end = 0, rlo = 0, rin = 0;
        if (live) {
            beg = a.rowptr[v];
            end = a.rowptr[v + 1];
            rlo = a.win_lo[v];
            rin = a.win_in[v];
        }
        int deg = end - beg;
        if (deg > a.skip_above) {                   // split row: its pieces produce the output
            deg = 0;
            live = false;
        }
        const int beg0 = __builtin_amdgcn_readfirstlane(beg);
        int off = 0, total = 0;
        bool contiguous = true;
#pragma unroll
        for (int s = 0; s < R; ++s) {
            const int ds = __builtin_amdgcn_readlane(deg, s * G);
            const int bs = __builtin_amdgcn_readlane(beg, s * G);
            off += (s < sub) ? ds : 0;
            contiguous = contiguous && (ds == 0 || bs == beg0 + total);
            total += ds;
        }

        float acc[1][4];
        int arg[1][4];
        init_acc<1, 4, IS_MAX>(acc, arg);
        for (int cb = 0; cb < total; cb += kWinChunk) {
            const int cn = min(kWinChunk, total - cb);
            E er[NT];
#pragma unroll
            for (int t = 0; t < NT; ++t) {
                if (t * 64 < cn) {
                    const int q = cb + min(t * 64 + lane, cn - 1);
                    int p;
                    if (contiguous) {
                        p = beg0 + q;
                    } else {
                        p = 0;
                        int o = 0;
#pragma unroll
                        for (int s = 0; s < R; ++s) {
                            const int ds = __builtin_amdgcn_readlane(deg, s * G);
                            const int bs = __builtin_amdgcn_readlane(beg, s * G);
                            p = (q >= o && q < o + ds) ? bs + (q - o) : p;
                            o += ds;
                        }
                    }
                    if constexpr (HAS_VAL) er[t] = i32x2{win_key(a.col[p], wlo), __float_as_int(a.val[p])};
                    else er[t] = win_key(a.col[p], wlo);
                }
            }
#pragma unroll
            for (int t = 0; t < NT; ++t)
                if (t * 64 < cn) se[t * 64 + lane] = er[t];
            wave_lds_sync();
            // the row's stretch of this chunk and its run boundaries, in chunk positions
            const int lo = max(off, cb) - cb;
            const int hi = max(lo, min(off + deg, cb + cn) - cb);
            const int q1 = min(max(off + rlo - cb, lo), hi);
            const int q2 = min(max(off + rlo + rin - cb, lo), hi);
            win_hbm_run<HAS_VAL, IS_MAX, 2>(se, lo, q1, a, colf, ok, acc, arg);
            win_lds_run<HAS_VAL, IS_MAX>(se, q1, q2, s_B, g16m1, wlo, acc, arg);
            win_hbm_run<HAS_VAL, IS_MAX, 2>(se, q2, hi, a, colf, ok, acc, arg);
            wave_lds_sync();
        }
        const int colv[1] = {colf};
        const bool okv[1] = {ok};
        if (live) store_out<1, 4, IS_MAX, false>(a, v, deg, colv, okv, acc, arg);
    }
}

// Lookup of one instantiated kernel; G = 64 also gets the piece-mode kernels,
// G = 4 and 8 the row-tile kernels.
template <int G, int VEC, int F>
RowKernelFn pick_row_kernel(const RowKernelKey &k) {
    if (k.tiled) {
        if constexpr (G == 4 || G == 8) {
            if (k.pieces) return nullptr;
            if (k.batch4) {
                // sum and mean only (max measured no faster in batches of 4)
                if constexpr (G == 4 && VEC == 4 && F == 1) {
                    if (k.is_max) return nullptr;
                    if (k.compact)
                        return k.has_val ? tile_kernel_t<G, VEC, F, true, false, true, 4>
                                         : tile_kernel_t<G, VEC, F, false, false, true, 4>;
                    return k.has_val ? tile_kernel_t<G, VEC, F, true, false, false, 4>
                                     : tile_kernel_t<G, VEC, F, false, false, false, 4>;
                } else {
                    return nullptr;
                }
            }
            if (k.compact) {
                if (k.is_max)
                    return k.has_val ? tile_kernel_t<G, VEC, F, true, true, true>
                                     : tile_kernel_t<G, VEC, F, false, true, true>;
                return k.has_val ? tile_kernel_t<G, VEC, F, true, false, true>
                                 : tile_kernel_t<G, VEC, F, false, false, true>;
            }
            if (k.is_max)
                return k.has_val ? tile_kernel_t<G, VEC, F, true, true, false>
                                 : tile_kernel_t<G, VEC, F, false, true, false>;
            return k.has_val ? tile_kernel_t<G, VEC, F, true, false, false>
                             : tile_kernel_t<G, VEC, F, false, false, false>;
        } else {
            return nullptr;
        }
    }
    if (k.pieces) {
        if constexpr (G == 64) {
            if (k.is_max)
                return k.has_val ? row_kernel_t<G, VEC, F, true, true, true>
                                 : row_kernel_t<G, VEC, F, false, true, true>;
            return k.has_val ? row_kernel_t<G, VEC, F, true, false, true>
                             : row_kernel_t<G, VEC, F, false, false, true>;
        } else {
            return nullptr;
        }
    }
    if (k.is_max)
        return k.has_val ? row_kernel_t<G, VEC, F, true, true, false>
                         : row_kernel_t<G, VEC, F, false, true, false>;
    return k.has_val ? row_kernel_t<G, VEC, F, true, false, false>
                     : row_kernel_t<G, VEC, F, false, false, false>;
}

template <int VEC>
RowKernelFn pick_row_kernel_vec(const RowKernelKey &k) {
    if (k.coarsen == 1) {
        switch (k.lanes) {
            case 4: return pick_row_kernel<4, VEC, 1>(k);
            case 8: return pick_row_kernel<8, VEC, 1>(k);
            case 16: return pick_row_kernel<16, VEC, 1>(k);
            case 32: return pick_row_kernel<32, VEC, 1>(k);
            case 64: return pick_row_kernel<64, VEC, 1>(k);
        }
    } else if (k.coarsen == 2) {
        switch (k.lanes) {
            case 4: return pick_row_kernel<4, VEC, 2>(k);
            case 8: return pick_row_kernel<8, VEC, 2>(k);
            case 16: return pick_row_kernel<16, VEC, 2>(k);
            case 32: return pick_row_kernel<32, VEC, 2>(k);
            case 64: return pick_row_kernel<64, VEC, 2>(k);
        }
    }
    return nullptr;
}

}  // namespace gspmm
