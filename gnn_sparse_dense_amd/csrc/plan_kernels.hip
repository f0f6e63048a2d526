// Plan-time kernels: CSR validation, degree descriptors, index narrowing and
// the row split.  All are single passes over rowptr or col (O(M) / O(nnz)),
// run once per graph and amortised over every later product (RA-SpMM,
// abstract and "Matched lifecycle timing": descriptors come from one O(M)
// pass over the row pointer; formats are built once and reused).
//
// Each block reduces its slice to one record; the host folds the records in
// block order, so every result is exact and independent of scheduling.
#include <climits>

#include <hipcub/hipcub.hpp>

#include "alloc.h"
#include "spmm_internal.h"

namespace gspmm {

namespace {

__device__ __forceinline__ void block_reduce5(int64_t &mn, uint64_t &s1, uint64_t &s2, int64_t &mx,
                                              int64_t &ne) {
    __shared__ int64_t sh_mn[kBlock], sh_mx[kBlock], sh_ne[kBlock];
    __shared__ uint64_t sh_s1[kBlock], sh_s2[kBlock];
    const int t = threadIdx.x;
    sh_mn[t] = mn; sh_s1[t] = s1; sh_s2[t] = s2; sh_mx[t] = mx; sh_ne[t] = ne;
    __syncthreads();
    for (int o = kBlock / 2; o > 0; o >>= 1) {
        if (t < o) {
            sh_mn[t] = min(sh_mn[t], sh_mn[t + o]);
            sh_s1[t] += sh_s1[t + o];
            sh_s2[t] += sh_s2[t + o];
            sh_mx[t] = max(sh_mx[t], sh_mx[t + o]);
            sh_ne[t] += sh_ne[t + o];
        }
        __syncthreads();
    }
    mn = sh_mn[0]; s1 = sh_s1[0]; s2 = sh_s2[0]; mx = sh_mx[0]; ne = sh_ne[0];
}

// Rows [b*kRowsPerScanBlock, ...): monotonicity (and rowptr[0] == 0), degree
// sums, largest degree, empty rows; also writes the int32 copy of rowptr.
// Callers guarantee rowptr[M] < 2^31.
__global__ __launch_bounds__(kBlock) void rowscan_kernel(const int64_t *__restrict__ rowptr, int64_t M,
                                                         int *__restrict__ rowptr32,
                                                         RowScanOut *__restrict__ out) {
    const int64_t base = (int64_t)blockIdx.x * kRowsPerScanBlock;
    int64_t bad = INT64_MAX, mx = 0, ne = 0;
    uint64_t s1 = 0, s2 = 0;
    for (int j = threadIdx.x; j < kRowsPerScanBlock; j += kBlock) {
        const int64_t i = base + j;
        if (i >= M) break;
        const int64_t a0 = rowptr[i];
        const int64_t a1 = rowptr[i + 1];
        const int64_t d = a1 - a0;
        if (d < 0 || (i == 0 && a0 != 0)) bad = min(bad, i);
        rowptr32[i] = (int)a0;
        if (i == M - 1) rowptr32[M] = (int)a1;
        const uint64_t du = (uint64_t)d;
        s1 += du;
        s2 += du * du;
        mx = max(mx, d);
        ne += (d == 0);
    }
    block_reduce5(bad, s1, s2, mx, ne);
    if (threadIdx.x == 0) out[blockIdx.x] = RowScanOut{bad, (int64_t)s1, (int64_t)s2, mx, ne};
}

constexpr int kColsPerThread = 8;
constexpr int kColsPerBlock = kBlock * kColsPerThread;

// Column range check and int32 narrowing; one record per block: the first bad
// entry position or INT64_MAX.
__global__ __launch_bounds__(kBlock) void colscan_kernel(const int64_t *__restrict__ col, int64_t nnz,
                                                         int64_t K, int *__restrict__ col32,
                                                         int64_t *__restrict__ bad_pos) {
    const int64_t base = (int64_t)blockIdx.x * kColsPerBlock;
    int64_t bad = INT64_MAX;
#pragma unroll
    for (int j = 0; j < kColsPerThread; ++j) {
        const int64_t p = base + j * kBlock + threadIdx.x;
        if (p < nnz) {
            const int64_t c = col[p];
            if (c < 0 || c >= K) bad = min(bad, p);
            col32[p] = (int)c;
        }
    }
    __shared__ int64_t sh[kBlock];
    sh[threadIdx.x] = bad;
    __syncthreads();
    for (int o = kBlock / 2; o > 0; o >>= 1) {
        if (threadIdx.x < o) sh[threadIdx.x] = min(sh[threadIdx.x], sh[threadIdx.x + o]);
        __syncthreads();
    }
    if (threadIdx.x == 0) bad_pos[blockIdx.x] = sh[0];
}

constexpr int kRowsPerThread = kRowsPerScanBlock / kBlock;   // consecutive rows per thread

__device__ __forceinline__ int64_t pieces_of(int64_t deg, int64_t L) { return (deg + L - 1) / L; }

__global__ __launch_bounds__(kBlock) void part_count_kernel(const int *__restrict__ rowptr, int64_t M,
                                                            int64_t T, int64_t L,
                                                            PartCount *__restrict__ out) {
    const int64_t base = (int64_t)blockIdx.x * kRowsPerScanBlock + (int64_t)threadIdx.x * kRowsPerThread;
    int64_t nh = 0, ns = 0, nl = 0;
    for (int j = 0; j < kRowsPerThread; ++j) {
        const int64_t i = base + j;
        if (i >= M) break;
        const int64_t d = rowptr[i + 1] - rowptr[i];
        if (d > T) {
            nh += 1;
            ns += pieces_of(d, L);
        } else {
            nl += 1;
        }
    }
    __shared__ int64_t sh[3][kBlock];
    sh[0][threadIdx.x] = nh; sh[1][threadIdx.x] = ns; sh[2][threadIdx.x] = nl;
    __syncthreads();
    for (int o = kBlock / 2; o > 0; o >>= 1) {
        if (threadIdx.x < o)
            for (int c = 0; c < 3; ++c) sh[c][threadIdx.x] += sh[c][threadIdx.x + o];
        __syncthreads();
    }
    if (threadIdx.x == 0) out[blockIdx.x] = PartCount{sh[0][0], sh[1][0], sh[2][0]};
}

// Ordered compaction: thread t of block b owns kRowsPerThread consecutive
// rows, so a block-wide exclusive scan of per-thread counts plus the block's
// global offset gives every heavy row, piece and light row its final index.
__global__ __launch_bounds__(kBlock) void part_write_kernel(
    const int *__restrict__ rowptr, int64_t M, int64_t T, int64_t L,
    const PartCount *__restrict__ block_off, int *__restrict__ heavy_rows, int *__restrict__ seg_first,
    int *__restrict__ seg_begin, int *__restrict__ seg_end, int *__restrict__ light_rows) {
    const int64_t base = (int64_t)blockIdx.x * kRowsPerScanBlock + (int64_t)threadIdx.x * kRowsPerThread;
    int64_t cnt[3] = {0, 0, 0};
    for (int j = 0; j < kRowsPerThread; ++j) {
        const int64_t i = base + j;
        if (i >= M) break;
        const int64_t d = rowptr[i + 1] - rowptr[i];
        if (d > T) {
            cnt[0] += 1;
            cnt[1] += pieces_of(d, L);
        } else {
            cnt[2] += 1;
        }
    }
    __shared__ int64_t sh[3][kBlock];
    for (int c = 0; c < 3; ++c) sh[c][threadIdx.x] = cnt[c];
    __syncthreads();
    for (int o = 1; o < kBlock; o <<= 1) {        // inclusive Hillis-Steele scan
        int64_t y[3];
        for (int c = 0; c < 3; ++c) y[c] = threadIdx.x >= o ? sh[c][threadIdx.x - o] : 0;
        __syncthreads();
        for (int c = 0; c < 3; ++c) sh[c][threadIdx.x] += y[c];
        __syncthreads();
    }
    const PartCount bo = block_off[blockIdx.x];
    int64_t ho = bo.n_heavy + sh[0][threadIdx.x] - cnt[0];
    int64_t so = bo.n_seg + sh[1][threadIdx.x] - cnt[1];
    int64_t lo = bo.n_light + sh[2][threadIdx.x] - cnt[2];
    for (int j = 0; j < kRowsPerThread; ++j) {
        const int64_t i = base + j;
        if (i >= M) break;
        const int64_t r0 = rowptr[i], r1 = rowptr[i + 1];
        if (r1 - r0 > T) {
            heavy_rows[ho] = (int)i;
            seg_first[ho] = (int)so;
            ho += 1;
            for (int64_t b = r0; b < r1; b += L) {
                seg_begin[so] = (int)b;
                seg_end[so] = (int)min(b + L, r1);
                so += 1;
            }
        } else if (light_rows) {
            light_rows[lo] = (int)i;
            lo += 1;
        }
    }
}

// One wave per row tile (record layouts in row_kernel_impl.h).  A tile with
// more than cap entries, or (compact) a column span beyond 16 bits, gets the
// overflow mark; each block reports how many of its tiles overflowed.
__global__ __launch_bounds__(kBlock) void tile_build_kernel(const int *__restrict__ rowptr,
                                                            const int *__restrict__ col,
                                                            const float *__restrict__ val, int64_t M,
                                                            int cap, int rs, int compact,
                                                            int *__restrict__ tiles,
                                                            int64_t *__restrict__ overflow,
                                                            int64_t block_base) {
    __shared__ int s_ovf[kWaves];
    const int lane = threadIdx.x & 63;
    const int wv = threadIdx.x >> 6;
    const int64_t blk = block_base + blockIdx.x;
    const int64_t t = blk * kWaves + wv;
    const int64_t ntiles = (M + kTileRows - 1) / kTileRows;
    int ovf = 0;
    if (t < ntiles) {
        const int64_t r0 = t * kTileRows;
        const int rb = rowptr[r0];
        const int re = rowptr[min(r0 + kTileRows, M)];
        const int total = re - rb;
        int *rec = tiles + t * rs;
        ovf = total > cap;
        int mn = INT_MAX, mx = INT_MIN;
        if (!ovf && compact) {
            for (int k = lane; k < total; k += 64) {
                const int c = col[rb + k];
                mn = min(mn, c);
                mx = max(mx, c);
            }
            for (int o = 32; o > 0; o >>= 1) {
                mn = min(mn, __shfl_xor(mn, o));
                mx = max(mx, __shfl_xor(mx, o));
            }
            ovf = total > 0 && (int64_t)mx - (int64_t)mn > 65535;
        }
        if (ovf) {
            if (compact) {
                if (lane == 0) rec[0] = -1;
            } else if (lane < kTileRows) {
                rec[lane] = (lane == kTileRows - 1) ? -1 : 0;
            }
        } else {
            const int e = rowptr[min(r0 + (lane & (kTileRows - 1)) + 1, M)] - rb;   // lanes 0..7: row ends
            const int hdr = compact ? 3 : kTileRows;
            const int idx_words = compact ? cap / 2 : cap;
            if (compact) {
                const int base = total > 0 ? mn : 0;
                int w1 = 0, w2 = 0;
                for (int j = 0; j < 4; ++j) {
                    w1 |= (__shfl(e, j) & 255) << (8 * j);
                    w2 |= (__shfl(e, 4 + j) & 255) << (8 * j);
                }
                if (lane == 0) {
                    rec[0] = base;
                    rec[1] = w1;
                    rec[2] = w2;
                }
                unsigned short *rec16 = reinterpret_cast<unsigned short *>(rec + hdr);
                for (int k = lane; k < total; k += 64) rec16[k] = (unsigned short)(col[rb + k] - base);
            } else {
                if (lane < kTileRows) rec[lane] = e;
                for (int k = lane; k < total; k += 64) rec[hdr + k] = col[rb + k];
            }
            if (val)
                for (int k = lane; k < total; k += 64) rec[hdr + idx_words + k] = __float_as_int(val[rb + k]);
        }
    }
    if (lane == 0) s_ovf[wv] = ovf;
    __syncthreads();
    if (threadIdx.x == 0) {
        int64_t n = 0;
        for (int w = 0; w < kWaves; ++w) n += s_ovf[w];
        overflow[blk] = n;
    }
}

// Per scan block: out[2b] = entries whose column lies in the same aligned
// block of kWinRows rows as their row, out[2b+1] = rows whose columns are not
// in non-decreasing order.  A thread takes each short row; rows longer than
// kScanLong entries are walked by the whole block afterwards (one thread per
// row would leave a hub of 50,000 entries to a single thread).
constexpr int kScanLong = 64;

__global__ __launch_bounds__(kBlock) void window_scan_kernel(const int *__restrict__ rowptr,
                                                             const int *__restrict__ col, int64_t M,
                                                             int64_t *__restrict__ out) {
    __shared__ int s_long[kRowsPerScanBlock];
    __shared__ int s_nlong;
    if (threadIdx.x == 0) s_nlong = 0;
    __syncthreads();
    const int64_t base = (int64_t)blockIdx.x * kRowsPerScanBlock;
    int64_t cnt = 0, unsorted = 0;
    for (int j = threadIdx.x; j < kRowsPerScanBlock; j += kBlock) {
        const int64_t i = base + j;
        if (i >= M) break;
        const int pb = rowptr[i], pe = rowptr[i + 1];
        if (pe - pb > kScanLong) {
            s_long[atomicAdd(&s_nlong, 1)] = j;
            continue;
        }
        const int blk = (int)(i / kWinRows);
        int prev = INT_MIN;
        bool up = true;
        for (int p = pb; p < pe; ++p) {
            const int c = col[p];
            cnt += (c / kWinRows == blk);
            up = up && c >= prev;
            prev = c;
        }
        unsorted += up ? 0 : 1;
    }
    __syncthreads();
    const int nlong = s_nlong;
    for (int t = 0; t < nlong; ++t) {              // counts are order-free: any list order
        const int64_t i = base + s_long[t];
        const int blk = (int)(i / kWinRows);
        const int pb = rowptr[i], pe = rowptr[i + 1];
        bool up = true;
        for (int64_t p = (int64_t)pb + threadIdx.x; p < pe; p += kBlock) {
            const int c = col[p];
            cnt += (c / kWinRows == blk);
            if (p > pb) up = up && c >= col[p - 1];
        }
        if (__syncthreads_or(up ? 0 : 1) && threadIdx.x == 0) ++unsorted;
    }
    __shared__ int64_t sh[2][kBlock];
    sh[0][threadIdx.x] = cnt;
    sh[1][threadIdx.x] = unsorted;
    __syncthreads();
    for (int o = kBlock / 2; o > 0; o >>= 1) {
        if (threadIdx.x < o) {
            sh[0][threadIdx.x] += sh[0][threadIdx.x + o];
            sh[1][threadIdx.x] += sh[1][threadIdx.x + o];
        }
        __syncthreads();
    }
    if (threadIdx.x == 0) {
        out[2 * blockIdx.x] = sh[0][0];
        out[2 * blockIdx.x + 1] = sh[1][0];
    }
}

// Rows with non-decreasing columns: entries below row i's aligned window of
// kWinRows rows and entries inside it, by two binary searches per row.
__global__ __launch_bounds__(kBlock) void window_runs_kernel(const int *__restrict__ rowptr,
                                                             const int *__restrict__ col, int64_t M,
                                                             int *__restrict__ win_lo, int *__restrict__ win_in) {
    const int64_t i = (int64_t)blockIdx.x * kBlock + threadIdx.x;
    if (i >= M) return;
    const int64_t w0 = (i / kWinRows) * kWinRows;
    const int pb = rowptr[i], pe = rowptr[i + 1];
    int lo = pb, hi = pe;
    while (lo < hi) {                                 // first column >= w0
        const int m = lo + ((hi - lo) >> 1);
        if (col[m] < w0) lo = m + 1;
        else hi = m;
    }
    const int first_in = lo;
    hi = pe;
    while (lo < hi) {                                 // first column >= w0 + kWinRows
        const int m = lo + ((hi - lo) >> 1);
        if (col[m] < w0 + kWinRows) lo = m + 1;
        else hi = m;
    }
    win_lo[i] = first_in - pb;
    win_in[i] = lo - first_in;
}

}  // namespace

hipError_t launch_window_runs(const int *rowptr, const int *col, int64_t M, int *win_lo, int *win_in,
                              hipStream_t s) {
    if (M <= 0) return hipSuccess;
    hipLaunchKernelGGL(window_runs_kernel, dim3((unsigned)((M + kBlock - 1) / kBlock)), dim3(kBlock), 0, s, rowptr,
                       col, M, win_lo, win_in);
    return hipGetLastError();
}

hipError_t launch_window_scan(const int *rowptr, const int *col, int64_t M, int64_t *out, int64_t nblocks,
                              hipStream_t s) {
    if (nblocks <= 0) return hipSuccess;
    hipLaunchKernelGGL(window_scan_kernel, dim3((unsigned)nblocks), dim3(kBlock), 0, s, rowptr, col, M, out);
    return hipGetLastError();
}

int64_t tile_build_blocks(int64_t M) {
    const int64_t ntiles = (M + kTileRows - 1) / kTileRows;
    return (ntiles + kWaves - 1) / kWaves;
}

hipError_t launch_tile_build(const int *rowptr, const int *col, const float *val, int64_t M, int cap, int rs,
                             bool compact, int *tiles, int64_t *overflow, int64_t nblocks, hipStream_t s) {
    // one wave per tile: above 2^26 tiles one grid would pass the 2^32
    // work-item limit of a dispatch, so the blocks go out in several
    const int64_t max_blocks = (int64_t)(UINT32_MAX / kBlock);
    for (int64_t b0 = 0; b0 < nblocks; b0 += max_blocks) {
        const int64_t n = std::min(nblocks - b0, max_blocks);
        hipLaunchKernelGGL(tile_build_kernel, dim3((unsigned)n), dim3(kBlock), 0, s, rowptr, col, val, M, cap,
                           rs, compact ? 1 : 0, tiles, overflow, b0);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

hipError_t launch_rowscan(const int64_t *rowptr, int64_t M, int *rowptr32, RowScanOut *out,
                          int64_t nblocks, hipStream_t s) {
    if (nblocks <= 0) return hipSuccess;
    hipLaunchKernelGGL(rowscan_kernel, dim3((unsigned)nblocks), dim3(kBlock), 0, s, rowptr, M,
                       rowptr32, out);
    return hipGetLastError();
}

hipError_t launch_colscan(const int64_t *col, int64_t nnz, int64_t K, int *col32, int64_t *bad_pos,
                          int64_t nblocks, hipStream_t s) {
    if (nblocks <= 0) return hipSuccess;
    hipLaunchKernelGGL(colscan_kernel, dim3((unsigned)nblocks), dim3(kBlock), 0, s, col, nnz, K,
                       col32, bad_pos);
    return hipGetLastError();
}

int64_t colscan_blocks(int64_t nnz) { return (nnz + kColsPerBlock - 1) / kColsPerBlock; }

hipError_t launch_part_count(const int *rowptr32, int64_t M, int64_t T, int64_t L, PartCount *out,
                             int64_t nblocks, hipStream_t s) {
    if (nblocks <= 0) return hipSuccess;
    hipLaunchKernelGGL(part_count_kernel, dim3((unsigned)nblocks), dim3(kBlock), 0, s, rowptr32, M,
                       T, L, out);
    return hipGetLastError();
}

hipError_t launch_part_write(const int *rowptr32, int64_t M, int64_t T, int64_t L,
                             const PartCount *offsets, int *heavy_rows, int *seg_first,
                             int *seg_begin, int *seg_end, int *light_rows, int64_t nblocks,
                             hipStream_t s) {
    if (nblocks <= 0) return hipSuccess;
    hipLaunchKernelGGL(part_write_kernel, dim3((unsigned)nblocks), dim3(kBlock), 0, s, rowptr32, M, T,
                       L, offsets, heavy_rows, seg_first, seg_begin, seg_end, light_rows);
    return hipGetLastError();
}

// Piece keys (column of the first entry, piece id): unique, so the radix sort
// gives the order with ties by piece id.  Every piece holds at least one entry.
__global__ __launch_bounds__(kBlock) void piece_keys_kernel(const int *__restrict__ col,
                                                            const int *__restrict__ seg_begin, int64_t n_seg,
                                                            uint64_t *__restrict__ keys) {
    const int64_t stride = (int64_t)gridDim.x * kBlock;
    for (int64_t p = (int64_t)blockIdx.x * kBlock + threadIdx.x; p < n_seg; p += stride)
        keys[p] = ((uint64_t)(uint32_t)col[seg_begin[p]] << 32) | (uint64_t)(uint32_t)p;
}

__global__ __launch_bounds__(kBlock) void piece_ids_kernel(const uint64_t *__restrict__ keys, int64_t n_seg,
                                                           int *__restrict__ order) {
    const int64_t stride = (int64_t)gridDim.x * kBlock;
    for (int64_t p = (int64_t)blockIdx.x * kBlock + threadIdx.x; p < n_seg; p += stride)
        order[p] = (int)(uint32_t)keys[p];
}

hipError_t build_piece_order(const int *col, const int *seg_begin, int64_t n_seg, int *order) {
    if (n_seg <= 0) return hipSuccess;
    const unsigned grid = (unsigned)std::min<int64_t>((n_seg + kBlock - 1) / kBlock, 4096);
    uint64_t *ka = nullptr, *kb = nullptr;
    void *tmp = nullptr;
    size_t tmp_bytes = 0;
    hipError_t e = dmalloc(&ka, sizeof(uint64_t) * n_seg, "piece order keys");
    if (e == hipSuccess) e = dmalloc(&kb, sizeof(uint64_t) * n_seg, "piece order keys (alternate)");
    if (e == hipSuccess) {
        hipLaunchKernelGGL(piece_keys_kernel, dim3(grid), dim3(kBlock), 0, nullptr, col, seg_begin, n_seg, ka);
        e = hipGetLastError();
    }
    hipcub::DoubleBuffer<uint64_t> keys(ka, kb);
    if (e == hipSuccess) e = hipcub::DeviceRadixSort::SortKeys(nullptr, tmp_bytes, keys, (int)n_seg);
    if (e == hipSuccess) e = dmalloc(&tmp, tmp_bytes > 0 ? tmp_bytes : 1, "piece order sort storage");
    if (e == hipSuccess) e = hipcub::DeviceRadixSort::SortKeys(tmp, tmp_bytes, keys, (int)n_seg);
    if (e == hipSuccess) {
        hipLaunchKernelGGL(piece_ids_kernel, dim3(grid), dim3(kBlock), 0, nullptr, keys.Current(), n_seg, order);
        e = hipGetLastError();
    }
    if (e == hipSuccess) e = hipDeviceSynchronize();
    if (tmp) dfree(tmp);
    if (ka) dfree(ka);
    if (kb) dfree(kb);
    return e;
}

}  // namespace gspmm
