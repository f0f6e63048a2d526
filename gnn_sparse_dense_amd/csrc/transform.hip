// Graph construction and backward support.
//
//  * Edge list -> CSR (graph-spmm kernel card, API table:
//    SparseAdj.from_edge_index sorts an unsorted [2, E] edge list into CSR):
//    a stable LSD radix sort of the rows (hipCUB) keeps each row's entries in
//    edge-list order, so the result and every later product are deterministic.
//  * Transposed CSR of a plan (card, "Requirements and limits": the card is
//    forward only and points to the reversed-edge adjacency A^T for the
//    gradient of a sum), optionally with weights a / deg_i for the backward of
//    a mean.
//  * Max-pool backward (card, "Method": the forward max reports its winning
//    neighbour, and that index routes the gradient back): dB[j][k] sums dC[i][k] over
//    rows i with argmax[i][k] == j, walking row j of the transpose in
//    ascending i, with no atomics.
#include <hipcub/hipcub.hpp>

#include <algorithm>
#include <mutex>
#include <vector>

#include <climits>

#include "alloc.h"
#include "spmm_internal.h"

namespace gspmm {

namespace {

constexpr int kEdgesPerBlock = kBlock * 4;

// Range check of an edge list and the sort inputs: key = row (int32), value =
// edge index.  One record per block: the first bad edge or INT64_MAX.
__global__ __launch_bounds__(kBlock) void coo_prepare_kernel(const int64_t *__restrict__ row,
                                                             const int64_t *__restrict__ col, int64_t E,
                                                             int64_t M, int64_t K, int *__restrict__ keys,
                                                             int *__restrict__ idx, int64_t *__restrict__ bad) {
    int64_t first_bad = INT64_MAX;
    for (int j = 0; j < 4; ++j) {
        const int64_t e = (int64_t)blockIdx.x * kEdgesPerBlock + j * kBlock + threadIdx.x;
        if (e < E) {
            const int64_t r = row[e], c = col[e];
            if (r < 0 || r >= M || c < 0 || c >= K) first_bad = min(first_bad, e);
            keys[e] = (int)r;
            idx[e] = (int)e;
        }
    }
    __shared__ int64_t sh[kBlock];
    sh[threadIdx.x] = first_bad;
    __syncthreads();
    for (int o = kBlock / 2; o > 0; o >>= 1) {
        if (threadIdx.x < o) sh[threadIdx.x] = min(sh[threadIdx.x], sh[threadIdx.x + o]);
        __syncthreads();
    }
    if (threadIdx.x == 0) bad[blockIdx.x] = sh[0];
}

// Sort inputs of a plan's transpose: key = column of entry p, value = p, and
// the row id of every entry.
// A thread takes each short row of its block's kBlock rows; rows longer than
// kPrepLong entries are written by the whole block afterwards.
constexpr int kPrepLong = 64;

__global__ __launch_bounds__(kBlock) void transpose_prepare_kernel(const int *__restrict__ rowptr,
                                                                   const int *__restrict__ col, int64_t M,
                                                                   int *__restrict__ keys, int *__restrict__ idx,
                                                                   int *__restrict__ rowid) {
    __shared__ int s_long[kBlock];
    __shared__ int s_nlong;
    if (threadIdx.x == 0) s_nlong = 0;
    __syncthreads();
    const int64_t i = (int64_t)blockIdx.x * kBlock + threadIdx.x;
    if (i < M) {
        const int pb = rowptr[i], pe = rowptr[i + 1];
        if (pe - pb > kPrepLong) {
            s_long[atomicAdd(&s_nlong, 1)] = (int)i;
        } else {
            for (int p = pb; p < pe; ++p) {
                keys[p] = col[p];
                idx[p] = p;
                rowid[p] = (int)i;
            }
        }
    }
    __syncthreads();
    const int nlong = s_nlong;
    for (int t = 0; t < nlong; ++t) {
        const int r = s_long[t];
        const int pe = rowptr[r + 1];
        for (int64_t p = (int64_t)rowptr[r] + threadIdx.x; p < pe; p += kBlock) {
            keys[p] = col[p];
            idx[p] = (int)p;
            rowid[p] = r;
        }
    }
}

// rowptr of a CSR with sorted row keys: every boundary k (0..E) writes the
// starts of the rows between the previous key and its own.
__global__ __launch_bounds__(kBlock) void rowptr_from_sorted_kernel(const int *__restrict__ sorted, int64_t E,
                                                                    int64_t M, int64_t *__restrict__ rowptr) {
    const int64_t k = (int64_t)blockIdx.x * kBlock + threadIdx.x;
    if (k > E) return;
    const int64_t prev = k > 0 ? sorted[k - 1] : -1;
    const int64_t cur = k < E ? sorted[k] : M;
    for (int64_t r = prev + 1; r <= cur; ++r) rowptr[r] = k;
}

// Entries in sorted order: column ids from the original columns (edge list)
// or from the row ids (transpose); values copied, or scaled by 1 / deg(row).
__global__ __launch_bounds__(kBlock) void gather_entries_kernel(const int *__restrict__ perm, int64_t E,
                                                                const int64_t *__restrict__ col64,
                                                                const int *__restrict__ rowid,
                                                                const float *__restrict__ val,
                                                                const int *__restrict__ deg_rowptr,
                                                                int64_t *__restrict__ col_out,
                                                                float *__restrict__ val_out) {
    const int64_t k = (int64_t)blockIdx.x * kBlock + threadIdx.x;
    if (k >= E) return;
    const int p = perm[k];
    col_out[k] = col64 ? col64[p] : (int64_t)rowid[p];
    if (val_out) {
        float a = val ? val[p] : 1.0f;
        if (deg_rowptr) {
            const int r = rowid[p];
            a = a / (float)(deg_rowptr[r + 1] - deg_rowptr[r]);
        }
        val_out[k] = a;
    }
}

int key_bits(int64_t n) {
    int b = 1;
    while (b < 31 && ((int64_t)1 << b) <= n) ++b;
    return b;
}

// Bytes of hipCUB storage that stable_sort needs for n keys in [0, key_range).
hipError_t sort_storage_bytes(int64_t n, int64_t key_range, size_t *bytes) {
    *bytes = 0;
    return hipcub::DeviceRadixSort::SortPairs(nullptr, *bytes, (const int *)nullptr, (int *)nullptr,
                                              (const int *)nullptr, (int *)nullptr, (int)n, 0, key_bits(key_range),
                                              (hipStream_t) nullptr);
}

// Stable sort of (keys, idx) by key into (skeys, perm) with the caller's
// hipCUB storage; returns once the sort has finished on stream s.
hipError_t stable_sort(const int *keys, const int *idx, int *skeys, int *perm, int64_t n, int64_t key_range,
                       void *tmp, size_t tmp_bytes, hipStream_t s) {
    const hipError_t e = hipcub::DeviceRadixSort::SortPairs(tmp, tmp_bytes, keys, skeys, idx, perm, (int)n, 0,
                                                            key_bits(key_range), s);
    const hipError_t e2 = hipStreamSynchronize(s);
    return e != hipSuccess ? e : e2;
}

size_t align256(size_t b) { return (b + 255) & ~(size_t)255; }

// Scratch of one call as slices of a single allocation (one allocation and
// one free per call instead of one per buffer), freed on scope exit.
struct Pool {
    unsigned char *base = nullptr;
    size_t off = 0;
    hipError_t alloc(size_t bytes, const char *what) {
        void *q = nullptr;
        const hipError_t e = dmalloc(&q, std::max<size_t>(bytes, 1), what);
        base = static_cast<unsigned char *>(q);
        return e;
    }
    template <typename T>
    T *take(size_t count) {
        T *p = reinterpret_cast<T *>(base + off);
        off += align256(sizeof(T) * std::max<size_t>(count, 1));
        return p;
    }
    ~Pool() { dfree(base); }
};

}  // namespace

int64_t coo_check_blocks(int64_t E) { return (E + kEdgesPerBlock - 1) / kEdgesPerBlock; }

// Edge list -> CSR in the caller's workspace: check the ranges (the host
// reads one record per block), stable-sort the rows, gather the entries, and
// write rowptr.  Synchronous on stream s.
hipError_t coo_to_csr_in(const int64_t *row, const int64_t *col, const float *val, int64_t E, int64_t M, int64_t K,
                         int64_t *rowptr_out, int64_t *col_out, float *val_out, int64_t *first_bad,
                         const CooWorkspace &w, hipStream_t s) {
    *first_bad = -1;
    hipError_t e;
    if (E > 0) {
        const int64_t nb = coo_check_blocks(E);
        hipLaunchKernelGGL(coo_prepare_kernel, dim3((unsigned)nb), dim3(kBlock), 0, s, row, col, E, M, K, w.keys,
                           w.idx, w.bad);
        e = hipMemcpyAsync(w.bad_host, w.bad, sizeof(int64_t) * nb, hipMemcpyDeviceToHost, s);
        if (e == hipSuccess) e = hipStreamSynchronize(s);
        if (e != hipSuccess) return e;
        const int64_t b = *std::min_element(w.bad_host, w.bad_host + nb);
        if (b != INT64_MAX) {
            *first_bad = b;
            return hipSuccess;
        }
        e = stable_sort(w.keys, w.idx, w.skeys, w.perm, E, M, w.sort, w.sort_bytes, s);
        if (e != hipSuccess) return e;
        hipLaunchKernelGGL(gather_entries_kernel, dim3((unsigned)((E + kBlock - 1) / kBlock)), dim3(kBlock), 0, s,
                           w.perm, E, col, (const int *)nullptr, val, (const int *)nullptr, col_out, val_out);
    }
    hipLaunchKernelGGL(rowptr_from_sorted_kernel, dim3((unsigned)((E + 1 + kBlock - 1) / kBlock)), dim3(kBlock), 0,
                       s, w.skeys, E, M, rowptr_out);
    e = hipGetLastError();
    if (e == hipSuccess) e = hipStreamSynchronize(s);
    return e;
}

hipError_t coo_sort_storage_bytes(int64_t E, int64_t M, size_t *bytes) { return sort_storage_bytes(E, M, bytes); }

// ---- allocation-free edge-list sort ----
// The workspace is this file-scope device array; each device holds its own
// copy from the time the library is loaded on it until the process ends.
// Host code never passes the array's name to a kernel: it takes the device
// address from hipGetSymbolAddress, resolved once per device.
static __device__ __align__(256) unsigned char scratch[kNoAllocScratchBytes];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu[kMaxDevices];     // one call at a time per device
unsigned char *g_scratch_ptr[kMaxDevices] = {};

}  // namespace

hipError_t coo_to_csr_noalloc(const int64_t *row, const int64_t *col, const float *val, int64_t E, int64_t M,
                              int64_t K, int64_t *rowptr_out, int64_t *col_out, float *val_out, int64_t *first_bad,
                              int *too_large) {
    *first_bad = -1;
    *too_large = 0;
    if (E > kNoAllocMaxEdges) {
        *too_large = 1;
        return hipSuccess;
    }
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lk(g_scratch_mu[dev]);
    if (!g_scratch_ptr[dev]) {
        void *ptr = nullptr;
        e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        g_scratch_ptr[dev] = static_cast<unsigned char *>(ptr);
    }
    unsigned char *base = g_scratch_ptr[dev];
    // carve: keys, idx, skeys, perm (int32 [E] each), range records, sort storage
    CooWorkspace w;
    const int64_t nb = coo_check_blocks(E);
    int64_t bad_host[kNoAllocMaxEdges / (kBlock * 4)];
    w.bad_host = bad_host;
    const size_t arr = align256(sizeof(int) * (size_t)std::max<int64_t>(E, 1));
    size_t off = 0;
    w.keys = reinterpret_cast<int *>(base + off);
    off += arr;
    w.idx = reinterpret_cast<int *>(base + off);
    off += arr;
    w.skeys = reinterpret_cast<int *>(base + off);
    off += arr;
    w.perm = reinterpret_cast<int *>(base + off);
    off += arr;
    w.bad = reinterpret_cast<int64_t *>(base + off);
    off += align256(sizeof(int64_t) * (size_t)std::max<int64_t>(nb, 1));
    if (E > 0 && (e = coo_sort_storage_bytes(E, M, &w.sort_bytes)) != hipSuccess) return e;
    if (off + w.sort_bytes > kNoAllocScratchBytes) {
        *too_large = 1;
        return hipSuccess;
    }
    w.sort = base + off;
    return coo_to_csr_in(row, col, val, E, M, K, rowptr_out, col_out, val_out, first_bad, w, nullptr);
}

hipError_t coo_to_csr(const int64_t *row, const int64_t *col, const float *val, int64_t E, int64_t M, int64_t K,
                      int64_t *rowptr_out, int64_t *col_out, float *val_out, int64_t *first_bad, hipStream_t s) {
    *first_bad = -1;
    CooWorkspace w;
    const int64_t nb = coo_check_blocks(E);
    std::vector<int64_t> bad_host((size_t)std::max<int64_t>(nb, 1));
    w.bad_host = bad_host.data();
    hipError_t e = E > 0 ? coo_sort_storage_bytes(E, M, &w.sort_bytes) : hipSuccess;
    if (e != hipSuccess) return e;
    // edge keys, positions, sorted keys and positions (int32 [E] each), range
    // records, sort storage
    const size_t arr = align256(sizeof(int) * (size_t)std::max<int64_t>(E, 1));
    Pool pool;
    e = pool.alloc(4 * arr + align256(sizeof(int64_t) * (size_t)std::max<int64_t>(nb, 1)) +
                       align256(std::max<size_t>(w.sort_bytes, 1)),
                   "edge-list sort scratch");
    if (e != hipSuccess) return e;
    w.keys = pool.take<int>(E);
    w.idx = pool.take<int>(E);
    w.skeys = pool.take<int>(E);
    w.perm = pool.take<int>(E);
    w.bad = pool.take<int64_t>(nb);
    w.sort = pool.take<unsigned char>(w.sort_bytes);
    return coo_to_csr_in(row, col, val, E, M, K, rowptr_out, col_out, val_out, first_bad, w, s);
}

hipError_t transpose_csr(const int *rowptr, const int *col, const float *val, int64_t M, int64_t K, int64_t nnz,
                         bool scale, int64_t *rowptr_t, int64_t *col_t, float *val_t, hipStream_t s) {
    size_t sort_bytes = 0;
    hipError_t e = nnz > 0 ? sort_storage_bytes(nnz, K, &sort_bytes) : hipSuccess;
    if (e != hipSuccess) return e;
    // keys, positions, sorted keys and positions, row ids (int32 [nnz] each),
    // sort storage
    Pool pool;
    e = pool.alloc(5 * align256(sizeof(int) * (size_t)std::max<int64_t>(nnz, 1)) +
                       align256(std::max<size_t>(sort_bytes, 1)),
                   "transpose scratch");
    if (e != hipSuccess) return e;
    struct {
        int *keys, *idx, *skeys, *perm, *rowid;
        void *sort;
    } t;
    t.keys = pool.take<int>(nnz);
    t.idx = pool.take<int>(nnz);
    t.skeys = pool.take<int>(nnz);
    t.perm = pool.take<int>(nnz);
    t.rowid = pool.take<int>(nnz);
    t.sort = pool.take<unsigned char>(sort_bytes);
    if (nnz > 0) {
        hipLaunchKernelGGL(transpose_prepare_kernel, dim3((unsigned)((M + kBlock - 1) / kBlock)), dim3(kBlock), 0, s,
                           rowptr, col, M, t.keys, t.idx, t.rowid);
        e = stable_sort(t.keys, t.idx, t.skeys, t.perm, nnz, K, t.sort, sort_bytes, s);
        if (e != hipSuccess) return e;
        hipLaunchKernelGGL(gather_entries_kernel, dim3((unsigned)((nnz + kBlock - 1) / kBlock)), dim3(kBlock), 0, s,
                           t.perm, nnz, (const int64_t *)nullptr, t.rowid, val, scale ? rowptr : nullptr, col_t,
                           val_t);
    }
    hipLaunchKernelGGL(rowptr_from_sorted_kernel, dim3((unsigned)((nnz + 1 + kBlock - 1) / kBlock)), dim3(kBlock),
                       0, s, t.skeys, nnz, K, rowptr_t);
    e = hipGetLastError();
    if (e == hipSuccess) e = hipStreamSynchronize(s);
    return e;
}

// Max-pool backward over the rows j of the transposed (unweighted) plan.  A
// wave owns 64/G consecutive rows j, whose source rows i are contiguous in
// col_t: they are staged kChunk at a time in LDS with coalesced loads (as in
// the forward row kernel), then lane g of row j's group gathers dC[i][c..] and
// argmax[i][c..] in predicated batches and adds dC where argmax == j, in
// ascending i.  A repeated i (a duplicated edge) is counted once.  With VEC =
// 4 the rows need only element alignment (16-byte accesses at 4-byte aligned
// addresses), and when N is not a multiple of 4 the lane whose vector would
// run past column N reads the last four columns and writes only those past
// its neighbour lane's.
template <int G, int VEC>
__global__ __launch_bounds__(kBlock) void maxgrad_kernel_t(MaxGradArgs a) {
    typedef float f4 __attribute__((ext_vector_type(4), aligned(4)));
    typedef long long l2 __attribute__((ext_vector_type(2), aligned(8)));
    constexpr int R = 64 / G;
    constexpr int U = 4;
    constexpr int NT = kChunk / 64;
    __shared__ int s_idx[kWaves][kChunk];
    const int lane = threadIdx.x & 63;
    const int wv = threadIdx.x >> 6;
    const int sub = lane / G;
    const int g = lane - sub * G;
    const int64_t j0 = ((int64_t)blockIdx.x * kWaves + wv) * R;
    if (j0 >= a.rows) return;                               // uniform per wave
    const int64_t j = j0 + sub;
    const bool live = j < a.rows;
    const int64_t c0 = (int64_t)blockIdx.y * (G * VEC) + g * VEC;
    const bool ok = c0 < a.N;
    const int64_t c = (VEC > 1 && c0 > a.N - VEC) ? a.N - VEC : c0;   // a.N >= VEC
    const int beg = live ? a.rowptr_t[j] : 0;
    const int deg = live ? a.rowptr_t[j + 1] - beg : 0;
    const int beg0 = __builtin_amdgcn_readfirstlane(beg);
    int off = 0, total = 0;
#pragma unroll
    for (int s = 0; s < R; ++s) {          // rows are consecutive, so entries are too
        const int ds = __builtin_amdgcn_readlane(deg, s * G);
        off += (s < sub) ? ds : 0;
        total += ds;
    }
    int *sidx = s_idx[wv];
    float acc[VEC];
    for (int e = 0; e < VEC; ++e) acc[e] = 0.0f;
    int prev = -1;
    for (int64_t cb64 = 0; cb64 < total; cb64 += kChunk) {   // 64-bit: total may lie within kChunk of 2^31
        const int cb = (int)cb64;
        const int cn = min(kChunk, total - cb);
        const int nt = (cn + 63) >> 6;
        int r[NT];
#pragma unroll
        for (int t = 0; t < NT; ++t)
            if (t < nt) r[t] = a.col_t[beg0 + cb + min(t * 64 + lane, cn - 1)];
#pragma unroll
        for (int t = 0; t < NT; ++t)
            if (t < nt) sidx[t * 64 + lane] = r[t];
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
        const int lo = max(off, cb) - cb;
        const int hi = min(off + deg, cb + cn) - cb;
        for (int k = lo; k < hi; k += U) {
            int ii[U];
            bool use[U];
            float d[U][VEC];
            int64_t am[U][VEC];
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const bool in = k + u < hi;
                ii[u] = sidx[in ? k + u : lo];
                use[u] = in && ok && ii[u] != prev;
                if (in) prev = ii[u];
            }
#pragma unroll
            for (int u = 0; u < U; ++u) {
#pragma unroll
                for (int e = 0; e < VEC; ++e) {
                    d[u][e] = 0.0f;
                    am[u][e] = -1;
                }
                if (use[u]) {
                    const int64_t o = (int64_t)ii[u] * a.N + c;
                    if constexpr (VEC == 4) {
                        const f4 dv = *reinterpret_cast<const f4 *>(a.dC + o);
                        const l2 a0 = *reinterpret_cast<const l2 *>(a.argmax + o);
                        const l2 a1 = *reinterpret_cast<const l2 *>(a.argmax + o + 2);
                        d[u][0] = dv.x; d[u][1] = dv.y; d[u][2] = dv.z; d[u][3] = dv.w;
                        am[u][0] = a0.x; am[u][1] = a0.y; am[u][2] = a1.x; am[u][3] = a1.y;
                    } else {
#pragma unroll
                        for (int e = 0; e < VEC; ++e) {
                            d[u][e] = a.dC[o + e];
                            am[u][e] = a.argmax[o + e];
                        }
                    }
                }
            }
#pragma unroll
            for (int u = 0; u < U; ++u)
#pragma unroll
                for (int e = 0; e < VEC; ++e)
                    if (use[u] && am[u][e] == j) acc[e] = acc[e] + d[u][e];
        }
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    }
    if (!live || !ok) return;
    if constexpr (VEC == 4) {
        if (c == c0) {
            *reinterpret_cast<f4 *>(a.dB + j * a.N + c) = f4{acc[0], acc[1], acc[2], acc[3]};
        } else {
#pragma unroll
            for (int e = 1; e < VEC; ++e)
                if (c + e >= c0) a.dB[j * a.N + c + e] = acc[e];
        }
    } else {
        for (int e = 0; e < VEC; ++e) a.dB[j * a.N + c + e] = acc[e];
    }
}

hipError_t launch_maxgrad(const MaxGradArgs &a, hipStream_t s) {
    if (a.rows <= 0) return hipSuccess;
    // float4 lanes for any N >= 4 (element-aligned rows, the last vector of a
    // row ending at column N), float1 below
    const bool a4 = ((uintptr_t)a.dC % 4 == 0) && ((uintptr_t)a.argmax % 8 == 0) && ((uintptr_t)a.dB % 4 == 0);
    const int vec = (a.N >= 4 && a4) ? 4 : 1;
    const int64_t W = (a.N + vec - 1) / vec;
    int G = 4;
    while (G < W && G < 64) G <<= 1;
    const int64_t per_block = (int64_t)(64 / G) * kWaves;
    const int64_t slices = (W + G - 1) / G;
    const int64_t blocks = (a.rows + per_block - 1) / per_block;
    if (slices > 65535 || blocks > (int64_t)(UINT32_MAX / kBlock)) return hipErrorInvalidConfiguration;
    const dim3 grid((unsigned)blocks, (unsigned)slices);
#define GSPMM_MAXGRAD(GG, VV) hipLaunchKernelGGL((maxgrad_kernel_t<GG, VV>), grid, dim3(kBlock), 0, s, a)
    if (vec == 4) {
        switch (G) {
            case 4: GSPMM_MAXGRAD(4, 4); break;
            case 8: GSPMM_MAXGRAD(8, 4); break;
            case 16: GSPMM_MAXGRAD(16, 4); break;
            case 32: GSPMM_MAXGRAD(32, 4); break;
            default: GSPMM_MAXGRAD(64, 4); break;
        }
    } else {
        switch (G) {
            case 4: GSPMM_MAXGRAD(4, 1); break;
            case 8: GSPMM_MAXGRAD(8, 1); break;
            case 16: GSPMM_MAXGRAD(16, 1); break;
            case 32: GSPMM_MAXGRAD(32, 1); break;
            default: GSPMM_MAXGRAD(64, 1); break;
        }
    }
#undef GSPMM_MAXGRAD
    return hipGetLastError();
}

}  // namespace gspmm
