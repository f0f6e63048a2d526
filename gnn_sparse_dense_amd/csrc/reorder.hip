// Locality reordering (ParamSpMM section 4.4: reordering complements the
// kernels by putting nodes with shared neighbours close together; its own
// choice, Rabbit order, is a third-party method).  This file computes the
// reverse Cuthill-McKee order (Cuthill and McKee 1969, reversed as George
// 1971 proposed), a textbook bandwidth-reducing order, and builds P A P^T.
//
// Cuthill-McKee order on the symmetric pattern of A + A^T (distinct
// neighbours, no self loops): nodes are taken in ascending (degree, id)
// order; each one not yet placed starts a component, which is placed breadth
// first, every placed node appending its unplaced neighbours in ascending
// (degree, id) order.  Level by level this is: the nodes of the next level
// ordered by (position of their earliest-placed neighbour in the current
// level, degree, id), which is what the GPU computes, one level per step:
//   expand: every node of the level offers its position to its neighbours
//           (atomic minimum: the result does not depend on the order of the
//           offers); the offer that finds no parent yet claims the node.
//           Placed nodes always have a parent below the level's positions
//           (component starts get -1), so offers never change or claim them;
//   order:  the claimed nodes are sorted by id, then stably by (parent
//           position, degree), and placed.
// The permutation is therefore exactly the sequential one.
#include <hipcub/hipcub.hpp>

#include <algorithm>
#include <climits>
#include <vector>

#include "alloc.h"
#include "spmm_internal.h"

namespace gspmm {

namespace {

int64_t grid_for(int64_t n, int64_t per = kBlock) {
    return std::max<int64_t>(1, std::min<int64_t>((n + per - 1) / per, 1 << 20));
}

// Both directions of every off-diagonal entry; self loops become the
// all-ones key, which sorts last and is dropped.
__global__ void sym_keys_kernel(const int *__restrict__ rowptr, const int *__restrict__ col, int64_t M,
                                uint64_t *__restrict__ keys) {
    const int lane = threadIdx.x & 63;
    const int64_t stride = (int64_t)gridDim.x * kWaves;
    for (int64_t i = (int64_t)blockIdx.x * kWaves + (threadIdx.x >> 6); i < M; i += stride)
        for (int64_t p = (int64_t)rowptr[i] + lane; p < rowptr[i + 1]; p += 64) {
            const int64_t j = col[p];
            const bool self = j == i;
            keys[2 * (int64_t)p] = self ? ~0ull : (uint64_t)i * (uint64_t)M + (uint64_t)j;
            keys[2 * (int64_t)p + 1] = self ? ~0ull : (uint64_t)j * (uint64_t)M + (uint64_t)i;
        }
}

// Row starts of the symmetric pattern (sorted distinct keys) by binary search.
__global__ void sym_rowptr_kernel(const uint64_t *__restrict__ ukeys, int64_t n, int64_t M, int *__restrict__ srow) {
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t u = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; u <= M; u += stride) {
        const uint64_t target = (uint64_t)u * (uint64_t)M;
        int64_t lo = 0, hi = n;
        while (lo < hi) {
            const int64_t mid = (lo + hi) >> 1;
            if (ukeys[mid] < target) lo = mid + 1;
            else hi = mid;
        }
        srow[u] = (int)lo;
    }
}

__global__ void sym_col_deg_kernel(const uint64_t *__restrict__ ukeys, int64_t n, int64_t M,
                                   const int *__restrict__ srow, int *__restrict__ scol, int *__restrict__ deg,
                                   int *__restrict__ ids) {
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t q = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; q < n; q += stride)
        scol[q] = (int)(ukeys[q] % (uint64_t)M);
    for (int64_t u = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; u < M; u += stride) {
        deg[u] = srow[u + 1] - srow[u];
        ids[u] = (int)u;
    }
}

__global__ void fill_kernel(int *__restrict__ a, int64_t n, int v) {
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += stride) a[i] = v;
}

// Places order[0 .. n0) (the isolated nodes, degree 0) at positions 0 .. n0-1.
__global__ void place_isolated_kernel(const int *__restrict__ order, int64_t n0, int *__restrict__ pos) {
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; t < n0; t += stride) pos[order[t]] = (int)t;
}

// First t >= from with order[t] unplaced (one block; the caller guarantees
// one exists); places it at position `placed` and makes it the frontier.
__global__ __launch_bounds__(kBlock) void next_start_kernel(const int *__restrict__ order, int64_t from, int64_t M,
                                                            int *__restrict__ pos, int *__restrict__ parent,
                                                            int *__restrict__ frontier, int64_t placed,
                                                            int64_t *__restrict__ found) {
    __shared__ int64_t s_best;
    if (threadIdx.x == 0) s_best = INT64_MAX;
    __syncthreads();
    for (int64_t base = from; base < M; base += kBlock) {
        const int64_t t = base + threadIdx.x;
        if (t < M && pos[order[t]] < 0) atomicMin((unsigned long long *)&s_best, (unsigned long long)t);
        __syncthreads();
        const int64_t b = s_best;
        __syncthreads();
        if (b != INT64_MAX) break;
    }
    if (threadIdx.x == 0) {
        const int64_t t = s_best;
        *found = t;
        if (t != INT64_MAX) {
            const int s = order[t];
            pos[s] = (int)placed;
            parent[s] = -1;   // below every position: never claimed again
            frontier[0] = s;
        }
    }
}

// Every frontier node (position base + f) offers its position to its unplaced
// neighbours and claims each newly reached node once.
__global__ void expand_kernel(const int *__restrict__ srow, const int *__restrict__ scol,
                              const int *__restrict__ frontier, int64_t nf, int64_t base,
                              int *__restrict__ parent, int *__restrict__ next, int *__restrict__ nnext) {
    const int lane = threadIdx.x & 63;
    const int64_t stride = (int64_t)gridDim.x * (blockDim.x / 64);
    for (int64_t f = (int64_t)blockIdx.x * (blockDim.x / 64) + (threadIdx.x >> 6); f < nf; f += stride) {
        const int u = frontier[f];
        const int pu = (int)(base + f);
        for (int64_t q = (int64_t)srow[u] + lane; q < srow[u + 1]; q += 64) {
            const int v = scol[q];
            if (atomicMin(&parent[v], pu) == INT_MAX) next[atomicAdd(nnext, 1)] = v;
        }
    }
}

__global__ void level_keys_kernel(const int *__restrict__ ids, int64_t n, int64_t base, const int *__restrict__ parent,
                                  const int *__restrict__ deg, uint64_t *__restrict__ keys) {
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += stride) {
        const int v = ids[i];
        keys[i] = ((uint64_t)(parent[v] - base) << 32) | (uint64_t)(unsigned)deg[v];
    }
}

__global__ void place_level_kernel(const int *__restrict__ ids, int64_t n, int64_t base, int *__restrict__ pos) {
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += stride) pos[ids[i]] = (int)(base + i);
}

__global__ void reverse_kernel(const int *__restrict__ pos, int64_t M, int64_t *__restrict__ perm) {
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t u = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; u < M; u += stride)
        perm[M - 1 - pos[u]] = u;
}

// Consecutive levels of one component inside one workgroup, for levels of
// at most kSmallLevel nodes.  The level's edge ranges stay in LDS from one
// level to the next, so a level costs three dependent trips to memory: the
// neighbours' ids, the offers (atomic minimum on the parent, which also
// claims), and the claimed nodes' parent, degree and edge range.  The
// claimed nodes are ordered by (parent position, degree, id) with a counting
// sort by parent and a rank among each parent's few children.  Returns to
// the host when the component is finished or a level is larger than
// kSmallLevel (its claims are then in `next`, unsorted and unplaced, and the
// current level in `frontier`, for the multi-block path).
constexpr int kSmallLevel = 4096;
constexpr int kSmallBlock = 1024;
constexpr int kSmallWaves = kSmallBlock / 64;

struct BfsState {
    int64_t base, nf, placed, nn, levels;
    int64_t done;
};

// Exclusive prefix of x over the workgroup's threads in thread order; *total
// is the sum.  s_wave holds kSmallWaves + 1 ints.
__device__ __forceinline__ int block_exclusive_scan(int x, int *s_wave, int *total) {
    const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
    int inc = x;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        const int y = __shfl_up(inc, o);
        if (lane >= o) inc += y;
    }
    if (lane == 63) s_wave[wv] = inc;
    __syncthreads();
    if (wv == 0) {
        const int w = lane < kSmallWaves ? s_wave[lane] : 0;
        int winc = w;
#pragma unroll
        for (int o = 1; o < kSmallWaves; o <<= 1) {
            const int y = __shfl_up(winc, o);
            if (lane >= o) winc += y;
        }
        if (lane < kSmallWaves) s_wave[lane] = winc - w;
        if (lane == kSmallWaves - 1) s_wave[kSmallWaves] = winc;
    }
    __syncthreads();
    const int ex = s_wave[wv] + inc - x;
    *total = s_wave[kSmallWaves];
    __syncthreads();   // s_wave may be reused
    return ex;
}

__global__ __launch_bounds__(kSmallBlock) void small_levels_kernel(const int *__restrict__ srow,
                                                                   const int *__restrict__ scol,
                                                                   const int *__restrict__ deg, int *__restrict__ pos,
                                                                   int *__restrict__ parent, int *__restrict__ frontier,
                                                                   int *__restrict__ next, int64_t base, int64_t nf,
                                                                   BfsState *__restrict__ st) {
    __shared__ int s_beg[kSmallLevel], s_len[kSmallLevel];                         // edge ranges of the level
    __shared__ int s_next[kSmallLevel], s_par[kSmallLevel], s_deg[kSmallLevel];    // the claims
    __shared__ int s_cnt[kSmallLevel], s_grp[kSmallLevel];                         // the counting sort
    __shared__ int s_wave[kSmallWaves + 1];
    __shared__ int s_count;
    constexpr int PER = kSmallLevel / kSmallBlock;
    constexpr int EB = 4;   // edges per thread in flight together
    const int tid = threadIdx.x;
    for (int64_t f = tid; f < nf; f += kSmallBlock) {
        const int u = frontier[f];
        const int b = srow[u];
        s_beg[f] = b;
        s_len[f] = srow[u + 1] - b;
    }
    if (tid == 0) s_count = 0;
    __syncthreads();
    int64_t placed = 0, levels = 0;
    int64_t n = 0;
    for (;;) {
        // expand: the level's edges, flattened (s_par = first edge number of
        // each level node), each offered its node's position
        int len[PER];
        int sum = 0;
#pragma unroll
        for (int k = 0; k < PER; ++k) {
            const int f = tid * PER + k;
            len[k] = f < nf ? s_len[f] : 0;
            sum += len[k];
        }
        int edges = 0;
        int ex = block_exclusive_scan(sum, s_wave, &edges);
#pragma unroll
        for (int k = 0; k < PER; ++k) {
            const int f = tid * PER + k;
            if (f < nf) s_par[f] = ex;
            ex += len[k];
        }
        __syncthreads();
        for (int e0 = 0; e0 < edges; e0 += EB * kSmallBlock) {
            int vb[EB], fb[EB];
#pragma unroll
            for (int b = 0; b < EB; ++b) {
                const int e = e0 + b * kSmallBlock + tid;
                fb[b] = -1;
                if (e < edges) {
                    int lo = 0, hi = (int)nf - 1;     // last f with s_par[f] <= e
                    while (lo < hi) {
                        const int mid = (lo + hi + 1) >> 1;
                        if (s_par[mid] <= e) lo = mid;
                        else hi = mid - 1;
                    }
                    fb[b] = lo;
                    vb[b] = scol[s_beg[lo] + (e - s_par[lo])];
                }
            }
#pragma unroll
            for (int b = 0; b < EB; ++b) {
                if (fb[b] < 0) continue;
                const int v = vb[b];
                if (atomicMin(&parent[v], (int)(base + fb[b])) == INT_MAX) {
                    const int slot = atomicAdd(&s_count, 1);
                    if (slot < kSmallLevel) s_next[slot] = v;
                    next[slot] = v;
                }
            }
        }
        __syncthreads();
        n = s_count;
        levels += 1;
        if (n == 0 || n > kSmallLevel) break;
        for (int64_t f = tid; f < nf; f += kSmallBlock) s_cnt[f] = 0;
        __syncthreads();
        // the claims' final parent, degree and edge range; their place in
        // their parent's group
        int cv[PER], cp[PER], cd[PER], cs[PER], cb[PER], ce[PER];
#pragma unroll
        for (int k = 0; k < PER; ++k) {
            const int i = tid + k * kSmallBlock;
            if (i < n) {
                const int v = s_next[i];
                cv[k] = v;
                cp[k] = __hip_atomic_load(&parent[v], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) - (int)base;
                cd[k] = deg[v];
                cb[k] = srow[v];
                ce[k] = srow[v + 1];
            }
        }
#pragma unroll
        for (int k = 0; k < PER; ++k) {
            const int i = tid + k * kSmallBlock;
            if (i < n) {
                s_par[i] = cp[k];
                s_deg[i] = cd[k];
                cs[k] = atomicAdd(&s_cnt[cp[k]], 1);
            }
        }
        __syncthreads();
        {
            // group starts: exclusive prefix of the group sizes s_cnt[0 .. nf)
            int c[PER];
            sum = 0;
#pragma unroll
            for (int k = 0; k < PER; ++k) {
                const int f = tid * PER + k;
                c[k] = f < nf ? s_cnt[f] : 0;
                sum += c[k];
            }
            int tot = 0;
            ex = block_exclusive_scan(sum, s_wave, &tot);
#pragma unroll
            for (int k = 0; k < PER; ++k) {
                const int f = tid * PER + k;
                if (f < nf) s_cnt[f] = ex;
                ex += c[k];
            }
        }
        __syncthreads();
#pragma unroll
        for (int k = 0; k < PER; ++k) {
            const int i = tid + k * kSmallBlock;
            if (i < n) s_grp[s_cnt[cp[k]] + cs[k]] = i;
        }
        __syncthreads();
        // rank by (degree, id) inside the parent's group
#pragma unroll
        for (int k = 0; k < PER; ++k) {
            const int i = tid + k * kSmallBlock;
            if (i < n) {
                const int pi = cp[k], di = cd[k], vi = cv[k];
                const int g0 = s_cnt[pi];
                const int g1 = pi + 1 < nf ? s_cnt[pi + 1] : (int)n;
                int rank = g0;
                for (int q = g0; q < g1; ++q) {
                    const int j = s_grp[q];
                    const int dj = s_deg[j];
                    rank += (dj < di || (dj == di && s_next[j] < vi)) ? 1 : 0;
                }
                cs[k] = rank;
            }
        }
        __syncthreads();
        // the new level replaces the old one in LDS (no reader of it is left)
#pragma unroll
        for (int k = 0; k < PER; ++k) {
            const int i = tid + k * kSmallBlock;
            if (i < n) {
                const int rank = cs[k];
                s_beg[rank] = cb[k];
                s_len[rank] = ce[k] - cb[k];
                frontier[rank] = cv[k];
                pos[cv[k]] = (int)(base + nf + rank);
            }
        }
        if (tid == 0) s_count = 0;
        base += nf;
        nf = n;
        placed += n;
        __syncthreads();
    }
    if (tid == 0) {
        st->base = base;
        st->nf = nf;
        st->placed = placed;
        st->nn = n;
        st->levels = levels;
        st->done = n == 0 ? 1 : 0;
    }
}

int bits_for(uint64_t vmax) {
    int b = 1;
    while (b < 64 && (vmax >> b) != 0) ++b;
    return b;
}

// Device scratch freed on scope exit.
struct Scratch {
    std::vector<void *> ptrs;
    template <typename T>
    hipError_t get(T **p, size_t count) {
        *p = nullptr;
        hipError_t e = dmalloc(reinterpret_cast<void **>(p), std::max<size_t>(count, 1) * sizeof(T), "reordering scratch");
        if (e == hipSuccess) ptrs.push_back(*p);
        return e;
    }
    ~Scratch() {
        for (void *q : ptrs) dfree(q);
    }
};

#define TRY(x)                                  \
    do {                                        \
        hipError_t e_ = (x);                    \
        if (e_ != hipSuccess) return e_;        \
    } while (0)

}  // namespace

hipError_t rcm_order(const int *rowptr, const int *col, int64_t M, int64_t nnz, int64_t *perm, int64_t *levels) {
    *levels = 0;
    if (M == 0) return hipSuccess;
    Scratch sc;
    // ---- symmetric pattern ----
    const int64_t nk = 2 * nnz;
    uint64_t *ka, *kb, *ukeys;
    int64_t *d_count;
    TRY(sc.get(&ka, nk));
    TRY(sc.get(&kb, nk));
    TRY(sc.get(&ukeys, nk));
    TRY(sc.get(&d_count, 1));
    int64_t nsym = 0;
    if (nnz > 0) {
        hipLaunchKernelGGL(sym_keys_kernel, dim3((unsigned)grid_for(M, kWaves)), dim3(kBlock), 0, nullptr, rowptr, col,
                           M, ka);
        TRY(hipGetLastError());
        hipcub::DoubleBuffer<uint64_t> kd(ka, kb);
        size_t tb = 0;
        void *tmp;
        TRY(hipcub::DeviceRadixSort::SortKeys(nullptr, tb, kd, (int)nk, 0, 64));
        TRY(sc.get(reinterpret_cast<char **>(&tmp), tb));
        TRY(hipcub::DeviceRadixSort::SortKeys(tmp, tb, kd, (int)nk, 0, 64));
        size_t ub = 0;
        void *utmp;
        TRY(hipcub::DeviceSelect::Unique(nullptr, ub, kd.Current(), ukeys, d_count, (int)nk));
        TRY(sc.get(reinterpret_cast<char **>(&utmp), ub));
        TRY(hipcub::DeviceSelect::Unique(utmp, ub, kd.Current(), ukeys, d_count, (int)nk));
        TRY(hipMemcpy(&nsym, d_count, sizeof(int64_t), hipMemcpyDeviceToHost));
        uint64_t last = 0;
        if (nsym > 0) TRY(hipMemcpy(&last, ukeys + nsym - 1, sizeof(uint64_t), hipMemcpyDeviceToHost));
        if (nsym > 0 && last == ~0ull) nsym -= 1;   // the self-loop key
    }
    int *srow, *scol, *deg, *ids, *order, *degs_sorted;
    TRY(sc.get(&srow, M + 1));
    TRY(sc.get(&scol, nsym));
    TRY(sc.get(&deg, M));
    TRY(sc.get(&ids, M));
    TRY(sc.get(&order, M));
    TRY(sc.get(&degs_sorted, M));
    hipLaunchKernelGGL(sym_rowptr_kernel, dim3((unsigned)grid_for(M + 1)), dim3(kBlock), 0, nullptr, ukeys, nsym, M,
                       srow);
    TRY(hipGetLastError());
    hipLaunchKernelGGL(sym_col_deg_kernel, dim3((unsigned)grid_for(std::max(nsym, M))), dim3(kBlock), 0, nullptr,
                       ukeys, nsym, M, srow, scol, deg, ids);
    TRY(hipGetLastError());
    // ---- (degree, id) order: a stable sort by degree of ids in ascending order ----
    {
        size_t tb = 0;
        void *tmp;
        const int db = bits_for((uint64_t)std::max<int64_t>(nsym, 1));
        TRY(hipcub::DeviceRadixSort::SortPairs(nullptr, tb, deg, degs_sorted, ids, order, (int)M, 0, db));
        TRY(sc.get(reinterpret_cast<char **>(&tmp), tb));
        TRY(hipcub::DeviceRadixSort::SortPairs(tmp, tb, deg, degs_sorted, ids, order, (int)M, 0, db));
    }
    // ---- breadth-first placement ----
    int *pos, *parent, *fa, *fb, *d_nnext;
    uint64_t *lk, *lk2;
    int *li;
    int64_t *d_found;
    TRY(sc.get(&pos, M));
    TRY(sc.get(&parent, M));
    TRY(sc.get(&fa, M));
    TRY(sc.get(&fb, M));
    TRY(sc.get(&d_nnext, 1));
    TRY(sc.get(&lk, M));
    TRY(sc.get(&lk2, M));
    TRY(sc.get(&li, M));
    TRY(sc.get(&d_found, 1));
    const dim3 gM((unsigned)grid_for(M));
    hipLaunchKernelGGL(fill_kernel, gM, dim3(kBlock), 0, nullptr, pos, M, -1);
    hipLaunchKernelGGL(fill_kernel, gM, dim3(kBlock), 0, nullptr, parent, M, INT_MAX);
    TRY(hipGetLastError());
    // isolated nodes come first in (degree, id) order: each is its own component
    int64_t n0 = 0;
    {
        std::vector<int> hd((size_t)M);
        TRY(hipMemcpy(hd.data(), degs_sorted, sizeof(int) * M, hipMemcpyDeviceToHost));
        n0 = std::lower_bound(hd.begin(), hd.end(), 1) - hd.begin();
    }
    if (n0 > 0) {
        hipLaunchKernelGGL(place_isolated_kernel, dim3((unsigned)grid_for(n0)), dim3(kBlock), 0, nullptr, order, n0,
                           pos);
        TRY(hipGetLastError());
    }
    size_t sort1 = 0, sort2 = 0;
    TRY(hipcub::DeviceRadixSort::SortKeys(nullptr, sort1, fb, fa, (int)M, 0, bits_for((uint64_t)M)));
    TRY(hipcub::DeviceRadixSort::SortPairs(nullptr, sort2, lk, lk2, fa, li, (int)M, 0, 64));
    void *stmp;
    TRY(sc.get(reinterpret_cast<char **>(&stmp), std::max(sort1, sort2)));
    BfsState *d_state;
    TRY(sc.get(&d_state, 1));
    int64_t placed = n0, from = n0;
    int *frontier = fa, *next = fb;
    while (placed < M) {
        hipLaunchKernelGGL(next_start_kernel, dim3(1), dim3(kBlock), 0, nullptr, order, from, M, pos, parent, frontier,
                           placed, d_found);
        TRY(hipGetLastError());
        int64_t t = 0;
        TRY(hipMemcpy(&t, d_found, sizeof(int64_t), hipMemcpyDeviceToHost));
        if (t == INT64_MAX) return hipErrorUnknown;   // cannot happen: placed < M
        from = t + 1;
        int64_t base = placed, nf = 1;
        placed += 1;
        while (nf > 0) {
            int64_t nn = 0;
            if (nf <= kSmallLevel) {
                // small levels run on the device until the component ends or a level grows
                hipLaunchKernelGGL(small_levels_kernel, dim3(1), dim3(kSmallBlock), 0, nullptr, srow, scol, deg, pos,
                                   parent, frontier, next, base, nf, d_state);
                TRY(hipGetLastError());
                BfsState h;
                TRY(hipMemcpy(&h, d_state, sizeof(BfsState), hipMemcpyDeviceToHost));
                *levels += h.levels;
                placed += h.placed;
                base = h.base;
                nf = h.nf;
                if (h.done) break;
                nn = h.nn;
            } else {
                TRY(hipMemset(d_nnext, 0, sizeof(int)));
                hipLaunchKernelGGL(expand_kernel, dim3((unsigned)grid_for(nf, kWaves)), dim3(kBlock), 0, nullptr, srow,
                                   scol, frontier, nf, base, parent, next, d_nnext);
                TRY(hipGetLastError());
                int nn32 = 0;
                TRY(hipMemcpy(&nn32, d_nnext, sizeof(int), hipMemcpyDeviceToHost));
                nn = nn32;
                *levels += 1;
                if (nn == 0) break;
            }
            // ids ascending, then stably by (parent position - base, degree)
            size_t b1 = sort1, b2 = sort2;
            TRY(hipcub::DeviceRadixSort::SortKeys(stmp, b1, next, frontier, (int)nn, 0, bits_for((uint64_t)M)));
            hipLaunchKernelGGL(level_keys_kernel, dim3((unsigned)grid_for(nn)), dim3(kBlock), 0, nullptr, frontier, nn,
                               base, parent, deg, lk);
            TRY(hipGetLastError());
            TRY(hipcub::DeviceRadixSort::SortPairs(stmp, b2, lk, lk2, frontier, next, (int)nn, 0, 64));
            hipLaunchKernelGGL(place_level_kernel, dim3((unsigned)grid_for(nn)), dim3(kBlock), 0, nullptr, next, nn,
                               base + nf, pos);
            TRY(hipGetLastError());
            std::swap(frontier, next);
            base += nf;
            nf = nn;
            placed += nn;
        }
    }
    hipLaunchKernelGGL(reverse_kernel, gM, dim3(kBlock), 0, nullptr, pos, M, perm);
    TRY(hipGetLastError());
    return hipDeviceSynchronize();
}

namespace {

// inv[perm[i]] = i; bad when perm[i] is outside [0, M).
__global__ void invert_kernel(const int64_t *__restrict__ perm, int64_t M, int *__restrict__ inv,
                              int *__restrict__ bad) {
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < M; i += stride) {
        const int64_t o = perm[i];
        if (o < 0 || o >= M) *bad = 1;
        else inv[o] = (int)i;
    }
}

// A permutation leaves no slot of inv unwritten (inv was filled with -1).
__global__ void check_inv_kernel(const int *__restrict__ inv, int64_t M, int *__restrict__ bad) {
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < M; i += stride)
        if (inv[i] < 0) *bad = 1;
}

__global__ void perm_keys_kernel(const int *__restrict__ rowptr, const int *__restrict__ col, int64_t M,
                                 const int *__restrict__ inv, uint64_t *__restrict__ keys, int *__restrict__ idx) {
    const int lane = threadIdx.x & 63;
    const int64_t stride = (int64_t)gridDim.x * kWaves;
    for (int64_t i = (int64_t)blockIdx.x * kWaves + (threadIdx.x >> 6); i < M; i += stride) {
        const uint64_t r = (uint64_t)inv[i] * (uint64_t)M;
        for (int64_t p = (int64_t)rowptr[i] + lane; p < rowptr[i + 1]; p += 64) {
            keys[p] = r + (uint64_t)inv[col[p]];
            idx[p] = (int)p;
        }
    }
}

__global__ void perm_rowptr_kernel(const int64_t *__restrict__ perm, const int *__restrict__ rowptr, int64_t M,
                                   int64_t *__restrict__ deg_new) {
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < M; i += stride) {
        const int64_t o = perm[i];
        deg_new[i] = rowptr[o + 1] - rowptr[o];
    }
}

__global__ void perm_scatter_kernel(const uint64_t *__restrict__ skeys, const int *__restrict__ sidx, int64_t nnz,
                                    int64_t M, const float *__restrict__ val, int64_t *__restrict__ col_p,
                                    float *__restrict__ val_p) {
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t q = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; q < nnz; q += stride) {
        col_p[q] = (int64_t)(skeys[q] % (uint64_t)M);
        if (val_p) val_p[q] = val[sidx[q]];
    }
}

}  // namespace

hipError_t permute_csr(const int *rowptr, const int *col, const float *val, int64_t M, int64_t nnz,
                       const int64_t *perm, int64_t *rowptr_p, int64_t *col_p, float *val_p, bool *bad_perm) {
    *bad_perm = false;
    Scratch sc;
    int *inv, *d_bad;
    TRY(sc.get(&inv, M));
    TRY(sc.get(&d_bad, 1));
    TRY(hipMemset(d_bad, 0, sizeof(int)));
    const dim3 gM((unsigned)grid_for(M));
    hipLaunchKernelGGL(fill_kernel, gM, dim3(kBlock), 0, nullptr, inv, M, -1);
    hipLaunchKernelGGL(invert_kernel, gM, dim3(kBlock), 0, nullptr, perm, M, inv, d_bad);
    hipLaunchKernelGGL(check_inv_kernel, gM, dim3(kBlock), 0, nullptr, inv, M, d_bad);
    TRY(hipGetLastError());
    int bad = 0;
    TRY(hipMemcpy(&bad, d_bad, sizeof(int), hipMemcpyDeviceToHost));
    if (bad) {
        *bad_perm = true;
        return hipSuccess;
    }
    // new row degrees -> rowptr_p (exclusive scan over M + 1 with a trailing 0)
    int64_t *dn;
    TRY(sc.get(&dn, M + 1));
    TRY(hipMemset(dn + M, 0, sizeof(int64_t)));
    hipLaunchKernelGGL(perm_rowptr_kernel, gM, dim3(kBlock), 0, nullptr, perm, rowptr, M, dn);
    TRY(hipGetLastError());
    size_t tb = 0;
    void *tmp;
    TRY(hipcub::DeviceScan::ExclusiveSum(nullptr, tb, dn, rowptr_p, (int)(M + 1)));
    TRY(sc.get(reinterpret_cast<char **>(&tmp), tb));
    TRY(hipcub::DeviceScan::ExclusiveSum(tmp, tb, dn, rowptr_p, (int)(M + 1)));
    if (nnz > 0) {
        uint64_t *ka, *kb;
        int *ia, *ib;
        TRY(sc.get(&ka, nnz));
        TRY(sc.get(&kb, nnz));
        TRY(sc.get(&ia, nnz));
        TRY(sc.get(&ib, nnz));
        hipLaunchKernelGGL(perm_keys_kernel, dim3((unsigned)grid_for(M, kWaves)), dim3(kBlock), 0, nullptr, rowptr, col,
                           M, inv, ka, ia);
        TRY(hipGetLastError());
        hipcub::DoubleBuffer<uint64_t> kd(ka, kb);
        hipcub::DoubleBuffer<int> id(ia, ib);
        const int end_bit = bits_for((uint64_t)(M - 1) * (uint64_t)M + (uint64_t)(M - 1));
        size_t sb = 0;
        void *stmp;
        TRY(hipcub::DeviceRadixSort::SortPairs(nullptr, sb, kd, id, (int)nnz, 0, end_bit));
        TRY(sc.get(reinterpret_cast<char **>(&stmp), sb));
        TRY(hipcub::DeviceRadixSort::SortPairs(stmp, sb, kd, id, (int)nnz, 0, end_bit));
        hipLaunchKernelGGL(perm_scatter_kernel, dim3((unsigned)grid_for(nnz)), dim3(kBlock), 0, nullptr, kd.Current(),
                           id.Current(), nnz, M, val, col_p, val_p);
        TRY(hipGetLastError());
    }
    return hipDeviceSynchronize();
}

}  // namespace gspmm
