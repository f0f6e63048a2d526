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

// Number of leading zeros of the ascending degrees (one thread, binary search).
__global__ void count_isolated_kernel(const int *__restrict__ degs_sorted, int64_t M, int64_t *__restrict__ n0) {
    if (threadIdx.x != 0) return;
    int64_t lo = 0, hi = M;   // first index with degree >= 1
    while (lo < hi) {
        const int64_t mid = (lo + hi) >> 1;
        if (degs_sorted[mid] < 1) lo = mid + 1;
        else hi = mid;
    }
    *n0 = lo;
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

// Edge records for the level kernel: for every symmetric entry q (u -> v),
// the edge range start and degree of v beside v itself, so that reaching a
// node also brings what its own expansion and ordering need.
__global__ void nbr_records_kernel(const int *__restrict__ srow, const int *__restrict__ scol,
                                   const int *__restrict__ deg, int64_t nsym, int *__restrict__ nsrow,
                                   int *__restrict__ ndeg) {
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t q = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; q < nsym; q += stride) {
        const int v = scol[q];
        nsrow[q] = srow[v];
        ndeg[q] = deg[v];
    }
}

// Consecutive levels of one component inside one workgroup, for levels of
// at most kSmallLevel nodes.  Breadth first on a symmetric pattern, the
// neighbours of level L lie in levels L-1, L and L+1 only, so a neighbour is
// new exactly when it is in neither of the two levels the workgroup already
// holds: those two levels are LDS hash sets, and the new level's claims go
// into a third one, keyed by node with the smallest offering position (LDS
// atomic minimum: independent of the order of the offers).  A level then
// costs one dependent trip to memory (the level's edge records: neighbour,
// its edge range start and its degree); the first level after entry, whose
// previous level is not in LDS, asks the global parent array instead.  The
// claims are ordered by (parent position, degree, id): one scan over the
// parents gives each parent's first child and first edge number, a rank
// among the parent's few children gives the rest, and each new node writes
// its own edges into an LDS map from edge number to node, so that the next
// level finds the node of an edge with one read.  Placed nodes get pos,
// parent and frontier written to memory for the multi-block path.  Returns
// to the host when the component is finished, or, with the level unexpanded
// and in `frontier`, when its claims would exceed kSmallLevel.
constexpr int kSmallLevel = 2048;
constexpr int kSmallBlock = 1024;
constexpr int kSmallWaves = kSmallBlock / 64;
constexpr int kHashBits = 12;
constexpr int kHashSlots = 1 << kHashBits;   // >= 2 kSmallLevel: load factor at most 1/2
constexpr int kEdgeMap = 8192;               // levels with more edges search the edge numbers
static_assert(kHashSlots >= 2 * kSmallLevel, "hash sets hold a level at load <= 1/2");
static_assert(kSmallLevel <= 65535, "16-bit node numbers in the edge map and group counts");

struct BfsState {
    int64_t base, nf, placed, levels;
    int64_t done;   // 1 component finished, 0 a level left to the host, 2 inconsistent
};

// Barrier for LDS traffic only: waits for this wave's LDS operations, not
// for its global stores (nothing in the level kernel reads them back).
__device__ __forceinline__ void lds_barrier() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// Inclusive prefix sum over the 64 lanes of a wave with DPP lane moves:
// shifts by 1, 2, 4 and 8 inside each row of 16 lanes, then the last lane
// of row 0 (and of row 2) added to row 1 (and row 3), then the last lane of
// row 1 added to rows 2 and 3.
__device__ __forceinline__ int wave_inclusive_scan(int x) {
    x += __builtin_amdgcn_update_dpp(0, x, 0x111, 0xf, 0xf, false);   // row_shr:1
    x += __builtin_amdgcn_update_dpp(0, x, 0x112, 0xf, 0xf, false);   // row_shr:2
    x += __builtin_amdgcn_update_dpp(0, x, 0x114, 0xf, 0xf, false);   // row_shr:4
    x += __builtin_amdgcn_update_dpp(0, x, 0x118, 0xf, 0xf, false);   // row_shr:8
    x += __builtin_amdgcn_update_dpp(0, x, 0x142, 0xa, 0xf, false);   // row_bcast:15
    x += __builtin_amdgcn_update_dpp(0, x, 0x143, 0xc, 0xf, false);   // row_bcast:31
    return x;
}

// Exclusive prefixes of x and y over the workgroup's threads in thread
// order, and their totals, with one barrier: every wave adds up the wave
// totals itself.  s_wave holds 2 kSmallWaves ints; the caller keeps a
// barrier between the reads of one call and the writes of the next.
__device__ __forceinline__ void block_exclusive_scan2(int x, int y, int *s_wave, int *ex_x, int *ex_y, int *tot_x,
                                                      int *tot_y) {
    const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
    const int ix = wave_inclusive_scan(x), iy = wave_inclusive_scan(y);
    if (lane == 63) {
        s_wave[wv] = ix;
        s_wave[kSmallWaves + wv] = iy;
    }
    lds_barrier();
    int px = 0, py = 0, tx = 0, ty = 0;
#pragma unroll
    for (int w = 0; w < kSmallWaves; ++w) {
        const int a = s_wave[w], b = s_wave[kSmallWaves + w];
        px += w < wv ? a : 0;
        py += w < wv ? b : 0;
        tx += a;
        ty += b;
    }
    *ex_x = px + ix - x;
    *ex_y = py + iy - y;
    *tot_x = tx;
    *tot_y = ty;
}

__device__ __forceinline__ int hash_home(int v) {
    return (int)(((uint32_t)v * 2654435761u) >> (32 - kHashBits));
}

// v is a key of set a or of set b (linear probing, -1 marks an empty slot;
// the two probe sequences advance together).
__device__ __forceinline__ bool hash_has2(const int *a, const int *b, int v) {
    int ha = hash_home(v), hb = ha;
    bool open_a = true, open_b = true, found = false;
    for (int i = 0; i < kHashSlots && (open_a || open_b); ++i) {
        const int ka = open_a ? a[ha] : -1;
        const int kb = open_b ? b[hb] : -1;
        if (open_a) {
            if (ka == v) found = true;
            if (ka == v || ka < 0) open_a = false;
            ha = (ha + 1) & (kHashSlots - 1);
        }
        if (open_b) {
            if (kb == v) found = true;
            if (kb == v || kb < 0) open_b = false;
            hb = (hb + 1) & (kHashSlots - 1);
        }
    }
    return found;
}

// Slot of v, inserted when absent (*fresh tells which); -1 when the set is full.
__device__ __forceinline__ int hash_put(int *keys, int v, bool *fresh) {
    int h = hash_home(v);
    for (int i = 0; i < kHashSlots; ++i) {
        const int k = atomicCAS(&keys[h], -1, v);
        if (k < 0 || k == v) {
            *fresh = k < 0;
            return h;
        }
        h = (h + 1) & (kHashSlots - 1);
    }
    *fresh = false;
    return -1;
}

__global__ __launch_bounds__(kSmallBlock) void lds_levels_kernel(
    const int *__restrict__ srow, const int *__restrict__ scol, const int *__restrict__ nsrow,
    const int *__restrict__ ndeg, const int *__restrict__ deg, int *__restrict__ pos, int *__restrict__ parent,
    int *__restrict__ frontier, int64_t M, int64_t nsym, int64_t base, int64_t nf, BfsState *__restrict__ st) {
    __shared__ int s_beg[kSmallLevel], s_off[kSmallLevel];     // the level's edge ranges, first edge numbers
    __shared__ uint16_t s_emap[kEdgeMap];                       // edge number -> level node
    __shared__ int s_keys[3][kHashSlots];                       // two levels + the claims
    __shared__ int s_hval[kHashSlots];                          // smallest offer per claim
    __shared__ int s_next[kSmallLevel], s_slot[kSmallLevel];    // claims: node, hash slot,
    __shared__ int s_csrow[kSmallLevel], s_cdeg[kSmallLevel];   //   edge range start, degree
    __shared__ int s_gcnt[kSmallLevel], s_gdeg[kSmallLevel];    // per parent: children, their degrees
    __shared__ int s_grp[kSmallLevel];                          // claims grouped by parent
    __shared__ int s_wave[2 * kSmallWaves];
    __shared__ int s_count, s_flag;                             // s_flag: 1 overflow, 2 inconsistent
    constexpr int PER = kSmallLevel / kSmallBlock;
    constexpr int EB = 4;   // edges per thread in flight together
    const int tid = threadIdx.x, lane = tid & 63;
    int prv = 0, cur = 1, nxt = 2;
    for (int i = tid; i < kHashSlots; i += kSmallBlock) {
        s_keys[0][i] = -1;
        s_keys[1][i] = -1;
        s_keys[2][i] = -1;
        s_hval[i] = INT_MAX;
    }
    if (tid == 0) {
        s_count = 0;
        s_flag = 0;
    }
    lds_barrier();
    // entry: the level from memory; its first edge numbers by a scan of the degrees
    int edges = 0;
    {
        int ld[PER], dsum = 0;
#pragma unroll
        for (int k = 0; k < PER; ++k) {
            const int f = tid * PER + k;
            ld[k] = 0;
            if (f < nf) {
                const int u = frontier[f];
                s_beg[f] = srow[u];
                ld[k] = deg[u];
                bool fresh;
                (void)hash_put(s_keys[cur], u, &fresh);   // nf <= kSmallLevel: always room
            }
            dsum += ld[k];
        }
        int ex, unused, etot, utot;
        block_exclusive_scan2(dsum, 0, s_wave, &ex, &unused, &etot, &utot);
#pragma unroll
        for (int k = 0; k < PER; ++k) {
            const int f = tid * PER + k;
            if (f < nf) {
                s_off[f] = ex;
                if (etot <= kEdgeMap)
                    for (int j = 0; j < ld[k]; ++j) s_emap[ex + j] = (uint16_t)f;
            }
            ex += ld[k];
        }
        edges = etot;
    }
    lds_barrier();
    int64_t placed = 0, levels = 0;
    bool first = true, finished = false;
    for (;;) {
        // expand: each edge of the level offers its node's position
        for (int64_t f = tid; f < nf; f += kSmallBlock) {
            s_gcnt[f] = 0;
            s_gdeg[f] = 0;
        }
        const bool mapped = edges <= kEdgeMap;
        for (int e0 = 0; e0 < edges; e0 += EB * kSmallBlock) {
            int vb[EB], sb[EB], db[EB], fb[EB];
#pragma unroll
            for (int b = 0; b < EB; ++b) {
                const int e = e0 + b * kSmallBlock + tid;
                fb[b] = -1;
                vb[b] = sb[b] = db[b] = 0;
                if (e < edges) {
                    int f;
                    if (mapped) {
                        f = s_emap[e];
                    } else {
                        int lo = 0, hi = (int)nf - 1;     // last f with s_off[f] <= e
                        while (lo < hi) {
                            const int mid = (lo + hi + 1) >> 1;
                            if (s_off[mid] <= e) lo = mid;
                            else hi = mid - 1;
                        }
                        f = lo;
                    }
                    const int64_t q = f < nf ? (int64_t)s_beg[f] + (e - s_off[f]) : -1;
                    if (q >= 0 && q < nsym) {
                        fb[b] = f;
                        vb[b] = scol[q];
                        sb[b] = nsrow[q];
                        db[b] = ndeg[q];
                    } else {
                        s_flag = 2;   // cannot happen: the edge map covers the level
                    }
                }
            }
            if (first) {
                // placed nodes hold a parent (component starts -1), others INT_MAX
                int pb[EB];
#pragma unroll
                for (int b = 0; b < EB; ++b) pb[b] = fb[b] >= 0 ? parent[vb[b]] : INT_MAX;
#pragma unroll
                for (int b = 0; b < EB; ++b)
                    if (pb[b] != INT_MAX) fb[b] = -1;
            }
#pragma unroll
            for (int b = 0; b < EB; ++b) {
                if (e0 + b * kSmallBlock >= edges) break;   // uniform
                const int v = vb[b];
                bool want = fb[b] >= 0;
                if (want && !first) want = !hash_has2(s_keys[prv], s_keys[cur], v);
                int h = -1;
                bool fresh = false;
                if (want) {
                    h = hash_put(s_keys[nxt], v, &fresh);
                    if (h < 0) s_flag = 1;
                }
                // claim numbers, one LDS atomic per wave
                const unsigned long long m = __ballot(fresh);
                if (m != 0) {
                    const int leader = __ffsll((long long)m) - 1;
                    int c0 = 0;
                    if (lane == leader) c0 = atomicAdd(&s_count, __popcll(m));
                    c0 = __builtin_amdgcn_readlane(c0, leader);
                    if (fresh) {
                        const int c = c0 + __popcll(m & ((1ull << lane) - 1));
                        if (c < kSmallLevel) {
                            s_next[c] = v;
                            s_slot[c] = h;
                            s_csrow[c] = sb[b];
                            s_cdeg[c] = db[b];
                        }
                    }
                }
                if (h >= 0) atomicMin(&s_hval[h], fb[b]);
            }
        }
        lds_barrier();
        const int n = s_count;
        const int flag = s_flag;
        if (flag == 0 && base + nf + n > M) {   // cannot happen: every node is placed once
            s_flag = 2;
            break;
        }
        if (flag != 0 || n > kSmallLevel) break;   // overflow: the host expands this level
        levels += 1;
        if (n == 0) {
            finished = true;
            break;
        }
        // the claims' parent, degree and edge range; their arrival in their
        // parent's group, and the group's degree sum
        int cv[PER], cp[PER], cd[PER], cs[PER], cb[PER], co[PER];
#pragma unroll
        for (int k = 0; k < PER; ++k) {
            const int i = tid + k * kSmallBlock;
            cp[k] = -1;
            if (i < n) {
                cv[k] = s_next[i];
                cp[k] = s_hval[s_slot[i]];
                cd[k] = s_cdeg[i];
                cb[k] = s_csrow[i];
                cs[k] = atomicAdd(&s_gcnt[cp[k]], 1);
                atomicAdd(&s_gdeg[cp[k]], cd[k]);
            }
        }
        lds_barrier();
        {
            // group starts and first edge numbers: exclusive prefixes over the parents
            int c[PER], d[PER], csum = 0, dsum = 0;
#pragma unroll
            for (int k = 0; k < PER; ++k) {
                const int f = tid * PER + k;
                c[k] = f < nf ? s_gcnt[f] : 0;
                d[k] = f < nf ? s_gdeg[f] : 0;
                csum += c[k];
                dsum += d[k];
            }
            int exc, exd, ctot, dtot;
            block_exclusive_scan2(csum, dsum, s_wave, &exc, &exd, &ctot, &dtot);
#pragma unroll
            for (int k = 0; k < PER; ++k) {
                const int f = tid * PER + k;
                if (f < nf) {
                    s_gcnt[f] = exc;
                    s_gdeg[f] = exd;
                }
                exc += c[k];
                exd += d[k];
            }
            edges = dtot;   // edges of the new level
        }
        lds_barrier();
#pragma unroll
        for (int k = 0; k < PER; ++k) {
            const int i = tid + k * kSmallBlock;
            if (i < n) {
                const int at = s_gcnt[cp[k]] + cs[k];
                if (at < n) s_grp[at] = i;
            }
        }
        lds_barrier();
        // rank by (degree, id) inside the parent's group; the degrees of the
        // children ranked before give the first edge number
#pragma unroll
        for (int k = 0; k < PER; ++k) {
            const int i = tid + k * kSmallBlock;
            if (i < n) {
                const int pi = cp[k], di = cd[k], vi = cv[k];
                const int g0 = s_gcnt[pi];
                const int g1 = min(pi + 1 < nf ? s_gcnt[pi + 1] : n, n);
                int rank = g0, off = s_gdeg[pi];
                for (int q = g0; q < g1; ++q) {
                    const int j = s_grp[q];
                    const int dj = s_cdeg[j];
                    const bool before = dj < di || (dj == di && s_next[j] < vi);
                    rank += before ? 1 : 0;
                    off += before ? dj : 0;
                }
                cs[k] = rank;
                co[k] = off;
            }
        }
        // the new level replaces the old one in LDS (no reader of it is
        // left); the claims' set becomes the current level's, the previous
        // level's set is emptied for the next claims
        const bool map_next = edges <= kEdgeMap;
#pragma unroll
        for (int k = 0; k < PER; ++k) {
            const int i = tid + k * kSmallBlock;
            if (i < n) {
                const int rank = cs[k];
                if (rank < n) {
                    s_beg[rank] = cb[k];
                    s_off[rank] = co[k];
                    if (map_next && co[k] >= 0 && co[k] + cd[k] <= kEdgeMap)
                        for (int j = 0; j < cd[k]; ++j) s_emap[co[k] + j] = (uint16_t)rank;
                    frontier[rank] = cv[k];
                }
                pos[cv[k]] = (int)(base + nf + rank);
                parent[cv[k]] = (int)(base + cp[k]);
            }
        }
        const int freed = prv;
        prv = cur;
        cur = nxt;
        nxt = freed;
        for (int i = tid; i < kHashSlots; i += kSmallBlock) {
            s_keys[nxt][i] = -1;
            s_hval[i] = INT_MAX;
        }
        if (tid == 0) s_count = 0;
        base += nf;
        nf = n;
        placed += n;
        first = false;
        lds_barrier();
    }
    if (tid == 0) {
        st->base = base;
        st->nf = nf;
        st->placed = placed;
        st->levels = levels;
        st->done = s_flag == 2 ? 2 : finished ? 1 : 0;
    }
}

int bits_for(uint64_t vmax) {
    int b = 1;
    while (b < 64 && (vmax >> b) != 0) ++b;
    return b;
}

// Device scratch freed on scope exit.  With reserve(), the buffers are
// slices of one allocation (an allocation and a free per call instead of
// one per buffer: device frees cost about 0.2 ms each); a request beyond the
// reserve gets its own allocation.
struct Scratch {
    std::vector<void *> ptrs;
    char *pool = nullptr;
    size_t used = 0, cap = 0;
    static size_t round_up(size_t b) { return (b + 255) & ~size_t(255); }
    hipError_t reserve(size_t bytes) {
        void *q = nullptr;
        const hipError_t e = dmalloc(&q, std::max<size_t>(bytes, 1), "reordering scratch");
        if (e != hipSuccess) return e;
        ptrs.push_back(q);
        pool = static_cast<char *>(q);
        cap = bytes;
        return hipSuccess;
    }
    template <typename T>
    hipError_t get(T **p, size_t count) {
        const size_t b = round_up(std::max<size_t>(count, 1) * sizeof(T));
        if (pool && used + b <= cap) {
            *p = reinterpret_cast<T *>(pool + used);
            used += b;
            return hipSuccess;
        }
        *p = nullptr;
        hipError_t e = dmalloc(reinterpret_cast<void **>(p), b, "reordering scratch");
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
    {
        // one reserve for every buffer below, sized from upper bounds (the
        // symmetric pattern has at most nk entries; sort storage for the
        // widest keys)
        size_t tb_keys = 0, tb_unique = 0, tb_deg = 0, tb_ids = 0, tb_level = 0;
        hipcub::DoubleBuffer<uint64_t> nb(nullptr, nullptr);
        TRY(hipcub::DeviceRadixSort::SortKeys(nullptr, tb_keys, nb, (int)nk, 0, 64));
        TRY(hipcub::DeviceSelect::Unique(nullptr, tb_unique, (uint64_t *)nullptr, (uint64_t *)nullptr,
                                         (int64_t *)nullptr, (int)nk));
        TRY(hipcub::DeviceRadixSort::SortPairs(nullptr, tb_deg, (int *)nullptr, (int *)nullptr, (int *)nullptr,
                                               (int *)nullptr, (int)M, 0, 32));
        TRY(hipcub::DeviceRadixSort::SortKeys(nullptr, tb_ids, (int *)nullptr, (int *)nullptr, (int)M, 0,
                                              bits_for((uint64_t)M)));
        TRY(hipcub::DeviceRadixSort::SortPairs(nullptr, tb_level, (uint64_t *)nullptr, (uint64_t *)nullptr,
                                               (int *)nullptr, (int *)nullptr, (int)M, 0, 64));
        const size_t n1 = (size_t)std::max<int64_t>(nk, 1), m1 = (size_t)M + 1;
        auto r = Scratch::round_up;
        const size_t total = 3 * r(n1 * 8) + r(8) + r(tb_keys) + r(tb_unique) + r(m1 * 4) + 3 * r(n1 * 4) +
                             9 * r((size_t)M * 4) + r(tb_deg) + 2 * r(4) + 2 * r((size_t)M * 8) + r(8) +
                             r(std::max(tb_ids, tb_level)) + r(sizeof(BfsState)) + 4 * 256;
        TRY(sc.reserve(total));
    }
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
    int *nsrow, *ndeg;
    TRY(sc.get(&nsrow, nsym));
    TRY(sc.get(&ndeg, nsym));
    if (nsym > 0) {
        hipLaunchKernelGGL(nbr_records_kernel, dim3((unsigned)grid_for(nsym)), dim3(kBlock), 0, nullptr, srow, scol,
                           deg, nsym, nsrow, ndeg);
        TRY(hipGetLastError());
    }
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
    hipLaunchKernelGGL(count_isolated_kernel, dim3(1), dim3(64), 0, nullptr, degs_sorted, M, d_found);
    TRY(hipGetLastError());
    TRY(hipMemcpy(&n0, d_found, sizeof(int64_t), hipMemcpyDeviceToHost));
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
            if (nf <= kSmallLevel) {
                // small levels run on the device until the component ends or
                // a level's claims outgrow the workgroup
                hipLaunchKernelGGL(lds_levels_kernel, dim3(1), dim3(kSmallBlock), 0, nullptr, srow, scol, nsrow, ndeg,
                                   deg, pos, parent, frontier, M, nsym, base, nf, d_state);
                TRY(hipGetLastError());
                BfsState h;
                TRY(hipMemcpy(&h, d_state, sizeof(BfsState), hipMemcpyDeviceToHost));
                *levels += h.levels;
                placed += h.placed;
                base = h.base;
                nf = h.nf;
                if (h.done == 2) return hipErrorUnknown;
                if (h.done) break;
            }
            // a level with many claims: expanded by the whole device
            TRY(hipMemset(d_nnext, 0, sizeof(int)));
            hipLaunchKernelGGL(expand_kernel, dim3((unsigned)grid_for(nf, kWaves)), dim3(kBlock), 0, nullptr, srow,
                               scol, frontier, nf, base, parent, next, d_nnext);
            TRY(hipGetLastError());
            int nn32 = 0;
            TRY(hipMemcpy(&nn32, d_nnext, sizeof(int), hipMemcpyDeviceToHost));
            const int64_t nn = nn32;
            *levels += 1;
            if (nn == 0) break;
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
    {
        // one reserve for the buffers below (sort storage for the widest keys)
        size_t tb_scan = 0, tb_sort = 0;
        TRY(hipcub::DeviceScan::ExclusiveSum(nullptr, tb_scan, (int64_t *)nullptr, (int64_t *)nullptr,
                                             (int)(M + 1)));
        if (nnz > 0) {
            hipcub::DoubleBuffer<uint64_t> nk(nullptr, nullptr);
            hipcub::DoubleBuffer<int> ni(nullptr, nullptr);
            TRY(hipcub::DeviceRadixSort::SortPairs(nullptr, tb_sort, nk, ni, (int)nnz, 0, 64));
        }
        auto r = Scratch::round_up;
        const size_t n1 = (size_t)std::max<int64_t>(nnz, 1);
        TRY(sc.reserve(r((size_t)M * 4) + r(4) + r(((size_t)M + 1) * 8) + r(tb_scan) + 2 * r(n1 * 8) +
                       2 * r(n1 * 4) + r(tb_sort) + 2 * 256));
    }
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
