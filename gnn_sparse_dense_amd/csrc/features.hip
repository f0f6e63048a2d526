// Data-locality features of a plan's sparsity pattern (ParamSpMM section 5.1,
// Table 3): row bandwidth, distinct entries and the nonzero vectors of V-row
// blocking (section 3.1), whose count gives the padding ratio of eq. 2.
//
// Bandwidth: one wave per row reduces the row's smallest and largest column;
// each block writes one (sum, max, rows) record, folded on the host in block
// order, so the result does not depend on scheduling.
// Vectors: every entry becomes the 64-bit key ((row / V) * K + col) * V +
// row % V; after a radix sort, distinct keys are distinct (row, col) pairs and
// distinct key / V values are the blocks' nonzero vectors.
#include <hipcub/hipcub.hpp>

#include <algorithm>
#include <climits>
#include <vector>

#include "alloc.h"
#include "spmm_internal.h"

namespace gspmm {

namespace {

constexpr int kFeatBlocks = 2048;

__device__ __forceinline__ int64_t wave_sum64(int64_t v) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
    return v;
}
__device__ __forceinline__ int wave_min(int v) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v = min(v, __shfl_xor(v, o));
    return v;
}
__device__ __forceinline__ int wave_max(int v) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v = max(v, __shfl_xor(v, o));
    return v;
}

__global__ __launch_bounds__(kBlock) void bandwidth_kernel(const int *__restrict__ rowptr,
                                                           const int *__restrict__ col, int64_t M,
                                                           FeatureRecord *__restrict__ out) {
    __shared__ int64_t s_sum[kWaves], s_max[kWaves], s_rows[kWaves];
    const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
    int64_t sum = 0, mx = 0, rows = 0;
    const int64_t stride = (int64_t)gridDim.x * kWaves;
    for (int64_t row = (int64_t)blockIdx.x * kWaves + wv; row < M; row += stride) {
        const int beg = rowptr[row], end = rowptr[row + 1];
        if (beg == end) continue;   // wave-uniform
        int lo = INT_MAX, hi = INT_MIN;
        for (int64_t p = (int64_t)beg + lane; p < end; p += 64) {
            const int c = col[p];
            lo = min(lo, c);
            hi = max(hi, c);
        }
        lo = wave_min(lo);
        hi = wave_max(hi);
        sum += hi - lo;
        mx = max(mx, (int64_t)(hi - lo));
        rows += 1;
    }
    if (lane == 0) {
        s_sum[wv] = sum;
        s_max[wv] = mx;
        s_rows[wv] = rows;
    }
    __syncthreads();
    if (threadIdx.x == 0) {
        FeatureRecord r{0, 0, 0};
        for (int w = 0; w < kWaves; ++w) {
            r.a += s_sum[w];
            r.b = max(r.b, s_max[w]);
            r.c += s_rows[w];
        }
        out[blockIdx.x] = r;
    }
}

__global__ __launch_bounds__(kBlock) void block_keys_kernel(const int *__restrict__ rowptr,
                                                            const int *__restrict__ col, int64_t M, int64_t K,
                                                            int64_t V, uint64_t *__restrict__ keys) {
    const int lane = threadIdx.x & 63;
    const int64_t stride = (int64_t)gridDim.x * kWaves;
    for (int64_t row = (int64_t)blockIdx.x * kWaves + (threadIdx.x >> 6); row < M; row += stride) {
        const uint64_t base = (uint64_t)(row / V) * (uint64_t)K;
        const uint64_t sub = (uint64_t)(row % V);
        for (int64_t p = (int64_t)rowptr[row] + lane; p < rowptr[row + 1]; p += 64)
            keys[p] = (base + (uint64_t)col[p]) * (uint64_t)V + sub;
    }
}

// Per block: a = distinct keys, b = distinct key / V (sorted keys).
__global__ __launch_bounds__(kBlock) void distinct_kernel(const uint64_t *__restrict__ keys, int64_t n, int64_t V,
                                                          FeatureRecord *__restrict__ out) {
    __shared__ int64_t s_a[kWaves], s_b[kWaves];
    const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
    int64_t a = 0, b = 0;
    const uint64_t uv = (uint64_t)V;
    for (int64_t i = (int64_t)blockIdx.x * kBlock + threadIdx.x; i < n; i += (int64_t)gridDim.x * kBlock) {
        const uint64_t k = keys[i];
        const bool first = i == 0;
        const uint64_t prev = first ? 0 : keys[i - 1];
        a += (first || k != prev) ? 1 : 0;
        b += (first || k / uv != prev / uv) ? 1 : 0;
    }
    a = wave_sum64(a);
    b = wave_sum64(b);
    if (lane == 0) {
        s_a[wv] = a;
        s_b[wv] = b;
    }
    __syncthreads();
    if (threadIdx.x == 0) {
        FeatureRecord r{0, 0, 0};
        for (int w = 0; w < kWaves; ++w) {
            r.a += s_a[w];
            r.b += s_b[w];
        }
        out[blockIdx.x] = r;
    }
}

int64_t feature_grid(int64_t items, int64_t per_block) {
    return std::max<int64_t>(1, std::min<int64_t>((items + per_block - 1) / per_block, kFeatBlocks));
}

}  // namespace

hipError_t pattern_features(const int *rowptr, const int *col, int64_t M, int64_t K, int64_t nnz, int64_t V,
                            int64_t *bw_sum, int64_t *bw_max, int64_t *nonempty, int64_t *distinct,
                            int64_t *vectors) {
    *bw_sum = *bw_max = *nonempty = *distinct = *vectors = 0;
    if (M == 0) return hipSuccess;
    FeatureRecord *rec = nullptr;
    hipError_t e = dmalloc(&rec, sizeof(FeatureRecord) * kFeatBlocks, "feature records");
    if (e != hipSuccess) return e;
    std::vector<FeatureRecord> h(kFeatBlocks);
    const int64_t gb = feature_grid(M, kWaves);
    hipLaunchKernelGGL(bandwidth_kernel, dim3((unsigned)gb), dim3(kBlock), 0, nullptr, rowptr, col, M, rec);
    e = hipGetLastError();
    if (e == hipSuccess) e = hipMemcpy(h.data(), rec, sizeof(FeatureRecord) * gb, hipMemcpyDeviceToHost);
    if (e == hipSuccess)
        for (int64_t b = 0; b < gb; ++b) {
            *bw_sum += h[b].a;
            *bw_max = std::max(*bw_max, h[b].b);
            *nonempty += h[b].c;
        }
    uint64_t *ka = nullptr, *kb = nullptr;
    void *tmp = nullptr;
    if (e == hipSuccess && nnz > 0) {
        e = dmalloc(&ka, sizeof(uint64_t) * nnz, "feature sort keys");
        if (e == hipSuccess) e = dmalloc(&kb, sizeof(uint64_t) * nnz, "feature sort keys (alternate)");
        if (e == hipSuccess) {
            hipLaunchKernelGGL(block_keys_kernel, dim3((unsigned)gb), dim3(kBlock), 0, nullptr, rowptr, col, M, K,
                               V, ka);
            e = hipGetLastError();
        }
        // largest key: ((M-1)/V * K + K-1) * V + V-1 < (M/V + 1) * K * V
        const uint64_t kmax = ((uint64_t)((M - 1) / V) * (uint64_t)K + (uint64_t)(K - 1)) * (uint64_t)V +
                              (uint64_t)(V - 1);
        int end_bit = 1;
        while (end_bit < 64 && (kmax >> end_bit) != 0) ++end_bit;
        hipcub::DoubleBuffer<uint64_t> keys(ka, kb);
        size_t tmp_bytes = 0;
        if (e == hipSuccess) e = hipcub::DeviceRadixSort::SortKeys(nullptr, tmp_bytes, keys, (int)nnz, 0, end_bit);
        if (e == hipSuccess) e = dmalloc(&tmp, tmp_bytes > 0 ? tmp_bytes : 1, "feature sort storage");
        if (e == hipSuccess) e = hipcub::DeviceRadixSort::SortKeys(tmp, tmp_bytes, keys, (int)nnz, 0, end_bit);
        const int64_t gd = feature_grid(nnz, kBlock);
        if (e == hipSuccess) {
            hipLaunchKernelGGL(distinct_kernel, dim3((unsigned)gd), dim3(kBlock), 0, nullptr, keys.Current(), nnz, V,
                               rec);
            e = hipGetLastError();
        }
        if (e == hipSuccess) e = hipMemcpy(h.data(), rec, sizeof(FeatureRecord) * gd, hipMemcpyDeviceToHost);
        if (e == hipSuccess)
            for (int64_t b = 0; b < gd; ++b) {
                *distinct += h[b].a;
                *vectors += h[b].b;
            }
    }
    if (tmp) dfree(tmp);
    if (ka) dfree(ka);
    if (kb) dfree(kb);
    dfree(rec);
    return e;
}

}  // namespace gspmm
