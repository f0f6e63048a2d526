// One dispatch for a split product: the pieces of the long rows and the light
// rows of the row kernel run as two ranges of blocks of one launch (pieces
// first, so their long waves start early and the light rows fill the CUs
// around them), instead of two launches with a drain between them.  Each
// block runs exactly the code of its own kernel (row_task with the same
// template arguments), so every result bit is the two-launch route's.  The
// ordered combine of the pieces still follows as its own launch.
#include "row_kernel_impl.h"

namespace gspmm {

namespace {

template <int GL, bool HAS_VAL, bool IS_MAX>
__global__ __launch_bounds__(kBlock) void split_fused_kernel_t(RowArgs light, RowArgs pieces, int64_t piece_blocks,
                                                               int64_t light_blocks_x, int light_slices) {
    constexpr int VEC = 4;
    __shared__ int s_col[kWaves][kChunk];
    __shared__ int s_val[kWaves][HAS_VAL ? kChunk : 1];
    const int lane = threadIdx.x & 63;
    const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);   // uniform per wave
    const int64_t b = blockIdx.x;
    int colf[1];
    bool ok[1];
    if (b < piece_blocks) {
        // one piece per wave, 64 lanes x float4 over the columns of this pass
        const int64_t task0 = b * kWaves + wv;
        if (task0 >= pieces.ntasks) return;
        lane_columns<64, VEC, 1>(pieces, pieces.c_begin, lane, colf, ok);
        row_task<64, VEC, 1, HAS_VAL, IS_MAX, true>(pieces, task0, lane, s_col[wv], s_val[wv], colf, ok);
        return;
    }
    // light rows: 64 / GL rows per wave, column slices of GL x 4 floats, the
    // blocks in the row kernel's order (slice-major, XCD remap over the range)
    constexpr int R = 64 / GL, SL = GL * VEC;
    int64_t lin = b - piece_blocks;
    if (light.xcd_remap) lin = xcd_remap_block(lin, light_blocks_x * light_slices);
    const int64_t by = light_slices == 1 ? 0 : lin / light_blocks_x;
    const int64_t bx = lin - by * light_blocks_x;
    const int64_t task0 = (bx * kWaves + wv) * R;
    if (task0 >= light.ntasks) return;
    lane_columns<GL, VEC, 1>(light, light.c_begin + by * SL, lane % GL, colf, ok);
    row_task<GL, VEC, 1, HAS_VAL, IS_MAX, false>(light, task0, lane, s_col[wv], s_val[wv], colf, ok);
}

template <int GL>
void *pick_fused(bool has_val, bool is_max) {
    if (is_max)
        return has_val ? (void *)split_fused_kernel_t<GL, true, true> : (void *)split_fused_kernel_t<GL, false, true>;
    return has_val ? (void *)split_fused_kernel_t<GL, true, false> : (void *)split_fused_kernel_t<GL, false, false>;
}

}  // namespace

bool split_fused_available(int lanes, int vec, int coarsen) {
    return vec == 4 && coarsen == 1 && (lanes == 16 || lanes == 32);
}

hipError_t launch_split_fused(int lanes, bool has_val, bool is_max, const RowArgs &light, const RowArgs &pieces,
                              int light_slices, hipStream_t s, bool *launched) {
    *launched = false;
    void *fn = lanes == 16 ? pick_fused<16>(has_val, is_max) : lanes == 32 ? pick_fused<32>(has_val, is_max) : nullptr;
    if (!fn || light.task_base != 0 || pieces.task_base != 0 || pieces.c_end - pieces.c_begin > 64 * 4)
        return hipSuccess;
    const int64_t rows_per_block = (int64_t)(64 / lanes) * kWaves;
    const int64_t light_blocks_x = (light.ntasks + rows_per_block - 1) / rows_per_block;
    const int64_t piece_blocks = (pieces.ntasks + kWaves - 1) / kWaves;
    const int64_t total = piece_blocks + light_blocks_x * light_slices;
    if (total <= 0 || total > (int64_t)(UINT32_MAX / kBlock)) return hipSuccess;
    *launched = true;
    RowArgs la = light, pa = pieces;
    int64_t pb = piece_blocks, lbx = light_blocks_x;
    int ls = light_slices;
    void *args[] = {&la, &pa, &pb, &lbx, &ls};
    return hipLaunchKernel(fn, dim3((unsigned)total), dim3(kBlock), args, 0, s);
}

}  // namespace gspmm
