// Gather / compaction of the kept rows (spke.com page, three-phase list,
// third bullet: layers above the gate layer see only the K kept tokens).
//
// hidden_kept[r] = hidden[kept[r]] bit for bit; scores_kept[r] = scores[kept[r]].
// Pure data movement, bound by HBM: each wave copies one row with 16-byte
// lane accesses, several loads in flight before the matching stores.  The row
// index is wave-uniform (the kept id comes through a scalar load) and the
// row's loads are issued before the score's, so a wave waits for two memory
// round trips rather than three.
#include "tg_device.h"
#include "tg_kernels.h"

namespace tg {

namespace {

constexpr int GATHER_THREADS = 256;
constexpr int ROWS_PER_BLOCK = GATHER_THREADS / WAVE;
constexpr int UNROLL = 4;

__global__ __launch_bounds__(GATHER_THREADS) void gather_rows_kernel(
    const u32x4* __restrict__ hidden, int64_t T, int row_vecs, const float* __restrict__ scores,
    const int32_t* __restrict__ kept, int64_t Kt, u32x4* __restrict__ out,
    float* __restrict__ s_out) {
    const int lane = lane_id();
    const int64_t stride = (int64_t)gridDim.x * ROWS_PER_BLOCK;
    const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x / WAVE);
    for (int64_t row = (int64_t)blockIdx.x * ROWS_PER_BLOCK + wv; row < Kt; row += stride) {
        const int32_t src = kept[row];
        const bool ok = src >= 0 && (int64_t)src < T;
        if (ok) {
            const u32x4* s = hidden + (int64_t)src * row_vecs;
            u32x4* d = out + row * row_vecs;
            int c = lane;
            for (; c + (UNROLL - 1) * WAVE < row_vecs; c += UNROLL * WAVE) {
                u32x4 t[UNROLL];
#pragma unroll
                for (int u = 0; u < UNROLL; ++u) t[u] = s[c + u * WAVE];
#pragma unroll
                for (int u = 0; u < UNROLL; ++u) d[c + u * WAVE] = t[u];
            }
            for (; c < row_vecs; c += WAVE) d[c] = s[c];
        }
        if (s_out != nullptr && lane == 0) s_out[row] = ok ? scores[src] : __builtin_nanf("");
    }
}

}  // namespace

hipError_t launch_gather(const void* hidden, int64_t T, int row_bytes, const float* scores,
                         const int32_t* kept, int64_t Kt, void* hidden_kept, float* scores_kept,
                         hipStream_t st) {
    const int64_t want = (Kt + ROWS_PER_BLOCK - 1) / ROWS_PER_BLOCK;
    const int blocks = (int)(want < 65536 ? want : 65536);
    hipLaunchKernelGGL(gather_rows_kernel, dim3(blocks), dim3(GATHER_THREADS), 0, st,
                       (const u32x4*)hidden, T, row_bytes / 16, scores, kept, Kt,
                       (u32x4*)hidden_kept, scores_kept);
    return hipGetLastError();
}

}  // namespace tg
