// Projections of the layers above the gate, run on the kept rows only
// (spke.com page, three-phase list, third bullet).
//     y[M][N] (+)= x[M][K] . w[N][K]^T
//
// bf16 path: 4-wave workgroups own a 128x128 tile of y; each wave a 64x64
// sub-tile as 2x2 tiles of the 32x32x16 bf16 MFMA.  The product is formed
// transposed (y^T = w . x^T) so a lane owns one output row m and four
// consecutive columns n per accumulator group: stores are 8-byte runs.
// x and w k-chunks of 64 are double buffered in LDS; within a chunk lane half
// h covers k in [32h, 32h+32) for both operands.
#include "tg_device.h"
#include "tg_kernels.h"

namespace tg {

namespace {

// ---------------------------------------------------------------- fp32 ----
__global__ __launch_bounds__(256) void linear_f32_kernel(const float* __restrict__ x,
                                                         const float* __restrict__ w,
                                                         float* __restrict__ y, int64_t M, int N,
                                                         int K, int accumulate) {
    const int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (gid >= M * N) return;
    const int64_t m = gid / N;
    const int nn = (int)(gid % N);
    const float* xr = x + m * K;
    const float* wr = w + (int64_t)nn * K;
    float acc = 0.f;
    for (int kk = 0; kk < K; ++kk) acc = fmaf(xr[kk], wr[kk], acc);
    y[gid] = accumulate ? y[gid] + acc : acc;
}

// ---------------------------------------------------------------- bf16 ----
constexpr int LB = 128;        // tile rows (m) and cols (n)
constexpr int LK = 64;         // k chunk
constexpr int LS = LK + 8;     // LDS row stride (bf16 elements)

__global__ __launch_bounds__(256, 2) void linear_bf16_kernel(const bf16* __restrict__ x,
                                                             const bf16* __restrict__ w,
                                                             bf16* __restrict__ y, int64_t M,
                                                             int N, int K, int accumulate) {
    __shared__ __attribute__((aligned(16))) bf16 Xs[2][LB * LS];
    __shared__ __attribute__((aligned(16))) bf16 Ws[2][LB * LS];

    const int tid = threadIdx.x;
    const int lane = lane_id();
    const int wv = tid / WAVE;
    const int wm = wv % 2, wn = wv / 2;
    const int hh = lane / 32, l32 = lane % 32;
    const int64_t m0 = (int64_t)blockIdx.x * LB;
    const int n0 = blockIdx.y * LB;

    // 16-byte units of one 128x64 chunk: 1024, four per thread.
    u32x4 xr[4], wr[4];
    auto load = [&](int k0) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int uu = tid + i * 256;
            const int row = uu / (LK / 8), c = uu % (LK / 8);
            int64_t mr = m0 + row;
            if (mr > M - 1) mr = M - 1;
            int nr = n0 + row;
            if (nr > N - 1) nr = N - 1;
            xr[i] = ld16(x + mr * K + k0 + 8 * c);
            wr[i] = ld16(w + (int64_t)nr * K + k0 + 8 * c);
        }
    };
    auto store = [&](int buf) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int uu = tid + i * 256;
            const int row = uu / (LK / 8), c = uu % (LK / 8);
            st16(&Xs[buf][row * LS + 8 * c], xr[i]);
            st16(&Ws[buf][row * LS + 8 * c], wr[i]);
        }
    };

    f32x16 acc[2][2];  // [nt][mt]: D[n][m]
#pragma unroll
    for (int a = 0; a < 2; ++a)
#pragma unroll
        for (int b = 0; b < 2; ++b)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[a][b][r] = 0.f;

    const int nsteps = K / LK;
    load(0);
    store(0);
    __syncthreads();
    for (int s = 0; s < nsteps; ++s) {
        const int buf = s & 1;
        const bool more = s + 1 < nsteps;
        if (more) load((s + 1) * LK);
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) {
            bf16x8 af[2], bfv[2];
#pragma unroll
            for (int t = 0; t < 2; ++t) {
                af[t] = as_bf16x8(ld16(&Ws[buf][(64 * wn + 32 * t + l32) * LS + 32 * hh + 8 * kk]));
                bfv[t] = as_bf16x8(ld16(&Xs[buf][(64 * wm + 32 * t + l32) * LS + 32 * hh + 8 * kk]));
            }
#pragma unroll
            for (int nt = 0; nt < 2; ++nt)
#pragma unroll
                for (int mt = 0; mt < 2; ++mt) acc[nt][mt] = mfma32(af[nt], bfv[mt], acc[nt][mt]);
        }
        if (more) store(buf ^ 1);
        __syncthreads();
    }

    // D[n][m]: lane owns m = 64wm + 32mt + l32, n = 64wn + 32nt + 8(r/4) + 4hh + r%4.
#pragma unroll
    for (int mt = 0; mt < 2; ++mt) {
        const int64_t m = m0 + 64 * wm + 32 * mt + l32;
        if (m >= M) continue;
#pragma unroll
        for (int nt = 0; nt < 2; ++nt) {
#pragma unroll
            for (int rq = 0; rq < 4; ++rq) {
                const int nn = n0 + 64 * wn + 32 * nt + 8 * rq + 4 * hh;
                if (nn >= N) continue;
                bf16x4* dst = reinterpret_cast<bf16x4*>(y + m * N + nn);
                bf16x4 ov;
                if (accumulate) {
                    const bf16x4 old = *dst;
#pragma unroll
                    for (int e = 0; e < 4; ++e) ov[e] = to_bf16(to_f32(old[e]) + acc[nt][mt][4 * rq + e]);
                } else {
#pragma unroll
                    for (int e = 0; e < 4; ++e) ov[e] = to_bf16(acc[nt][mt][4 * rq + e]);
                }
                *dst = ov;
            }
        }
    }
}

}  // namespace

hipError_t launch_linear_f32(const float* x, const float* w, float* y, int64_t M, int N, int K,
                             int accumulate, hipStream_t st) {
    const int64_t n = M * N;
    hipLaunchKernelGGL(linear_f32_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st, x,
                       w, y, M, N, K, accumulate);
    return hipGetLastError();
}

hipError_t launch_linear_bf16(const void* x, const void* w, void* y, int64_t M, int N, int K,
                              int accumulate, hipStream_t st) {
    const dim3 grid((unsigned)((M + LB - 1) / LB), (unsigned)((N + LB - 1) / LB));
    hipLaunchKernelGGL(linear_bf16_kernel, grid, dim3(256), 0, st, (const bf16*)x,
                       (const bf16*)w, (bf16*)y, M, N, K, accumulate);
    return hipGetLastError();
}

}  // namespace tg
