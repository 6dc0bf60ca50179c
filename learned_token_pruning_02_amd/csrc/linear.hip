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
// WM x WN tiles of 32x32 per wave, GM x GN waves per workgroup, k chunks of
// KC.  The operands stream through L2, so the workgroup tile sets the
// FLOPs per byte fetched: <2,2,64,2,2> 128x128 (64 FLOP/B, two workgroups
// per CU), <4,2,32,2,2> 256x128 (85 FLOP/B), <4,2,32,2,4> 256x256 with eight
// waves (128 FLOP/B, one workgroup per CU).  Every variant stays under 256
// registers, so the accumulators live in ordinary VGPRs.
// Split over k (blockIdx.z = slice): the workgroup contracts k in
// [z K, (z + 1) K) of rows that are ldk long, and with `part` set writes its
// fp32 partial to part[z][M][N] instead of y.
// Several products of the same x in one launch (the q, k and v projections):
// the columns of segment i are [nend[i-1], nend[i]) of the grid, each
// boundary a multiple of the workgroup tile, with their own weights and
// output (rows of nend[i] - nend[i-1]).  One product is one segment.
struct LinSegs {
    const bf16* w[LINEAR_MAX_SEG];
    bf16* y[LINEAR_MAX_SEG];
    int nend[LINEAR_MAX_SEG];
    int nseg;
};

// GLU: the grid's columns are the 2F rows of a stacked [gate; up] weight,
// arranged so that each wave's two 32-column tiles are the gate and the up
// rows of the same 32 units; the epilogue stores silu(gate) * up to an
// [M][F] output instead of both products.
template <int WM, int WN, int KC, int GM, int GN, bool GLU = false>
__global__ __launch_bounds__(64 * GM * GN, GM * GN == 4 ? 2 : 1) void linear_bf16_kernel(
        const bf16* __restrict__ x, LinSegs sg, int64_t M, int K, int accumulate, int64_t ldk,
        float* __restrict__ part) {
    constexpr int THREADS = 64 * GM * GN;
    constexpr int LK = KC;                       // k chunk
    constexpr int LS = LK + 8;                   // LDS row stride (bf16 elements)
    constexpr int BM = 32 * WM * GM, BN = 32 * WN * GN;  // workgroup tile rows (m), cols (n)
    constexpr int XU = BM * (LK / 8) / THREADS;  // 16-byte units per thread of x
    constexpr int WU = BN * (LK / 8) / THREADS;  // and of w
    static_assert(XU * THREADS == BM * (LK / 8) && WU * THREADS == BN * (LK / 8), "staging");
    constexpr int KSTEPS = LK / 16;
    __shared__ __attribute__((aligned(16))) bf16 Xs[2][BM * LS];
    __shared__ __attribute__((aligned(16))) bf16 Ws[2][BN * LS];

    const int tid = threadIdx.x;
    const int lane = lane_id();
    const int wv = tid / WAVE;
    const int wm = wv % GM, wn = wv / GM;
    const int hh = lane / 32, l32 = lane % 32;
    const int64_t m0 = (int64_t)blockIdx.x * BM;
    // This workgroup's segment, and its columns within it.
    int n0 = blockIdx.y * BN, sgi = 0;
#pragma unroll
    for (int i = 0; i + 1 < LINEAR_MAX_SEG; ++i)
        if (sgi + 1 < sg.nseg && n0 >= sg.nend[sgi]) ++sgi;
    const int nbeg = sgi > 0 ? sg.nend[sgi - 1] : 0;
    const bf16* __restrict__ w = sg.w[sgi];
    bf16* __restrict__ y = sg.y[sgi];
    const int N = sg.nend[sgi] - nbeg;
    n0 -= nbeg;
    static_assert(!GLU || WN == 2, "GLU: a wave's two column tiles are gate and up");
    const int F = N / 2, fbase = n0 / 2;  // GLU: units of this workgroup start at fbase
    x += (int64_t)blockIdx.z * K;
    w += (int64_t)blockIdx.z * K;

    // Chunks stream from HBM through a ring of two register sets, issued two
    // chunks before their compute: chunk s+1 is stored into LDS at the end of
    // step s, after which its registers take the loads of chunk s+3.
    struct Regs {
        u32x4 x[XU], w[WU];
    };
    // Row and 16-byte column of staging unit uu.  The LDS takes a 16-byte
    // store eight lanes at a time over 32 four-byte banks.  With 32-wide k
    // chunks (four units per 80-byte row) eight consecutive lanes store two
    // rows four apart, whose units fall on disjoint bank quads; two adjacent
    // rows would share one quad.  With 64-wide chunks a row is eight units.
    auto unit_rc = [&](int uu, int& row, int& c) {
        if constexpr (LK / 8 == 4) {
            const int q = uu / 32, l = uu % 32, g = l / 8, j = l % 8;
            row = 8 * q + g + 4 * (j / 4);
            c = j % 4;
        } else {
            row = uu / (LK / 8);
            c = uu % (LK / 8);
        }
    };
    auto load = [&](Regs& r, int k0) {
#pragma unroll
        for (int i = 0; i < XU; ++i) {
            const int uu = tid + i * THREADS;
            int row, c;
            unit_rc(uu, row, c);
            int64_t mr = m0 + row;
            if (mr > M - 1) mr = M - 1;
            r.x[i] = ld16(x + mr * ldk + k0 + 8 * c);
        }
#pragma unroll
        for (int i = 0; i < WU; ++i) {
            const int uu = tid + i * THREADS;
            int row, c;
            unit_rc(uu, row, c);
            int nr = n0 + row;
            if constexpr (GLU) {  // row 64 wn + 32 t + j: gate (t = 0) or up row of unit 32 wn + j
                nr = (row % 64) / 32 * F + fbase + 32 * (row / 64) + row % 32;
            }
            if (nr > N - 1) nr = N - 1;
            r.w[i] = ld16(w + (int64_t)nr * ldk + k0 + 8 * c);
        }
    };
    auto store = [&](const Regs& r, int buf) {
#pragma unroll
        for (int i = 0; i < XU; ++i) {
            int row, c;
            unit_rc(tid + i * THREADS, row, c);
            st16(&Xs[buf][row * LS + 8 * c], r.x[i]);
        }
#pragma unroll
        for (int i = 0; i < WU; ++i) {
            int row, c;
            unit_rc(tid + i * THREADS, row, c);
            st16(&Ws[buf][row * LS + 8 * c], r.w[i]);
        }
    };

    f32x16 acc[WN][WM];  // [nt][mt]: D[n][m]
#pragma unroll
    for (int a = 0; a < WN; ++a)
#pragma unroll
        for (int b = 0; b < WM; ++b)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[a][b][r] = 0.f;

    const int nsteps = K / LK;
    const int last = (nsteps - 1) * LK;
    Regs ra, rb;
    load(ra, 0);
    store(ra, 0);
    load(ra, min(LK, last));
    load(rb, min(2 * LK, last));
    __syncthreads();
    // Branch-free so that every wait for a register set is a partial one:
    // past the end the chunk index clamps to the last chunk, and the extra
    // loads and stores go to a buffer nobody reads again.
    auto mma = [&](int buf) {
        // Within a chunk, lane half hh covers k in [hh*LK/2, (hh+1)*LK/2) for
        // both operands (a permutation of k shared by A and B).
#pragma unroll
        for (int kk = 0; kk < KSTEPS; ++kk) {
            bf16x8 af[WN], bfv[WM];
#pragma unroll
            for (int t = 0; t < WN; ++t)
                af[t] = as_bf16x8(ld16(&Ws[buf][(32 * WN * wn + 32 * t + l32) * LS + (LK / 2) * hh + 8 * kk]));
#pragma unroll
            for (int t = 0; t < WM; ++t)
                bfv[t] = as_bf16x8(ld16(&Xs[buf][(32 * WM * wm + 32 * t + l32) * LS + (LK / 2) * hh + 8 * kk]));
#pragma unroll
            for (int nt = 0; nt < WN; ++nt)
#pragma unroll
                for (int mt = 0; mt < WM; ++mt) acc[nt][mt] = mfma32(af[nt], bfv[mt], acc[nt][mt]);
        }
    };
    // step s: compute chunk s from LDS; nx holds chunk s+1 (stored now) and
    // then takes the loads of chunk s+3.
    auto step = [&](int s, Regs& nx) {
        mma(s & 1);
        store(nx, (s + 1) & 1);
        load(nx, min((s + 3) * LK, last));
        __syncthreads();
    };
    int s = 0;
    for (; s + 1 < nsteps; s += 2) {  // two steps per trip: the register sets alternate
        step(s, ra);
        step(s + 1, rb);
    }
    if (s < nsteps) mma(s & 1);  // odd count: the last chunk is already in LDS

    if constexpr (GLU) {
        // acc[0] holds gate and acc[1] up of units fbase + 32 wn + 8(r/4) + 4hh + r%4.
#pragma unroll
        for (int mt = 0; mt < WM; ++mt) {
            const int64_t m = m0 + 32 * WM * wm + 32 * mt + l32;
            if (m >= M) continue;
#pragma unroll
            for (int rq = 0; rq < 4; ++rq) {
                const int f = fbase + 32 * wn + 8 * rq + 4 * hh;
                bf16x4 ov;
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const float g = acc[0][mt][4 * rq + e], u = acc[1][mt][4 * rq + e];
                    ov[e] = to_bf16(g / (1.0f + __expf(-g)) * u);
                }
                *reinterpret_cast<bf16x4*>(y + m * F + f) = ov;
            }
        }
        return;
    }
    // D[n][m]: lane owns m = 32WM wm + 32mt + l32, n = 32WN wn + 32nt + 8(r/4) + 4hh + r%4.
#pragma unroll
    for (int mt = 0; mt < WM; ++mt) {
        const int64_t m = m0 + 32 * WM * wm + 32 * mt + l32;
        if (m >= M) continue;
#pragma unroll
        for (int nt = 0; nt < WN; ++nt) {
#pragma unroll
            for (int rq = 0; rq < 4; ++rq) {
                const int nn = n0 + 32 * WN * wn + 32 * nt + 8 * rq + 4 * hh;
                if (nn >= N) continue;
                if (part != nullptr) {
                    const f32x4 pv = {acc[nt][mt][4 * rq], acc[nt][mt][4 * rq + 1], acc[nt][mt][4 * rq + 2],
                                      acc[nt][mt][4 * rq + 3]};
                    st16(part + ((int64_t)blockIdx.z * M + m) * N + nn, __builtin_bit_cast(u32x4, pv));
                    continue;
                }
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

hipError_t launch_linear_bf16_multi(const void* x, int nseg, const void* const* w, void* const* y,
                                    const int* n, int64_t M, int K, int accumulate, int tile,
                                    hipStream_t st) {
    LinSegs sg{};
    int N = 0;
    for (int i = 0; i < nseg; ++i) {
        sg.w[i] = (const bf16*)w[i];
        sg.y[i] = (bf16*)y[i];
        N += n[i];
        sg.nend[i] = N;
    }
    sg.nseg = nseg;
    // tile 0: the largest tile that still gives every CU at least one
    // workgroup (two for the 256x128 tile, which runs two per CU);
    // 1, 2, 3 force the 128x128, 256x128 or 256x256 tile.
    const int64_t t256 = ((M + 255) / 256) * ((N + 255) / 256);
    const int64_t t128 = ((M + 255) / 256) * ((N + 127) / 128);
    const int choice = tile > 0 ? tile - 1 : (t256 >= 256 ? 2 : t128 >= 512 ? 1 : 0);
    if (choice == 2) {
        const dim3 grid((unsigned)((M + 255) / 256), (unsigned)((N + 255) / 256));
        hipLaunchKernelGGL((linear_bf16_kernel<4, 2, 32, 2, 4>), grid, dim3(512), 0, st,
                           (const bf16*)x, sg, M, K, accumulate, (int64_t)K, nullptr);
    } else if (choice == 1) {
        const dim3 grid((unsigned)((M + 255) / 256), (unsigned)((N + 127) / 128));
        hipLaunchKernelGGL((linear_bf16_kernel<4, 2, 32, 2, 2>), grid, dim3(256), 0, st,
                           (const bf16*)x, sg, M, K, accumulate, (int64_t)K, nullptr);
    } else {
        const dim3 grid((unsigned)((M + 127) / 128), (unsigned)((N + 127) / 128));
        hipLaunchKernelGGL((linear_bf16_kernel<2, 2, 64, 2, 2>), grid, dim3(256), 0, st,
                           (const bf16*)x, sg, M, K, accumulate, (int64_t)K, nullptr);
    }
    return hipGetLastError();
}

hipError_t launch_linear_bf16_swiglu(const void* x, const void* wgu, void* out, int64_t M, int F,
                                     int K, int tile, hipStream_t st) {
    LinSegs sg{};
    const int N = 2 * F;
    sg.w[0] = (const bf16*)wgu;
    sg.y[0] = (bf16*)out;
    sg.nend[0] = N;
    sg.nseg = 1;
    const int64_t t256 = ((M + 255) / 256) * ((N + 255) / 256);
    const int64_t t128 = ((M + 255) / 256) * ((N + 127) / 128);
    const int choice = tile > 0 ? tile - 1 : (t256 >= 256 ? 2 : t128 >= 512 ? 1 : 0);
    if (choice == 2) {
        const dim3 grid((unsigned)((M + 255) / 256), (unsigned)(N / 256));
        hipLaunchKernelGGL((linear_bf16_kernel<4, 2, 32, 2, 4, true>), grid, dim3(512), 0, st,
                           (const bf16*)x, sg, M, K, 0, (int64_t)K, nullptr);
    } else if (choice == 1) {
        const dim3 grid((unsigned)((M + 255) / 256), (unsigned)(N / 128));
        hipLaunchKernelGGL((linear_bf16_kernel<4, 2, 32, 2, 2, true>), grid, dim3(256), 0, st,
                           (const bf16*)x, sg, M, K, 0, (int64_t)K, nullptr);
    } else {
        const dim3 grid((unsigned)((M + 127) / 128), (unsigned)(N / 128));
        hipLaunchKernelGGL((linear_bf16_kernel<2, 2, 64, 2, 2, true>), grid, dim3(256), 0, st,
                           (const bf16*)x, sg, M, K, 0, (int64_t)K, nullptr);
    }
    return hipGetLastError();
}

hipError_t launch_linear_bf16(const void* x, const void* w, void* y, int64_t M, int N, int K,
                              int accumulate, int tile, hipStream_t st) {
    return launch_linear_bf16_multi(x, 1, &w, &y, &N, M, K, accumulate, tile, st);
}

hipError_t launch_linear_bf16_splitk(const void* x, const void* w, float* part, int64_t M, int N,
                                     int K, int slices, hipStream_t st) {
    const int ks = K / slices;  // a multiple of 64 (checked by the caller)
    const dim3 grid((unsigned)((M + 127) / 128), (unsigned)((N + 127) / 128), (unsigned)slices);
    LinSegs sg{};
    sg.w[0] = (const bf16*)w;
    sg.y[0] = nullptr;
    sg.nend[0] = N;
    sg.nseg = 1;
    hipLaunchKernelGGL((linear_bf16_kernel<2, 2, 64, 2, 2>), grid, dim3(256), 0, st, (const bf16*)x,
                       sg, M, ks, 0, (int64_t)K, part);
    return hipGetLastError();
}

}  // namespace tg
