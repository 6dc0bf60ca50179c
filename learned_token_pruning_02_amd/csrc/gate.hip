// Gate MLP score (spke.com page, three-phase list, second bullet: an MLP
// scores every token from its post-attention residual at the gate layer).
//     s_t = w2 . GELU(W1 x_t + b1) + b2,  GELU in its exact erf form.
//
// bf16 path: one workgroup of 2*WM waves scores BM = 64*WM tokens against all
// d_gate gate units.  Wave (wm, wn) owns 64 tokens x d_gate/2 units, i.e.
// 2 x (d_gate/64) tiles of the 32x32x16 bf16 MFMA with fp32 accumulators.
// The residual streams from HBM straight into registers (each lane reads
// 64 contiguous bytes of one token row per 64-wide k chunk, one chunk ahead);
// W1 chunks [d_gate][64] are staged through double-buffered LDS and shared by
// all waves.  Inside a 64-wide k chunk, lane half h covers k in [32h, 32h+32)
// for both operands, so every operand fetch is a contiguous 16-byte access.
// The epilogue adds b1, applies GELU, weights by w2, reduces over the units
// (lane butterfly, then the two unit halves through LDS) and adds b2.
#include "tg_device.h"
#include "tg_kernels.h"

namespace tg {

namespace {

// --------------------------------------------------------------- fp32 ----
constexpr int GF_THREADS = 256;

__global__ __launch_bounds__(GF_THREADS) void gate_f32_kernel(
    const float* __restrict__ hidden, int64_t T, int d, const float* __restrict__ w1,
    const float* __restrict__ b1, const float* __restrict__ w2, const float* __restrict__ b2,
    int dg, float* __restrict__ scores) {
    extern __shared__ float xs[];
    __shared__ float red[GF_THREADS / WAVE];
    const int tid = threadIdx.x;
    for (int64_t t = blockIdx.x; t < T; t += gridDim.x) {
        for (int k = tid; k < d; k += GF_THREADS) xs[k] = hidden[t * d + k];
        __syncthreads();
        float part = 0.f;
        for (int u = tid; u < dg; u += GF_THREADS) {
            const float* wr = w1 + (int64_t)u * d;
            float z = 0.f;
            for (int k = 0; k < d; ++k) z = fmaf(wr[k], xs[k], z);
            if (b1 != nullptr) z += b1[u];
            part = fmaf(w2[u], gelu_erf(z), part);
        }
        part = wave_sum(part);
        if (lane_id() == 0) red[tid / WAVE] = part;
        __syncthreads();
        if (tid == 0) {
            float sum = 0.f;
            for (int i = 0; i < GF_THREADS / WAVE; ++i) sum += red[i];
            if (b2 != nullptr) sum += b2[0];
            scores[t] = sum;
        }
        __syncthreads();
    }
}

// --------------------------------------------------------------- bf16 ----
constexpr int GK = 64;            // k chunk
constexpr int W_STRIDE = GK + 8;  // LDS row stride of a W1 chunk (bf16 elements)

template <int DG, int WM>
__global__ __launch_bounds__(128 * WM) void gate_bf16_kernel(
    const bf16* __restrict__ hidden, int64_t T, int d, const bf16* __restrict__ w1,
    const bf16* __restrict__ b1, const bf16* __restrict__ w2, const bf16* __restrict__ b2,
    float* __restrict__ scores) {
    constexpr int THREADS = 128 * WM;
    constexpr int BM = 64 * WM;
    constexpr int NT = DG / 64;                   // 32-unit tiles per wave
    constexpr int WUNITS = (DG * GK / 8) / THREADS;  // 16-byte W1 units per thread per chunk
    static_assert(WUNITS >= 1 && (DG * GK / 8) % THREADS == 0, "W1 chunk split");

    __shared__ __attribute__((aligned(16))) bf16 wl[2][DG * W_STRIDE];
    __shared__ float red[2][BM];

    const int tid = threadIdx.x;
    const int lane = lane_id();
    const int w = tid / WAVE;
    const int wm = w % WM;
    const int wn = w / WM;
    const int hh = lane / 32;
    const int l32 = lane % 32;
    const int64_t tok0 = (int64_t)blockIdx.x * BM;

    // Token rows this lane feeds to the MFMA A operand (clamped in range).
    const bf16* arow[2];
#pragma unroll
    for (int mt = 0; mt < 2; ++mt) {
        int64_t r = tok0 + 64 * wm + 32 * mt + l32;
        if (r > T - 1) r = T - 1;
        arow[mt] = hidden + r * d + 32 * hh;
    }

    uint4 acur[2][4], anext[2][4];
    uint4 wreg[WUNITS];
    f32x16 acc[2][NT];
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
#pragma unroll
        for (int nt = 0; nt < NT; ++nt)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[mt][nt][r] = 0.f;

    auto load_a = [&](uint4 (&dst)[2][4], int k0) {
#pragma unroll
        for (int mt = 0; mt < 2; ++mt)
#pragma unroll
            for (int kk = 0; kk < 4; ++kk)
                dst[mt][kk] = *reinterpret_cast<const uint4*>(arow[mt] + k0 + 8 * kk);
    };
    auto load_w = [&](int k0) {
#pragma unroll
        for (int i = 0; i < WUNITS; ++i) {
            const int u = tid + i * THREADS;
            const int row = u / (GK / 8), c = u % (GK / 8);
            wreg[i] = *reinterpret_cast<const uint4*>(w1 + (int64_t)row * d + k0 + 8 * c);
        }
    };
    auto store_w = [&](int buf) {
#pragma unroll
        for (int i = 0; i < WUNITS; ++i) {
            const int u = tid + i * THREADS;
            const int row = u / (GK / 8), c = u % (GK / 8);
            *reinterpret_cast<uint4*>(&wl[buf][row * W_STRIDE + 8 * c]) = wreg[i];
        }
    };

    const int nsteps = d / GK;
    load_a(acur, 0);
    load_w(0);
    store_w(0);
    __syncthreads();

    for (int s = 0; s < nsteps; ++s) {
        const int buf = s & 1;
        const bool more = s + 1 < nsteps;
        if (more) {
            load_a(anext, (s + 1) * GK);
            load_w((s + 1) * GK);
        }
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) {
#pragma unroll
            for (int nt = 0; nt < NT; ++nt) {
                const int row = wn * (DG / 2) + 32 * nt + l32;
                const bf16x8 bv = as_bf16x8(
                    *reinterpret_cast<const uint4*>(&wl[buf][row * W_STRIDE + 32 * hh + 8 * kk]));
#pragma unroll
                for (int mt = 0; mt < 2; ++mt)
                    acc[mt][nt] = mfma32(as_bf16x8(acur[mt][kk]), bv, acc[mt][nt]);
            }
        }
        if (more) store_w(buf ^ 1);
        __syncthreads();
        if (more) {
#pragma unroll
            for (int mt = 0; mt < 2; ++mt)
#pragma unroll
                for (int kk = 0; kk < 4; ++kk) acur[mt][kk] = anext[mt][kk];
        }
    }

    // Epilogue: lane holds unit wn*DG/2 + 32nt + l32, tokens 8(r/4)+4hh+r%4 (+32mt).
    float bias[NT], wout[NT];
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
        const int u = wn * (DG / 2) + 32 * nt + l32;
        bias[nt] = b1 != nullptr ? to_f32(b1[u]) : 0.f;
        wout[nt] = to_f32(w2[u]);
    }
#pragma unroll
    for (int mt = 0; mt < 2; ++mt) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            float p = 0.f;
#pragma unroll
            for (int nt = 0; nt < NT; ++nt) p = fmaf(wout[nt], gelu_erf(acc[mt][nt][r] + bias[nt]), p);
#pragma unroll
            for (int o = 16; o > 0; o >>= 1) p += __shfl_xor(p, o, WAVE);
            if (l32 == 0) red[wn][64 * wm + 32 * mt + 8 * (r / 4) + 4 * hh + (r % 4)] = p;
        }
    }
    __syncthreads();
    if (tid < BM && tok0 + tid < T) {
        float sum = red[0][tid] + red[1][tid];
        if (b2 != nullptr) sum += to_f32(b2[0]);
        scores[tok0 + tid] = sum;
    }
}

template <int DG>
hipError_t launch_gate_bf16_dg(const bf16* hidden, int64_t T, int d, const bf16* w1,
                               const bf16* b1, const bf16* w2, const bf16* b2, float* scores,
                               hipStream_t st) {
    // Largest token tile that still gives at least two workgroups per CU.
    if (T >= 256 * 512) {
        const int64_t blocks = (T + 255) / 256;
        hipLaunchKernelGGL((gate_bf16_kernel<DG, 4>), dim3(blocks), dim3(512), 0, st, hidden, T,
                           d, w1, b1, w2, b2, scores);
    } else if (T >= 128 * 512) {
        const int64_t blocks = (T + 127) / 128;
        hipLaunchKernelGGL((gate_bf16_kernel<DG, 2>), dim3(blocks), dim3(256), 0, st, hidden, T,
                           d, w1, b1, w2, b2, scores);
    } else {
        const int64_t blocks = (T + 63) / 64;
        hipLaunchKernelGGL((gate_bf16_kernel<DG, 1>), dim3(blocks), dim3(128), 0, st, hidden, T,
                           d, w1, b1, w2, b2, scores);
    }
    return hipGetLastError();
}

}  // namespace

hipError_t launch_gate_f32(const float* hidden, int64_t T, int d, const float* w1, const float* b1,
                           const float* w2, const float* b2, int dg, float* scores,
                           hipStream_t st) {
    const int64_t blocks = T < 4096 ? T : 4096;
    hipLaunchKernelGGL(gate_f32_kernel, dim3((unsigned)blocks), dim3(GF_THREADS),
                       (size_t)d * sizeof(float), st, hidden, T, d, w1, b1, w2, b2, dg, scores);
    return hipGetLastError();
}

hipError_t launch_gate_bf16(const void* hidden, int64_t T, int d, const void* w1, const void* b1,
                            const void* w2, const void* b2, int dg, float* scores,
                            hipStream_t st) {
    const bf16* h = (const bf16*)hidden;
    const bf16* W1 = (const bf16*)w1;
    const bf16* B1 = (const bf16*)b1;
    const bf16* W2 = (const bf16*)w2;
    const bf16* B2 = (const bf16*)b2;
    switch (dg) {
        case 64: return launch_gate_bf16_dg<64>(h, T, d, W1, B1, W2, B2, scores, st);
        case 128: return launch_gate_bf16_dg<128>(h, T, d, W1, B1, W2, B2, scores, st);
        case 256: return launch_gate_bf16_dg<256>(h, T, d, W1, B1, W2, B2, scores, st);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace tg
