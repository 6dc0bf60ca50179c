// Gate MLP score (spke.com page, three-phase list, second bullet: an MLP
// scores every token from its post-attention residual at the gate layer).
//     s_t = w2 . GELU(W1 x_t + b1) + b2,  GELU in its exact erf form.
//
// bf16 path: a workgroup of WAVES waves scores 64*WAVES tokens; each wave owns
// 64 tokens against ALL d_gate gate units (2 x d_gate/32 tiles of the
// 32x32x16 bf16 MFMA, fp32 accumulators held in the accumulation registers,
// one wave per SIMD).  The residual streams from HBM straight into registers:
// each lane reads 64 contiguous bytes of one token row per 64-wide k chunk,
// through a ring of three register sets issued two chunks ahead, so about
// 64 KB per CU is in flight.  W1 chunks [d_gate][64] are read coalesced into
// registers and stored into double-buffered LDS in a fragment-major layout,
// so each MFMA B fragment is one conflict-free 16-byte LDS read; they are
// requested before the residual so that waiting for them (in-order load
// counter) never waits for the residual prefetch.  Inside a 64-wide k chunk, lane half h covers k in
// [32h, 32h+32) for both operands, so every operand fetch is one contiguous
// 16-byte access.  The epilogue adds b1, applies GELU (branch-free erf of
// Abramowitz & Stegun 7.1.26), weights by w2, reduces over the units with a
// lane butterfly and adds b2.
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
constexpr int GK = 64;   // k chunk
constexpr int RING = 3;  // residual fragment sets per wave (two chunks in flight)
constexpr int RED_STRIDE = 36;  // floats per row of the unit-sum tile (16-byte aligned, skewed banks)

// US = 2 splits the gate units between two waves of the same tokens (each
// owns DG/2 units; their partial scores are summed in LDS in a fixed order),
// so that a short prompt still gives every SIMD a wave.
template <int DG, int WAVES, int MT, int OCC, int US = 1>
__global__ __launch_bounds__(64 * WAVES, OCC) void gate_bf16_kernel(
    const bf16* __restrict__ hidden, int64_t T, int d, const bf16* __restrict__ w1,
    const bf16* __restrict__ b1, const bf16* __restrict__ w2, const bf16* __restrict__ b2,
    float* __restrict__ scores) {
    constexpr int BM = 32 * MT * WAVES / US;  // tokens per workgroup (MT 32-token blocks per wave)
    constexpr int NTA = DG / 32;           // 32-unit tiles staged per k chunk
    constexpr int NT = NTA / US;           // 32-unit tiles of one wave
    constexpr int NFRAG = NTA * 4;         // W1 fragments (1 KB each) per k chunk
    static_assert(US == 1 || US == 2, "unit split");

    // W1 chunks in fragment layout: [buf][nt*4 + kk][lane] 16-byte units.
    __shared__ __attribute__((aligned(16))) u32x4 wl[2][NFRAG * WAVE];
    // Per-wave tile for the final unit sum: 64 rows (token slot, half) of 32
    // unit-lane partials, rows padded to RED_STRIDE floats.  It lives in the
    // W1 buffers (dead after the last barrier) whenever they are big enough,
    // so that it costs no extra LDS.
    constexpr int RED_FLOATS = 32 * MT * RED_STRIDE;
    constexpr bool RED_IN_WL = WAVES * RED_FLOATS * 4 <= 2 * NFRAG * WAVE * 16;
    __shared__ __attribute__((aligned(16))) float red_own[RED_IN_WL ? 4 : WAVES * RED_FLOATS];

    const int lane = lane_id();
    const int w = threadIdx.x / WAVE;
    const int tgw = w / US;        // token group of this wave
    const int uh = w % US;         // unit half of this wave (US = 2)
    const int nt0 = uh * NT;       // first 32-unit tile of this wave
    const int hh = lane / 32;
    const int l32 = lane % 32;
    const int64_t tok0 = (int64_t)blockIdx.x * BM;

    const bf16* arow[MT];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
        int64_t r = tok0 + 32 * MT * tgw + 32 * mt + l32;
        if (r > T - 1) r = T - 1;
        arow[mt] = hidden + r * d + 32 * hh;
    }
    // W1 chunk staging: each wave stores 8 rows x 8 sixteen-byte columns of a
    // chunk per round (rows r0 + R*i, column 8*c0).  It lands in the
    // fragment-major LDS layout (fragment f = nt*4 + kk, 64 lanes of 16 bytes)
    // at position lane ^ swz(kk, half) with swz = 2*kk + 8*half: a bijection
    // on the low four position bits, so the fragment reads stay
    // conflict-free.  The LDS takes a 16-byte store eight lanes at a time
    // over 32 four-byte banks, so each group of eight lanes holds two rows x
    // four kk of one half (positions distinct modulo 8), and each group of
    // sixteen lanes both halves (distinct modulo 16); one row per group of
    // eight lanes, as a row-major assignment gives, hits each bank quad twice
    // (measured: SQ_LDS_BANK_CONFLICT 4.3 M cycles per 128k call, now none).
    constexpr int THREADS = 64 * WAVES;
    constexpr int WUNITS = NFRAG * WAVE / THREADS;
    constexpr int R = THREADS / 8;
    static_assert(32 % R == 0 || R % 32 == 0, "rows per staging round");
    const int wv_ = threadIdx.x / WAVE, l_ = threadIdx.x % WAVE;
    const int r0 = 8 * wv_ + 2 * (l_ / 16) + (l_ % 8) / 4, c0 = (l_ % 4) + 4 * ((l_ % 16) / 8);
    const bf16* wbase = w1 + (int64_t)r0 * d + 8 * c0;
    const int wkk = c0 % 4, whq = c0 / 4;
    auto wpos = [&](int i) {
        const int row = r0 + R * i;
        const int ln = (row % 32) + 32 * whq;
        return ((row / 32) * 4 + wkk) * WAVE + (ln ^ (2 * wkk + 8 * whq));
    };
    int rd_pos[4];  // this lane's read position inside a fragment, per kk
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) rd_pos[kk] = lane ^ (2 * kk + 8 * hh);
    u32x4 wreg[WUNITS];

    u32x4 a0[MT][4], a1[MT][4], a2[MT][4];
    f32x16 acc[MT][NT];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int nt = 0; nt < NT; ++nt)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[mt][nt][r] = 0.f;

    // This lane's epilogue units (b1 and w2 of units 32nt + l32), loaded before
    // the main loop and branch-free (w2 stands in for a missing b1 and the
    // value is dropped), so that no wait for them follows the loop.
    float bias[NT], wout[NT];
    {
        const bf16* bsrc = b1 != nullptr ? b1 : w2;
        const float bkeep = b1 != nullptr ? 1.0f : 0.0f;
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) {
            const int u = 32 * (nt0 + nt) + l32;
            bias[nt] = to_f32(bsrc[u]) * bkeep;
            wout[nt] = to_f32(w2[u]);
        }
    }

    const int nsteps = d / GK;
    // Each workgroup walks the k chunks starting at its own offset, so that
    // concurrent workgroups read different column slices of their rows (and
    // different memory channels); the contraction order does not matter.
    const int rot = (int)(blockIdx.x % (unsigned)nsteps);

    auto rot_k = [&](int step) {
        const int r = step + rot;
        return (r >= nsteps ? r - nsteps : r) * GK;
    };
#define TG_LOAD_A1(dst, step, li) dst[(li) / 4][(li) % 4] = ld16(arow[(li) / 4] + rot_k(step) + 8 * ((li) % 4))
#define TG_LOAD_W1(step, li) wreg[li] = ld16(wbase + (int64_t)(R * (li)) * d + rot_k(step))
#define TG_LOAD_A(dst, step)                                                                 \
    do {                                                                                     \
        _Pragma("unroll") for (int li = 0; li < 4 * MT; ++li) TG_LOAD_A1(dst, step, li);     \
    } while (0)
#define TG_LOAD_W(step)                                                                      \
    do {                                                                                     \
        _Pragma("unroll") for (int li = 0; li < WUNITS; ++li) TG_LOAD_W1(step, li);          \
    } while (0)
#define TG_STORE_W(buf)                                                                      \
    do {                                                                                     \
        _Pragma("unroll") for (int i = 0; i < WUNITS; ++i)                                   \
            wl[buf][wpos(i)] = wreg[i];                                                       \
    } while (0)
#define TG_READ_B(dst, buf, kk)                                                              \
    do {                                                                                     \
        _Pragma("unroll") for (int nt = 0; nt < NT; ++nt)                                    \
            dst[nt] = as_bf16x8(wl[buf][((nt0 + nt) * 4 + (kk)) * WAVE + rd_pos[kk]]);        \
    } while (0)
    // The 2*NT MFMAs of one k slice, with NL loads (LOAD1(li)) spread evenly
    // between them, so that the vector-memory pipe fills while MFMAs run
    // instead of stalling the wave at the top of the chunk.
#define TG_MMA_LOADS(cur, b, kk, NL, LOAD1)                                                  \
    do {                                                                                     \
        _Pragma("unroll") for (int j = 0; j < MT * NT; ++j) {                                \
            acc[j % MT][j / MT] = mfma32(as_bf16x8(cur[j % MT][kk]), b[j / MT], acc[j % MT][j / MT]); \
            _Pragma("unroll") for (int li = j * (NL) / (MT * NT); li < (j + 1) * (NL) / (MT * NT); ++li) \
                LOAD1(li);                                                                   \
            __builtin_amdgcn_sched_barrier(0);                                               \
        }                                                                                    \
    } while (0)
#define TG_MMA(cur, b, kk)                                                                   \
    do {                                                                                     \
        _Pragma("unroll") for (int nt = 0; nt < NT; ++nt)                                    \
            _Pragma("unroll") for (int mt = 0; mt < MT; ++mt)                                \
                acc[mt][nt] = mfma32(as_bf16x8(cur[mt][kk]), b[nt], acc[mt][nt]);            \
    } while (0)
    // Two waves per SIMD (two workgroups, or eight waves) leave no room for
    // a whole slice of B fragments.
    constexpr bool STREAM = WAVES * OCC >= 8;
    bf16x8 bA[STREAM ? 1 : NT], bB[STREAM ? 1 : NT];

    // One k chunk: the B fragments of slices 0 and 1 are read from LDS; W1 of
    // the next chunk is requested between slice 0's MFMAs and the residual
    // two chunks ahead between slice 1's; then slices 2 and 3 run and the W1
    // registers go to LDS (the in-order load counter lets that wait skip the
    // residual loads).  Prefetch addresses are clamped to the last chunk
    // instead of branching, so the three-step body is straight-line code and
    // the register ring rotates without copies; the clamped extra loads are
    // never used.
#define TG_LW(li) TG_LOAD_W1(min(s_ + 1, nsteps - 1), li)
#define TG_LA(li) TG_LOAD_A1(ahead_, min(s_ + 2, nsteps - 1), li)
    // Two workgroups per CU (OCC = 2) leave no room for a whole slice of B
    // fragments: they are read PD MFMAs ahead, one at a time, with W1 loads
    // spread over slice 0 and residual loads over slice 1.
    constexpr int PD = 4;
#define TG_BFRAG(buf, i) as_bf16x8(wl[buf][((nt0 + (i) % NT) * 4 + (i) / NT) * WAVE + rd_pos[(i) / NT]])
#define TG_STEP_STREAM(s, cur, ahead)                                                        \
    do {                                                                                     \
        const int s_ = (s);                                                                  \
        auto& ahead_ = ahead;                                                                \
        const int buf_ = s_ & 1;                                                             \
        bf16x8 bq[PD];                                                                       \
        _Pragma("unroll") for (int i = 0; i < PD; ++i) bq[i] = TG_BFRAG(buf_, i);            \
        __builtin_amdgcn_sched_barrier(0);                                                   \
        _Pragma("unroll") for (int i = 0; i < 4 * NT; ++i) {                                 \
            const int kk = i / NT, nt = i % NT;                                              \
            acc[0][nt] = mfma32(as_bf16x8(cur[0][kk]), bq[i % PD], acc[0][nt]);              \
            if (i + PD < 4 * NT) bq[i % PD] = TG_BFRAG(buf_, i + PD);                        \
            if (kk == 0) {                                                                   \
                _Pragma("unroll") for (int li = nt * WUNITS / NT; li < (nt + 1) * WUNITS / NT; ++li) \
                    TG_LW(li);                                                               \
            } else if (kk == 1) {                                                            \
                _Pragma("unroll") for (int li = nt * 4 / NT; li < (nt + 1) * 4 / NT; ++li)   \
                    TG_LA(li);                                                               \
            }                                                                                \
            __builtin_amdgcn_sched_barrier(0);                                               \
        }                                                                                    \
        TG_STORE_W(buf_ ^ 1);                                                                \
        __syncthreads();                                                                     \
    } while (0)
#define TG_STEP(s, cur, ahead)                                                               \
    do {                                                                                     \
        const int s_ = (s);                                                                  \
        auto& ahead_ = ahead;                                                                \
        const int buf_ = s_ & 1;                                                             \
        TG_READ_B(bA, buf_, 0);                                                              \
        TG_READ_B(bB, buf_, 1);                                                              \
        __builtin_amdgcn_sched_barrier(0);                                                   \
        TG_MMA_LOADS(cur, bA, 0, WUNITS, TG_LW);                                             \
        TG_READ_B(bA, buf_, 2);                                                              \
        __builtin_amdgcn_sched_barrier(0);                                                   \
        TG_MMA_LOADS(cur, bB, 1, 4 * MT, TG_LA);                                             \
        TG_READ_B(bB, buf_, 3);                                                              \
        __builtin_amdgcn_sched_barrier(0);                                                   \
        TG_MMA(cur, bA, 2);                                                                  \
        __builtin_amdgcn_sched_barrier(0);                                                   \
        TG_MMA(cur, bB, 3);                                                                  \
        TG_STORE_W(buf_ ^ 1);                                                                \
        __syncthreads();                                                                     \
    } while (0)

    TG_LOAD_W(0);
    TG_LOAD_A(a0, 0);
    TG_LOAD_A(a1, min(1, nsteps - 1));
    TG_STORE_W(0);
    __syncthreads();
    const int groups = nsteps / RING;
    if constexpr (STREAM) {
        static_assert(MT == 1, "two waves per SIMD use 32-token waves");
        for (int g = 0; g < groups; ++g) {
            const int s = g * RING;
            TG_STEP_STREAM(s, a0, a2);
            TG_STEP_STREAM(s + 1, a1, a0);
            TG_STEP_STREAM(s + 2, a2, a1);
        }
        const int rest = nsteps - groups * RING;
        if (rest > 0) TG_STEP_STREAM(groups * RING, a0, a2);
        if (rest > 1) TG_STEP_STREAM(groups * RING + 1, a1, a0);
    } else {
        for (int g = 0; g < groups; ++g) {
            const int s = g * RING;
            TG_STEP(s, a0, a2);
            TG_STEP(s + 1, a1, a0);
            TG_STEP(s + 2, a2, a1);
        }
        const int rest = nsteps - groups * RING;
        if (rest > 0) TG_STEP(groups * RING, a0, a2);
        if (rest > 1) TG_STEP(groups * RING + 1, a1, a0);
    }
#undef TG_STEP
#undef TG_STEP_STREAM
#undef TG_BFRAG
#undef TG_LW
#undef TG_LA
#undef TG_MMA
#undef TG_MMA_LOADS
#undef TG_LOAD_A1
#undef TG_LOAD_W1
#undef TG_READ_B
#undef TG_STORE_W
#undef TG_LOAD_W
#undef TG_LOAD_A

    // Epilogue: lane holds unit 32nt + l32 and tokens 8(r/4)+4hh+r%4 (+32mt).
    // Each lane folds its NT units per token, then the 32 unit-lanes of every
    // token are summed through a per-wave LDS tile: lane (l32, hh) writes its
    // partial of token slot j = 16mt + r into row 2j + hh, and lane i then adds
    // up row i (token slot i/2, half i%2), a transpose instead of 32
    // five-level shuffle butterflies.
    float* rt = (RED_IN_WL ? reinterpret_cast<float*>(&wl[0][0]) : red_own) + w * RED_FLOATS;
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            float p = 0.f;
#pragma unroll
            for (int nt = 0; nt < NT; ++nt) p = fmaf(wout[nt], gelu_fast(acc[mt][nt][r] + bias[nt]), p);
            rt[(2 * (16 * mt + r) + hh) * RED_STRIDE + l32] = p;
        }
    }
    __builtin_amdgcn_wave_barrier();
    float sum = 0.f;
    if (lane < 32 * MT) {
        sum = (b2 != nullptr && uh == 0) ? to_f32(b2[0]) : 0.f;
#pragma unroll
        for (int c = 0; c < 8; ++c) {
            const f32x4 v = *reinterpret_cast<const f32x4*>(&rt[lane * RED_STRIDE + 4 * c]);
            sum += (v[0] + v[1]) + (v[2] + v[3]);
        }
    }
    if constexpr (US == 2) {
        // The second half's partial score of each token, added to the first's.
        __shared__ float half1[WAVES / 2][32 * MT];
        if (uh == 1 && lane < 32 * MT) half1[tgw][lane] = sum;
        __syncthreads();
        if (uh == 1) return;
        if (lane < 32 * MT) sum += half1[tgw][lane];
    }
    if (lane < 32 * MT) {
        const int j = lane / 2, half = lane % 2, mt = j / 16, r = j % 16;
        const int64_t t = tok0 + 32 * MT * tgw + 32 * mt + 8 * (r / 4) + 4 * half + (r % 4);
        if (t < T) scores[t] = sum;
    }
}

template <int DG>
hipError_t launch_gate_bf16_dg(const bf16* hidden, int64_t T, int d, const bf16* w1,
                               const bf16* b1, const bf16* w2, const bf16* b2, float* scores,
                               hipStream_t st) {
    if (T >= 256 * 256) {
        // Largest token tile that still gives at least one workgroup per CU:
        // fewer, larger workgroups read each W1 chunk for more tokens.
        hipLaunchKernelGGL((gate_bf16_kernel<DG, 4, 2, 1>), dim3((T + 255) / 256), dim3(256), 0, st,
                           hidden, T, d, w1, b1, w2, b2, scores);
    } else if constexpr (DG == 256) {
        if (T <= 128 * 256 / 2) {
            // A short prompt (up to 16384 tokens): 64-token workgroups whose
            // two pairs of waves split the gate units, so that every SIMD
            // gets a wave (128-token workgroups leave half of them idle).
            // One workgroup per CU, so each wave holds whole slices of W1
            // fragments.
            hipLaunchKernelGGL((gate_bf16_kernel<DG, 4, 1, 1, 2>), dim3((T + 63) / 64), dim3(256), 0,
                               st, hidden, T, d, w1, b1, w2, b2, scores);
        } else {
            // Below 65536 tokens, 128-token workgroups of 32-token waves, two
            // per CU: more waves, and one workgroup's GELU epilogue overlaps
            // the other's MFMAs and loads.
            hipLaunchKernelGGL((gate_bf16_kernel<DG, 4, 1, 2>), dim3((T + 127) / 128), dim3(256), 0, st,
                               hidden, T, d, w1, b1, w2, b2, scores);
        }
    } else if (T >= 128 * 512) {
        hipLaunchKernelGGL((gate_bf16_kernel<DG, 2, 2, 1>), dim3((T + 127) / 128), dim3(128), 0, st,
                           hidden, T, d, w1, b1, w2, b2, scores);
    } else {
        hipLaunchKernelGGL((gate_bf16_kernel<DG, 1, 2, 1>), dim3((T + 63) / 64), dim3(64), 0, st,
                           hidden, T, d, w1, b1, w2, b2, scores);
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
