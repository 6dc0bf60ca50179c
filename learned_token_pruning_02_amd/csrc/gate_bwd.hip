// Backward of the gate MLP over the kept rows.
//
// The gate learns through the score bias of the attention above it; the top-K
// choice has no gradient, so only kept tokens receive a score gradient ds
// (spke.com page, "Comment TokenGate a-t-il appris ...").  For a kept row x,
// z = W1 x + b1, s = w2 . GELU(z) + b2:
//   dz  = ds * w2 * GELU'(z),  GELU'(z) = Phi(z) + z phi(z)
//   dW1 = sum_t dz_t x_t^T,  db1 = sum_t dz_t,  dw2 = sum_t ds_t GELU(z_t),
//   db2 = sum_t ds_t,        dx_t = W1^T dz_t
// The three products run on the matrix-core projection kernel (z = X W1^T,
// dx = dZ W1, dW1 = dZ^T X through zero-padded transposes so that the
// contraction over kept rows is a plain row-major product); the elementwise
// part and the column sums are two small kernels here, the sums reduced in a
// fixed order (no atomics).

#include <algorithm>

#include "tg_device.h"
#include "tg_kernels.h"

namespace tg {
namespace {

constexpr int DZ_ROWS = 16;     // kept rows per workgroup of the dz kernel
constexpr int DZ_THREADS = 256;

template <class T>
__device__ __forceinline__ float ld1(const T* p) { return to_f32(*p); }

// out[c][r] = in[r][c] for r < R, 0 for R <= r < Rpad; in is [R][C].
template <class T>
__global__ __launch_bounds__(256) void transpose_kernel(const T* __restrict__ in, int64_t R, int C,
                                                        T* __restrict__ out, int64_t Rpad) {
    __shared__ T tile[32][33];
    const int c0 = blockIdx.x * 32;
    const int64_t r0 = (int64_t)blockIdx.y * 32;
    const int tx = threadIdx.x % 32, ty = threadIdx.x / 32;  // 32 x 8
#pragma unroll
    for (int k = 0; k < 32; k += 8) {
        const int64_t r = r0 + ty + k;
        const int c = c0 + tx;
        tile[ty + k][tx] = (r < R && c < C) ? in[r * C + c] : from_f32<T>(0.0f);
    }
    __syncthreads();
#pragma unroll
    for (int k = 0; k < 32; k += 8) {
        const int c = c0 + ty + k;
        const int64_t r = r0 + tx;
        if (c < C && r < Rpad) out[(int64_t)c * Rpad + r] = tile[tx][ty + k];
    }
}

// dz[t][u] from zlin = X W1^T, given as S fp32 partials zlin[s][t][u] summed
// here in slice order; per-workgroup partial sums of ds*GELU(z) (for dw2), dz
// (for db1) and ds (for db2).
template <class T>
__global__ __launch_bounds__(DZ_THREADS) void gate_dz_kernel(const float* __restrict__ zlin, int S,
                                                             const T* __restrict__ b1,
                                                             const T* __restrict__ w2,
                                                             const float* __restrict__ ds,
                                                             int64_t Kt, int dg,
                                                             T* __restrict__ dz,
                                                             float* __restrict__ part) {
    const int64_t t0 = (int64_t)blockIdx.x * DZ_ROWS;
    const int64_t t1 = std::min<int64_t>(Kt, t0 + DZ_ROWS);
    float* pb = part + (int64_t)blockIdx.x * (2 * dg + 1);
    for (int u = threadIdx.x; u < dg; u += DZ_THREADS) {
        const float bu = b1 != nullptr ? ld1(b1 + u) : 0.0f;
        const float wu = ld1(w2 + u);
        float sw = 0.0f, sz = 0.0f;
        for (int64_t t = t0; t < t1; ++t) {
            float zs = zlin[t * dg + u];
            for (int q = 1; q < S; ++q) zs += zlin[((int64_t)q * Kt + t) * dg + u];
            const float z = zs + bu;
            const float Phi = 0.5f * (1.0f + erff(z * 0.70710678118654752f));
            const float phi = 0.39894228040143268f * __expf(-0.5f * z * z);
            const float d = ds[t];
            const float g = d * wu * fmaf(z, phi, Phi);
            dz[t * dg + u] = from_f32<T>(g);
            sw = fmaf(d, z * Phi, sw);
            sz += g;
        }
        pb[u] = sw;
        pb[dg + u] = sz;
    }
    if (threadIdx.x == 0) {
        float s = 0.0f;
        for (int64_t t = t0; t < t1; ++t) s += ds[t];
        pb[2 * dg] = s;
    }
}

// One wave per output: lanes sum a strided share of the partials, then a
// fixed shuffle tree combines the lanes (deterministic).
__global__ __launch_bounds__(256) void gate_bwd_reduce_kernel(const float* __restrict__ part,
                                                              int nblk, int dg,
                                                              float* __restrict__ dw2,
                                                              float* __restrict__ db1,
                                                              float* __restrict__ db2) {
    const int i = blockIdx.x * (256 / WAVE) + threadIdx.x / WAVE;  // output index
    if (i >= 2 * dg + 1) return;
    const int lane = lane_id();
    float acc = 0.0f;
    for (int b = lane; b < nblk; b += WAVE) acc += part[(int64_t)b * (2 * dg + 1) + i];
    acc = wave_sum(acc);
    if (lane != 0) return;
    if (i < dg) dw2[i] = acc;
    else if (i < 2 * dg) { if (db1 != nullptr) db1[i - dg] = acc; }
    else db2[0] = acc;
}

// dW1 = dZ^T X contracts over the kept rows into only d_gate x d outputs, too
// few tiles to fill the chip: the contraction is split into S slices of at
// least 512 rows (S <= 16), each writing an fp32 partial, summed in slice
// order by split_sum_kernel (deterministic).
__global__ __launch_bounds__(256) void split_sum_kernel(const float* __restrict__ part, int S, int64_t n,
                                                        bf16* __restrict__ y) {
    const int64_t i = ((int64_t)blockIdx.x * 256 + threadIdx.x) * 4;
    if (i >= n) return;
    f32x4 acc = __builtin_bit_cast(f32x4, ld16(part + i));
    for (int z = 1; z < S; ++z) {
        const f32x4 v = __builtin_bit_cast(f32x4, ld16(part + z * n + i));
#pragma unroll
        for (int e = 0; e < 4; ++e) acc[e] += v[e];
    }
    bf16x4 o;
#pragma unroll
    for (int e = 0; e < 4; ++e) o[e] = to_bf16(acc[e]);
    st8(y + i, __builtin_bit_cast(u32x2, o));
}

int dw1_slices(tg_dtype dt, int64_t Kt) {
    if (dt != TG_BF16) return 1;
    return (int)std::min<int64_t>(16, std::max<int64_t>(1, (Kt + 511) / 512));
}

// z = X W1^T has d_gate outputs per row: split its contraction over d in up
// to four slices while the 128x128 tiles alone number fewer than 512.
int z_slices(tg_dtype dt, int64_t Kt, int d, int dg) {
    if (dt != TG_BF16) return 1;
    const int64_t tiles = ((Kt + 127) / 128) * ((dg + 127) / 128);
    int S = 1;
    while (S < 4 && tiles * S < 512 && d % (64 * 2 * S) == 0) S *= 2;
    return S;
}

struct GateBwdLayout {
    int64_t kt_pad, nblk;
    int slices, zs;
    size_t zlin, dz, dzT, xT, w1T, part, dw1p, total;
};

GateBwdLayout layout(tg_dtype dt, int64_t Kt, int d, int dg) {
    const int64_t eb = dt == TG_BF16 ? 2 : 4;
    const auto up = [](int64_t x) { return (size_t)((x + 255) / 256 * 256); };
    GateBwdLayout L;
    L.slices = dw1_slices(dt, Kt);
    L.zs = z_slices(dt, Kt, d, dg);
    const int64_t q = 64 * L.slices;  // every slice a whole number of 64-row chunks
    L.kt_pad = (Kt + q - 1) / q * q;
    L.nblk = (Kt + DZ_ROWS - 1) / DZ_ROWS;
    size_t o = 0;
    L.zlin = o; o += up((int64_t)L.zs * Kt * dg * 4);  // fp32 partials of X W1^T
    L.dz = o;   o += up(Kt * dg * eb);
    L.dzT = o;  o += up((int64_t)dg * L.kt_pad * eb);
    L.xT = o;   o += up((int64_t)d * L.kt_pad * eb);
    L.w1T = o;  o += up((int64_t)d * dg * eb);
    L.part = o; o += up(std::max<int64_t>(1, L.nblk) * (2 * dg + 1) * 4);
    L.dw1p = o; o += L.slices > 1 ? up((int64_t)L.slices * dg * d * 4) : 0;
    L.total = o;
    return L;
}

template <class T>
hipError_t transpose(const T* in, int64_t R, int C, T* out, int64_t Rpad, hipStream_t st) {
    const dim3 grid((unsigned)((C + 31) / 32), (unsigned)((Rpad + 31) / 32));
    hipLaunchKernelGGL(transpose_kernel<T>, grid, dim3(256), 0, st, in, R, C, out, Rpad);
    return hipGetLastError();
}

template <class T>
hipError_t run(tg_dtype dt, const T* x, int64_t Kt, int d, const T* w1, const T* b1, const T* w2,
               int dg, const float* ds, T* dx, T* dw1, float* db1, float* dw2, float* db2, char* ws,
               hipStream_t st) {
    const GateBwdLayout L = layout(dt, Kt, d, dg);
    float* zlin = (float*)(ws + L.zlin);
    T* dz = (T*)(ws + L.dz);
    T* dzT = (T*)(ws + L.dzT);
    T* xT = (T*)(ws + L.xT);
    T* w1T = (T*)(ws + L.w1T);
    float* part = (float*)(ws + L.part);
    const auto lin = [&](const T* a, const T* b, T* y, int64_t M, int N, int K) {
        return dt == TG_BF16 ? launch_linear_bf16(a, b, y, M, N, K, 0, 0, st)
                             : launch_linear_f32((const float*)a, (const float*)b, (float*)y, M, N,
                                                 K, 0, st);
    };
    hipError_t e;
    if (dt == TG_BF16)                                                           // z - b1
        e = launch_linear_bf16_splitk(x, w1, zlin, Kt, dg, d, L.zs, st);
    else
        e = lin(x, w1, (T*)zlin, Kt, dg, d);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(gate_dz_kernel<T>, dim3((unsigned)L.nblk), dim3(DZ_THREADS), 0, st, zlin, L.zs, b1,
                       w2, ds, Kt, dg, dz, part);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    hipLaunchKernelGGL(gate_bwd_reduce_kernel, dim3((unsigned)((2 * dg + 1 + 3) / 4)), dim3(256), 0, st,
                       part, (int)L.nblk, dg, dw2, db1, db2);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    if ((e = transpose(w1, dg, d, w1T, dg, st)) != hipSuccess) return e;        // W1^T [d][dg]
    if ((e = lin(dz, w1T, dx, Kt, d, dg)) != hipSuccess) return e;              // dx = dZ W1
    if ((e = transpose(dz, Kt, dg, dzT, L.kt_pad, st)) != hipSuccess) return e; // dZ^T [dg][Kt_pad]
    if ((e = transpose(x, Kt, d, xT, L.kt_pad, st)) != hipSuccess) return e;    // X^T  [d][Kt_pad]
    if (L.slices == 1) return lin(dzT, xT, dw1, dg, d, (int)L.kt_pad);         // dW1 = dZ^T X
    float* dw1p = (float*)(ws + L.dw1p);
    if ((e = launch_linear_bf16_splitk(dzT, xT, dw1p, dg, d, (int)L.kt_pad, L.slices, st)) != hipSuccess)
        return e;
    const int64_t nout = (int64_t)dg * d;
    hipLaunchKernelGGL(split_sum_kernel, dim3((unsigned)((nout / 4 + 255) / 256)), dim3(256), 0, st, dw1p,
                       L.slices, nout, (bf16*)dw1);
    return hipGetLastError();
}

}  // namespace

size_t gate_bwd_workspace_bytes(tg_dtype dt, int64_t Kt, int d, int dg) {
    return layout(dt, Kt, d, dg).total;
}

hipError_t launch_gate_bwd(tg_dtype dt, const void* x, int64_t Kt, int d, const void* w1,
                           const void* b1, const void* w2, int dg, const float* ds, void* dx,
                           void* dw1, float* db1, float* dw2, float* db2, void* ws,
                           hipStream_t st) {
    if (dt == TG_BF16)
        return run<bf16>(dt, (const bf16*)x, Kt, d, (const bf16*)w1, (const bf16*)b1,
                         (const bf16*)w2, dg, ds, (bf16*)dx, (bf16*)dw1, db1, dw2, db2, (char*)ws, st);
    return run<float>(dt, (const float*)x, Kt, d, (const float*)w1, (const float*)b1,
                      (const float*)w2, dg, ds, (float*)dx, (float*)dw1, db1, dw2, db2, (char*)ws,
                      st);
}

}  // namespace tg
