// The rest of a pruned decoder layer on the kept rows: RMSNorm, the per-head
// RMSNorm of q and k followed by the rotary embedding at each kept token's
// original position, the SwiGLU product, and the kept rows' positions.
//
// Layers above the gate run on the kept tokens only (spke.com page,
// three-phase list, third bullet); the layer itself is the published Qwen3
// decoder layer (the backbone the pages name).  Every kernel here is a
// streaming, HBM-bound pass: one read and one write of each element, fp32
// arithmetic, one rounding at the store.

#include <math.h>

#include "tg_device.h"
#include "tg_kernels.h"

namespace tg {
namespace {

template <class T> struct Vec;
template <> struct Vec<bf16> {
    static constexpr int N = 8;
    __device__ static void load(const void* p, float* f) {
        const bf16x8 h = as_bf16x8(ld16(p));
#pragma unroll
        for (int e = 0; e < 8; ++e) f[e] = (float)h[e];
    }
    __device__ static void store(void* p, const float* f) {
        bf16x8 h;
#pragma unroll
        for (int e = 0; e < 8; ++e) h[e] = (bf16)f[e];
        st16(p, __builtin_bit_cast(u32x4, h));
    }
};
template <> struct Vec<float> {
    static constexpr int N = 4;
    __device__ static void load(const void* p, float* f) {
        const f32x4 x = __builtin_bit_cast(f32x4, ld16(p));
#pragma unroll
        for (int e = 0; e < 4; ++e) f[e] = x[e];
    }
    __device__ static void store(void* p, const float* f) {
        st16(p, __builtin_bit_cast(u32x4, f32x4{f[0], f[1], f[2], f[3]}));
    }
};

constexpr int ROWS_PER_BLOCK = 4;  // one wave per row

// y[m] = x[m] / sqrt(mean(x[m]^2) + eps) * w.  Two passes over the row: the
// second read of a 4 KiB row is served by the cache.
template <class T>
__global__ __launch_bounds__(ROWS_PER_BLOCK * WAVE) void rmsnorm_kernel(
        const T* __restrict__ x, const T* __restrict__ w, float eps, int64_t M, int d,
        T* __restrict__ y) {
    constexpr int V = Vec<T>::N;
    const int64_t m = (int64_t)blockIdx.x * ROWS_PER_BLOCK + threadIdx.x / WAVE;
    if (m >= M) return;
    const int lane = lane_id();
    const T* xr = x + m * d;
    float ss = 0.0f;
    for (int c = lane * V; c < d; c += WAVE * V) {
        float f[V];
        Vec<T>::load(xr + c, f);
#pragma unroll
        for (int e = 0; e < V; ++e) ss = fmaf(f[e], f[e], ss);
    }
    ss = wave_sum(ss);
    const float r = 1.0f / sqrtf(ss / (float)d + eps);
    T* yr = y + m * d;
    for (int c = lane * V; c < d; c += WAVE * V) {
        float f[V], g[V];
        Vec<T>::load(xr + c, f);
        Vec<T>::load(w + c, g);
#pragma unroll
        for (int e = 0; e < V; ++e) f[e] = f[e] * r * g[e];
        Vec<T>::store(yr + c, f);
    }
}

struct RopeArgs {
    void* q;
    void* k;
    const void* qw;  // [DH] or null
    const void* kw;  // [DH] or null
    const int32_t* pos;
    int64_t M;
    int32_t Hq, Hkv;
    float eps;
    double inv_freq[64];  // theta^(-2i/DH), i < DH/2, computed on the host in double
};

// In place on one row of q (Hq heads) and k (Hkv heads): per head, RMSNorm
// over DH elements (when a weight is given), then the pair (i, i + DH/2)
// turns by pos * inv_freq[i].  Lanes of a head: LPR = DH / V, each holding V
// contiguous elements; the partner of an element sits DH/2 further, i.e. in
// lane ^ (LPR / 2).  The angle is formed and reduced modulo 2 pi in double,
// so positions up to 2^31 keep full fp32 accuracy in sin and cos.
template <class T, int DH>
__global__ __launch_bounds__(ROWS_PER_BLOCK * WAVE) void qk_norm_rope_kernel(RopeArgs a) {
    constexpr int V = Vec<T>::N;
    constexpr int LPR = DH / V;
    constexpr int HPW = WAVE / LPR;  // heads per wave pass
    constexpr int HALF = DH / 2;
    const int64_t m = (int64_t)blockIdx.x * ROWS_PER_BLOCK + threadIdx.x / WAVE;
    if (m >= a.M) return;
    const int lane = lane_id();
    const int sub = lane % LPR, hsub = lane / LPR;
    const int col = sub * V;
    const bool first = col < HALF;

    const double p = (double)a.pos[m];
    float cs[V], sn[V];
#pragma unroll
    for (int e = 0; e < V; ++e) {
        const double ang = p * a.inv_freq[(col + e) % HALF];
        const double two_pi = 6.283185307179586476925;
        const float red = (float)(ang - two_pi * rint(ang / two_pi));
        sincosf(red, &sn[e], &cs[e]);
    }
    float qwf[V], kwf[V];
#pragma unroll
    for (int e = 0; e < V; ++e) qwf[e] = kwf[e] = 1.0f;
    if (a.qw != nullptr) Vec<T>::load((const T*)a.qw + col, qwf);
    if (a.kw != nullptr) Vec<T>::load((const T*)a.kw + col, kwf);

    const int H = a.Hq + a.Hkv;
    for (int h0 = 0; h0 < H; h0 += HPW) {
        const int h = h0 + hsub;
        const bool live = h < H;
        const bool isq = h < a.Hq;
        T* base = isq ? (T*)a.q + (m * a.Hq + h) * DH
                      : (T*)a.k + (m * a.Hkv + (h - a.Hq)) * DH;
        float f[V];
#pragma unroll
        for (int e = 0; e < V; ++e) f[e] = 0.0f;
        if (live) Vec<T>::load(base + col, f);
        const bool norm = isq ? a.qw != nullptr : a.kw != nullptr;
        float ss = 0.0f;
#pragma unroll
        for (int e = 0; e < V; ++e) ss = fmaf(f[e], f[e], ss);
#pragma unroll
        for (int o = 1; o < LPR; o <<= 1) ss += __shfl_xor(ss, o, WAVE);
        const float r = norm ? 1.0f / sqrtf(ss / (float)DH + a.eps) : 1.0f;
#pragma unroll
        for (int e = 0; e < V; ++e) f[e] = f[e] * r * (isq ? qwf[e] : kwf[e]);
        float g[V];
#pragma unroll
        for (int e = 0; e < V; ++e) g[e] = __shfl_xor(f[e], LPR / 2, WAVE);
        float out[V];
#pragma unroll
        for (int e = 0; e < V; ++e)
            out[e] = first ? fmaf(f[e], cs[e], -g[e] * sn[e]) : fmaf(f[e], cs[e], g[e] * sn[e]);
        if (live) Vec<T>::store(base + col, out);
    }
}

// out[m][j] = silu(gu[m][j]) * gu[m][F + j], silu(z) = z / (1 + e^-z).
template <class T>
__global__ __launch_bounds__(256) void silu_mul_kernel(const T* __restrict__ gu, int64_t M, int F,
                                                        T* __restrict__ out) {
    constexpr int V = Vec<T>::N;
    const int per_row = F / V;
    const int64_t n = M * per_row;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n;
         i += (int64_t)gridDim.x * blockDim.x) {
        const int64_t m = i / per_row;
        const int c = (int)(i % per_row) * V;
        float g[V], u[V];
        Vec<T>::load(gu + m * 2 * F + c, g);
        Vec<T>::load(gu + m * 2 * F + F + c, u);
#pragma unroll
        for (int e = 0; e < V; ++e) g[e] = g[e] / (1.0f + __expf(-g[e])) * u[e];
        Vec<T>::store(out + m * F + c, g);
    }
}

// pos[r] = kept[r] - cu_seq[b] for the request b whose kept rows hold r.
__global__ __launch_bounds__(256) void kept_positions_kernel(const int32_t* __restrict__ kept,
                                                              int64_t Kt, BatchArgs a,
                                                              int32_t* __restrict__ pos) {
    const int64_t r = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (r >= Kt) return;
    int lo = 0, hi = a.batch - 1;  // last b with cu_kept[b] <= r
    while (lo < hi) {
        const int mid = (lo + hi + 1) / 2;
        if (a.cu_kept[mid] <= r) lo = mid; else hi = mid - 1;
    }
    pos[r] = kept[r] - a.cu_seq[lo];
}

int grid_for(int64_t rows) { return (int)((rows + ROWS_PER_BLOCK - 1) / ROWS_PER_BLOCK); }

}  // namespace

hipError_t launch_rmsnorm(tg_dtype dt, const void* x, const void* w, float eps, int64_t M, int d,
                          void* y, hipStream_t st) {
    if (dt == TG_BF16)
        hipLaunchKernelGGL(rmsnorm_kernel<bf16>, dim3(grid_for(M)), dim3(ROWS_PER_BLOCK * WAVE), 0,
                           st, (const bf16*)x, (const bf16*)w, eps, M, d, (bf16*)y);
    else
        hipLaunchKernelGGL(rmsnorm_kernel<float>, dim3(grid_for(M)), dim3(ROWS_PER_BLOCK * WAVE), 0,
                           st, (const float*)x, (const float*)w, eps, M, d, (float*)y);
    return hipGetLastError();
}

hipError_t launch_qk_norm_rope(tg_dtype dt, void* q, void* k, const void* qw, const void* kw,
                               const int32_t* pos, int64_t M, int Hq, int Hkv, int dh, float theta,
                               float eps, hipStream_t st) {
    RopeArgs a;
    a.q = q;
    a.k = k;
    a.qw = qw;
    a.kw = kw;
    a.pos = pos;
    a.M = M;
    a.Hq = Hq;
    a.Hkv = Hkv;
    a.eps = eps;
    for (int i = 0; i < 64; ++i) a.inv_freq[i] = i < dh / 2 ? pow((double)theta, -2.0 * i / dh) : 0.0;
    const dim3 grid(grid_for(M)), block(ROWS_PER_BLOCK * WAVE);
    if (dt == TG_BF16) {
        if (dh == 128) hipLaunchKernelGGL((qk_norm_rope_kernel<bf16, 128>), grid, block, 0, st, a);
        else hipLaunchKernelGGL((qk_norm_rope_kernel<bf16, 64>), grid, block, 0, st, a);
    } else {
        if (dh == 128) hipLaunchKernelGGL((qk_norm_rope_kernel<float, 128>), grid, block, 0, st, a);
        else hipLaunchKernelGGL((qk_norm_rope_kernel<float, 64>), grid, block, 0, st, a);
    }
    return hipGetLastError();
}

hipError_t launch_silu_mul(tg_dtype dt, const void* gu, int64_t M, int F, void* out,
                           hipStream_t st) {
    const int V = dt == TG_BF16 ? 8 : 4;
    const int64_t n = M * (F / V);
    const int grid = (int)std::min<int64_t>((n + 255) / 256, 256 * 32);
    if (dt == TG_BF16)
        hipLaunchKernelGGL(silu_mul_kernel<bf16>, dim3(grid), dim3(256), 0, st, (const bf16*)gu, M,
                           F, (bf16*)out);
    else
        hipLaunchKernelGGL(silu_mul_kernel<float>, dim3(grid), dim3(256), 0, st, (const float*)gu,
                           M, F, (float*)out);
    return hipGetLastError();
}

hipError_t launch_kept_positions(const int32_t* kept, int64_t Kt, const BatchArgs& a, int32_t* pos,
                                 hipStream_t st) {
    hipLaunchKernelGGL(kept_positions_kernel, dim3((unsigned)((Kt + 255) / 256)), dim3(256), 0, st,
                       kept, Kt, a, pos);
    return hipGetLastError();
}

}  // namespace tg
