// Token-gated decode attention over the kept-only KV cache.
//
// After a pruned prefill the cache holds only the kept tokens (spke.com page,
// three-phase list, third bullet: no KV record for a pruned token), each row
// with its gate score.  One new query per request attends to every cached row
// with the same logit as the prefill (page "Qu'est-ce que l'attention gérée
// par des tokens ?"):  l_j = tau_h (q . k_j) / sqrt(dh) + g_h s_j.
//
// The step reads every cached K/V row once and does a few FLOP per byte, so it
// is bound by HBM bandwidth, not by the matrix cores.  Split-K layout:
//   * one workgroup per (128-row chunk, KV head, request); the G = Hq/Hkv
//     query heads that share the KV head share every K/V byte read;
//   * each lane owns 16 contiguous bytes of a row (LPR lanes cover a row) and
//     issues all of its K and V loads before any arithmetic, so a workgroup
//     has its whole 128-row chunk in flight at once;
//   * per chunk the workgroup leaves (max, sum, unnormalised output) in the
//     caller's workspace, in the log2 domain; a second kernel merges the
//     chunks of each (request, head).
// Lengths and row offsets are device arrays, so a decode loop needs no host
// synchronisation; rows outside [0, cache_rows) are never dereferenced.

#include "tg_device.h"
#include "tg_kernels.h"

namespace tg {
namespace {

constexpr int DEC_THREADS = 256;
constexpr int DEC_WAVES = DEC_THREADS / WAVE;

struct DecArgs {
    const void* q;        // [B][Hq][DH]
    const void* k;        // [R][Hkv][DH]
    const void* v;        // [R][Hkv][DH]
    const float* s;       // [R] or null (no bias)
    const int64_t* row_off;    // [B] device
    const int32_t* cache_len;  // [B] device
    const float* gain;    // [Hq] or null
    const float* temp;    // [Hq]
    float* part_o;        // [B][Hq][nch][DH]
    float* part_ml;       // [B][Hq][nch][2]
    void* out;            // [B][Hq][DH]
    float* lse;           // [B][Hq] or null
    int64_t rows;         // R
    int32_t max_len;
    int32_t nch;          // chunks per request
    int32_t Hq, Hkv, G;
    float qscale;         // log2(e) / sqrt(DH)
};

template <class T> struct Elt;
template <> struct Elt<bf16> {
    static constexpr int PER16 = 8;
    __device__ static void unpack(u32x4 u, float* f) {
        const bf16x8 h = as_bf16x8(u);
#pragma unroll
        for (int e = 0; e < 8; ++e) f[e] = (float)h[e];
    }
};
template <> struct Elt<float> {
    static constexpr int PER16 = 4;
    __device__ static void unpack(u32x4 u, float* f) {
        const f32x4 x = __builtin_bit_cast(f32x4, u);  // whole-vector cast, then index
#pragma unroll
        for (int e = 0; e < 4; ++e) f[e] = x[e];
    }
};

// Sum over the LPR consecutive lanes that hold one row.
template <int LPR>
__device__ __forceinline__ float row_sum(float x) {
#pragma unroll
    for (int o = 1; o < LPR; o <<= 1) x += __shfl_xor(x, o, WAVE);
    return x;
}

// Reduce over the row groups of a wave (lanes that differ in bits >= log2 LPR).
template <int LPR>
__device__ __forceinline__ float groups_max(float x) {
#pragma unroll
    for (int o = LPR; o < WAVE; o <<= 1) x = fmaxf(x, __shfl_xor(x, o, WAVE));
    return x;
}
template <int LPR>
__device__ __forceinline__ float groups_sum(float x) {
#pragma unroll
    for (int o = LPR; o < WAVE; o <<= 1) x += __shfl_xor(x, o, WAVE);
    return x;
}

template <class T, int DH, int MAXG>
__global__ __launch_bounds__(DEC_THREADS) void decode_chunk_kernel(DecArgs a) {
    constexpr int EPL = Elt<T>::PER16;       // elements per 16-byte lane load
    constexpr int LPR = DH / EPL;            // lanes per row
    constexpr int RPW = WAVE / LPR;          // rows per wave and load
    constexpr int ITER = TG_DECODE_CHUNK / (DEC_WAVES * RPW);
    static_assert(ITER >= 1 && ITER * DEC_WAVES * RPW == TG_DECODE_CHUNK, "chunk tiling");

    __shared__ float red[DEC_WAVES][MAXG];
    __shared__ float red_o[DEC_WAVES][MAXG][DH];

    const int c = blockIdx.x, kvh = blockIdx.y, b = blockIdx.z;
    const int len = min(max(a.cache_len[b], 0), a.max_len);
    const int j0 = c * TG_DECODE_CHUNK;
    if (j0 >= len) return;  // uniform: the merge reads only chunks below len
    const int64_t off = a.row_off[b];
    const int tid = threadIdx.x, w = tid / WAVE, lane = tid % WAVE;
    const int col = (lane % LPR) * EPL;
    const int G = a.G;
    const int h0 = kvh * G;

    // Raw query slices first; they are unpacked only after the K/V loads
    // below are in flight, so their latency overlaps the stream.
    u32x4 qr[MAXG];
    float qsc[MAXG], gain2[MAXG];
#pragma unroll
    for (int g = 0; g < MAXG; ++g) {  // branch-free: padded heads reread the last one, scaled by 0
        const int h = h0 + min(g, G - 1);
        qr[g] = ld16((const T*)a.q + ((int64_t)b * a.Hq + h) * DH + col);
        qsc[g] = g < G ? a.temp[h] * a.qscale : 0.0f;
        gain2[g] = (g < G && a.gain != nullptr) ? a.gain[h] * 1.4426950408889634f : 0.0f;
    }

    // Issue every K, V and score load of this lane before using any.
    u32x4 kr[ITER], vr[ITER];
    float sj[ITER];
    bool ok[ITER];
#pragma unroll
    for (int it = 0; it < ITER; ++it) {
        const int j = j0 + it * (DEC_WAVES * RPW) + w * RPW + lane / LPR;
        const int64_t row = off + j;
        ok[it] = j < len && row >= 0 && row < a.rows;
        kr[it] = u32x4{0u, 0u, 0u, 0u};
        vr[it] = u32x4{0u, 0u, 0u, 0u};
        sj[it] = 0.0f;
        if (ok[it]) {
            const int64_t e0 = (row * a.Hkv + kvh) * DH + col;
            // Each cached byte is read once per step: nontemporal loads keep
            // the stream from evicting the partials and small operands.
            kr[it] = __builtin_nontemporal_load((const u32x4*)((const T*)a.k + e0));
            vr[it] = __builtin_nontemporal_load((const u32x4*)((const T*)a.v + e0));
            if (a.s != nullptr) sj[it] = a.s[row];
        }
    }

    // Query slices pre-scaled so that the dot product is
    // tau_h q.k / sqrt(DH) in log2 units.
    float qf[MAXG][EPL];
#pragma unroll
    for (int g = 0; g < MAXG; ++g) {
        Elt<T>::unpack(qr[g], qf[g]);
#pragma unroll
        for (int e = 0; e < EPL; ++e) qf[g][e] *= qsc[g];
    }

    // Logits (log2 units) and the chunk maximum of each head.
    float y[ITER][MAXG], m[MAXG];
#pragma unroll
    for (int g = 0; g < MAXG; ++g) m[g] = -INFINITY;
#pragma unroll
    for (int it = 0; it < ITER; ++it) {
        float kf[EPL];
        Elt<T>::unpack(kr[it], kf);
#pragma unroll
        for (int g = 0; g < MAXG; ++g) {
            float d = 0.0f;
#pragma unroll
            for (int e = 0; e < EPL; ++e) d = fmaf(qf[g][e], kf[e], d);
            d = row_sum<LPR>(d);
            y[it][g] = ok[it] ? fmaf(gain2[g], sj[it], d) : -INFINITY;
            m[g] = fmaxf(m[g], y[it][g]);
        }
    }
#pragma unroll
    for (int g = 0; g < MAXG; ++g) m[g] = groups_max<LPR>(m[g]);
    if (lane == 0) {
#pragma unroll
        for (int g = 0; g < MAXG; ++g) red[w][g] = m[g];
    }
    __syncthreads();
#pragma unroll
    for (int g = 0; g < MAXG; ++g) {
        float mm = red[0][g];
#pragma unroll
        for (int i = 1; i < DEC_WAVES; ++i) mm = fmaxf(mm, red[i][g]);
        m[g] = mm == -INFINITY ? 0.0f : mm;  // no valid row: every p below is 0
    }
    __syncthreads();  // red is reused for the sums

    // p_j = 2^(y_j - m); per-lane output slice sum_j p_j v_j.
    float l[MAXG], acc[MAXG][EPL];
#pragma unroll
    for (int g = 0; g < MAXG; ++g) {
        l[g] = 0.0f;
#pragma unroll
        for (int e = 0; e < EPL; ++e) acc[g][e] = 0.0f;
    }
#pragma unroll
    for (int it = 0; it < ITER; ++it) {
        float vf[EPL];
        Elt<T>::unpack(vr[it], vf);
#pragma unroll
        for (int g = 0; g < MAXG; ++g) {
            const float p = __builtin_amdgcn_exp2f(y[it][g] - m[g]);  // exp2(-inf) = 0
            l[g] += p;
#pragma unroll
            for (int e = 0; e < EPL; ++e) acc[g][e] = fmaf(p, vf[e], acc[g][e]);
        }
    }
#pragma unroll
    for (int g = 0; g < MAXG; ++g) {
        l[g] = groups_sum<LPR>(l[g]);
#pragma unroll
        for (int e = 0; e < EPL; ++e) acc[g][e] = groups_sum<LPR>(acc[g][e]);
    }
    if (lane < LPR) {
#pragma unroll
        for (int g = 0; g < MAXG; ++g)
#pragma unroll
            for (int e = 0; e < EPL; ++e) red_o[w][g][col + e] = acc[g][e];
    }
    if (lane == 0) {
#pragma unroll
        for (int g = 0; g < MAXG; ++g) red[w][g] = l[g];
    }
    __syncthreads();

    // Cross-wave sums; one thread per (head, column) writes the partial.
    const int64_t pbase = ((int64_t)b * a.Hq + h0) * a.nch + c;  // head h0 + g adds g * nch
    for (int i = tid; i < MAXG * DH; i += DEC_THREADS) {
        const int g = i / DH, d = i % DH;
        if (g < G) {
            float o = 0.0f;
#pragma unroll
            for (int ww = 0; ww < DEC_WAVES; ++ww) o += red_o[ww][g][d];
            a.part_o[(pbase + (int64_t)g * a.nch) * DH + d] = o;
        }
    }
#pragma unroll
    for (int g = 0; g < MAXG; ++g) {  // static indexing keeps m[] in registers
        if (g < G && tid == g) {
            float ls = 0.0f;
#pragma unroll
            for (int ww = 0; ww < DEC_WAVES; ++ww) ls += red[ww][g];
            float* ml = a.part_ml + (pbase + (int64_t)g * a.nch) * 2;
            ml[0] = m[g];
            ml[1] = ls;
        }
    }
}

// Merge the chunks of one (request, head): out = sum_c 2^(m_c - M) o_c / L
// with M the largest chunk maximum and L = sum_c 2^(m_c - M) l_c.  The chunk
// weights are computed once (kept in LDS for the first MERGE_LDS_CHUNKS
// chunks); each thread then sums one column over every R-th chunk with
// independent loads, and the R partial sums meet in LDS.
constexpr int MERGE_THREADS = 256;
constexpr int MERGE_LDS_CHUNKS = 2048;

template <class T, int DH>
__global__ __launch_bounds__(MERGE_THREADS) void decode_merge_kernel(DecArgs a) {
    constexpr int R = MERGE_THREADS / DH;
    constexpr int NW = MERGE_THREADS / WAVE;
    __shared__ float fac[MERGE_LDS_CHUNKS];
    __shared__ float red_m[NW], red_l[NW];
    __shared__ float red_o[R][DH];

    const int bh = blockIdx.x;
    const int b = bh / a.Hq;
    const int t = threadIdx.x, w = t / WAVE, lane = t % WAVE;
    const int len = min(max(a.cache_len[b], 0), a.max_len);
    const int nch = (len + TG_DECODE_CHUNK - 1) / TG_DECODE_CHUNK;
    const float* ml = a.part_ml + (int64_t)bh * a.nch * 2;
    const float* po = a.part_o + (int64_t)bh * a.nch * DH;

    float mx = -INFINITY;
    for (int c = t; c < nch; c += MERGE_THREADS)
        if (ml[2 * c + 1] > 0.0f) mx = fmaxf(mx, ml[2 * c]);
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) mx = fmaxf(mx, __shfl_xor(mx, o, WAVE));
    if (lane == 0) red_m[w] = mx;
    __syncthreads();
    float M = red_m[0];
#pragma unroll
    for (int i = 1; i < NW; ++i) M = fmaxf(M, red_m[i]);
    const bool none = M == -INFINITY;  // no chunk holds a present row

    float lp = 0.0f;
    for (int c = t; c < nch; c += MERGE_THREADS) {
        const float lc = ml[2 * c + 1];
        const float f = (lc > 0.0f && !none) ? __builtin_amdgcn_exp2f(ml[2 * c] - M) : 0.0f;
        if (c < MERGE_LDS_CHUNKS) fac[c] = f;
        lp = fmaf(lc, f, lp);
    }
    lp = wave_sum(lp);
    if (lane == 0) red_l[w] = lp;
    __syncthreads();
    float L = 0.0f;
#pragma unroll
    for (int i = 0; i < NW; ++i) L += red_l[i];

    const int r = t / DH, d = t % DH;
    float o = 0.0f;
#pragma unroll 8
    for (int c = r; c < nch; c += R) {
        float f;
        if (c < MERGE_LDS_CHUNKS) {
            f = fac[c];
        } else {
            const float lc = ml[2 * c + 1];
            f = (lc > 0.0f && !none) ? __builtin_amdgcn_exp2f(ml[2 * c] - M) : 0.0f;
        }
        o = fmaf(po[(int64_t)c * DH + d], f, o);
    }
    red_o[r][d] = o;
    __syncthreads();
    if (t < DH) {
        float os = 0.0f;
#pragma unroll
        for (int i = 0; i < R; ++i) os += red_o[i][t];
        const bool any = L > 0.0f;
        ((T*)a.out)[(int64_t)bh * DH + t] = from_f32<T>(any ? os / L : 0.0f);
        if (a.lse != nullptr && t == 0)
            a.lse[bh] = any ? (M + __log2f(L)) * 0.6931471805599453f : -INFINITY;
    }
}

template <class T, int DH>
hipError_t launch_dh(const DecArgs& a, int batch, hipStream_t st) {
    const dim3 grid(a.nch, a.Hkv, batch);
    if (a.nch == 0)  // max_len == 0: only the merge runs (zero output, lse = -inf)
        ;
    else if (a.G <= 1)
        hipLaunchKernelGGL((decode_chunk_kernel<T, DH, 1>), grid, dim3(DEC_THREADS), 0, st, a);
    else if (a.G <= 2)
        hipLaunchKernelGGL((decode_chunk_kernel<T, DH, 2>), grid, dim3(DEC_THREADS), 0, st, a);
    else if (a.G <= 4)
        hipLaunchKernelGGL((decode_chunk_kernel<T, DH, 4>), grid, dim3(DEC_THREADS), 0, st, a);
    else
        hipLaunchKernelGGL((decode_chunk_kernel<T, DH, 8>), grid, dim3(DEC_THREADS), 0, st, a);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((decode_merge_kernel<T, DH>), dim3(batch * a.Hq), dim3(MERGE_THREADS), 0, st,
                       a);
    return hipGetLastError();
}

}  // namespace

size_t decode_workspace_bytes(int32_t batch, int32_t Hq, int32_t d_head, int32_t max_len) {
    const int64_t nch = ((int64_t)max_len + TG_DECODE_CHUNK - 1) / TG_DECODE_CHUNK;
    const int64_t per = (int64_t)batch * Hq * nch;
    const int64_t o_bytes = (per * d_head * 4 + 255) / 256 * 256;
    return (size_t)(o_bytes + per * 2 * 4);
}

hipError_t launch_decode(tg_dtype dt, const DecodeShape& sh, const void* q, const void* k,
                         const void* v, const float* s, const int64_t* row_off,
                         const int32_t* cache_len, const float* gain, const float* temp, void* out,
                         float* lse, void* ws, hipStream_t st) {
    DecArgs a;
    a.q = q;
    a.k = k;
    a.v = v;
    a.s = s;
    a.row_off = row_off;
    a.cache_len = cache_len;
    a.gain = gain;
    a.temp = temp;
    a.out = out;
    a.lse = lse;
    a.rows = sh.rows;
    a.max_len = sh.max_len;
    a.nch = (sh.max_len + TG_DECODE_CHUNK - 1) / TG_DECODE_CHUNK;
    a.Hq = sh.Hq;
    a.Hkv = sh.Hkv;
    a.G = sh.Hq / sh.Hkv;
    a.qscale = 1.4426950408889634f / sqrtf((float)sh.d_head);
    const int64_t per = (int64_t)sh.batch * sh.Hq * a.nch;
    a.part_o = (float*)ws;
    a.part_ml = (float*)((char*)ws + (per * sh.d_head * 4 + 255) / 256 * 256);
    if (dt == TG_BF16)
        return sh.d_head == 128 ? launch_dh<bf16, 128>(a, sh.batch, st)
                                : launch_dh<bf16, 64>(a, sh.batch, st);
    return sh.d_head == 128 ? launch_dh<float, 128>(a, sh.batch, st)
                            : launch_dh<float, 64>(a, sh.batch, st);
}

}  // namespace tg
