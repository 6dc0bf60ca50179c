// Backward of the token-gated attention: gradients with respect to q, k, v,
// the kept tokens' scores s_j, the per-head gains g_h and temperatures tau_h.
//
// The score bias is the only path by which the gate receives a gradient
// (spke.com page, "Qu'est-ce que l'attention gérée par des tokens ?"; the
// top-K choice has none).  With l_ij = tau_h r_ij + g_h s_j,
// r_ij = q_i.k_j / sqrt(dh), P = softmax_j(l), the forward's lse and output O:
//   D_i = dO_i . O_i,   dP_ij = dO_i . v_j,   dL_ij = P_ij (dP_ij - D_i)
//   dq_i = tau/sqrt(dh) sum_j dL_ij k_j,  dk_j = sum_h tau_h/sqrt(dh) sum_i dL_ij q_i
//   dv_j = sum_h sum_i P_ij dO_i,         ds_j = sum_h g_h sum_i dL_ij
//   dg_h = sum_ij dL_ij s_j,              dtau_h = sum_ij dL_ij r_ij
//
// Two deterministic MFMA passes (no floating-point atomics):
//   * KV-major: a wave owns 32 keys of one KV head and walks the query blocks
//     of every query head in its group.  S = Q K^T and dP = dO V^T come out
//     with lane = key; their fp32 registers, rounded to bf16, are used
//     directly as the B operand of dK^T += Q^T dS and dV^T += dO^T P (the
//     contraction over queries runs in the C-register order, and the A
//     operand -- Q^T and dO^T staged transposed in LDS -- is read in that
//     same order).  Column sums of dL give the score gradient per KV head;
//     gain and temperature sums are left per wave.
//   * Q-major: a wave owns 32 queries of one head and walks the key blocks;
//     S^T = K Q^T and dP^T = V dO^T come out with lane = query and feed
//     dQ^T += K^T dS^T the same way (K^T staged in LDS).
// A small kernel then sums the per-KV-head score gradients and the per-wave
// gain/temperature partials in a fixed order.  P and dL enter the matrix
// cores rounded to bf16; everything else accumulates in fp32.

#include <algorithm>

#include "tg_device.h"
#include "tg_kernels.h"

namespace tg {
namespace {

constexpr float LOG2E = 1.4426950408889634f;
constexpr int BW = 4;            // waves per workgroup
constexpr int BT = BW * WAVE;
constexpr int TB = 32;           // rows per wave (keys or queries) and per tile
constexpr int BWD_MAX_GROUP = 64;  // query heads per KV head (Hq / Hkv) supported

struct BwdArgs {
    const bf16* q;      // [Kt][Hq][DH]
    const bf16* k;      // [Kt][Hkv][DH]
    const bf16* v;
    const float* s;     // [Kt] or null
    const float* gain;  // [Hq] or null
    const float* temp;  // [Hq]
    const bf16* out;    // [Kt][Hq][DH]
    const float* lse;   // [Hq][Kt]
    const bf16* dout;   // [Kt][Hq][DH]
    bf16* dq;
    bf16* dk;
    bf16* dv;
    float* ds;          // [Kt] or null
    float* dgain;       // [Hq] or null
    float* dtemp;       // [Hq]
    float* D;           // ws: [Hq][Kt]
    float* ds_part;     // ws: [Hkv][Kt]
    float* gt_part;     // ws: [batch][nkb][Hkv][BW][G][2]
    int64_t Kt;
    int32_t Hq, Hkv, G;
    int32_t nkb;        // key blocks of BW*TB per request (grid.x of the KV pass)
    int32_t batch;
    float inv_sqrt_dh;
    int32_t cu[TG_MAX_BATCH + 1];
};

__device__ __forceinline__ bf16x8 pack8(const float* f) {
    bf16x8 r;
#pragma unroll
    for (int e = 0; e < 8; ++e) r[e] = (bf16)f[e];
    return r;
}

// Row l%32 of a row-major tile as an MFMA operand: k-step t covers elements
// [16t, 16t+16) of the row, this lane holds 8 of them.  Rows past `rows`
// read as zero.
template <int DH>
__device__ __forceinline__ void load_rows(const bf16* base, int64_t row_stride, int row, int rows,
                                          int lane, u32x4 (&r)[DH / 16]) {
    const bool ok = row < rows;
    const bf16* p = base + (int64_t)(ok ? row : 0) * row_stride + 8 * (lane / 32);
#pragma unroll
    for (int t = 0; t < DH / 16; ++t) r[t] = ok ? ld16(p + 16 * t) : u32x4{0u, 0u, 0u, 0u};
}

// A operand for a contraction over the 32 rows (keys or queries) of a
// row-major LDS tile T[TB][RT]: rows 32m + (lane % 32) of the head
// dimension, rows 16c + 4(lane / 32) + {0..3} and 16c + 8 + 4(lane / 32) +
// {0..3} of the tile (the order of the C registers that feed the B
// operand).  gfx950's transposing LDS read returns, in each group of 16
// lanes where lane i points at four values of one row, to lane j value j % 4
// of the rows that lanes j/4, j/4 + 4, j/4 + 8 and j/4 + 12 point at; so
// lane i of a group points at tile row 4(lane / 32) + i/4 and head dims
// 16 (group % 2) + 4 (i % 4), and two reads, eight rows apart, give the
// operand.  A row stride of DH + 32 (16 or 48 dwords modulo 64 banks) keeps
// the four rows a half-wave reads on disjoint banks.
template <int DH>
constexpr int tr_stride() { return DH + 32; }
template <int RT>
__device__ __forceinline__ bf16x8 lds_tr_operand(const bf16* T, int m, int c, int lane) {
    typedef short v4i16_t __attribute__((ext_vector_type(4)));
    const int off = (4 * (lane / 32) + (lane % 16) / 4) * RT + 16 * ((lane / 16) % 2) + 4 * (lane % 4);
    const bf16* p0 = T + (16 * c) * RT + 32 * m + off;
    const v4i16_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) v4i16_t*)p0);
    const v4i16_t hi =
        __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) v4i16_t*)(p0 + 8 * RT));
    const u32x2 x = __builtin_bit_cast(u32x2, lo), y = __builtin_bit_cast(u32x2, hi);
    return as_bf16x8(u32x4{x[0], x[1], y[0], y[1]});
}

// D[h][i] = dO_i . O_i over DH: DH/8 lanes per (row, head), 16 bytes each,
// so that a wave reads 1 KB of each matrix contiguously per load; a lane
// butterfly sums the partial dots.
template <int DH>
__global__ __launch_bounds__(256) void bwd_dot_kernel(BwdArgs a) {
    constexpr int LPR = DH / 8;
    const int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    const int64_t idx = gid / LPR;  // (row, head) pair: row-major [Kt][Hq]
    const int sub = (int)(gid % LPR);
    const bool ok = idx < a.Kt * a.Hq;
    const int64_t at = (ok ? idx : 0) * DH + sub * 8;
    const bf16x8 x = as_bf16x8(ld16(a.out + at)), y = as_bf16x8(ld16(a.dout + at));
    float acc = 0.0f;
#pragma unroll
    for (int e = 0; e < 8; ++e) acc = fmaf((float)x[e], (float)y[e], acc);
#pragma unroll
    for (int o = 1; o < LPR; o <<= 1) acc += __shfl_xor(acc, o, WAVE);
    if (ok && sub == 0) a.D[(idx % a.Hq) * a.Kt + idx / a.Hq] = acc;
}

// Staging of two 32-row tiles (`mats` row-major [rows][stride] bf16
// matrices, DH columns each) for one pipeline step: every thread fetches
// PER 16-byte segments into registers, then writes them into an LDS buffer,
// row-major with rows of RP (row-form operands: conflict-free 16-byte
// reads) and, for the first `ntrans` matrices, a second row-major copy with
// rows of RT (operands that contract over the rows, read by transposing
// reads).  All stores are 16 bytes.  Consecutive threads take consecutive
// segments of a row: the LDS takes a 16-byte store eight lanes at a time over
// 32 four-byte banks, and eight segments of one row fall on eight distinct
// bank quads in both copies (eight rows of one segment, at RT = DH + 32,
// would share two quads).
template <int DH>
struct TileStage {
    static constexpr int SEGS = DH / 8;
    static constexpr int RP = DH + 8;               // padded row-major row (bf16)
    static constexpr int RT = tr_stride<DH>();      // row of the copy read transposed
    static constexpr int PER = 2 * TB * SEGS / BT;  // segments per thread
    u32x4 r[PER];

    // Rows past `rows` clamp to the last row (no branch, so no wait at a
    // join); the kernels mask everything those rows contribute.
    __device__ __forceinline__ void fetch(const bf16* m0, const bf16* m1, int64_t stride, int row0,
                                          int rows, int tid) {
#pragma unroll
        for (int u = 0; u < PER; ++u) {
            const int idx = tid + BT * u;
            const int mat = idx / (TB * SEGS), rem = idx % (TB * SEGS);
            const int rr = rem / SEGS, seg = rem % SEGS;
            const int row = min(row0 + rr, rows - 1);
            const bf16* base = mat == 0 ? m0 : m1;
            r[u] = ld16(base + (int64_t)row * stride + seg * 8);
        }
    }
    // rm: [2][TB*RP] row-major tiles; tr: [ntrans][TB*RT] their second copies
    __device__ __forceinline__ void put(bf16* rm, bf16* tr, int ntrans, int tid) const {
#pragma unroll
        for (int u = 0; u < PER; ++u) {
            const int idx = tid + BT * u;
            const int mat = idx / (TB * SEGS), rem = idx % (TB * SEGS);
            const int rr = rem / SEGS, seg = rem % SEGS;
            st16(rm + mat * TB * RP + rr * RP + seg * 8, r[u]);
            if (mat < ntrans) st16(tr + mat * TB * RT + rr * RT + seg * 8, r[u]);
        }
    }
};

// KV-major pass: dK, dV, score-gradient and gain/temperature partials.  The
// workgroup walks (32-query block, query head of the group) pairs; the Q and
// dO tiles of the next pair are fetched into registers while the current
// pair is computed from the other LDS buffer (one barrier per step).
// Consecutive workgroup ids cycle over the KV heads, so that (with as many
// KV heads as XCDs) the workgroups of one KV head share one XCD's L2, and
// every workgroup walks the query blocks from the request's last one down,
// heads inner: the workgroups running at the same time then read the same
// Q and dO tiles at about the same time, from L2 after the first.
template <int DH>
__global__ __launch_bounds__(BT) void bwd_kv_kernel(BwdArgs a) {
    constexpr int KS = DH / 16;   // k-steps over the head dimension
    constexpr int MT = DH / 32;   // 32-row output tiles over the head dimension
    using Stage = TileStage<DH>;
    constexpr int RP = Stage::RP;
    constexpr int RT = Stage::RT;
    __shared__ __align__(16) bf16 Rm[2][2 * TB * RP];     // [buffer] Q | dO, row-major
    __shared__ __align__(16) bf16 Tr[2][2 * TB * RT];     // [buffer] Q | dO, copies read transposed
    __shared__ float lse2[2][TB], Dq[2][TB];
    __shared__ float s_tau[BWD_MAX_GROUP], s_gain[BWD_MAX_GROUP];
    __shared__ float s_gt[BW][BWD_MAX_GROUP][2];  // per wave and head: (dgain, dtemp) sums

    const int kvh = (int)(blockIdx.x % (unsigned)a.Hkv);
    const int kb = (int)((blockIdx.x / (unsigned)a.Hkv) % (unsigned)a.nkb);
    const int b = (int)(blockIdx.x / (unsigned)(a.Hkv * a.nkb));
    const int lo = a.cu[b], n = a.cu[b + 1] - lo;
    const int tid = threadIdx.x, w = tid / WAVE, lane = tid % WAVE;
    const int col = lane % 32;
    // This wave's own slot of gain/temperature partials: the G heads of its
    // KV head, (dgain, dtemp) each.
    float* gtp = a.gt_part + ((((int64_t)b * a.nkb + kb) * a.Hkv + kvh) * BW + w) * a.G * 2;
    const int q0 = kb * BW * TB;
    if (q0 >= n) {  // uniform: no key of this block exists
        for (int i = lane; i < a.G * 2; i += WAVE) gtp[i] = 0.0f;
        return;
    }
    const int j0 = q0 + w * TB;                    // first key of this wave (request-local)
    const bool wave_on = j0 < n;
    const int key = j0 + col;
    const bool key_ok = key < n;

    u32x4 kr[KS], vr[KS];
    load_rows<DH>(a.k + (int64_t)lo * a.Hkv * DH + kvh * DH, (int64_t)a.Hkv * DH, key, n, lane, kr);
    load_rows<DH>(a.v + (int64_t)lo * a.Hkv * DH + kvh * DH, (int64_t)a.Hkv * DH, key, n, lane, vr);
    const float s_key = (a.s != nullptr && key_ok) ? a.s[lo + key] : 0.0f;

    f32x16 dkT[MT], dvT[MT];
#pragma unroll
    for (int m = 0; m < MT; ++m)
#pragma unroll
        for (int r = 0; r < 16; ++r) dkT[m][r] = dvT[m][r] = 0.0f;
    float ds_acc = 0.0f, dg_acc = 0.0f, dt_acc = 0.0f;

    // Per-head constants staged once: loads issued inside the loop after the
    // prefetch would make every wait for them a wait for the prefetch too
    // (the vector-memory counter retires in order).
    for (int g = tid; g < a.G; g += BT) {
        s_tau[g] = a.temp[kvh * a.G + g];
        s_gain[g] = a.gain != nullptr ? a.gain[kvh * a.G + g] : 0.0f;
    }
    for (int i = tid; i < BW * BWD_MAX_GROUP * 2; i += BT) (&s_gt[0][0][0])[i] = 0.0f;

    const int nqb = (n - q0 + TB - 1) / TB;       // query blocks from the block's first key
    const int nbt = (n + TB - 1) / TB;            // query blocks of the request
    const int iters = a.G * nqb;
    // Step it: head g = it % G of query block nbt - 1 - it / G.
    auto step_head = [&](int it) { return it % a.G; };
    auto step_row = [&](int it) { return TB * (nbt - 1 - it / a.G); };
    const int64_t hs = (int64_t)a.Hq * DH;        // row stride of q and dout
    Stage st;
    float pl = 0.0f;
    bool pl_ok = false;
    const float* const lse_p = a.lse;
    const float* const d_p = a.D;
    const float* const row_src = tid < TB ? lse_p : d_p;  // this thread's per-row value
    auto fetch = [&](int it) {
        const int h = kvh * a.G + step_head(it), i0 = step_row(it);
        st.fetch(a.q + (int64_t)lo * hs + h * DH, a.dout + (int64_t)lo * hs + h * DH, hs, i0, n, tid);
        // branch-free: the row index clamps, the value is masked when stored
        const int rr = tid % TB;
        pl_ok = i0 + rr < n;
        const int64_t at = (int64_t)h * a.Kt + lo + min(i0 + rr, n - 1);
        pl = row_src[at];
    };
    auto put = [&](int buf) {
        st.put(Rm[buf], Tr[buf], 2, tid);
        if (tid < TB) lse2[buf][tid] = pl_ok ? pl * LOG2E : 0.0f;
        else if (tid < 2 * TB) Dq[buf][tid - TB] = pl_ok ? pl : 0.0f;
    };
    fetch(0);
    put(0);
    for (int it = 0; it < iters; ++it) {
        const int buf = it & 1;
        __syncthreads();  // buffer `buf` complete, buffer buf^1 no longer read
        if (it + 1 < iters) fetch(it + 1);
        const int g = step_head(it), i0 = step_row(it);
        // Branch-free: a block no query of which sees these keys (or a wave
        // past the request) is masked to P = dL = 0 below.  A branch here
        // would make the compiler copy the loop-carried accumulators.
        {
            const float tau = s_tau[g];
            const float gn = s_gain[g];
            const float c1 = tau * a.inv_sqrt_dh * LOG2E;
            const float bias2 = gn * s_key * LOG2E;
            const float kscale = tau * a.inv_sqrt_dh;
            const bf16* qrow = Rm[buf] + col * RP + 8 * (lane / 32);
            const bf16* orow = qrow + TB * RP;
            f32x16 S, dP;
#pragma unroll
            for (int r = 0; r < 16; ++r) S[r] = dP[r] = 0.0f;
#pragma unroll
            for (int t = 0; t < KS; ++t) {
                S = mfma32(as_bf16x8(ld16(qrow + 16 * t)), as_bf16x8(kr[t]), S);
                dP = mfma32(as_bf16x8(ld16(orow + 16 * t)), as_bf16x8(vr[t]), dP);
            }
            float P[16], dS[16];
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int qq = 8 * (r / 4) + 4 * (lane / 32) + r % 4;
                const int qi = i0 + qq;
                const bool ok = key_ok && qi < n && qi >= key;
                // operands read unconditionally so the mask is a select, not a branch
                const float e = __builtin_amdgcn_exp2f(fmaf(S[r], c1, bias2) - lse2[buf][qq]);
                const float p = ok ? e : 0.0f;
                const float dl = p * (dP[r] - Dq[buf][qq]);
                P[r] = p;
                dS[r] = dl * kscale;
                ds_acc = fmaf(dl, gn, ds_acc);
                dg_acc = fmaf(dl, s_key, dg_acc);
                dt_acc = fmaf(dl, S[r] * a.inv_sqrt_dh, dt_acc);
            }
            const bf16* qt = Tr[buf];
            const bf16* ot = Tr[buf] + TB * RT;
#pragma unroll
            for (int c = 0; c < 2; ++c) {
                const bf16x8 pb = pack8(P + 8 * c), sb = pack8(dS + 8 * c);
#pragma unroll
                for (int m = 0; m < MT; ++m) {
                    dvT[m] = mfma32(lds_tr_operand<RT>(ot, m, c, lane), pb, dvT[m]);
                    dkT[m] = mfma32(lds_tr_operand<RT>(qt, m, c, lane), sb, dkT[m]);
                }
            }
        }
        {  // this step's gain/temperature terms into the wave's sums of head g
            const float dg = wave_sum(dg_acc), dt = wave_sum(dt_acc);
            if (lane == 0) {
                s_gt[w][g][0] += dg;
                s_gt[w][g][1] += dt;
            }
            dg_acc = dt_acc = 0.0f;
        }
        if (it + 1 < iters) put(buf ^ 1);
    }
    __builtin_amdgcn_wave_barrier();
    for (int i = lane; i < a.G * 2; i += WAVE) gtp[i] = s_gt[w][i / 2][i % 2];
    if (!wave_on) return;
    ds_acc += __shfl_xor(ds_acc, 32, WAVE);
    if (lane < 32 && key_ok && a.ds_part != nullptr) a.ds_part[(int64_t)kvh * a.Kt + lo + key] = ds_acc;
    if (!key_ok) return;
    bf16* dkp = a.dk + ((int64_t)(lo + key) * a.Hkv + kvh) * DH;
    bf16* dvp = a.dv + ((int64_t)(lo + key) * a.Hkv + kvh) * DH;
#pragma unroll
    for (int m = 0; m < MT; ++m)
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
            const int d0 = 32 * m + 8 * q4 + 4 * (lane / 32);
            bf16x4 xk, xv;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                xk[e] = (bf16)dkT[m][4 * q4 + e];
                xv[e] = (bf16)dvT[m][4 * q4 + e];
            }
            st8(dkp + d0, __builtin_bit_cast(u32x2, xk));
            st8(dvp + d0, __builtin_bit_cast(u32x2, xv));
        }
}

// Q-major pass: dQ.  The workgroup walks 32-key blocks; the K and V tiles of
// the next block are fetched while the current one is computed.
template <int DH>
__global__ __launch_bounds__(BT, 2) void bwd_q_kernel(BwdArgs a) {
    constexpr int KS = DH / 16;
    constexpr int MT = DH / 32;
    using Stage = TileStage<DH>;
    constexpr int RP = Stage::RP;
    constexpr int RT = Stage::RT;
    __shared__ __align__(16) bf16 Rm[2][2 * TB * RP];  // [buffer] K | V, row-major
    __shared__ __align__(16) bf16 Tr[2][TB * RT];      // [buffer] K, the copy read transposed
    __shared__ float sb2[2][TB];

    // Consecutive workgroup ids cycle over the KV heads (the workgroups of one
    // KV head share an XCD's L2, and all walk its key blocks from the first
    // in step), then over the heads of the group; query blocks with the most
    // keys come first.
    const int kvh_u = (int)(blockIdx.x % (unsigned)a.Hkv);
    const int rest = (int)(blockIdx.x / (unsigned)a.Hkv);
    const int h = kvh_u * a.G + rest % a.G;
    const int qb = a.nkb - 1 - (rest / a.G) % a.nkb;
    const int b = rest / (a.G * a.nkb);
    const int lo = a.cu[b], n = a.cu[b + 1] - lo;
    if (qb * BW * TB >= n) return;
    const int tid = threadIdx.x, w = tid / WAVE, lane = tid % WAVE;
    const int col = lane % 32;
    const int kvh = h / a.G;
    const int i0 = qb * BW * TB + w * TB;
    const bool wave_on = i0 < n;
    const int qi = i0 + col;
    const bool q_ok = qi < n;

    u32x4 qr[KS], orr[KS];
    load_rows<DH>(a.q + (int64_t)lo * a.Hq * DH + h * DH, (int64_t)a.Hq * DH, qi, n, lane, qr);
    load_rows<DH>(a.dout + (int64_t)lo * a.Hq * DH + h * DH, (int64_t)a.Hq * DH, qi, n, lane, orr);
    const float tau = a.temp[h];
    const float gn = a.gain != nullptr ? a.gain[h] : 0.0f;
    const float c1 = tau * a.inv_sqrt_dh * LOG2E;
    const float lq = q_ok ? a.lse[(int64_t)h * a.Kt + lo + qi] * LOG2E : 0.0f;
    const float Dv = q_ok ? a.D[(int64_t)h * a.Kt + lo + qi] : 0.0f;
    const int64_t ks = (int64_t)a.Hkv * DH;
    const bf16* kh = a.k + (int64_t)lo * ks + kvh * DH;
    const bf16* vh = a.v + (int64_t)lo * ks + kvh * DH;

    f32x16 dqT[MT];
#pragma unroll
    for (int m = 0; m < MT; ++m)
#pragma unroll
        for (int r = 0; r < 16; ++r) dqT[m][r] = 0.0f;

    const int jend = min(n, qb * BW * TB + BW * TB);
    const int iters = (jend + TB - 1) / TB;
    Stage st;
    float pb = 0.0f;
    bool pb_ok = false;
    const float* sp = a.s != nullptr ? a.s : a.temp;  // any readable array when there is no bias
    auto fetch = [&](int it) {
        const int j0 = TB * it;
        st.fetch(kh, vh, ks, j0, n, tid);
        // branch-free: the key index clamps, the value is masked when stored
        pb_ok = a.s != nullptr && j0 + (tid % TB) < n;
        pb = sp[a.s != nullptr ? lo + min(j0 + tid % TB, n - 1) : 0];
    };
    auto put = [&](int buf) {
        st.put(Rm[buf], Tr[buf], 1, tid);
        if (tid < TB) sb2[buf][tid] = pb_ok ? gn * pb * LOG2E : 0.0f;
    };
    fetch(0);
    put(0);
    for (int it = 0; it < iters; ++it) {
        const int buf = it & 1;
        __syncthreads();
        if (it + 1 < iters) fetch(it + 1);
        const int j0 = TB * it;
        {  // branch-free, as in the KV pass: the mask zeroes what no query sees
            const bf16* krow = Rm[buf] + col * RP + 8 * (lane / 32);
            const bf16* vrow = krow + TB * RP;
            f32x16 S, dP;
#pragma unroll
            for (int r = 0; r < 16; ++r) S[r] = dP[r] = 0.0f;
#pragma unroll
            for (int t = 0; t < KS; ++t) {
                S = mfma32(as_bf16x8(ld16(krow + 16 * t)), as_bf16x8(qr[t]), S);
                dP = mfma32(as_bf16x8(ld16(vrow + 16 * t)), as_bf16x8(orr[t]), dP);
            }
            float dS[16];
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int kk = 8 * (r / 4) + 4 * (lane / 32) + r % 4;
                const int kj = j0 + kk;
                const bool ok = q_ok && kj < n && qi >= kj;
                const float e = __builtin_amdgcn_exp2f(fmaf(S[r], c1, sb2[buf][kk]) - lq);
                const float p = ok ? e : 0.0f;
                dS[r] = p * (dP[r] - Dv);
            }
#pragma unroll
            for (int c = 0; c < 2; ++c) {
                const bf16x8 sbv = pack8(dS + 8 * c);
#pragma unroll
                for (int m = 0; m < MT; ++m)
                    dqT[m] = mfma32(lds_tr_operand<RT>(Tr[buf], m, c, lane), sbv, dqT[m]);
            }
        }
        if (it + 1 < iters) put(buf ^ 1);
    }
    if (!q_ok) return;
    const float qs = tau * a.inv_sqrt_dh;
    bf16* dqp = a.dq + ((int64_t)(lo + qi) * a.Hq + h) * DH;
#pragma unroll
    for (int m = 0; m < MT; ++m)
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
            const int d0 = 32 * m + 8 * q4 + 4 * (lane / 32);
            bf16x4 x;
#pragma unroll
            for (int e = 0; e < 4; ++e) x[e] = (bf16)(dqT[m][4 * q4 + e] * qs);
            st8(dqp + d0, __builtin_bit_cast(u32x2, x));
        }
}

// ds[j] = sum over KV heads of the partial column sums (one thread per key);
// dgain, dtemp: one wave per (head, which) output, lanes summing strided
// per-wave partials, then a fixed shuffle tree (deterministic).
__global__ __launch_bounds__(256) void bwd_reduce_kernel(BwdArgs a) {
    const int64_t j = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (a.ds != nullptr && j < a.Kt) {
        float acc = 0.0f;
        for (int kv = 0; kv < a.Hkv; ++kv) acc += a.ds_part[(int64_t)kv * a.Kt + j];
        a.ds[j] = acc;
    }
    const int hh = blockIdx.x * (256 / WAVE) + threadIdx.x / WAVE;  // 2 * head + which
    if (hh >= 2 * a.Hq) return;
    const int h = hh / 2, kv = h / a.G, g = h % a.G;
    const int lane = lane_id();
    const int64_t nslot = (int64_t)a.batch * a.nkb * BW;          // (block, wave) slots
    float acc = 0.0f;
    for (int64_t sl = lane; sl < nslot; sl += WAVE) {
        const int64_t blk = sl / BW, ww = sl % BW;
        acc += a.gt_part[((blk * a.Hkv + kv) * BW + ww) * a.G * 2 + 2 * g + hh % 2];
    }
    acc = wave_sum(acc);
    if (lane != 0) return;
    if (hh % 2 == 0) {
        if (a.dgain != nullptr) a.dgain[h] = acc;
    } else {
        a.dtemp[h] = acc;
    }
}

int key_blocks(const AttnShape& sh) {
    int mx = 0;
    for (int b = 0; b < sh.batch; ++b) mx = std::max(mx, sh.cu[b + 1] - sh.cu[b]);
    return (mx + BW * TB - 1) / (BW * TB);
}

template <int DH>
hipError_t launch_dh(BwdArgs& a, const AttnShape& sh, hipStream_t st) {
    const int64_t rows = a.Kt * a.Hq;
    hipLaunchKernelGGL(bwd_dot_kernel<DH>, dim3((unsigned)((rows * (DH / 8) + 255) / 256)), dim3(256), 0, st, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(bwd_kv_kernel<DH>, dim3((unsigned)(a.nkb * a.Hkv * sh.batch)), dim3(BT), 0, st, a);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    hipLaunchKernelGGL(bwd_q_kernel<DH>, dim3((unsigned)(a.nkb * a.Hq * sh.batch)), dim3(BT), 0, st, a);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    const int64_t red_blocks = std::max<int64_t>((a.Kt + 255) / 256, (2 * a.Hq + 3) / 4);
    hipLaunchKernelGGL(bwd_reduce_kernel, dim3((unsigned)std::max<int64_t>(1, red_blocks)), dim3(256), 0,
                       st, a);
    return hipGetLastError();
}

}  // namespace

size_t attn_bwd_workspace_bytes(const AttnShape& sh) {
    const int64_t nkb = key_blocks(sh);
    const auto up = [](int64_t x) { return (x + 255) / 256 * 256; };
    return (size_t)(up(sh.Kt * sh.Hq * 4) + up(sh.Kt * sh.Hkv * 4) +
                    up((int64_t)sh.batch * nkb * BW * sh.Hq * 2 * 4));
}

hipError_t launch_attn_bwd(const AttnShape& sh, const void* q, const void* k, const void* v,
                           const float* s, const float* gain, const float* temp, const void* out,
                           const float* lse, const void* dout, void* dq, void* dk, void* dv,
                           float* ds, float* dgain, float* dtemp, void* ws, hipStream_t st) {
    BwdArgs a;
    a.q = (const bf16*)q;
    a.k = (const bf16*)k;
    a.v = (const bf16*)v;
    a.s = s;
    a.gain = gain;
    a.temp = temp;
    a.out = (const bf16*)out;
    a.lse = lse;
    a.dout = (const bf16*)dout;
    a.dq = (bf16*)dq;
    a.dk = (bf16*)dk;
    a.dv = (bf16*)dv;
    a.ds = ds;
    a.dgain = dgain;
    a.dtemp = dtemp;
    a.Kt = sh.Kt;
    a.Hq = sh.Hq;
    a.Hkv = sh.Hkv;
    a.G = sh.Hq / sh.Hkv;
    a.nkb = key_blocks(sh);
    a.batch = sh.batch;
    a.inv_sqrt_dh = 1.0f / sqrtf((float)sh.d_head);
    for (int i = 0; i <= sh.batch; ++i) a.cu[i] = sh.cu[i];
    const auto up = [](int64_t x) { return (x + 255) / 256 * 256; };
    char* w = (char*)ws;
    a.D = (float*)w;
    w += up(sh.Kt * sh.Hq * 4);
    a.ds_part = (float*)w;
    w += up(sh.Kt * sh.Hkv * 4);
    a.gt_part = (float*)w;
    return sh.d_head == 128 ? launch_dh<128>(a, sh, st) : launch_dh<64>(a, sh, st);
}

}  // namespace tg
