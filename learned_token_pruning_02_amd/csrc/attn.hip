// Token-gated causal GQA attention over the kept tokens (spke.com page,
// "Qu'est-ce que l'attention gérée par des tokens ?": each kept token's gate
// score is a bias on the attention logits, with a per-head gain and a
// per-head temperature).  For query row i, key j <= i of one request:
//     l_ij = temp[h] * (q_i . k_j) / sqrt(d_head) + gain[h] * s_j
//
// bf16 path, flash style (exact softmax computed online, never materialising
// the score matrix): a workgroup of 8 waves (two per SIMD, so one wave's
// softmax overlaps the other's MFMAs) owns one KV head, HPB query heads that
// share it and BQ = 256/HPB query rows of one request; each wave owns 32 query
// rows of one head, and every K/V tile staged in LDS feeds all eight waves.
// Per 64-key tile:
//   S^T[key][query] = K . Q^T with the 32x32x16 bf16 MFMA: K fragments from
//     LDS (A operand), Q fragments resident in registers (B operand), so each
//     lane holds all scores of ONE query row and the row max / row sum need
//     only one exchange with the partner lane half;
//   scale and bias are one FMA in the exp2 domain: x = c1*S + g2*s_j with
//     c1 = temp*log2(e)/sqrt(d), g2 = gain*log2(e);
//   O^T[dh][query] += V^T . P^T: V is stored transposed in LDS (A operand) and
//     the probabilities, converted to bf16, are fed straight from the S
//     registers as the B operand, again one query per lane, so the online
//     rescale of O needs no data exchange.
// Only the tiles on the diagonal (or past the end of the request) are masked,
// and a wave skips tiles whose keys all lie after its rows.  The exponent base
// of each row only moves when the row max exceeds it by more than 2^8, so the
// rescale of O is rare; the final O / l and lse are exact either way.
// K/V tiles are double buffered: the next tile is fetched into registers
// while the current one is consumed.  Heavy query tiles (many keys) are
// dispatched first and consecutive workgroup ids cycle over the KV heads, so
// the 8 XCDs each keep one head's K/V in their own L2.
#include "tg_device.h"
#include "tg_kernels.h"

namespace tg {

namespace {

constexpr float LOG2E = 1.4426950408889634f;
constexpr float LN2 = 0.6931471805599453f;

// ---------------------------------------------------------------- fp32 ----
template <int DH>
__global__ __launch_bounds__(128) void attn_f32_kernel(const float* __restrict__ q,
                                                       const float* __restrict__ k,
                                                       const float* __restrict__ v,
                                                       const float* __restrict__ s,
                                                       const float* __restrict__ gain,
                                                       const float* __restrict__ temp,
                                                       AttnShape sh, float* __restrict__ out,
                                                       float* __restrict__ lse) {
    const int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (gid >= sh.Kt * sh.Hq) return;
    const int64_t r = gid / sh.Hq;
    const int h = (int)(gid % sh.Hq);
    int b = 0;
    while (b + 1 < sh.batch && sh.cu[b + 1] <= r) ++b;
    const int64_t lo = sh.cu[b];
    const int kvh = h / (sh.Hq / sh.Hkv);
    const float c1 = temp[h] / sqrtf((float)DH);
    const float g = s != nullptr ? gain[h] : 0.f;
    const float* qr = q + (r * sh.Hq + h) * DH;
    float qv[DH], acc[DH];
#pragma unroll
    for (int e = 0; e < DH; ++e) {
        qv[e] = qr[e];
        acc[e] = 0.f;
    }
    float m = -INFINITY, l = 0.f;
    for (int64_t j = lo; j <= r; ++j) {
        const float* kr = k + (j * sh.Hkv + kvh) * DH;
        float dot = 0.f;
#pragma unroll
        for (int e = 0; e < DH; ++e) dot = fmaf(qv[e], kr[e], dot);
        const float x = s != nullptr ? c1 * dot + g * s[j] : c1 * dot;
        const float mn = fmaxf(m, x);
        const float sc = expf(m - mn);
        const float p = expf(x - mn);
        l = l * sc + p;
        const float* vr = v + (j * sh.Hkv + kvh) * DH;
#pragma unroll
        for (int e = 0; e < DH; ++e) acc[e] = fmaf(acc[e], sc, p * vr[e]);
        m = mn;
    }
    float* orow = out + (r * sh.Hq + h) * DH;
#pragma unroll
    for (int e = 0; e < DH; ++e) orow[e] = acc[e] / l;
    if (lse != nullptr) lse[(int64_t)h * sh.Kt + r] = m + logf(l);
}

// ---------------------------------------------------------------- bf16 ----
struct AttnArgs {
    const bf16* q;
    const bf16* k;
    const bf16* v;
    const float* s;
    const float* gain;
    const float* temp;
    bf16* out;
    float* lse;
    int64_t Kt;
    int32_t Hq, Hkv, n_hg, batch, max_tiles;
    int32_t cu[TG_MAX_BATCH + 1];
    int32_t ntiles[TG_MAX_BATCH];
};

constexpr int KVT = 64;          // keys per tile
// Fourth word of a raw buffer resource (32-bit data format, no swizzle).
constexpr int BUFFER_RSRC_WORD3 = 0x00020000;
constexpr int VT_STRIDE = KVT + 8;  // LDS row stride of V^T (bf16 elements)

// Number of query tiles whose local index is >= t.
__device__ __forceinline__ int tiles_at_or_above(const AttnArgs& a, int t) {
    int c = 0;
    for (int b = 0; b < a.batch; ++b) c += max(0, a.ntiles[b] - t);
    return c;
}

template <int DH, int HPB, int NWAVE, bool BIAS>
__global__ __launch_bounds__(64 * NWAVE, 8 / NWAVE) void attn_bf16_kernel(AttnArgs a) {
    // NWAVE = 8: two waves per SIMD from one workgroup; 4: two workgroups per CU.
    constexpr int WPH = NWAVE / HPB;   // waves per head
    constexpr int BQ = 32 * WPH;       // query rows per head per workgroup
    constexpr int KS = DH + 8;         // LDS row stride of K (bf16 elements)
    constexpr int KU = KVT * DH / 8 / 256;  // 16-byte K units per staging thread per tile
    constexpr int VU = (KVT / 4) * (DH / 8);  // V units (4 keys x 8 dh) per tile
    constexpr int NKK = DH / 16;       // k steps of the QK^T product
    constexpr int NMD = DH / 32;       // 32-row dh tiles of O^T
    constexpr float RESCALE_SLACK = 8.0f;  // log2 headroom before O is rescaled
    // Four waves (two workgroups per CU) interleave the softmax with the PV
    // MFMAs by hand, slice by slice; eight waves (one workgroup per CU) leave
    // the interleave to scheduling groups, which measures faster there.
    constexpr bool FUSED = NWAVE == 4;
    constexpr int NKB = 2;  // K / bias buffers

    __shared__ __attribute__((aligned(16))) bf16 Ks[NKB][KVT * KS];
    __shared__ __attribute__((aligned(16))) bf16 Vt[2][DH * VT_STRIDE];
    // Per key of the tile and per head of the workgroup: g_h log2(e) s_j.
    __shared__ __attribute__((aligned(16))) float Bs[NKB][HPB][KVT];

    const int tid = threadIdx.x;
    const int lane = lane_id();
    // Wave index, read through a scalar register so that the compiler treats
    // everything derived from it (rows, loop bounds, buffer bases) as uniform.
    const int w = __builtin_amdgcn_readfirstlane(tid / WAVE);
    const int hh = lane / 32;
    const int l32 = lane % 32;

    // ---- which (request, query tile, head group) this workgroup owns ------
    const int hg = blockIdx.x % a.n_hg;
    const int u = blockIdx.x / a.n_hg;
    int b, t;
    if (a.batch == 1) {
        b = 0;
        t = a.ntiles[0] - 1 - u;
    } else {
        int lo = 0, hi = a.max_tiles - 1;
        while (lo < hi) {
            const int mid = (lo + hi + 1) / 2;
            if (tiles_at_or_above(a, mid) > u) lo = mid;
            else hi = mid - 1;
        }
        t = lo;
        int j = u - tiles_at_or_above(a, t + 1);
        for (b = 0; b < a.batch; ++b) {
            if (a.ntiles[b] > t) {
                if (j == 0) break;
                --j;
            }
        }
        if (b >= a.batch) return;  // unreachable for a consistent tile count
    }
    const int64_t rbase = a.cu[b];
    const int n = a.cu[b + 1] - a.cu[b];
    const int q0 = t * BQ;
    const int kend = min(q0 + BQ, n);
    const int nkv = (kend + KVT - 1) / KVT;
    const int group = a.Hq / a.Hkv;
    const int kvh = (hg * HPB) / group;
    const int hp = w / WPH;  // head of this wave within the workgroup
    const int h = hg * HPB + hp;
    const int qmin = q0 + 32 * (w % WPH);  // first query row of this wave
    const int qi = qmin + l32;               // this lane's query row
    const bool qvalid = qi < n;

    // ---- resident Q fragments (B operand of S^T = K Q^T) ----------------
    bf16x8 qf[NKK];
    {
        const bf16* qp = a.q + ((rbase + (qvalid ? qi : 0)) * a.Hq + h) * DH + (DH / 2) * hh;
        const u32x4 zero = {0u, 0u, 0u, 0u};
#pragma unroll
        for (int kk = 0; kk < NKK; ++kk) qf[kk] = as_bf16x8(qvalid ? ld16(qp + 8 * kk) : zero);
    }
    const float c1 = a.temp[h] * LOG2E / sqrtf((float)DH);
    float gbias[HPB];
#pragma unroll
    for (int j = 0; j < HPB; ++j) gbias[j] = BIAS ? a.gain[hg * HPB + j] * LOG2E : 0.f;

    // ---- K/V/s tile staging ------------------------------------------------
    // K (with the score bias) is staged for tile jt+1 while V is staged one
    // tile behind, for tile jt: iteration jt computes QK and the softmax of
    // tile jt next to the PV product of tile jt-1, so each wave overlaps its
    // own VALU work with MFMAs.  With 8 waves, threads [0, 256) stage V and
    // threads [256, 512) stage K and the bias; with 4 waves every thread does both.
    // With 8 waves a thread stages either K or V, so both share one register array.
    constexpr int NSTG = NWAVE == 8 ? (KU > 4 ? KU : 4) : KU + 4;
    u32x4 stg[NSTG];
    u32x4* const kreg = stg;
    u32x4* const vreg = NWAVE == 8 ? stg : stg + KU;
    float sreg = 0.f;
    const bool kstager = NWAVE == 8 ? w >= 4 : true;
    const bool vstager = NWAVE == 8 ? w < 4 : true;
    const int st = tid & 255;
    // Tiles are read through buffer resources whose base is the tile's first
    // key and whose size ends at the request's last key: the per-lane offsets
    // stay fixed from tile to tile, and keys past the request read as zero
    // (those keys are masked, and 0 * V = 0 keeps the PV product finite).
    const int64_t row_elems = (int64_t)a.Hkv * DH;
    auto tile_rsrc = [&](const bf16* base, int j0) {
        return __builtin_amdgcn_make_buffer_rsrc(
            (void*)(base + (rbase + j0) * row_elems + kvh * DH), (short)0,
            (int)((n - j0) * row_elems * 2), BUFFER_RSRC_WORD3);
    };
    auto load_k = [&](int jt) {
        const int j0 = jt * KVT;
        if (kstager) {
            const __amdgpu_buffer_rsrc_t rk = tile_rsrc(a.k, j0);
#pragma unroll
            for (int i = 0; i < KU; ++i) {
                const int uu = st + i * 256;
                const int row = uu / (DH / 8), c = uu % (DH / 8);
                kreg[i] = __builtin_amdgcn_raw_buffer_load_b128(
                    rk, (int)(row * row_elems * 2) + 16 * c, 0, 0);
            }
            if (BIAS && st < KVT) {
                const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
                    (void*)(a.s + rbase + j0), (short)0, (n - j0) * 4, BUFFER_RSRC_WORD3);
                sreg = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rs, 4 * st, 0, 0));
            }
        }
    };
    auto load_v = [&](int jt) {
        const int j0 = jt * KVT;
        if (vstager && st < VU) {
            const __amdgpu_buffer_rsrc_t rv = tile_rsrc(a.v, j0);
            const int kg = st % (KVT / 4), dg = st / (KVT / 4);
#pragma unroll
            for (int i = 0; i < 4; ++i)
                vreg[i] = __builtin_amdgcn_raw_buffer_load_b128(
                    rv, (int)((4 * kg + i) * row_elems * 2) + 16 * dg, 0, 0);
        }
    };
    auto store_k = [&](int buf) {
        if (kstager) {
#pragma unroll
            for (int i = 0; i < KU; ++i) {
                const int uu = st + i * 256;
                const int row = uu / (DH / 8), c = uu % (DH / 8);
                st16(&Ks[buf][row * KS + 8 * c], kreg[i]);
            }
            if (BIAS && st < KVT) {
#pragma unroll
                for (int j = 0; j < HPB; ++j) Bs[buf][j][st] = gbias[j] * sreg;
            }
        }
    };
    auto store_v = [&](int buf) {
        if (vstager && st < VU) {
            const int kg = st % (KVT / 4), dg = st / (KVT / 4);
            // Keys 16G + 4h + {0..3} and 16G + 8 + 4h + {0..3} (one PV operand
            // of lane half h) are stored next to each other at 16G + 8h.
            const int vpos = 16 * (kg / 4) + 8 * (kg & 1) + 4 * ((kg >> 1) & 1);
            // Transpose 4 keys x 8 dh: element e of a row is half e%2 of word e/2.
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const int wd = e / 2;
                // Byte select: low (e even) or high (e odd) halves of two words.
                const unsigned sel = e % 2 ? 0x07060302u : 0x05040100u;
                u32x2 pk;
                pk[0] = __builtin_amdgcn_perm(vreg[1][wd], vreg[0][wd], sel);
                pk[1] = __builtin_amdgcn_perm(vreg[3][wd], vreg[2][wd], sel);
                st8(&Vt[buf][(8 * dg + e) * VT_STRIDE + vpos], pk);
            }
        }
    };

    f32x16 o[NMD];
#pragma unroll
    for (int md = 0; md < NMD; ++md)
#pragma unroll
        for (int r = 0; r < 16; ++r) o[md][r] = 0.f;
    float m = -INFINITY, lpart = 0.f;  // exponent base (log2 units) and this lane's row-sum half
    bf16x8 pold[4];                    // probabilities of the previous tile (PV operand)
    float alpha_prev = 1.f;            // rescale of O owed before the next PV product
    bool pend = false;                 // some row of the wave owes a rescale

    f32x16 sacc[2];  // S^T of one tile

    // S^T of tile T from its staged K.
#define TG_QK(T)                                                                             \
    do {                                                                                     \
        const int kb = (T) % NKB;                                                            \
        _Pragma("unroll") for (int mt = 0; mt < 2; ++mt)                                     \
            _Pragma("unroll") for (int r = 0; r < 16; ++r) sacc[mt][r] = 0.f;                \
        _Pragma("unroll") for (int kk = 0; kk < NKK; ++kk) {                                 \
            _Pragma("unroll") for (int mt = 0; mt < 2; ++mt) {                               \
                const bf16x8 kf = as_bf16x8(                                                 \
                    ld16(&Ks[kb][(32 * mt + l32) * KS + (DH / 2) * hh + 8 * kk]));           \
                sacc[mt] = mfma32(kf, qf[kk], sacc[mt]);                                     \
            }                                                                                \
        }                                                                                    \
    } while (0)

    // DO_S: softmax of tile jt from sacc (MASKED on the diagonal tile);
    // DO_PV: O += V(jt-1) P(jt-1).  The exponent base of a row moves only when
    // its max exceeds it by more than RESCALE_SLACK; the rescale of O this
    // causes is owed until the start of the next step (TG_RESCALE), before
    // the next PV product, so that the QK product, the PV product and the
    // softmax form one straight run of independent MFMA and VALU work.
#define TG_RESCALE()                                                                         \
    do {                                                                                     \
        if (pend) {                                                                          \
            _Pragma("unroll") for (int md = 0; md < NMD; ++md)                               \
                _Pragma("unroll") for (int r = 0; r < 16; ++r) o[md][r] *= alpha_prev;       \
        }                                                                                    \
    } while (0)
#define TG_PVSM(MASKED, DO_S, DO_PV)                                                         \
    do {                                                                                     \
        if (DO_PV) {                                                                         \
            const int vb = (jt - 1) & 1;                                                     \
            bf16x8 v0[4];                                                                    \
            _Pragma("unroll") for (int kk = 0; kk < 4; ++kk) v0[kk] = as_bf16x8(             \
                ld16(&Vt[vb][l32 * VT_STRIDE + 16 * kk + 8 * hh]));                          \
            /* QK above, then PV interleaved with the softmax below. */                      \
            if (DO_S) __builtin_amdgcn_sched_barrier(0);                                     \
            _Pragma("unroll") for (int md = 0; md < NMD; ++md) {                             \
                _Pragma("unroll") for (int kk = 0; kk < 4; ++kk) {                           \
                    const bf16x8 vf = md == 0 ? v0[kk] : as_bf16x8(                          \
                        ld16(&Vt[vb][(32 * md + l32) * VT_STRIDE + 16 * kk + 8 * hh]));      \
                    o[md] = mfma32(vf, pold[kk], o[md]);                                     \
                }                                                                            \
            }                                                                                \
        }                                                                                    \
        if (DO_S) {                                                                          \
            const int bb = jt % NKB;                                                         \
            const int j0 = jt * KVT;                                                         \
            float mx = -INFINITY;                                                            \
            _Pragma("unroll") for (int mt = 0; mt < 2; ++mt) {                               \
                _Pragma("unroll") for (int rq = 0; rq < 4; ++rq) {                           \
                    const int kl = 32 * mt + 8 * rq + 4 * hh;                                \
                    const f32x4 sv = BIAS ? *reinterpret_cast<const f32x4*>(&Bs[bb][hp][kl]) \
                                          : f32x4{0.f, 0.f, 0.f, 0.f};                       \
                    _Pragma("unroll") for (int e = 0; e < 4; ++e) {                          \
                        float x = fmaf(c1, sacc[mt][4 * rq + e], sv[e]);                     \
                        if (MASKED && j0 + kl + e > qi) x = -INFINITY;                       \
                        sacc[mt][4 * rq + e] = x;                                            \
                        mx = fmaxf(mx, x);                                                   \
                    }                                                                        \
                }                                                                            \
            }                                                                                \
            mx = fmaxf(mx, __shfl_xor(mx, 32, WAVE));                                        \
            const bool grow = mx > m + RESCALE_SLACK;                                        \
            const float m_new = grow ? mx : m;                                               \
            const float alpha = grow ? __builtin_amdgcn_exp2f(m - m_new) : 1.f;              \
            m = m_new;                                                                       \
            const float mb = m == -INFINITY ? 0.f : m;                                       \
            float psum = 0.f;                                                                \
            bf16x8 pnew[4];                                                                  \
            _Pragma("unroll") for (int kk = 0; kk < 4; ++kk) {                               \
                _Pragma("unroll") for (int e = 0; e < 8; ++e) {                              \
                    const float p = __builtin_amdgcn_exp2f(sacc[kk / 2][8 * (kk % 2) + e] - mb); \
                    psum += p;                                                               \
                    pnew[kk][e] = to_bf16(p);                                                \
                }                                                                            \
            }                                                                                \
            /* Pin the probabilities here: left alone, the compiler sinks the   */         \
            /* exponentials below the staging stores, away from the PV MFMAs.   */         \
            _Pragma("unroll") for (int kk = 0; kk < 4; ++kk) asm volatile("" : "+v"(pnew[kk])); \
            if (DO_PV) {                                                                     \
                _Pragma("unroll") for (int i = 0; i < 4 * NMD; ++i) {                        \
                    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);                       \
                    __builtin_amdgcn_sched_group_barrier(0x002, 256 / (4 * NMD), 0);         \
                    __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);                       \
                }                                                                            \
            }                                                                                \
            lpart = fmaf(lpart, alpha, psum);                                                \
            alpha_prev = alpha;                                                              \
            pend = __any(grow);                                                              \
            _Pragma("unroll") for (int kk = 0; kk < 4; ++kk) pold[kk] = pnew[kk];            \
        }                                                                                    \
    } while (0)

    // Softmax of tile jt and PV(jt-1) together, interleaved by hand: the
    // first half of the PV MFMAs each go with a slice of the logits and their
    // max, the second half each with a slice of the exponentials.  Scheduling
    // fences keep every slice next to its MFMA; V operands are read four
    // MFMAs ahead and bias vectors one slice ahead.
    constexpr int NPV = 4 * NMD;            // PV MFMAs per tile
    constexpr int NA = NPV / 2;             // MFMAs next to the logits
    constexpr int CA = 8 / NA;              // logit slices (4 keys each) per MFMA
    constexpr int EB = 32 / (NPV - NA);     // exponentials per MFMA
#define TG_VFRAG(I)                                                                          \
    as_bf16x8(ld16(&Vt[vb][(32 * ((I) / 4) + l32) * VT_STRIDE + 16 * ((I) % 4) + 8 * hh]))
#define TG_BIAS(C)                                                                           \
    (BIAS ? *reinterpret_cast<const f32x4*>(&Bs[bb][hp][32 * ((C) / 4) + 8 * ((C) % 4) + 4 * hh]) \
          : f32x4{0.f, 0.f, 0.f, 0.f})
#define TG_PVSM_FUSED(MASKED)                                                                \
    do {                                                                                     \
        const int vb = (jt - 1) & 1;                                                         \
        const int bb = jt % NKB;                                                             \
        const int j0 = jt * KVT;                                                             \
        bf16x8 vq[4];                                                                        \
        _Pragma("unroll") for (int i = 0; i < 4; ++i) vq[i] = TG_VFRAG(i);                   \
        f32x4 sv = TG_BIAS(0);                                                               \
        float mx = -INFINITY;                                                                \
        __builtin_amdgcn_sched_barrier(0);                                                   \
        _Pragma("unroll") for (int i = 0; i < NA; ++i) {                                     \
            o[i / 4] = mfma32(vq[i % 4], pold[i % 4], o[i / 4]);                             \
            if (i + 4 < NPV) vq[i % 4] = TG_VFRAG(i + 4);                                    \
            _Pragma("unroll") for (int c = i * CA; c < (i + 1) * CA; ++c) {                  \
                const f32x4 cur = sv;                                                        \
                if (c + 1 < 8) sv = TG_BIAS(c + 1);                                          \
                const int mt = c / 4, rq = c % 4;                                            \
                const int kl = 32 * mt + 8 * rq + 4 * hh;                                    \
                _Pragma("unroll") for (int e = 0; e < 4; ++e) {                              \
                    float x = fmaf(c1, sacc[mt][4 * rq + e], cur[e]);                        \
                    if (MASKED && j0 + kl + e > qi) x = -INFINITY;                           \
                    sacc[mt][4 * rq + e] = x;                                                \
                    mx = fmaxf(mx, x);                                                       \
                }                                                                            \
            }                                                                                \
            __builtin_amdgcn_sched_barrier(0);                                               \
        }                                                                                    \
        mx = fmaxf(mx, __shfl_xor(mx, 32, WAVE));                                            \
        const bool grow = mx > m + RESCALE_SLACK;                                            \
        const float m_new = grow ? mx : m;                                                   \
        const float alpha = grow ? __builtin_amdgcn_exp2f(m - m_new) : 1.f;                  \
        m = m_new;                                                                           \
        const float mb = m == -INFINITY ? 0.f : m;                                           \
        float psum = 0.f;                                                                    \
        bf16x8 pnew[4];                                                                      \
        _Pragma("unroll") for (int i = NA; i < NPV; ++i) {                                   \
            o[i / 4] = mfma32(vq[i % 4], pold[i % 4], o[i / 4]);                             \
            if (i + 4 < NPV) vq[i % 4] = TG_VFRAG(i + 4);                                    \
            _Pragma("unroll") for (int x = (i - NA) * EB; x < (i - NA + 1) * EB; ++x) {      \
                const int kk = x / 8, e = x % 8;                                             \
                const float p = __builtin_amdgcn_exp2f(sacc[kk / 2][8 * (kk % 2) + e] - mb); \
                psum += p;                                                                   \
                pnew[kk][e] = to_bf16(p);                                                    \
            }                                                                                \
            __builtin_amdgcn_sched_barrier(0);                                               \
        }                                                                                    \
        _Pragma("unroll") for (int kk = 0; kk < 4; ++kk) asm volatile("" : "+v"(pnew[kk])); \
        lpart = fmaf(lpart, alpha, psum);                                                    \
        alpha_prev = alpha;                                                                  \
        pend = __any(grow);                                                                  \
        _Pragma("unroll") for (int kk = 0; kk < 4; ++kk) pold[kk] = pnew[kk];                \
    } while (0)

    // One step of the workgroup: stage K(jt+1) and V(jt) around BODY.
    // Every wave takes nkv + 1 steps, each ending in one barrier.
    int jt = 0;
#define TG_STEP(BODY)                                     \
    do {                                                  \
        const bool knext = jt + 1 < nkv;                  \
        const bool vnow = jt < nkv;                       \
        if (knext) load_k(jt + 1);                        \
        if (vnow) load_v(jt);                             \
        BODY;                                             \
        if (knext) store_k((jt + 1) % NKB);               \
        if (vnow) store_v(jt & 1);                        \
        __syncthreads();                                  \
        ++jt;                                             \
    } while (0)

    // Tiles strictly before this wave's rows need no mask; the tile holding
    // the wave's first row is the diagonal one; later tiles are skipped by
    // this wave (the workgroup still stages them).
    const int jt_diag = qmin / KVT;  // <= nkv - 1
    load_k(0);
    store_k(0);
    __syncthreads();
    if (jt_diag == 0) {
        TG_STEP({ TG_QK(jt); TG_PVSM(true, true, false); });
    } else {
        TG_STEP({ TG_QK(jt); TG_PVSM(false, true, false); });
        if (FUSED) {
            while (jt < jt_diag) TG_STEP({ TG_RESCALE(); TG_QK(jt); TG_PVSM_FUSED(false); });
            TG_STEP({ TG_RESCALE(); TG_QK(jt); TG_PVSM_FUSED(true); });
        } else {
            while (jt < jt_diag) TG_STEP({ TG_RESCALE(); TG_QK(jt); TG_PVSM(false, true, true); });
            TG_STEP({ TG_RESCALE(); TG_QK(jt); TG_PVSM(true, true, true); });
        }
    }
    TG_STEP({ TG_RESCALE(); TG_PVSM(false, false, true); });
    while (jt <= nkv) TG_STEP((void)0);
#undef TG_STEP
#undef TG_PVSM
#undef TG_RESCALE
#undef TG_PVSM_FUSED
#undef TG_VFRAG
#undef TG_BIAS
#undef TG_QK

    // ---- normalise and store ------------------------------------------------
    const float l = lpart + __shfl_xor(lpart, 32, WAVE);
    const float inv = 1.0f / l;
    if (qvalid) {
        bf16* op = a.out + ((rbase + qi) * a.Hq + h) * DH + 4 * hh;
#pragma unroll
        for (int md = 0; md < NMD; ++md) {
#pragma unroll
            for (int rq = 0; rq < 4; ++rq) {
                bf16x4 ov;
#pragma unroll
                for (int e = 0; e < 4; ++e) ov[e] = to_bf16(o[md][4 * rq + e] * inv);
                *reinterpret_cast<bf16x4*>(op + 32 * md + 8 * rq) = ov;
            }
        }
        if (a.lse != nullptr && hh == 0) a.lse[(int64_t)h * a.Kt + rbase + qi] = (m + log2f(l)) * LN2;
    }
}

template <int DH, int HPB, int NWAVE>
hipError_t launch_bf16(const AttnArgs& a, int total_tiles, hipStream_t st) {
    const int blocks = total_tiles * a.n_hg;
    if (a.s != nullptr)
        hipLaunchKernelGGL((attn_bf16_kernel<DH, HPB, NWAVE, true>), dim3(blocks), dim3(64 * NWAVE), 0, st, a);
    else
        hipLaunchKernelGGL((attn_bf16_kernel<DH, HPB, NWAVE, false>), dim3(blocks), dim3(64 * NWAVE), 0, st, a);
    return hipGetLastError();
}

template <int DH, int HPB>
hipError_t launch_bf16_w(AttnArgs& a, const AttnShape& sh, hipStream_t st) {
    // Eight-wave workgroups (K/V staged once for 256 query rows) unless that
    // leaves fewer than two workgroups per CU; then four-wave workgroups.
    auto tiles = [&](int bq) {
        int total = 0, mx = 0;
        for (int b = 0; b < sh.batch; ++b) {
            const int nt = (sh.cu[b + 1] - sh.cu[b] + bq - 1) / bq;
            a.ntiles[b] = nt;
            total += nt;
            mx = nt > mx ? nt : mx;
        }
        a.max_tiles = mx;
        return total;
    };
    const int t8 = tiles(256 / HPB);
    if (t8 * a.n_hg >= 512) return launch_bf16<DH, HPB, 8>(a, t8, st);
    const int t4 = tiles(128 / HPB);
    if (t4 == 0) return hipSuccess;
    return launch_bf16<DH, HPB, 4>(a, t4, st);
}

}  // namespace

hipError_t launch_attn_f32(const float* q, const float* k, const float* v, const float* s,
                           const float* gain, const float* temp, const AttnShape& sh, float* out,
                           float* lse, hipStream_t st) {
    const int64_t n = sh.Kt * sh.Hq;
    const int blocks = (int)((n + 127) / 128);
    if (sh.d_head == 64)
        hipLaunchKernelGGL(attn_f32_kernel<64>, dim3(blocks), dim3(128), 0, st, q, k, v, s, gain,
                           temp, sh, out, lse);
    else
        hipLaunchKernelGGL(attn_f32_kernel<128>, dim3(blocks), dim3(128), 0, st, q, k, v, s, gain,
                           temp, sh, out, lse);
    return hipGetLastError();
}

hipError_t launch_attn_bf16(const void* q, const void* k, const void* v, const float* s,
                            const float* gain, const float* temp, const AttnShape& sh, void* out,
                            float* lse, hipStream_t st) {
    const int group = sh.Hq / sh.Hkv;
    const int hpb = group % 4 == 0 ? 4 : (group % 2 == 0 ? 2 : 1);
    AttnArgs a;
    a.q = (const bf16*)q;
    a.k = (const bf16*)k;
    a.v = (const bf16*)v;
    a.s = s;
    a.gain = gain;
    a.temp = temp;
    a.out = (bf16*)out;
    a.lse = lse;
    a.Kt = sh.Kt;
    a.Hq = sh.Hq;
    a.Hkv = sh.Hkv;
    a.n_hg = sh.Hq / hpb;
    a.batch = sh.batch;
    for (int b = 0; b <= sh.batch; ++b) a.cu[b] = sh.cu[b];
    if (sh.Kt == 0) return hipSuccess;
    if (sh.d_head == 64) {
        if (hpb == 4) return launch_bf16_w<64, 4>(a, sh, st);
        if (hpb == 2) return launch_bf16_w<64, 2>(a, sh, st);
        return launch_bf16_w<64, 1>(a, sh, st);
    }
    if (hpb == 4) return launch_bf16_w<128, 4>(a, sh, st);
    if (hpb == 2) return launch_bf16_w<128, 2>(a, sh, st);
    return launch_bf16_w<128, 1>(a, sh, st);
}

}  // namespace tg
