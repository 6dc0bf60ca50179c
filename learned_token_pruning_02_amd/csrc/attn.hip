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
//   one extra k step of the product multiplies a per-key column [s split into
//     two bf16 halves, 1] with a per-query one [gain*log2(e)/c1 and -base/c1,
//     each split likewise], where c1 = temp*log2(e)/sqrt(d), so that one
//     multiply by c1 per element gives the exp2-domain logit with the bias
//     added and the row's exponent base subtracted;
//   O^T[dh][query] += V^T . P^T: V is stored transposed in LDS (A operand) and
//     the probabilities, converted to bf16, are fed straight from the S
//     registers as the B operand, again one query per lane, so the online
//     rescale of O needs no data exchange.
// Only the tiles on the diagonal (or past the end of the request) are masked,
// and a wave skips tiles whose keys all lie after its rows.  The exponent base
// of each row only moves when the row max exceeds it by more than 2^8 (and
// then from the next tile on), so the rescale of O is rare; the final O / l
// and lse are exact either way.  Row sums are taken from the bf16
// probabilities that feed the PV product, two per dot instruction.
// K/V tiles are double buffered: the next tile is fetched into registers,
// in four loads spread between the QK MFMAs, while the current one is
// consumed.  Heavy query tiles (many keys) are
// dispatched first and consecutive workgroup ids cycle over the KV heads, so
// the 8 XCDs each keep one head's K/V in their own L2.
// A single request too short to fill the chip (four-wave workgroups, fewer
// than two per CU) can, given a workspace, cut each query tile into pieces of
// at most 24 key tiles, one workgroup each: every piece leaves its
// unnormalised output, exponent base and row sum in fp32, takes a ticket, and
// the last piece of the tile combines all of them in piece order, so the
// result does not depend on which piece finished last.
#include "tg_device.h"
#include "tg_kernels.h"

namespace tg {

namespace {

constexpr float LOG2E = 1.4426950408889634f;
constexpr float LN2 = 0.6931471805599453f;
constexpr bf16x2 ONES = {(bf16)1.0f, (bf16)1.0f};

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
    // Key split (one request, four-wave workgroups): query tile t is cut into
    // ceil(nkv / split_len) pieces of near-equal key ranges, one workgroup
    // each; every piece leaves its partial result in part, and the last piece
    // of a tile to finish (ticket in cnt) combines them.
    int32_t split_len;
    uint32_t* cnt;  // [n_hg][ntiles[0]] tickets (< SPLIT_MAX_TILES), zero between calls
    float* part;    // [gridDim.x][SPLIT_SLOT_FLOATS<DH>()] partial results
};

constexpr int KVT = 64;          // keys per tile
constexpr int VT_STRIDE = KVT + 8;  // LDS row stride of V^T (bf16 elements)
// LDS row stride of V kept key-major (bf16 elements): 80 dwords, 16 modulo the
// 64 banks, so the four key rows a half-wave's transposing read touches fall
// on disjoint banks.
template <int DH>
constexpr int vs_stride() { return DH + 32; }

// The key split serves grids of fewer than SPLIT_MAX_TILES (query tile, head
// group) pairs; their tickets fill a counter region of fixed size at the start
// of the workspace, so that the partial results of any shape start after it
// and a workspace zeroed once keeps every ticket at zero between calls of any
// shapes.
constexpr int SPLIT_MAX_TILES = 512;
constexpr size_t SPLIT_CNT_BYTES = SPLIT_MAX_TILES * 4;

// Partial result of one piece of a split query tile, per four-wave workgroup:
// the unnormalised output registers (two per 8-byte word, lane-minor, so each
// wave's store of one register pair is 512 contiguous bytes), then each
// lane's (exponent base, row-sum half).
template <int DH>
constexpr int split_slot_floats() { return 4 * 64 * (DH / 32 * 16 + 2); }

// Key tiles of query tile t (BQ rows per head) of a request of n rows.
__device__ __forceinline__ int tile_keys(int t, int bq, int n) {
    return (min(bq * (t + 1), n) + KVT - 1) / KVT;
}

// Query tile t, piece p of np of the u-th workgroup (per head group) of a
// key-split launch: tiles from the last (most keys) down, each taking
// ceil(nkv / split_len) consecutive ids.
__device__ __forceinline__ void split_locate(const AttnArgs& a, int u, int bq, int& t, int& p,
                                             int& np) {
    const int n = a.cu[1] - a.cu[0];
    t = a.ntiles[0] - 1;
    for (;;) {
        np = (tile_keys(t, bq, n) + a.split_len - 1) / a.split_len;
        if (u < np || t == 0) break;
        u -= np;
        --t;
    }
    p = u;
}


// Number of query tiles whose local index is >= t.
__device__ __forceinline__ int tiles_at_or_above(const AttnArgs& a, int t) {
    int c = 0;
    for (int b = 0; b < a.batch; ++b) c += max(0, a.ntiles[b] - t);
    return c;
}

// Request b and query tile t of the u-th workgroup (per head group): tiles
// with more keys first, so that the heaviest work starts earliest.  With
// PAIR (one request, four-wave workgroups, two per CU, the whole grid
// resident at once) the first half of the ids takes the heavy half of the
// tiles from the heaviest down and the second half the light ones from the
// lightest up, so that the two workgroups sharing a CU (ids u and u + half)
// hold tiles t and nt - 1 - t: equal work on every CU.
template <bool PAIR>
__device__ __forceinline__ bool locate_tile(const AttnArgs& a, int u, int& b, int& t) {
    if (a.batch == 1) {
        b = 0;
        const int nt = a.ntiles[0];
        const int half = (nt + 1) / 2;
        t = !PAIR || u < half ? nt - 1 - u : u - half;
        return true;
    }
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
    return b < a.batch;  // false only for an inconsistent tile count
}

template <int DH, int HPB, int NWAVE, bool BIAS, bool SPLIT>
__global__ __launch_bounds__(64 * NWAVE, 8 / NWAVE) void attn_bf16_kernel(AttnArgs a) {
    // NWAVE = 8: two waves per SIMD from one workgroup; 4: two workgroups per CU.
    constexpr int WPH = NWAVE / HPB;   // waves per head
    constexpr int BQ = 32 * WPH;       // query rows per head per workgroup
    constexpr int KS = DH + 8;         // LDS row stride of K: DH values, then the 8-value bias column
    constexpr int KU = KVT * DH / 8 / 256;  // 16-byte K units per staging thread per tile
    constexpr int VU = (KVT / 4) * (DH / 8);  // V units (4 keys x 8 dh) per tile
    constexpr int NKK = DH / 16;       // k steps of the QK^T product (plus one for the bias column)
    constexpr int NMD = DH / 32;       // 32-row dh tiles of O^T
    constexpr float RESCALE_SLACK = 8.0f;   // log2 headroom before a row's base moves
    constexpr float REBASE_LIMIT = 64.0f;   // beyond it, exponentials are redone against the new base
    // Four waves (two workgroups per CU) interleave the softmax with the PV
    // MFMAs by hand, slice by slice; eight waves (one workgroup per CU) leave
    // the interleave to scheduling groups, which measures faster there.
    constexpr bool FUSED = NWAVE == 4;
    // Staging distance and LDS buffers.  The four-wave kernels stage K one
    // tile ahead (V of the current tile) into two buffers each and take a
    // barrier after every step.  The eight-wave kernel (one workgroup per CU,
    // room for more LDS) stages K two tiles ahead and V one ahead into four
    // buffers each and takes a barrier after every second step: a tile
    // written in step s is first read in step s + 2, always after the next
    // barrier, and each buffer it overwrites was last read before the
    // previous one.  Waves then meet half as often.
    constexpr int AHEAD = NWAVE == 8 ? 2 : 1;
    constexpr int NKB = 2 * AHEAD;  // K buffers
    constexpr int NVB = 2 * AHEAD;  // V buffers
    // A split piece needs every wave's rows inside the tile's last key tile
    // (at most 64 query rows per head), so that only the last piece masks.
    static_assert(!SPLIT || (NWAVE == 4 && BQ <= KVT), "key split: four waves, <= 64 rows per head");

    __shared__ __attribute__((aligned(16))) bf16 Ks[NKB][KVT * KS];
    // V in LDS: the four-wave kernel keeps it key-major, as loaded, and reads
    // the PV operands with gfx950's transposing LDS reads (no register
    // transpose when staging); the eight-wave kernel, whose step is bound by
    // LDS instruction issue, stores it transposed so that each operand is one
    // 16-byte read.
    constexpr bool VTR = NWAVE == 4;
    constexpr int VS = vs_stride<DH>();
    __shared__ __attribute__((aligned(16))) bf16 Vt[NVB][VTR ? KVT * VS : DH * VT_STRIDE];

    const int tid = threadIdx.x;
    const int lane = lane_id();
    // Wave index, read through a scalar register so that the compiler treats
    // everything derived from it (rows, loop bounds, buffer bases) as uniform.
    const int w = __builtin_amdgcn_readfirstlane(tid / WAVE);
    const int hh = lane / 32;
    const int l32 = lane % 32;

    // ---- which (request, query tile, head group) this workgroup owns ------
    const int hg = blockIdx.x % a.n_hg;
    int b = 0, t, piece = 0, npiece = 1;
    if (SPLIT) split_locate(a, (int)(blockIdx.x / a.n_hg), BQ, t, piece, npiece);
    else if (!locate_tile<NWAVE == 4>(a, (int)(blockIdx.x / a.n_hg), b, t)) return;
    const int64_t rbase = a.cu[b];
    const int n = a.cu[b + 1] - a.cu[b];
    const int q0 = t * BQ;
    const int kend = min(q0 + BQ, n);
    const int nkv = (kend + KVT - 1) / KVT;
    // Key tiles [jbeg, jend) of this workgroup: all of them, or one piece.
    const int jbeg = SPLIT ? piece * nkv / npiece : 0;
    const int jend = SPLIT ? (piece + 1) * nkv / npiece : nkv;
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
    // Scale of the exp2-domain logit: c1 = temp * log2(e) / sqrt(d), kept at
    // least 2^-60 in magnitude so that it can divide (a zero temperature then
    // contributes q.k * 2^-60, far below fp32 resolution of the bias).
    float c1 = a.temp[h] * LOG2E / sqrtf((float)DH);
    if (fabsf(c1) < 0x1p-60f) c1 = c1 < 0.f ? -0x1p-60f : 0x1p-60f;
    const float inv_c1 = 1.0f / c1;
    // ---- the bias column --------------------------------------------------
    // One more k step of the same product adds the gate bias and subtracts
    // the row's exponent base, both divided by c1, so that a single multiply
    // by c1 turns the MFMA result into the exp2-domain logit less the base.
    // Per key, the K side holds
    //     [s_hi, s_hi, s_lo, s_lo, 1, 1, 0, 0]      (s = s_hi + s_lo in bf16)
    // and lane half 0 of each query holds
    //     [g_hi, g_lo, g_hi, g_lo, -b_hi, -b_lo, 0, 0]
    // with g = gain * log2(e) / c1 and b = base / c1 split likewise (lane
    // half 1: zeros), so the step contributes (g_hi + g_lo)(s_hi + s_lo) - b
    // with bf16 products that are exact in the fp32 accumulator.  The base is
    // kept as c1 times the value its two bf16 halves represent.
    uint32_t qx_g = 0u;
    if (BIAS && hh == 0) {
        const float g = a.gain[h] * LOG2E * inv_c1;
        const bf16 g_hi = to_bf16(g);
        const bf16 g_lo = to_bf16(g - (float)g_hi);
        qx_g = __builtin_bit_cast(uint32_t, bf16x2{g_hi, g_lo});
    }
    u32x4 qx = {qx_g, qx_g, 0u, 0u};
    float mcur = 0.f;  // base subtracted by the bias column in the next QK product
    auto set_base = [&](float m_new) {
        const float nb = -m_new * inv_c1;
        const bf16 b_hi = to_bf16(nb);
        const bf16 b_lo = to_bf16(nb - (float)b_hi);
        mcur = -((float)b_hi + (float)b_lo) * c1;
        qx[2] = hh == 0 ? __builtin_bit_cast(uint32_t, bf16x2{b_hi, b_lo}) : 0u;
    };

    // ---- K/V/s tile staging ------------------------------------------------
    // K (with its bias column) is staged for tile jt+1 while V is staged one
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
    // Load i (0..3) of this thread's share of K tile jt (with the bias of
    // its keys at i = 0) and of V tile jv.  The four loads are issued at
    // separate points of a step, between MFMAs, so that the vector memory
    // pipe works through them in the background instead of holding up every
    // wave at the top of the step.
    // The loads are branch-free: a tile that is not needed gets a buffer of
    // size zero, and lanes without a unit get an offset past the buffer, so
    // both read zeros without touching memory.
    constexpr int OFF_NONE = 0x7ffffff0;
    auto k_rsrc = [&](bool kdo, int jt) {
        const int j0 = jt * KVT;
        return __builtin_amdgcn_make_buffer_rsrc(
            (void*)(a.k + (rbase + j0) * row_elems + kvh * DH), (short)0,
            kdo ? (int)((n - j0) * row_elems * 2) : 0, BUFFER_RSRC_WORD3);
    };
    auto v_rsrc = [&](bool vdo, int jv) {
        const int j0 = jv * KVT;
        return __builtin_amdgcn_make_buffer_rsrc(
            (void*)(a.v + (rbase + j0) * row_elems + kvh * DH), (short)0,
            vdo ? (int)((n - j0) * row_elems * 2) : 0, BUFFER_RSRC_WORD3);
    };
    auto k_off = [&](int i) {
        const int uu = st + i * 256;
        const int row = uu / (DH / 8), c = uu % (DH / 8);
        return (int)(row * row_elems * 2) + 16 * c;
    };
    // Thread st stages keys 4kg + {0..3}, dims 8dg + {0..7} of the V tile:
    // for the key-major layout sixteen consecutive threads cover one key row
    // (coalesced loads, whole-row LDS stores); for the transposed one they
    // cover sixteen keys of the same dims.
    auto v_off = [&](int i) {
        const int kg = VTR ? st / (DH / 8) : st % (KVT / 4), dg = VTR ? st % (DH / 8) : st / (KVT / 4);
        return st < VU ? (int)((4 * kg + i) * row_elems * 2) + 16 * dg : OFF_NONE;
    };
    // With eight waves a thread stages either K or V (one shared register
    // array); the tile base and size are chosen arithmetically so that the
    // wave-uniform choice needs no branch.
    const uint64_t kmask = kstager ? ~0ull : 0ull;
    auto load_part = [&](int i, bool kdo, int jt, bool vdo, int jv) {
        if (NWAVE == 8) {
            if (i < KU || !kstager) {
                const int jk0 = jt * KVT, jv0 = jv * KVT;
                const uint64_t kb = (uint64_t)(a.k + (rbase + jk0) * row_elems + kvh * DH);
                const uint64_t vb = (uint64_t)(a.v + (rbase + jv0) * row_elems + kvh * DH);
                const uint32_t ksz = kdo ? (uint32_t)((n - jk0) * row_elems * 2) : 0u;
                const uint32_t vsz = vdo ? (uint32_t)((n - jv0) * row_elems * 2) : 0u;
                const uint64_t base = vb + ((kb - vb) & kmask);
                const uint32_t size = vsz + ((ksz - vsz) & (uint32_t)kmask);
                const __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc(
                    (void*)base, (short)0, (int)size, BUFFER_RSRC_WORD3);
                stg[i] = __builtin_amdgcn_raw_buffer_load_b128(r, kstager ? k_off(i) : v_off(i), 0, 0);
            }
        } else {
            if (i < KU) kreg[i] = __builtin_amdgcn_raw_buffer_load_b128(k_rsrc(kdo, jt), k_off(i), 0, 0);
            vreg[i] = __builtin_amdgcn_raw_buffer_load_b128(v_rsrc(vdo, jv), v_off(i), 0, 0);
        }
        if (BIAS && i == 0) {
            const int j0 = jt * KVT;
            const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
                (void*)(a.s + rbase + j0), (short)0, kdo && kstager ? (n - j0) * 4 : 0, BUFFER_RSRC_WORD3);
            sreg = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(
                rs, st < KVT ? 4 * st : OFF_NONE, 0, 0));
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
            if (st < KVT) {
                uint32_t w_hi = 0u, w_lo = 0u;
                if (BIAS) {
                    const bf16 s_hi = to_bf16(sreg);
                    const bf16 s_lo = to_bf16(sreg - (float)s_hi);
                    w_hi = __builtin_bit_cast(uint32_t, bf16x2{s_hi, s_hi});
                    w_lo = __builtin_bit_cast(uint32_t, bf16x2{s_lo, s_lo});
                }
                const u32x4 col = {w_hi, w_lo, 0x3F803F80u /* bf16 1, 1 */, 0u};
                st16(&Ks[buf][st * KS + DH], col);
            }
        }
    };
    auto store_v = [&](int buf) {
        if (VTR && st < VU) {
            const int kg = st / (DH / 8), dg = st % (DH / 8);
#pragma unroll
            for (int i = 0; i < 4; ++i) st16(&Vt[buf][(4 * kg + i) * VS + 8 * dg], vreg[i]);
        } else if (!VTR && vstager && st < VU) {
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

    // PV operand of dh tile md, k step kk: keys 16kk + 4hh + {0..3} and
    // 16kk + 8 + 4hh + {0..3} (the order of the probabilities in the score
    // registers) of dim 32md + l32.  Key-major V: two transposing reads; in
    // each 16-lane group, lane i points at four dims of one key row, and lane
    // j receives dim j of the group's rows j/4, j/4 + 4, j/4 + 8 and j/4 + 12,
    // so lane i of a group points at key 4hh + i/4 and dims 16 (group % 2) +
    // 4 (i % 4).  Transposed V: one 16-byte read.
    const int vtr = (4 * hh + (lane % 16) / 4) * VS + 16 * ((lane / 16) % 2) + 4 * (lane % 4);
    typedef short v4i16_t __attribute__((ext_vector_type(4)));
    auto vfrag_tr = [&](int vb, int md, int kk) {
        const bf16* p0 = &Vt[vb][(16 * kk) * VS + 32 * md + vtr];
        const v4i16_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) v4i16_t*)p0);
        const v4i16_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (__attribute__((address_space(3))) v4i16_t*)(p0 + 8 * VS));
        const u32x2 a = __builtin_bit_cast(u32x2, lo), c = __builtin_bit_cast(u32x2, hi);
        return as_bf16x8(u32x4{a[0], a[1], c[0], c[1]});
    };

    f32x16 o[NMD];
#pragma unroll
    for (int md = 0; md < NMD; ++md)
#pragma unroll
        for (int r = 0; r < 16; ++r) o[md][r] = 0.f;
    // Online softmax state.  The exponentials of a tile are taken against the
    // base its QK product subtracted (mcur at the time), whatever the tile's
    // max turns out to be: pf is the base of the latest probabilities, O and
    // lpart are kept against pf, and a change of pf rescales them by
    // alpha = 2^(pf_old - pf_new).  The base only moves when a row's max
    // exceeds it by more than RESCALE_SLACK, and then for the next tile, so
    // the probabilities of a tile are at most 2^REBASE_LIMIT; a row past that
    // redoes its exponentials against its new base (a rare, separate path).
    float pf = 0.f, lpart = 0.f;       // base of O / lpart, and this lane's row-sum half
    bf16x8 pold[4];                    // probabilities of the previous tile (PV operand)
    float alpha_prev = 1.f;            // rescale of O owed before the next PV product
    bool pend = false;                 // some row of the wave owes a rescale

    f32x16 sacc[2];  // S^T of one tile: (log2-domain logits - mcur) / c1, then times c1

    // S^T of tile T from its staged K: the bias column first, then d_head;
    // LD(i) issues staging load i after the MFMAs of k step i.
#define TG_KFRAG(KK, MT)                                                                     \
    as_bf16x8(ld16(&Ks[kb][(32 * (MT) + l32) * KS + ((KK) < 0 ? DH : (DH / 2) * hh + 8 * (KK))]))
#define TG_QK(T, LD)                                                                         \
    do {                                                                                     \
        const int kb = (T) % NKB;                                                            \
        bf16x8 kc[2], kn[2];                                                                 \
        _Pragma("unroll") for (int mt = 0; mt < 2; ++mt) {                                   \
            _Pragma("unroll") for (int r = 0; r < 16; ++r) sacc[mt][r] = 0.f;                \
            kc[mt] = TG_KFRAG(-1, mt);                                                       \
        }                                                                                    \
        /* K fragments are read one k step ahead; the fences keep the two */                 \
        /* accumulators alternating. */                                                      \
        _Pragma("unroll") for (int kk = -1; kk < NKK; ++kk) {                                \
            if (kk + 1 < NKK) { kn[0] = TG_KFRAG(kk + 1, 0); kn[1] = TG_KFRAG(kk + 1, 1); }  \
            _Pragma("unroll") for (int mt = 0; mt < 2; ++mt)                                 \
                sacc[mt] = mfma32(kc[mt], kk < 0 ? as_bf16x8(qx) : qf[kk < 0 ? 0 : kk], sacc[mt]); \
            if (kk >= 0 && kk < 4) LD(kk);                                                   \
            __builtin_amdgcn_sched_barrier(0);                                               \
            kc[0] = kn[0];                                                                   \
            kc[1] = kn[1];                                                                   \
        }                                                                                    \
    } while (0)

    // Logit element c (0..31) of this lane: S^T register 4rq + e of tile mt
    // holds key 32mt + 8rq + 4hh + e.  Probability element (kk, e) of the PV
    // operand is S^T register 8(kk%2) + e of tile kk/2.
#define TG_MASK_MAX(MASKED, C)                                                               \
    do {                                                                                     \
        const int mt_ = (C) / 16, r_ = (C) % 16;                                             \
        float y_ = sacc[mt_][r_] * c1;                                                       \
        if (MASKED && j0 + 32 * mt_ + 8 * (r_ / 4) + 4 * hh + (r_ % 4) > qi) y_ = -INFINITY; \
        sacc[mt_][r_] = y_;                                                                  \
        mx = fmaxf(mx, y_);                                                                  \
    } while (0)
// The same without the row max (tiles after the first: the max is only
// taken, in TG_SOFTMAX_TAIL, when a row's probabilities sum past 2^8).
#define TG_MASK(MASKED, C)                                                                   \
    do {                                                                                     \
        const int mt_ = (C) / 16, r_ = (C) % 16;                                             \
        float y_ = sacc[mt_][r_] * c1;                                                       \
        if (MASKED && j0 + 32 * mt_ + 8 * (r_ / 4) + 4 * hh + (r_ % 4) > qi) y_ = -INFINITY; \
        sacc[mt_][r_] = y_;                                                                  \
    } while (0)
#define TG_EXP_PAIR(X, SUB)                                                                  \
    do {                                                                                     \
        const int kk_ = (X) / 8, e_ = (X) % 8;                                               \
        const float p0_ = __builtin_amdgcn_exp2f(sacc[kk_ / 2][8 * (kk_ % 2) + e_] - (SUB)); \
        const float p1_ = __builtin_amdgcn_exp2f(sacc[kk_ / 2][8 * (kk_ % 2) + e_ + 1] - (SUB)); \
        const bf16x2 pp_ = {to_bf16(p0_), to_bf16(p1_)};                                     \
        pnew[kk_][e_] = pp_[0];                                                              \
        pnew[kk_][e_ + 1] = pp_[1];                                                          \
        psum[kk_ % 2] = __builtin_amdgcn_fdot2_f32_bf16(pp_, ONES, psum[kk_ % 2], false);    \
    } while (0)

    // After the exponentials of tile jt (against mcur): rows whose max grew
    // past the slack move their base for the next tile; rows past the limit
    // also redo this tile's exponentials against the new base.  Then the
    // rescale owed by a change of base is recorded and the row sum updated.
#define TG_SOFTMAX_TAIL()                                                                    \
    do {                                                                                     \
        /* Every probability is at most the row's sum, so a row whose sum  */                \
        /* stays within 2^8 cannot have grown past the slack: the row max */                 \
        /* is only needed when some row's sum exceeds it (or overflows).  */                 \
        const float ps_ = psum[0] + psum[1];                                                 \
        const float tot_ = ps_ + __shfl_xor(ps_, 32, WAVE);                                  \
        float pf_new = mcur;                                                                 \
        if (__any(!(tot_ <= 0x1p8f))) {                                                      \
            float mx = -INFINITY;                                                            \
            _Pragma("unroll") for (int c = 0; c < 32; ++c) mx = fmaxf(mx, sacc[c / 16][c % 16]); \
            mx = fmaxf(mx, __shfl_xor(mx, 32, WAVE));                                        \
            const bool grow = mx > RESCALE_SLACK;                                            \
            const float m_old = mcur;                                                        \
            if (grow) set_base(m_old + mx);                                                  \
            const bool redo = mx > REBASE_LIMIT;                                             \
            if (__any(redo)) {                                                               \
                const float sub = redo ? mcur - m_old : 0.f;                                 \
                psum[0] = psum[1] = 0.f;                                                     \
                _Pragma("unroll") for (int x = 0; x < 32; x += 2) TG_EXP_PAIR(x, sub);       \
                if (redo) pf_new = mcur;                                                     \
            }                                                                                \
        }                                                                                    \
        const float alpha = __builtin_amdgcn_exp2f(pf - pf_new);                             \
        pf = pf_new;                                                                         \
        lpart = fmaf(lpart, alpha, psum[0] + psum[1]);                                       \
        alpha_prev = alpha;                                                                  \
        pend = __any(alpha != 1.f);                                                          \
        _Pragma("unroll") for (int kk = 0; kk < 4; ++kk) pold[kk] = pnew[kk];                \
    } while (0)

    // The first tile of a wave: its row max becomes the base, and the
    // exponentials are taken against it (nothing accumulated yet).
#define TG_SOFTMAX_FIRST(MASKED)                                                             \
    do {                                                                                     \
        const int j0 = jt * KVT;                                                             \
        float mx = -INFINITY;                                                                \
        _Pragma("unroll") for (int c = 0; c < 32; ++c) TG_MASK_MAX(MASKED, c);               \
        mx = fmaxf(mx, __shfl_xor(mx, 32, WAVE));                                            \
        set_base(mx);                                                                        \
        pf = mcur;                                                                           \
        float psum[2] = {0.f, 0.f};                                                          \
        bf16x8 pnew[4];                                                                      \
        _Pragma("unroll") for (int x = 0; x < 32; x += 2) TG_EXP_PAIR(x, mcur);              \
        lpart = psum[0] + psum[1];                                                           \
        _Pragma("unroll") for (int kk = 0; kk < 4; ++kk) pold[kk] = pnew[kk];                \
    } while (0)

    // DO_S: softmax of tile jt from sacc (MASKED on the diagonal tile);
    // DO_PV: O += V(jt-1) P(jt-1).  The rescale of O owed by a change of base
    // is applied at the start of the next step (TG_RESCALE), before the next
    // PV product, so that the QK product, the PV product and the softmax form
    // one straight run of independent MFMA and VALU work.
#define TG_RESCALE()                                                                         \
    do {                                                                                     \
        if (pend) {                                                                          \
            _Pragma("unroll") for (int md = 0; md < NMD; ++md)                               \
                _Pragma("unroll") for (int r = 0; r < 16; ++r) o[md][r] *= alpha_prev;       \
        }                                                                                    \
    } while (0)
#define TG_PVSM(MASKED)                                                                      \
    do {                                                                                     \
        const int vb = (jt - 1) & (NVB - 1);                                                 \
        const int j0 = jt * KVT;                                                             \
        bf16x8 v0[NMD];                                                                      \
        _Pragma("unroll") for (int md = 0; md < NMD; ++md) v0[md] = TG_VFRAG(md);            \
        /* QK above, then PV interleaved with the softmax below. */                          \
        __builtin_amdgcn_sched_barrier(0);                                                   \
        _Pragma("unroll") for (int i = 0; i < NPV; ++i)                                      \
            o[i % NMD] = mfma32(i < NMD ? v0[i] : TG_VFRAG(i), pold[i / NMD], o[i % NMD]);   \
        _Pragma("unroll") for (int c = 0; c < 32; ++c) TG_MASK(MASKED, c);                   \
        float psum[2] = {0.f, 0.f};                                                          \
        bf16x8 pnew[4];                                                                      \
        _Pragma("unroll") for (int x = 0; x < 32; x += 2) TG_EXP_PAIR(x, 0.f);               \
        /* Pin the probabilities here: left alone, the compiler sinks the   */               \
        /* exponentials below the staging stores, away from the PV MFMAs.   */               \
        _Pragma("unroll") for (int kk = 0; kk < 4; ++kk) asm volatile("" : "+v"(pnew[kk])); \
        _Pragma("unroll") for (int i = 0; i < 4 * NMD; ++i) {                                \
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);                               \
            __builtin_amdgcn_sched_group_barrier(0x002, SG_VALU, 0);                         \
            __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);                               \
        }                                                                                    \
        TG_SOFTMAX_TAIL();                                                                   \
    } while (0)

    // Softmax of tile jt and PV(jt-1) together, interleaved by hand: each PV
    // MFMA goes with a slice of the logits (mask and max) and of the
    // exponentials.  Scheduling fences keep every slice next to its MFMA; V
    // operands are read four MFMAs ahead.
    constexpr int NPV = 4 * NMD;            // PV MFMAs per tile
    constexpr int CPM = 32 / NPV;           // logits per MFMA (even)
    constexpr int SG_VALU = (5 * 32 / 2 + NPV - 1) / NPV;  // VALU per MFMA in the scheduling groups
#define TG_VFRAG(I)                                                                          \
    (VTR ? vfrag_tr(vb, (I) % NMD, (I) / NMD)                                                \
         : as_bf16x8(ld16(&Vt[vb][(32 * ((I) % NMD) + l32) * VT_STRIDE + 16 * ((I) / NMD) + 8 * hh])))
#define TG_PVSM_FUSED(MASKED)                                                                \
    do {                                                                                     \
        const int vb = (jt - 1) & (NVB - 1);                                                 \
        const int j0 = jt * KVT;                                                             \
        bf16x8 vq[4];                                                                        \
        _Pragma("unroll") for (int i = 0; i < 4; ++i) vq[i] = TG_VFRAG(i);                   \
        float psum[2] = {0.f, 0.f};                                                          \
        bf16x8 pnew[4];                                                                      \
        __builtin_amdgcn_sched_barrier(0);                                                   \
        _Pragma("unroll") for (int i = 0; i < NPV; ++i) {                                    \
            o[i % NMD] = mfma32(vq[i % 4], pold[i / NMD], o[i % NMD]);                       \
            if (i + 4 < NPV) vq[i % 4] = TG_VFRAG(i + 4);                                    \
            _Pragma("unroll") for (int x = i * CPM; x < (i + 1) * CPM; x += 2) {             \
                const int kk = x / 8, e = x % 8;                                             \
                TG_MASK(MASKED, 16 * (kk / 2) + 8 * (kk % 2) + e);                           \
                TG_MASK(MASKED, 16 * (kk / 2) + 8 * (kk % 2) + e + 1);                       \
                TG_EXP_PAIR(x, 0.f);                                                         \
            }                                                                                \
            __builtin_amdgcn_sched_barrier(0);                                               \
        }                                                                                    \
        _Pragma("unroll") for (int kk = 0; kk < 4; ++kk) asm volatile("" : "+v"(pnew[kk])); \
        TG_SOFTMAX_TAIL();                                                                   \
    } while (0)

    // One step of the workgroup: stage K(jt+AHEAD) and V(jt+AHEAD-1) around
    // BODY.  Every wave takes nkv + 1 steps; a barrier ends every step (four
    // waves) or every second one (eight waves).
    int jt = jbeg;
#define TG_STEP(BODY)                                               \
    do {                                                            \
        const bool knext = jt + AHEAD < jend;                       \
        const bool vnow = jt + AHEAD - 1 < jend;                    \
        BODY;                                                       \
        if (knext) store_k((jt + AHEAD) % NKB);                     \
        if (vnow) store_v((jt + AHEAD - 1) % NVB);                  \
        if (AHEAD == 1 || ((jt - jbeg) & 1)) __syncthreads();       \
        ++jt;                                                       \
    } while (0)
#define TG_LD(i) load_part((i), knext, jt + AHEAD, vnow, jt + AHEAD - 1)
#define TG_LD_ALL() do { TG_LD(0); TG_LD(1); TG_LD(2); TG_LD(3); } while (0)

    // Tiles strictly before this wave's rows need no mask; the tile holding
    // the wave's first row is the diagonal one; later tiles are skipped by
    // this wave (the workgroup still stages them).  A wave whose rows all lie
    // past the end of the request (in a request's last tile) takes the last
    // key tile as its diagonal: its rows are never stored, and it runs the
    // same nkv + 1 steps (barriers) as the other waves instead of computing
    // on a key tile that was never staged.
    const int jt_diag = min(qmin / KVT, nkv - 1);
    // The last key tile this wave computes, and whether it is the diagonal
    // one (always, unless this is a piece before the last of a split tile).
    const int jlast = SPLIT ? jend - 1 : jt_diag;
    const bool mlast = !SPLIT || jend == nkv;
    // Waves 4-7 share each SIMD with one of waves 0-3, which the hardware
    // favours when both can issue; raising their priority evens out the
    // two waves' step times, so neither idles long at the barrier.
    if (NWAVE == 8 && w >= 4) __builtin_amdgcn_s_setprio(2);
    load_part(0, true, jbeg, false, 0);
    load_part(1, true, jbeg, false, 0);
    load_part(2, true, jbeg, false, 0);
    load_part(3, true, jbeg, false, 0);
    store_k(jbeg % NKB);
    if (AHEAD == 2) {  // the first epoch also reads K(jbeg+1) and V(jbeg)
        const bool k1 = jbeg + 1 < jend;
        load_part(0, k1, jbeg + 1, true, jbeg);
        load_part(1, k1, jbeg + 1, true, jbeg);
        load_part(2, k1, jbeg + 1, true, jbeg);
        load_part(3, k1, jbeg + 1, true, jbeg);
        if (k1) store_k((jbeg + 1) % NKB);
        store_v(jbeg % NVB);
    }
    __syncthreads();
    if (jlast == jbeg) {
        if (mlast) TG_STEP({ TG_QK(jt, TG_LD); TG_SOFTMAX_FIRST(true); });
        else TG_STEP({ TG_QK(jt, TG_LD); TG_SOFTMAX_FIRST(false); });
    } else {
        TG_STEP({ TG_QK(jt, TG_LD); TG_SOFTMAX_FIRST(false); });
        if (FUSED) {
            while (jt < jlast) TG_STEP({ TG_RESCALE(); TG_QK(jt, TG_LD); TG_PVSM_FUSED(false); });
            if (mlast) TG_STEP({ TG_RESCALE(); TG_QK(jt, TG_LD); TG_PVSM_FUSED(true); });
            else TG_STEP({ TG_RESCALE(); TG_QK(jt, TG_LD); TG_PVSM_FUSED(false); });
        } else {
            while (jt < jlast) TG_STEP({ TG_RESCALE(); TG_QK(jt, TG_LD); TG_PVSM(false); });
            TG_STEP({ TG_RESCALE(); TG_QK(jt, TG_LD); TG_PVSM(true); });
        }
    }
    // The PV product of the last tile.
    TG_STEP({
        TG_LD_ALL();
        TG_RESCALE();
        const int vb = (jt - 1) & (NVB - 1);
        _Pragma("unroll") for (int i = 0; i < NPV; ++i) o[i % NMD] = mfma32(TG_VFRAG(i), pold[i / NMD], o[i % NMD]);
    });
    while (jt <= jend) TG_STEP(TG_LD_ALL());
#undef TG_LD_ALL
#undef TG_LD
#undef TG_STEP
#undef TG_PVSM
#undef TG_PVSM_FUSED
#undef TG_RESCALE
#undef TG_SOFTMAX_FIRST
#undef TG_SOFTMAX_TAIL
#undef TG_EXP_PAIR
#undef TG_MASK_MAX
#undef TG_MASK
#undef TG_VFRAG
#undef TG_QK
#undef TG_KFRAG

    // ---- pieces of a split tile: the last one to finish combines them -------
    if (SPLIT && npiece > 1) {
        constexpr int NPAIR = NMD * 8;  // 8-byte words of output registers per lane
        constexpr int SLOT = split_slot_floats<DH>();
        uint64_t* const mine = reinterpret_cast<uint64_t*>(a.part + (int64_t)blockIdx.x * SLOT);
#pragma unroll
        for (int i = 0; i < NPAIR; ++i)
            coherent_st64(mine + (w * NPAIR + i) * WAVE + lane, o[i / 8][2 * (i % 8)], o[i / 8][2 * (i % 8) + 1]);
        coherent_st64(mine + 4 * NPAIR * WAVE + w * WAVE + lane, pf, lpart);
        __shared__ int s_last;
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // this wave's stores are performed
        __syncthreads();
        if (tid == 0) {
            uint32_t* const c = a.cnt + hg * a.ntiles[0] + t;
            const uint32_t old = __hip_atomic_fetch_add(c, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            const bool last = old == (uint32_t)(npiece - 1);
            // Every piece has taken its ticket: reset it for the next call.
            if (last) __hip_atomic_store(c, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            s_last = last;
        }
        __syncthreads();
        if (!s_last) return;
        // Combine the pieces in piece order (whichever finished last), each
        // rescaled from its own base to the largest: the result does not
        // depend on the order in which the pieces ran.
        const uint64_t* const first =
            reinterpret_cast<const uint64_t*>(a.part + (int64_t)(blockIdx.x - piece * a.n_hg) * SLOT);
        const int64_t stride = (int64_t)a.n_hg * SLOT / 2;  // 8-byte words between pieces
        const int mlw = 4 * NPAIR * WAVE + w * WAVE + lane;  // this lane's (base, sum) word
        // Largest base over the pieces, eight loads in flight at a time.
        float mx = -INFINITY;
        for (int i0 = 0; i0 < npiece; i0 += 8) {
            float2 ml[8];
#pragma unroll
            for (int i = 0; i < 8; ++i)
                ml[i] = i0 + i < npiece ? coherent_ld64(first + (i0 + i) * stride + mlw) : make_float2(-INFINITY, 0.f);
#pragma unroll
            for (int i = 0; i < 8; ++i) mx = fmaxf(mx, ml[i].x);
        }
        // Each piece's output registers are loaded while the previous
        // piece's are accumulated.
        auto load_piece = [&](int i, float2* v) {
            const uint64_t* const src = first + (int64_t)i * stride;
#pragma unroll
            for (int j = 0; j < NPAIR; ++j) v[j] = coherent_ld64(src + (w * NPAIR + j) * WAVE + lane);
            v[NPAIR] = coherent_ld64(src + mlw);
        };
        float2 cur[NPAIR + 1], nxt[NPAIR + 1] = {};
        load_piece(0, cur);
#pragma unroll
        for (int md = 0; md < NMD; ++md)
#pragma unroll
            for (int r = 0; r < 16; ++r) o[md][r] = 0.f;
        lpart = 0.f;
        for (int i = 0; i < npiece; ++i) {
            if (i + 1 < npiece) load_piece(i + 1, nxt);
            const float f = __builtin_amdgcn_exp2f(cur[NPAIR].x - mx);
            lpart = fmaf(cur[NPAIR].y, f, lpart);
#pragma unroll
            for (int j = 0; j < NPAIR; ++j) {
                o[j / 8][2 * (j % 8)] = fmaf(cur[j].x, f, o[j / 8][2 * (j % 8)]);
                o[j / 8][2 * (j % 8) + 1] = fmaf(cur[j].y, f, o[j / 8][2 * (j % 8) + 1]);
            }
#pragma unroll
            for (int j = 0; j <= NPAIR; ++j) cur[j] = nxt[j];
        }
        pf = mx;
    }

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
        if (a.lse != nullptr && hh == 0) a.lse[(int64_t)h * a.Kt + rbase + qi] = (pf + log2f(l)) * LN2;
    }
}

template <int DH, int HPB, int NWAVE, bool SPLIT>
hipError_t launch_bf16(const AttnArgs& a, int blocks, hipStream_t st) {
    if (a.s != nullptr)
        hipLaunchKernelGGL((attn_bf16_kernel<DH, HPB, NWAVE, true, SPLIT>), dim3(blocks), dim3(64 * NWAVE), 0, st, a);
    else
        hipLaunchKernelGGL((attn_bf16_kernel<DH, HPB, NWAVE, false, SPLIT>), dim3(blocks), dim3(64 * NWAVE), 0, st, a);
    return hipGetLastError();
}

// Key tiles per piece of a split query tile.  The 16k layer's 2048 kept rows
// (32 query tiles of 1..32 key tiles, 8 head groups) then run as 320
// workgroups of at most 16 steps instead of 256 whose longest walks 32 key
// tiles.  Shorter pieces balance better but each costs a partial result
// written, a ticket and a share of a merge (a few microseconds of memory
// round trips); measured at 1000, 2048 and 3000 rows, 24 was fastest.
#ifndef TG_ATTN_SPLIT_LEN
#define TG_ATTN_SPLIT_LEN 24
#endif
constexpr int SPLIT_LEN = TG_ATTN_SPLIT_LEN;
// A request whose longest query tile has 19..SPLIT_LEN key tiles (1153 to
// 1536 kept rows) would not be split at that length; pieces of at most
// SPLIT_SHORT key tiles still spread it (measured: 1536 rows 35.2 -> 28.9
// us, 1200 rows 27.9 -> 26.7 us; at 1025 rows the split lost, 24.5 -> 25.9).
constexpr int SPLIT_SHORT = 16;
constexpr int SPLIT_SHORT_MIN = 19;  // key tiles of the longest tile, at least

// How a packed batch is launched: eight-wave workgroups (K/V staged once for
// 256 query rows) unless that leaves fewer than two workgroups per CU; then
// four-wave workgroups, two per CU.  A single request whose four-wave grid
// still holds at most one workgroup per CU has its query tiles split over
// several workgroups (the key split), when it has a workspace and at least
// two query heads share a KV head.
struct AttnPlan {
    int nwave;         // 8 or 4
    int blocks;        // workgroups without the key split
    int tiles;         // query tiles over all requests
    bool split;
    int split_len;     // key tiles per piece, at most
    int split_blocks;  // workgroups with it
    size_t ws_bytes;   // workspace of the key split (0 without it)
};

AttnPlan plan_bf16(AttnArgs& a, const AttnShape& sh, int hpb) {
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
    AttnPlan pl{};
    const int t8 = tiles(256 / hpb);
    if (t8 * a.n_hg >= 512) {
        pl = {8, t8 * a.n_hg, t8, false, 0, 0, 0};
        return pl;
    }
    const int bq = 128 / hpb;
    const int t4 = tiles(bq);
    pl = {4, t4 * a.n_hg, t4, false, 0, 0, 0};
    if (sh.batch != 1 || hpb < 2 || t4 * a.n_hg >= SPLIT_MAX_TILES) return pl;
    const int n = sh.cu[1] - sh.cu[0];
    const int nkv_max = (n + KVT - 1) / KVT;  // key tiles of the last query tile
    const int len = nkv_max > SPLIT_LEN || nkv_max < SPLIT_SHORT_MIN ? SPLIT_LEN : SPLIT_SHORT;
    int pieces = 0;
    for (int t = 0; t < t4; ++t) {
        const int nkv = ((bq * (t + 1) < n ? bq * (t + 1) : n) + KVT - 1) / KVT;
        pieces += (nkv + len - 1) / len;
    }
    if (pieces == t4) return pl;  // no tile is long enough to split
    const size_t slot = (size_t)(sh.d_head == 64 ? split_slot_floats<64>() : split_slot_floats<128>()) * 4;
    pl.split = true;
    pl.split_len = len;
    pl.split_blocks = pieces * a.n_hg;
    pl.ws_bytes = SPLIT_CNT_BYTES + (size_t)pl.split_blocks * slot;
    return pl;
}

template <int DH, int HPB>
hipError_t launch_bf16_w(AttnArgs& a, const AttnShape& sh, void* ws, hipStream_t st) {
    const AttnPlan pl = plan_bf16(a, sh, HPB);
    if (pl.tiles == 0) return hipSuccess;
    if (pl.nwave == 8) return launch_bf16<DH, HPB, 8, false>(a, pl.blocks, st);
    if constexpr (HPB >= 2) {
        if (pl.split && ws != nullptr) {
            a.split_len = pl.split_len;
            a.cnt = (uint32_t*)ws;
            a.part = (float*)((char*)ws + SPLIT_CNT_BYTES);
            return launch_bf16<DH, HPB, 4, true>(a, pl.split_blocks, st);
        }
    }
    return launch_bf16<DH, HPB, 4, false>(a, pl.blocks, st);
}

int heads_per_block(const AttnShape& sh) {
    const int group = sh.Hq / sh.Hkv;
    return group % 4 == 0 ? 4 : (group % 2 == 0 ? 2 : 1);
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

size_t attn_prefill_workspace_bytes(const AttnShape& sh) {
    if (sh.Kt == 0) return 0;
    AttnArgs a{};
    const int hpb = heads_per_block(sh);
    a.n_hg = sh.Hq / hpb;
    return plan_bf16(a, sh, hpb).ws_bytes;
}

hipError_t launch_attn_bf16(const void* q, const void* k, const void* v, const float* s,
                            const float* gain, const float* temp, const AttnShape& sh, void* out,
                            float* lse, void* ws, size_t ws_bytes, hipStream_t st) {
    (void)ws_bytes;  // checked against attn_prefill_workspace_bytes by the caller
    const int hpb = heads_per_block(sh);
    AttnArgs a{};
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
        if (hpb == 4) return launch_bf16_w<64, 4>(a, sh, ws, st);
        if (hpb == 2) return launch_bf16_w<64, 2>(a, sh, ws, st);
        return launch_bf16_w<64, 1>(a, sh, ws, st);
    }
    if (hpb == 4) return launch_bf16_w<128, 4>(a, sh, ws, st);
    if (hpb == 2) return launch_bf16_w<128, 2>(a, sh, ws, st);
    return launch_bf16_w<128, 1>(a, sh, ws, st);
}

}  // namespace tg
