// Top-K selection with the question tail always kept (spke.com page,
// "Comment TokenGate a-t-il appris ...": the second bullet of the three-phase
// list for the top-K, the sentence after the list for the question, which is
// never pruned; "Comment déployer TokenGate ?" for the max_kept_prefill_tokens
// budget).
//
// Per request b:
//   * budget >= N_b: keep every token;
//   * otherwise keep the K_b - q_b best document tokens under the total order
//     (score descending, index ascending) plus the q_b question tokens.
// Kept ids come out ascending.
//
// Scores become order-preserving u32 keys (larger key = better score; -0 and
// +0 share a key; NaN maps to 0, below -inf).  The document of every request
// is cut into chunks of 2048 keys, one 256-thread workgroup per chunk, and
// the whole batch goes through four launches:
//   1. clear the per-request histograms and counters;
//   2. histogram of the keys over 2048 bins per chunk (LDS), summed into the
//      request's histogram with global atomics; the chunk that finishes last
//      (atomic ticket, no waiting) finds the bin d1 holding the K_doc-th best
//      key.  The bins are linear in the score over a range taken from the
//      document's first chunk (mean +- 8 standard deviations within its min
//      and max; every workgroup derives the same range from the same keys),
//      and clamped to the end bins, so monotone in the key;
//   3. per chunk, count the keys above d1 and append the keys in d1 with
//      their index; the last chunk ranks the candidates exactly under the
//      63-bit composite (key, then reversed index), which turns (key desc,
//      index asc) into a single descending order, by counting for each one
//      the candidates that beat it (a few hundred at most) or else by an LDS
//      radix select over the composite, then counts the kept tokens of every
//      chunk and scans them into output offsets;
//   4. per chunk, re-derive each key's keep flag from (d1, composite
//      threshold) and write the kept ids in index order (wave ballots + a
//      small count table per workgroup), and the question tail after them.
// A batch with a document above BIG_DOC tokens ranks its candidates with
// every workgroup instead, in separate launches (radix passes over the
// composite, then a counting launch).
// Results do not depend on which workgroup finishes last.
#include <algorithm>
#include <atomic>
#include <mutex>

#include "tg_device.h"
#include "tg_kernels.h"

namespace tg {

namespace {

constexpr int SB = 256;                 // threads per workgroup
constexpr int SWAVES = SB / WAVE;
constexpr int SITEMS = 8;               // keys per thread
constexpr int SCHUNK = SB * SITEMS;     // 2048 keys per chunk
constexpr int NBIN = 2048;
constexpr int META = 10;                // u32 words of per-request metadata
constexpr int CTR = 16;                 // u32 counters per request (tickets, candidate count)
constexpr int NPASS = 6;                // radix passes over the 63-bit candidate composite
constexpr uint32_t RC_MAX = 384;        // candidates ranked by counting (linear bins)
constexpr int BIG_DOC = 1 << 20;        // documents above this rank their candidates with every workgroup
constexpr int RANK_WG = 512;            // workgroups of the many-workgroup candidate passes, at most
constexpr uint32_t RANK_PER_WG = 4 * SB; // candidates per workgroup of those passes, at least
constexpr uint32_t CAND_LDS = 8192;     // threshold-bin candidates staged in LDS
constexpr int MAX_GROUPS = 2048;        // workgroups of launches 2-4 at most (chunks grouped beyond)
static_assert(SCHUNK <= (int)CAND_LDS, "one chunk's candidates fit the staging list");
static_assert(SCHUNK < 65536, "per-chunk counts share one 32-bit scan");

__device__ __forceinline__ uint32_t order_key(float f) {
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7fffffffu) > 0x7f800000u) return 0u;  // NaN: lowest of all
    if (u == 0x80000000u) u = 0u;                     // -0 -> +0
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Rank key of a candidate inside the threshold bin (whose keys share no key
// bits): the whole key, then 0x7fffffff - index, so that larger = better and
// unique (63 bits).  Its radix digits are 11 + 11 + 10 + 11 + 10 + 10 bits
// from the top.
__device__ __forceinline__ uint64_t composite(uint32_t key, uint32_t idx) {
    return ((uint64_t)key << 31) | (uint64_t)(0x7fffffffu - idx);
}
__device__ __forceinline__ int pass_shift(int p) {
    return p == 0 ? 52 : (p == 1 ? 41 : (p == 2 ? 31 : (p == 3 ? 20 : (p == 4 ? 10 : 0))));
}
__device__ __forceinline__ int pass_width(int p) { return (p == 0 || p == 1 || p == 3) ? 11 : 10; }

// Bin of score v among NBIN bins linear in the value over the range
// [vmin, vmin + (NBIN - 2) / scale], clamped to the end bins (NaN and -inf
// to bin 0, +inf to the last), so monotone in the selection order: a higher
// key never lands in a lower bin, and -0 and +0 share a bin.  A zero scale
// puts every score in bin 0.
__device__ __forceinline__ uint32_t lin_bin(float v, float vmin, float scale) {
    const float f = (v - vmin) * scale;
    if (!(f >= 1.0f)) return 0u;  // below the range, NaN
    return f < (float)(NBIN - 1) ? (uint32_t)f : (uint32_t)(NBIN - 1);
}

// The range of the linear bins from the finite scores among `vals` (n of
// them over the workgroup, `valid` marking this thread's): their mean +- 8
// standard deviations, within their min and max; *vlo and *scale as
// lin_bin takes them.  Every thread gets the same bits, and so does every
// workgroup that reduces the same values in the same thread layout.
template <int NT, int NV, class Vals>
__device__ __forceinline__ void value_range(Vals vals, float* red, float* out_lo, float* out_scale) {
    constexpr int NW = NT / WAVE;
    const int lane = lane_id(), w = threadIdx.x / WAVE;
    float vmin = INFINITY, vmax = -INFINITY, sum = 0.f, sq = 0.f, cnt_f = 0.f;
#pragma unroll
    for (int e = 0; e < NV; ++e) {
        bool ok;
        const float v = vals(e, &ok);
        if (ok && fabsf(v) <= 3.402823466e38f) {  // finite
            vmin = fminf(vmin, v);
            vmax = fmaxf(vmax, v);
            sum += v;
            sq = fmaf(v, v, sq);
            cnt_f += 1.f;
        }
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
        vmin = fminf(vmin, __shfl_xor(vmin, o, WAVE));
        vmax = fmaxf(vmax, __shfl_xor(vmax, o, WAVE));
        sum += __shfl_xor(sum, o, WAVE);
        sq += __shfl_xor(sq, o, WAVE);
        cnt_f += __shfl_xor(cnt_f, o, WAVE);
    }
    if (lane == 0) {
        red[w] = vmin;
        red[NW + w] = vmax;
        red[2 * NW + w] = sum;
        red[3 * NW + w] = sq;
        red[4 * NW + w] = cnt_f;
    }
    __syncthreads();
    sum = sq = cnt_f = 0.f;
#pragma unroll
    for (int i = 0; i < NW; ++i) {
        vmin = fminf(vmin, red[i]);
        vmax = fmaxf(vmax, red[NW + i]);
        sum += red[2 * NW + i];
        sq += red[3 * NW + i];
        cnt_f += red[4 * NW + i];
    }
    float lo = vmin, hi = vmax;
    if (cnt_f > 0.f) {
        const float mu = sum / cnt_f;
        const float sd = sqrtf(fmaxf(sq / cnt_f - mu * mu, 0.f));
        if (sd <= 3.402823466e38f) {
            lo = fmaxf(lo, mu - 8.f * sd);
            hi = fminf(hi, mu + 8.f * sd);
        }
    }
    // Bins of width (hi - lo) / (NBIN - 2) between the end bins; a
    // degenerate or non-finite range puts every score in bin 0.
    const float span = hi - lo;
    *out_scale = span > 0.f && span <= 3.402823466e38f ? (float)(NBIN - 2) / span : 0.f;
    *out_lo = lo >= -3.402823466e38f ? lo : 0.f;
}

__device__ __forceinline__ uint32_t coherent_load(const uint32_t* p) {
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ void coherent_store(uint32_t* p, uint32_t v) {
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ void coherent_store2(uint2* p, uint2 v) {
    __hip_atomic_store(reinterpret_cast<uint64_t*>(p), (uint64_t)v.x | ((uint64_t)v.y << 32),
                       __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Publishing to the last workgroup of a launch.  Everything one workgroup
// hands to another inside a launch is written with device-coherent atomic
// stores or atomic adds and read with device-coherent atomic loads, so no
// cache needs flushing; each wave only has to wait until its own writes are
// performed before the workgroup takes its ticket.  (A device-wide fence
// here would also write back and invalidate whole caches, which costs
// microseconds per workgroup.)
__device__ __forceinline__ void wait_own_writes() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

__device__ __forceinline__ uint2 coherent_load2(const uint2* p) {
    const uint64_t v = __hip_atomic_load(reinterpret_cast<const uint64_t*>(p), __ATOMIC_RELAXED,
                                         __HIP_MEMORY_SCOPE_AGENT);
    return make_uint2((uint32_t)v, (uint32_t)(v >> 32));
}

struct SelArgs {
    int32_t batch;
    int32_t off[TG_MAX_BATCH + 1];        // token offset of each request
    int32_t out[TG_MAX_BATCH + 1];        // kept-row offset of each request
    int32_t q[TG_MAX_BATCH];              // question tail
    int32_t p[TG_MAX_BATCH];              // template prefix (kept); the document is [p, N - q)
    int32_t doc_chunk0[TG_MAX_BATCH + 1]; // first document chunk (selecting requests only)
    int32_t all_chunk0[TG_MAX_BATCH + 1]; // first chunk over the whole request
    int32_t group;                        // chunks per workgroup of launches 2-4
    int32_t doc_group0[TG_MAX_BATCH + 1]; // first chunk group of each selecting request
    int32_t all_group0[TG_MAX_BATCH + 1]; // first chunk group over whole requests
    const float* scores;
    int32_t* kept;
    int32_t* cu_dev;
    uint32_t* hist;       // [B][NBIN]
    uint32_t* meta;       // [B][META]: d1, rem1, cnt1, cprefix lo/hi, cmask lo/hi, done,
                          //            bin range low, bin scale (float bits)
    uint32_t* ctr;        // [B][CTR]: hist ticket, candidate ticket, candidate count,
                          //           rank-pass tickets [4, 4+NPASS), count ticket 4+NPASS
    uint32_t* rank_hist;  // [B][NPASS][NBIN]: every pass of the many-workgroup ranking
    uint32_t* grp_kept;   // [doc groups]: kept candidates per chunk group (many-workgroup ranking only)
    int32_t big;          // rank candidates with every workgroup (some document > BIG_DOC)
    uint32_t* grp_def;    // [doc groups]: keys above d1 per chunk group
    uint32_t* grp_off;    // [doc groups]: output offset of the group's first kept document token
    uint2* cand;          // [T]: (key, local index), request b at off[b]
};

__device__ __forceinline__ int find_request(const int32_t* base, int batch, int blk) {
    int b = 0;
    while (b + 1 < batch && base[b + 1] <= blk) ++b;
    return b;
}

// Keys c*SCHUNK + 8*tid + e (e < 8) of a document's chunk c, as two 16-byte
// loads per thread through a buffer resource bounded by the chunk's end, so
// that positions past the document read as 0 (callers skip them).  The
// histogram and the candidate pass do not depend on which thread holds which
// key; the compaction, which writes in order, keeps its own layout.
struct Chunk8 {
    f32x4 v[2];
};
__device__ __forceinline__ Chunk8 load_chunk8(const float* doc, int ndoc, int c) {
    const int lo = c * SCHUNK;
    const int n = min(SCHUNK, ndoc - lo);
    const __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(doc + lo), (short)0, n > 0 ? n * 4 : 0, BUFFER_RSRC_WORD3);
    Chunk8 x;
    // Whole vectors are reinterpreted (a bit cast of one element of a
    // u32x4 yielded element 0 for every index with this toolchain).
    x.v[0] = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(r, 32 * (int)threadIdx.x, 0, 0));
    x.v[1] = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(r, 32 * (int)threadIdx.x + 16, 0, 0));
    return x;
}

// Inclusive block scan (256 threads) of v; *total gets the sum.
__device__ __forceinline__ uint32_t block_incl_scan(uint32_t v, uint32_t* wtot, uint32_t* total) {
    const int lane = lane_id(), w = threadIdx.x / WAVE;
#pragma unroll
    for (int o = 1; o < WAVE; o <<= 1) {
        const uint32_t n = __shfl_up(v, o, WAVE);
        if (lane >= o) v += n;
    }
    if (lane == WAVE - 1) wtot[w] = v;
    __syncthreads();
    uint32_t before = 0, all = 0;
#pragma unroll
    for (int i = 0; i < SWAVES; ++i) {
        if (i < w) before += wtot[i];
        all += wtot[i];
    }
    __syncthreads();
    if (total != nullptr) *total = all;
    return v + before;
}

// Over `nb` bins (multiple of SB) of hist (LDS or global via loader), find the
// bin d with count(bins > d) < rem <= count(bins >= d).  Results go to *out_d,
// *out_gt, *out_cnt (shared) from the owning thread.
template <class Get>
__device__ __forceinline__ void find_bin(Get get, int nb, uint32_t rem, uint32_t* wtot,
                                         uint32_t* out_d, uint32_t* out_gt, uint32_t* out_cnt) {
    const int per = nb / SB;
    const int g = SB - 1 - (int)threadIdx.x;  // descending bin groups in thread order
    uint32_t vals[NBIN / SB];
    uint32_t gs = 0;
    for (int j = 0; j < per; ++j) {
        vals[j] = get(g * per + j);
        gs += vals[j];
    }
    uint32_t incl = block_incl_scan(gs, wtot, nullptr);
    uint32_t ge = incl - gs;
    for (int j = per - 1; j >= 0; --j) {
        const uint32_t gt = ge;
        ge += vals[j];
        if (gt < rem && rem <= ge) {
            *out_d = (uint32_t)(g * per + j);
            *out_gt = gt;
            *out_cnt = vals[j];
        }
    }
    __syncthreads();
}

// ------------------------------------------------------------- launch 1 ----
__global__ __launch_bounds__(SB) void sel_clear_kernel(uint32_t* hist, uint32_t* ctr, int n_hist,
                                                       int n_ctr, uint32_t* rank_hist, int n_rank,
                                                       uint32_t* grp_kept, int n_kept) {
    const int i = blockIdx.x * SB + threadIdx.x;
    if (i < n_hist) hist[i] = 0u;
    if (i < n_ctr) ctr[i] = 0u;
    if (i < n_rank) rank_hist[i] = 0u;
    if (i < n_kept) grp_kept[i] = 0u;
}

// ------------------------------------------------------------- launch 2 ----
// The bin range comes from the document's first chunk, which every workgroup
// reduces the same way; the last one publishes it in the request's metadata
// for launches 3 and 4.
__global__ __launch_bounds__(SB) void sel_hist_kernel(SelArgs a) {
    __shared__ uint32_t h[NBIN];
    __shared__ uint32_t wtot[SWAVES];
    __shared__ float red[5 * SWAVES];
    __shared__ uint32_t sh_last, sh_d, sh_gt, sh_cnt;
    const int tid = threadIdx.x;
    const int b = find_request(a.doc_group0, a.batch, blockIdx.x);
    const int grp = blockIdx.x - a.doc_group0[b];
    const int ngrp = a.doc_group0[b + 1] - a.doc_group0[b];
    const int nck = a.doc_chunk0[b + 1] - a.doc_chunk0[b];
    const int N = a.off[b + 1] - a.off[b];
    const int ndoc = N - a.q[b] - a.p[b];
    const int kdoc = a.out[b + 1] - a.out[b] - a.q[b] - a.p[b];
    const float* s = a.scores + a.off[b] + a.p[b];  // document tokens, indexed from 0
    const int c_lo = grp * a.group, c_hi = min(c_lo + a.group, nck);

    for (int i = tid; i < NBIN; i += SB) h[i] = 0u;
    // The chunks of this group, the keys of the next one loaded before the
    // histogram of the current one.
    static_assert(SITEMS == 8, "two 16-byte loads per thread and chunk");
    Chunk8 nxt = load_chunk8(s, ndoc, c_lo);
    float vlo, scale;
    {
        const Chunk8 z = c_lo == 0 ? nxt : load_chunk8(s, ndoc, 0);
        value_range<SB, SITEMS>(
            [&](int e, bool* ok) {
                *ok = SITEMS * tid + e < ndoc;
                return z.v[e / 4][e % 4];
            },
            red, &vlo, &scale);
    }
    for (int c = c_lo; c < c_hi; ++c) {
        const Chunk8 cur = nxt;
        if (c + 1 < c_hi) nxt = load_chunk8(s, ndoc, c + 1);
#pragma unroll
        for (int e = 0; e < SITEMS; ++e) {
            const int i = c * SCHUNK + SITEMS * tid + e;
            const float v = cur.v[e / 4][e % 4];
            if (i < ndoc) atomicAdd(&h[lin_bin(v, vlo, scale)], 1u);
        }
    }
    __syncthreads();
    uint32_t* gh = a.hist + (size_t)b * NBIN;
    for (int i = tid; i < NBIN; i += SB)
        if (h[i] != 0u) atomicAdd(&gh[i], h[i]);
    wait_own_writes();
    __syncthreads();
    if (tid == 0) sh_last = atomicAdd(&a.ctr[b * CTR + 0], 1u) == (uint32_t)(ngrp - 1);
    __syncthreads();
    if (!sh_last) return;
    find_bin([&](int i) { return coherent_load(&gh[i]); }, NBIN, (uint32_t)kdoc, wtot, &sh_d,
             &sh_gt, &sh_cnt);
    if (tid == 0) {
        uint32_t* m = a.meta + b * META;
        m[0] = sh_d;
        m[1] = (uint32_t)kdoc - sh_gt;
        m[2] = sh_cnt;
        m[8] = __float_as_uint(vlo);
        m[9] = __float_as_uint(scale);
    }
}

// ------------------------------------------------------------- launch 3 ----
// BIG: the batch ranks its candidates with every workgroup afterwards
// (sel_rank_kernel), so the last workgroup here only publishes the start of
// the ranking, and LDS holds just the staging list (a chunk's candidates at
// most): four times as many workgroups per CU.  Else the last workgroup ranks.
template <bool BIG>
__global__ __launch_bounds__(SB) void sel_cand_kernel(SelArgs a) {
    constexpr uint32_t CL = BIG ? (uint32_t)SCHUNK : CAND_LDS;
    __shared__ uint32_t wtot[SWAVES];
    __shared__ uint32_t sh_base, sh_last, sh_d, sh_gt, sh_cnt, sh_total;
    __shared__ uint64_t sh_t;
    __shared__ uint32_t h[BIG ? 1 : NBIN];
    __shared__ uint2 cl[CL];
    const int tid = threadIdx.x;
    const int b = find_request(a.doc_group0, a.batch, blockIdx.x);
    const int grp = blockIdx.x - a.doc_group0[b];
    const int ngrp = a.doc_group0[b + 1] - a.doc_group0[b];
    const int nck = a.doc_chunk0[b + 1] - a.doc_chunk0[b];
    const int N = a.off[b + 1] - a.off[b];
    const int ndoc = N - a.q[b] - a.p[b];
    const float* s = a.scores + a.off[b] + a.p[b];  // document tokens, indexed from 0
    uint32_t* m = a.meta + b * META;
    const uint32_t d1 = m[0];
    const float vlo = __uint_as_float(m[8]), scale = __uint_as_float(m[9]);
    uint2* cand = a.cand + a.off[b];
    const int c_lo = grp * a.group, c_hi = min(c_lo + a.group, nck);

    // Per chunk of the group: the count of keys above d1 (summed over the
    // group for its output offset), and the keys in d1 staged in LDS with
    // their index; the group's candidates then go to the request's list with
    // one atomic.
    uint32_t run = 0;        // candidates staged in cl (the same in every thread)
    uint32_t grp_above = 0;  // keys above d1 in the group's chunks so far
    // Move the staged candidates to the request's list (one atomic for all);
    // `more`: the list is refilled afterwards.
    auto flush = [&](bool more) {
        if (tid == 0) sh_base = run ? atomicAdd(&a.ctr[b * CTR + 2], run) : 0u;
        __syncthreads();
        for (uint32_t j = tid; j < run; j += SB) coherent_store2(&cand[sh_base + j], cl[j]);
        if (more) __syncthreads();
        run = 0;
    };
    Chunk8 nxt = load_chunk8(s, ndoc, c_lo);
    for (int c = c_lo; c < c_hi; ++c) {
        float cur[SITEMS];
        uint32_t bn[SITEMS];
#pragma unroll
        for (int e = 0; e < SITEMS; ++e) {
            cur[e] = nxt.v[e / 4][e % 4];
            bn[e] = lin_bin(cur[e], vlo, scale);
        }
        if (c + 1 < c_hi) nxt = load_chunk8(s, ndoc, c + 1);
        uint32_t above = 0, ncand = 0;
#pragma unroll
        for (int e = 0; e < SITEMS; ++e) {
            const int i = c * SCHUNK + SITEMS * tid + e;
            if (i < ndoc) {
                above += bn[e] > d1;
                ncand += bn[e] == d1;
            }
        }
        // One scan for both counts (each at most SCHUNK per chunk, so the
        // two 16-bit halves never carry into each other).
        uint32_t tot2;
        const uint32_t incl2 = block_incl_scan((above << 16) | ncand, wtot, &tot2);
        const uint32_t tot_above = tot2 >> 16, tot_cand = tot2 & 0xffffu;
        const uint32_t incl = incl2 & 0xffffu;
        grp_above += tot_above;
        if (run + tot_cand > CL) flush(true);
        uint32_t pos = run + incl - ncand;
#pragma unroll
        for (int e = 0; e < SITEMS; ++e) {
            const int i = c * SCHUNK + SITEMS * tid + e;
            if (i < ndoc && bn[e] == d1) cl[pos++] = make_uint2(order_key(cur[e]), (uint32_t)i);
        }
        run += tot_cand;
    }
    flush(false);
    if (tid == 0) coherent_store(&a.grp_def[a.doc_group0[b] + grp], grp_above);
    wait_own_writes();
    __syncthreads();
    if (tid == 0) sh_last = atomicAdd(&a.ctr[b * CTR + 1], 1u) == (uint32_t)(ngrp - 1);
    __syncthreads();
    if (!sh_last) return;

    if constexpr (BIG) {
        // Ranking is left to the many-workgroup passes (sel_rank_kernel).
        if (tid == 0) {
            m[3] = m[4] = m[5] = m[6] = 0u;
            m[7] = 0u;
        }
        return;
    } else {

    // ---- the last chunk: exact rank inside bin d1 --------------------------
    // The bin's candidates (usually a few dozen to a few hundred) are staged
    // in LDS once, eight device-coherent loads in flight per thread.  Up to
    // RC_MAX of them are ranked by counting, for each, the candidates that
    // beat it under (key desc, index asc); the rem-th best gives the
    // threshold composite.  A bigger bin (heavy ties, or scores the first
    // chunk did not represent) is ranked by LDS radix passes over the
    // composite instead, read from global memory on every pass when it does
    // not fit in LDS.
    const uint32_t cnt1 = m[2];
    const bool in_lds = cnt1 <= CAND_LDS;
    constexpr int CB = 8;  // candidate loads in flight per thread
    auto for_cands = [&](auto f) {  // f(candidate) over all cnt1 candidates
        if (in_lds) {
            for (uint32_t j = tid; j < cnt1; j += SB) f(cl[j]);
            return;
        }
        for (uint32_t j0 = 0; j0 < cnt1; j0 += CB * SB) {
            uint2 e[CB];
#pragma unroll
            for (int u = 0; u < CB; ++u) {
                const uint32_t j = j0 + u * SB + tid;
                e[u] = j < cnt1 ? coherent_load2(&cand[j]) : make_uint2(0u, 0u);
            }
#pragma unroll
            for (int u = 0; u < CB; ++u)
                if (j0 + u * SB + tid < cnt1) f(e[u]);
        }
    };
    if (in_lds) {
        for (uint32_t j0 = 0; j0 < cnt1; j0 += CB * SB) {
            uint2 e[CB];
#pragma unroll
            for (int u = 0; u < CB; ++u) {
                const uint32_t j = j0 + u * SB + tid;
                e[u] = j < cnt1 ? coherent_load2(&cand[j]) : make_uint2(0u, 0u);
            }
#pragma unroll
            for (int u = 0; u < CB; ++u) {
                const uint32_t j = j0 + u * SB + tid;
                if (j < cnt1) cl[j] = e[u];
            }
        }
    }
    __syncthreads();
    uint32_t rem = m[1];  // 1 <= rem <= cnt1
    uint64_t cprefix = 0, cmask = 0;
    if (cnt1 <= RC_MAX) {
        for (uint32_t c = tid; c < cnt1; c += SB) {
            const uint2 me = cl[c];
            uint32_t r0 = 0, r1 = 0, r2 = 0, r3 = 0;
            uint32_t o = 0;
            for (; o + 4 <= cnt1; o += 4) {
                const uint2 e0 = cl[o], e1 = cl[o + 1], e2 = cl[o + 2], e3 = cl[o + 3];
                r0 += (e0.x > me.x) || (e0.x == me.x && e0.y < me.y);
                r1 += (e1.x > me.x) || (e1.x == me.x && e1.y < me.y);
                r2 += (e2.x > me.x) || (e2.x == me.x && e2.y < me.y);
                r3 += (e3.x > me.x) || (e3.x == me.x && e3.y < me.y);
            }
            for (; o < cnt1; ++o) {
                const uint2 e0 = cl[o];
                r0 += (e0.x > me.x) || (e0.x == me.x && e0.y < me.y);
            }
            if (r0 + r1 + r2 + r3 == rem - 1) sh_t = composite(me.x, me.y);
        }
        __syncthreads();
        cprefix = sh_t;  // the kept candidates: composite >= the rem-th best
        cmask = ~0ull;
    } else {
        uint32_t cnt = cnt1;  // candidates matching the prefix fixed so far
#pragma unroll 1
        for (int p = 0; p < NPASS && cnt != rem; ++p) {
            const int sh = pass_shift(p);
            const int nb = 1 << pass_width(p);
            for (int i = tid; i < NBIN; i += SB) h[i] = 0u;
            __syncthreads();
            for_cands([&](uint2 e) {
                const uint64_t cp = composite(e.x, e.y);
                if ((cp & cmask) == cprefix) atomicAdd(&h[(cp >> sh) & (uint64_t)(nb - 1)], 1u);
            });
            __syncthreads();
            find_bin([&](int i) { return h[i]; }, nb, rem, wtot, &sh_d, &sh_gt, &sh_cnt);
            rem -= sh_gt;
            cprefix |= (uint64_t)sh_d << sh;
            cmask |= (uint64_t)(nb - 1) << sh;
            cnt = sh_cnt;
            __syncthreads();
        }
        // Every composite with this prefix is kept (cnt == rem), or the
        // prefix covers all 63 bits.
    }

    // Kept candidates per chunk group, then exclusive offsets of all groups
    // (the compaction accumulates the chunks of its group itself).
    uint32_t* gcnt = h;  // reuse: up to NBIN groups handled per round
    const uint32_t* gdef = a.grp_def + a.doc_group0[b];
    uint32_t* goff = a.grp_off + a.doc_group0[b];
    const int G = a.group;
    uint32_t carry = 0;
    for (int g0 = 0; g0 < ngrp; g0 += NBIN) {
        for (int i = tid; i < NBIN; i += SB) h[i] = 0u;
        __syncthreads();
        for_cands([&](uint2 e) {
            const int gi = (int)(e.y / SCHUNK) / G - g0;
            if (gi >= 0 && gi < NBIN && (composite(e.x, e.y) & cmask) >= cprefix)
                atomicAdd(&gcnt[gi], 1u);
        });
        __syncthreads();
        // each thread owns NBIN/SB consecutive groups
        constexpr int per = NBIN / SB;
        uint32_t v[per];
        uint32_t sum = 0;
#pragma unroll
        for (int j = 0; j < per; ++j) {
            const int gg = g0 + tid * per + j;
            v[j] = gg < ngrp ? coherent_load(&gdef[gg]) : 0u;
        }
#pragma unroll
        for (int j = 0; j < per; ++j) {
            const int gg = g0 + tid * per + j;
            if (gg < ngrp) v[j] += gcnt[tid * per + j];
            sum += v[j];
        }
        const uint32_t incl2 = block_incl_scan(sum, wtot, &sh_total);
        uint32_t run = carry + incl2 - sum;
        for (int j = 0; j < per; ++j) {
            const int gg = g0 + tid * per + j;
            if (gg < ngrp) goff[gg] = run;
            run += v[j];
        }
        carry += sh_total;
        __syncthreads();
    }
    if (tid == 0) {
        m[3] = (uint32_t)cprefix;
        m[4] = (uint32_t)(cprefix >> 32);
        m[5] = (uint32_t)cmask;
        m[6] = (uint32_t)(cmask >> 32);
    }
    }  // !BIG
}

// ------------------------------------ large documents: ranking by all ----
// The same radix passes over the candidate composite as the last chunk runs
// above, with the candidate list of every selecting request spread over
// RANK_WG workgroups: each histograms its share of the candidates that match
// the prefix fixed so far (LDS, then global atomics), and the workgroup that
// finishes last picks the digit and updates the request's prefix.  Launched
// once per pass; a request whose rank is already fixed is skipped.  A request
// takes one workgroup per RANK_PER_WG candidates, at most RANK_WG (the others
// skip it), so that a few thousand candidates do not pay for hundreds of
// histogram flushes and tickets.
__device__ __forceinline__ uint32_t rank_workgroups(uint32_t cnt) {
    return min((uint32_t)RANK_WG, max(1u, (cnt + RANK_PER_WG - 1) / RANK_PER_WG));
}

__global__ __launch_bounds__(SB) void sel_rank_kernel(SelArgs a, int p) {
    __shared__ uint32_t h[NBIN];
    __shared__ uint32_t wtot[SWAVES];
    __shared__ uint32_t sh_last, sh_d, sh_gt, sh_cnt;
    const int tid = threadIdx.x;
    const int sh = pass_shift(p), nb = 1 << pass_width(p);
    for (int b = 0; b < a.batch; ++b) {
        if (a.doc_chunk0[b + 1] == a.doc_chunk0[b]) continue;  // not selecting
        uint32_t* m = a.meta + b * META;
        if (m[7] != 0u) continue;  // rank already fixed by an earlier pass
        const uint32_t cnt1 = m[2];
        const uint32_t nwg = rank_workgroups(cnt1);
        if (blockIdx.x >= nwg) continue;
        const uint64_t cprefix = (uint64_t)m[3] | ((uint64_t)m[4] << 32);
        const uint64_t cmask = (uint64_t)m[5] | ((uint64_t)m[6] << 32);
        const uint2* cand = a.cand + a.off[b];
        for (int i = tid; i < nb; i += SB) h[i] = 0u;
        __syncthreads();
        for (uint32_t j = blockIdx.x * SB + tid; j < cnt1; j += nwg * SB) {
            const uint2 e = cand[j];
            const uint64_t cp = composite(e.x, e.y);
            if ((cp & cmask) == cprefix) atomicAdd(&h[(cp >> sh) & (uint64_t)(nb - 1)], 1u);
        }
        __syncthreads();
        uint32_t* gh = a.rank_hist + ((size_t)b * NPASS + p) * NBIN;
        for (int i = tid; i < nb; i += SB)
            if (h[i] != 0u) atomicAdd(&gh[i], h[i]);
        wait_own_writes();
        __syncthreads();
        if (tid == 0) sh_last = atomicAdd(&a.ctr[b * CTR + 4 + p], 1u) == nwg - 1;
        __syncthreads();
        if (sh_last) {
            const uint32_t rem = m[1];
            find_bin([&](int i) { return coherent_load(&gh[i]); }, nb, rem, wtot, &sh_d, &sh_gt,
                     &sh_cnt);
            if (tid == 0) {
                const uint32_t rem2 = rem - sh_gt;
                const uint64_t np = cprefix | ((uint64_t)sh_d << sh);
                const uint64_t nm = cmask | ((uint64_t)(nb - 1) << sh);
                m[1] = rem2;
                m[3] = (uint32_t)np;
                m[4] = (uint32_t)(np >> 32);
                m[5] = (uint32_t)nm;
                m[6] = (uint32_t)(nm >> 32);
                if (sh_cnt == rem2) m[7] = 1u;  // every composite with this prefix is kept
            }
        }
        __syncthreads();
    }
}

// Kept candidates per chunk group (global atomics over the workgroups), then
// the workgroup finishing last scans the groups' kept counts into their
// output offsets, as the last chunk of sel_cand does for small documents.
__global__ __launch_bounds__(SB) void sel_rankcount_kernel(SelArgs a) {
    __shared__ uint32_t wtot[SWAVES];
    __shared__ uint32_t sh_last, sh_total;
    const int tid = threadIdx.x;
    const int G = a.group;
    for (int b = 0; b < a.batch; ++b) {
        if (a.doc_chunk0[b + 1] == a.doc_chunk0[b]) continue;
        const uint32_t* m = a.meta + b * META;
        const uint32_t cnt1 = m[2];
        const uint32_t nwg = rank_workgroups(cnt1);
        if (blockIdx.x >= nwg) continue;
        const uint64_t cprefix = (uint64_t)m[3] | ((uint64_t)m[4] << 32);
        const uint64_t cmask = (uint64_t)m[5] | ((uint64_t)m[6] << 32);
        const uint2* cand = a.cand + a.off[b];
        uint32_t* kc = a.grp_kept + a.doc_group0[b];
        // Candidates of one group sit next to each other in the list (each
        // group appends its candidates in one block), so a wave's kept
        // candidates usually span one or two groups: one atomic per distinct
        // group of the wave instead of one per candidate.
        const uint32_t lane = lane_id();
        for (uint32_t j0 = blockIdx.x * SB; j0 < cnt1; j0 += nwg * SB) {
            const uint32_t j = j0 + tid;
            bool kept = false;
            uint32_t gi = 0;
            if (j < cnt1) {
                const uint2 e = cand[j];
                kept = (composite(e.x, e.y) & cmask) >= cprefix;
                gi = e.y / SCHUNK / (uint32_t)G;
            }
            uint64_t todo = __ballot(kept);
            while (todo != 0ull) {
                const uint32_t lead = (uint32_t)__builtin_ctzll(todo);
                const uint32_t lg = (uint32_t)__shfl((int)gi, (int)lead, WAVE);
                const uint64_t same = __ballot(kept && gi == lg);
                if (lane == lead) atomicAdd(&kc[lg], (uint32_t)__popcll(same));
                todo &= ~same;
            }
        }
        wait_own_writes();
        __syncthreads();
        if (tid == 0) sh_last = atomicAdd(&a.ctr[b * CTR + 4 + NPASS], 1u) == nwg - 1;
        __syncthreads();
        if (!sh_last) continue;
        const int ngrp = a.doc_group0[b + 1] - a.doc_group0[b];  // at most MAX_GROUPS
        const uint32_t* gdef = a.grp_def + a.doc_group0[b];
        uint32_t* goff = a.grp_off + a.doc_group0[b];
        // Thread t owns the contiguous groups [t per, (t+1) per), per <= 8:
        // one batch of loads, one block scan.
        const int per = (ngrp + SB - 1) / SB;
        const int cb = min(tid * per, ngrp), ce = min(cb + per, ngrp);
        constexpr int LB = MAX_GROUPS / SB;
        uint32_t v[LB];
        uint32_t sum = 0;
#pragma unroll
        for (int u = 0; u < LB; ++u) {
            const int gg = cb + u;
            v[u] = gg < ce ? coherent_load(&kc[gg]) + coherent_load(&gdef[gg]) : 0u;
            sum += v[u];
        }
        const uint32_t incl = block_incl_scan(sum, wtot, &sh_total);
        uint32_t run = incl - sum;
#pragma unroll
        for (int u = 0; u < LB; ++u) {
            if (cb + u < ce) goff[cb + u] = run;
            run += v[u];
        }
        __syncthreads();
    }
}

// ------------------------------------------------------------- launch 4 ----
__global__ __launch_bounds__(SB) void sel_compact_kernel(SelArgs a) {
    __shared__ uint32_t wtot[SWAVES];
    const int tid = threadIdx.x;
    const int b = find_request(a.all_group0, a.batch, blockIdx.x);
    const int grp = blockIdx.x - a.all_group0[b];
    if (blockIdx.x == 0 && a.cu_dev != nullptr)
        for (int i = tid; i <= a.batch; i += SB) a.cu_dev[i] = a.out[i];
    const int off = a.off[b];
    const int N = a.off[b + 1] - off;
    const int q = a.q[b];
    const int pf = a.p[b];
    const int out = a.out[b];
    const int keep = a.out[b + 1] - out;
    const int ndoc = N - q - pf;
    const int kdoc = keep - q - pf;
    const float* s = a.scores + off + pf;
    const int c_lo = grp * a.group, c_hi = min(c_lo + a.group, (N + SCHUNK - 1) / SCHUNK);
    const bool doc = keep < N && kdoc > 0;  // the document is selected from
    // Scores of chunk c of the document, thread t holding positions
    // c*SCHUNK + 8t .. 8t+7; the next chunk's are loaded before the current
    // one is written.
    Chunk8 nxt = {};
    if (doc) nxt = load_chunk8(s, ndoc, c_lo);
    // Output position of the next kept document token of this group: the
    // group's offset, then the kept tokens of its chunks so far.
    uint32_t run_off = 0;
    bool have_off = false;
    for (int c = c_lo; c < c_hi; ++c) {  // the chunks of this group, in order
        const Chunk8 cur = nxt;
        if (doc && c + 1 < c_hi) nxt = load_chunk8(s, ndoc, c + 1);
        const int lo = c * SCHUNK;
        const int hi = min(lo + SCHUNK, N);
        if (keep >= N) {
            for (int i = lo + tid; i < hi; i += SB) a.kept[out + i] = off + i;
            continue;
        }
        // The always-kept tokens, prefix then question, as one list of
        // pf + q <= N entries shared out by chunk: prefix token f goes to
        // output f, question token f - pf after the prefix and the kept
        // document tokens.
        for (int f = lo + tid; f < min(lo + SCHUNK, pf + q); f += SB) {
            const int i = f < pf ? f : N - q + (f - pf);
            a.kept[out + (f < pf ? f : pf + kdoc + (f - pf))] = off + i;
        }
        // Chunk c of the document: document tokens [lo, lo + SCHUNK), at
        // request positions pf + i, written after the prefix in order: each
        // thread's kept keys (8 consecutive positions) after those of the
        // threads before it (one block scan).
        if (kdoc <= 0 || lo >= ndoc) continue;

        const uint32_t* m = a.meta + b * META;
        const uint32_t d1 = m[0];
        const uint64_t cprefix = (uint64_t)m[3] | ((uint64_t)m[4] << 32);
        const uint64_t cmask = (uint64_t)m[5] | ((uint64_t)m[6] << 32);
        const float vlo = __uint_as_float(m[8]), scale = __uint_as_float(m[9]);
        if (!have_off) {  // the first document chunk of this group
            run_off = a.grp_off[a.doc_group0[b] + grp];
            have_off = true;
        }
        const int i0 = lo + SITEMS * tid;
        uint32_t km = 0u;
#pragma unroll
        for (int e = 0; e < SITEMS; ++e) {
            const int i = i0 + e;
            if (i < ndoc) {
                const float v = cur.v[e / 4][e % 4];
                const uint32_t key = order_key(v);
                const uint32_t dg = lin_bin(v, vlo, scale);
                if (dg > d1 || (dg == d1 && (composite(key, (uint32_t)i) & cmask) >= cprefix))
                    km |= 1u << e;
            }
        }
        const uint32_t n = (uint32_t)__popc(km);
        uint32_t tot;
        uint32_t pos = run_off + block_incl_scan(n, wtot, &tot) - n;
        run_off += tot;
#pragma unroll
        for (int e = 0; e < SITEMS; ++e) {
            if ((km >> e) & 1u) {
                if (pos < (uint32_t)kdoc) a.kept[out + pf + pos] = off + pf + i0 + e;
                ++pos;
            }
        }
    }
}

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

struct WsLayout {
    size_t hist, meta, ctr, def, off, cand, rank, kept, total;
};

WsLayout ws_layout(int batch, int doc_chunks, int64_t T) {
    WsLayout L;
    size_t p = 0;
    L.hist = p; p = align256(p + (size_t)batch * NBIN * 4);
    L.meta = p; p = align256(p + (size_t)batch * META * 4);
    L.ctr = p;  p = align256(p + (size_t)batch * CTR * 4);
    L.def = p;  p = align256(p + (size_t)doc_chunks * 4);  // per group (groups <= chunks)
    L.off = p;  p = align256(p + (size_t)doc_chunks * 4);
    L.cand = p; p = align256(p + (size_t)T * 8);
    L.rank = p; p = align256(p + (size_t)batch * NPASS * NBIN * 4);
    L.kept = p; p = align256(p + (size_t)doc_chunks * 4);
    L.total = p;
    return L;
}

void chunk_plan(const BatchArgs& a, SelArgs* s, int* doc_chunks, int* all_chunks) {
    int dc = 0, ac = 0;
    for (int b = 0; b < a.batch; ++b) {
        const int N = a.cu_seq[b + 1] - a.cu_seq[b];
        const int keep = a.cu_kept[b + 1] - a.cu_kept[b];
        const int ndoc = N - a.q_len[b] - a.p_len[b];
        const bool selecting = keep < N && keep - a.q_len[b] - a.p_len[b] > 0;
        if (s != nullptr) {
            s->doc_chunk0[b] = dc;
            s->all_chunk0[b] = ac;
        }
        if (selecting) dc += (ndoc + SCHUNK - 1) / SCHUNK;
        ac += (N + SCHUNK - 1) / SCHUNK;
    }
    if (s != nullptr) {
        s->doc_chunk0[a.batch] = dc;
        s->all_chunk0[a.batch] = ac;
        // Chunks per workgroup: one, unless that would need more than
        // MAX_GROUPS workgroups; then consecutive chunks of a request are
        // grouped, so that tickets, histogram flushes and candidate appends
        // (same-address atomics, which serialise) happen once per group.
        const int most = std::max(dc, ac);
        const int g = std::max(1, (most + MAX_GROUPS - 1) / MAX_GROUPS);
        s->group = g;
        int dg = 0, ag = 0;
        for (int b = 0; b < a.batch; ++b) {
            s->doc_group0[b] = dg;
            s->all_group0[b] = ag;
            dg += (s->doc_chunk0[b + 1] - s->doc_chunk0[b] + g - 1) / g;
            ag += (s->all_chunk0[b + 1] - s->all_chunk0[b] + g - 1) / g;
        }
        s->doc_group0[a.batch] = dg;
        s->all_group0[a.batch] = ag;
    }
    *doc_chunks = dc;
    *all_chunks = ac;
}

// ------------------------------------------------ one-workgroup path ----
// When every document of the batch has at most SELECT_ONE_WG_AUTO tokens
// (SELECT_ONE_WG_MAX when forced), each request is selected by one
// 1024-thread workgroup, the whole batch in a single launch.  Above 32768
// tokens the chunked path is faster: one CU streams the document once per
// pass, while the chunks spread it over the chip (measured at 65536 tokens:
// 37 against 28 us per call).  The document is read in rows of 4096 keys, thread t taking
// positions 4t .. 4t+3 of a row in one 16-byte load (a wave reads 1 KiB of
// consecutive scores per load), four rows at a time; the first four rows
// (16384 keys) stay in registers for every pass, later ones are re-read.
//   1. the first rows give a value range: their mean +- 8 standard
//      deviations within their min and max;
//   2. every score goes to one of 2048 bins linear in that value range
//      (scores outside it, NaN and infinities to the end bins).  The map is
//      monotone, so every key of a higher bin beats every key of a lower one
//      whatever the first rows missed, and a few outliers (planted needles,
//      say) do not stretch the range over the bulk of the scores.  Linear in
//      the value, it spreads gate scores evenly (the top bits of the float,
//      or bins linear in the order key, crowd them into a few, and the
//      histogram then stalls on same-address LDS atomics).  A descending scan
//      over the bins finds the bin d holding the K_doc-th best key and how
//      many of its keys are kept;
//   3. one pass collects the keys of bin d with their positions (usually a
//      few dozen) and counts, per (row, wave), the keys of higher bins; the
//      candidates are ranked exactly under (key descending, position
//      ascending) in LDS, the kept ones marked in a bitmap and added to their
//      (row, wave) counts, which one block scan turns into output offsets;
//   4. one pass writes the kept positions in order (wave ballots).
// When bin d holds more than S1_CAND keys (heavy ties), its keys are ranked by
// three radix passes over the 32-bit key instead (11, 11, 10 bits), which give
// the threshold key T and how many keys equal to T are kept (the lowest
// positions), and the counting pass also counts keys equal to T.
constexpr int S1_THREADS = 1024;
constexpr int S1_WAVES = S1_THREADS / WAVE;
constexpr int S1_KPT = 4;                        // consecutive keys per thread per row
constexpr int S1_ROW = S1_THREADS * S1_KPT;      // 4096 keys per row
constexpr int S1_GR = 4;                         // rows per group (loads in flight per thread)
constexpr int S1_GROUP = S1_ROW * S1_GR;         // 16384 keys per group
constexpr int S1_MAX = SELECT_ONE_WG_MAX;        // document tokens per request
constexpr int S1_ROWS = S1_MAX / S1_ROW;         // rows at most
constexpr int S1_NB = NBIN;                      // bins of the first histogram
constexpr int S1_CAND = 1024;                    // candidates ranked in LDS
constexpr int S1_BPT = S1_NB / S1_THREADS;       // bins per thread in the bin scans
static_assert(S1_MAX % S1_GROUP == 0 && S1_ROWS * S1_WAVES <= S1_THREADS, "rows");

// Exclusive block scan over the S1_THREADS threads of v; *total gets the sum.
__device__ __forceinline__ uint32_t s1_scan_excl(uint32_t v, uint32_t* wtot, uint32_t* total) {
    const int lane = lane_id(), w = threadIdx.x / WAVE;
    uint32_t x = v;
#pragma unroll
    for (int o = 1; o < WAVE; o <<= 1) {
        const uint32_t n = __shfl_up(x, o, WAVE);
        if (lane >= o) x += n;
    }
    if (lane == WAVE - 1) wtot[w] = x;
    __syncthreads();
    uint32_t before = 0, all = 0;
#pragma unroll
    for (int i = 0; i < S1_WAVES; ++i) {
        if (i < w) before += wtot[i];
        all += wtot[i];
    }
    __syncthreads();
    *total = all;
    return x - v + before;
}

// Over the S1_NB bins of hist, the bin d holding the rem-th largest element
// (count(bins > d) < rem <= count(bins >= d)): *d, the rank within it
// (*rank_in) and its count (*cnt), set by the owning thread.  Thread t owns
// the S1_BPT bins below S1_NB - S1_BPT t (descending order in thread order).
__device__ __forceinline__ void s1_find_bin(const uint32_t* hist, uint32_t rem, uint32_t* wtot,
                                            uint32_t* d, uint32_t* rank_in, uint32_t* cnt) {
    const int top = S1_NB - 1 - S1_BPT * (int)threadIdx.x;
    uint32_t c[S1_BPT], sum = 0;
#pragma unroll
    for (int k = 0; k < S1_BPT; ++k) {
        c[k] = hist[top - k];
        sum += c[k];
    }
    uint32_t tot;
    uint32_t above = s1_scan_excl(sum, wtot, &tot);
#pragma unroll
    for (int k = 0; k < S1_BPT; ++k) {
        if (above < rem && rem <= above + c[k]) {
            *d = (uint32_t)(top - k);
            *rank_in = rem - above;
            *cnt = c[k];
        }
        above += c[k];
    }
}

// In-place exclusive scan of n <= S1_THREADS counts in LDS (one per thread).
__device__ __forceinline__ void s1_scan_counts(uint32_t* c, int n, uint32_t* wtot) {
    const int t = threadIdx.x;
    const uint32_t v = t < n ? c[t] : 0u;
    uint32_t tot;
    const uint32_t e = s1_scan_excl(v, wtot, &tot);
    if (t < n) c[t] = e;
    __syncthreads();
}

// The keys of this thread in one group of S1_GR rows: v[r][e] is position
// S1_GROUP g + S1_ROW r + 4t + e (positions past the document read as 0 and
// are excluded by the caller).  Whole vectors are reinterpreted: a bit cast
// of one element of a u32x4 yielded element 0 for every index with this
// toolchain.
struct S1Group {
    f32x4 v[S1_GR];
};
__device__ __forceinline__ S1Group s1_load(__amdgpu_buffer_rsrc_t r, int g) {
    S1Group x;
    const int base = (g * S1_GROUP + S1_KPT * (int)threadIdx.x) * 4;
#pragma unroll
    for (int k = 0; k < S1_GR; ++k)
        x.v[k] = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(r, base + 4 * S1_ROW * k, 0, 0));
    return x;
}

// Run body(row index, keys of that row as f32x4) over the rows of the
// document: group 0 from registers (c0), later groups loaded per pass.
template <class Body>
__device__ __forceinline__ void s1_rows(__amdgpu_buffer_rsrc_t rs, int nrows, const S1Group& c0,
                                        Body body) {
#pragma unroll
    for (int k = 0; k < S1_GR; ++k)
        if (k < nrows) body(k, c0.v[k]);
    const int ngroups = (nrows + S1_GR - 1) / S1_GR;
    for (int g = 1; g < ngroups; ++g) {
        const S1Group x = s1_load(rs, g);
#pragma unroll
        for (int k = 0; k < S1_GR; ++k)
            if (g * S1_GR + k < nrows) body(g * S1_GR + k, x.v[k]);
    }
}

__global__ __launch_bounds__(S1_THREADS) void sel_one_kernel(SelArgs a) {
    __shared__ uint32_t hist[S1_NB];
    __shared__ uint32_t cnt[S1_ROWS * S1_WAVES];    // per (row, wave): kept keys
    __shared__ uint32_t eqc[S1_ROWS * S1_WAVES];    // per (row, wave): keys == T (ties path)
    __shared__ uint32_t bits[S1_MAX / 32];          // kept candidates
    __shared__ uint2 cand[S1_CAND];                 // (key, position) of the keys in bin d
    __shared__ uint32_t wtot[S1_WAVES];
    __shared__ float red[5 * S1_WAVES];
    __shared__ uint32_t sh_d, sh_rem, sh_cnt, sh_ncand;

    const int b = blockIdx.x, tid = threadIdx.x, w = tid / WAVE, lane = lane_id();
    if (b == 0 && a.cu_dev != nullptr)
        for (int i = tid; i <= a.batch; i += S1_THREADS) a.cu_dev[i] = a.out[i];
    const int off = a.off[b], N = a.off[b + 1] - off;
    const int out = a.out[b], K = a.out[b + 1] - out;
    int32_t* kept = a.kept + out;
    if (K >= N) {  // the budget covers the request
        for (int i = tid; i < N; i += S1_THREADS) kept[i] = off + i;
        return;
    }
    const int q = a.q[b], p = a.p[b];
    const int ndoc = N - q - p, kdoc = K - q - p;
    for (int i = tid; i < p; i += S1_THREADS) kept[i] = off + i;
    for (int i = tid; i < q; i += S1_THREADS) kept[p + kdoc + i] = off + N - q + i;
    if (kdoc <= 0) return;  // only the prefix and the question are kept
    const float* s = a.scores + off + p;  // document keys, positions 0..ndoc-1
    const __amdgpu_buffer_rsrc_t rs =
        __builtin_amdgcn_make_buffer_rsrc((void*)s, (short)0, ndoc * 4, BUFFER_RSRC_WORD3);
    const int nrows = (ndoc + S1_ROW - 1) / S1_ROW;
    const int nslot = nrows * S1_WAVES;
    const int pos0 = S1_KPT * tid;  // this thread's first position in a row
    int32_t* dst = kept + p;
    // The ranks of this lane's keys within its wave's slice of a row: keys
    // of lower lanes first, then this lane's in position order.
    auto lane_offset = [&](uint32_t m4) {  // m4: this lane's 4 flags
        uint32_t o = 0;
#pragma unroll
        for (int e = 0; e < S1_KPT; ++e) o += lanes_below(__ballot((m4 >> e) & 1u));
        return o;
    };
    auto wave_count = [&](uint32_t m4) {
        uint32_t c = 0;
#pragma unroll
        for (int e = 0; e < S1_KPT; ++e) c += (uint32_t)__popcll(__ballot((m4 >> e) & 1u));
        return c;
    };

    // ---- 1. value range from the first row -----------------------------------
    // (The other rows of the first group are still arriving meanwhile.)
    const S1Group c0 = s1_load(rs, 0);
    for (int i = tid; i < S1_NB; i += S1_THREADS) hist[i] = 0u;
    float vlo, scale;
    value_range<S1_THREADS, S1_KPT>(
        [&](int e, bool* ok) {
            *ok = pos0 + e < ndoc;
            return c0.v[0][e];
        },
        red, &vlo, &scale);

    // ---- 2. histogram, threshold bin ------------------------------------------
    // The bins of the first group's keys (in registers) are kept, two 16-bit
    // bins per word, for the candidate pass.
    uint32_t bq[S1_GR][S1_KPT / 2] = {};
    s1_rows(rs, nrows, c0, [&](int r, f32x4 x) {
        const int i0 = r * S1_ROW + pos0;
#pragma unroll
        for (int e = 0; e < S1_KPT; ++e) {
            const uint32_t bn = lin_bin(x[e], vlo, scale);
            if (r < S1_GR) bq[r][e / 2] |= bn << (16 * (e % 2));
            if (i0 + e < ndoc) atomicAdd(&hist[bn], 1u);
        }
    });
    __syncthreads();
    s1_find_bin(hist, (uint32_t)kdoc, wtot, &sh_d, &sh_rem, &sh_cnt);
    if (tid == 0) sh_ncand = 0u;
    for (int i = tid; i < (ndoc + 31) / 32; i += S1_THREADS) bits[i] = 0u;
    __syncthreads();
    const uint32_t d = sh_d, rem = sh_rem;

    if (sh_cnt <= (uint32_t)S1_CAND) {
        // ---- 3. candidates of bin d, counts of higher bins ---------------------
        // For the first group's rows (in registers) the masks of keys above
        // bin d and in bin d are kept for the write pass.
        uint32_t up0 = 0u, eq0 = 0u;
        s1_rows(rs, nrows, c0, [&](int r, f32x4 x) {
            const int i0 = r * S1_ROW + pos0;
            uint32_t up = 0u, eq = 0u;
#pragma unroll
            for (int e = 0; e < S1_KPT; ++e) {
                if (i0 + e < ndoc) {
                    const uint32_t bn = r < S1_GR ? (bq[r][e / 2] >> (16 * (e % 2))) & 0xFFFFu
                                                  : lin_bin(x[e], vlo, scale);
                    if (bn > d) up |= 1u << e;
                    if (bn == d) {
                        eq |= 1u << e;
                        cand[atomicAdd(&sh_ncand, 1u)] = make_uint2(order_key(x[e]), (uint32_t)(i0 + e));
                    }
                }
            }
            if (r < S1_GR) {
                up0 |= up << (S1_KPT * r);
                eq0 |= eq << (S1_KPT * r);
            }
            const uint32_t c = wave_count(up);
            if (lane == 0) cnt[r * S1_WAVES + w] = c;
        });
        __syncthreads();
        // Exact rank of each candidate under (key desc, position asc); the
        // first rem are kept.
        const uint32_t nc = sh_ncand;
        for (uint32_t c = tid; c < nc; c += S1_THREADS) {
            const uint2 me = cand[c];
            uint32_t r0 = 0, r1 = 0, r2 = 0, r3 = 0;
            uint32_t o = 0;
            for (; o + 4 <= nc; o += 4) {
                const uint2 e0 = cand[o], e1 = cand[o + 1], e2 = cand[o + 2], e3 = cand[o + 3];
                r0 += (e0.x > me.x) || (e0.x == me.x && e0.y < me.y);
                r1 += (e1.x > me.x) || (e1.x == me.x && e1.y < me.y);
                r2 += (e2.x > me.x) || (e2.x == me.x && e2.y < me.y);
                r3 += (e3.x > me.x) || (e3.x == me.x && e3.y < me.y);
            }
            for (; o < nc; ++o) {
                const uint2 e0 = cand[o];
                r0 += (e0.x > me.x) || (e0.x == me.x && e0.y < me.y);
            }
            if (r0 + r1 + r2 + r3 < rem) {
                atomicOr(&bits[me.y / 32], 1u << (me.y % 32));
                atomicAdd(&cnt[(me.y / S1_ROW) * S1_WAVES + (me.y % S1_ROW) / (S1_KPT * WAVE)], 1u);
            }
        }
        __syncthreads();
        s1_scan_counts(cnt, nslot, wtot);
        // ---- 4. ordered write ------------------------------------------------
        s1_rows(rs, nrows, c0, [&](int r, f32x4 x) {
            const int i0 = r * S1_ROW + pos0;
            uint32_t km = 0u;
            if (r < S1_GR) {
                // Keys above bin d are kept; of those in bin d (a few per
                // request) only the candidates marked in bits.
                km = (up0 >> (S1_KPT * r)) & 0xFu;
                const uint32_t eq = (eq0 >> (S1_KPT * r)) & 0xFu;
                if (eq != 0u) {
#pragma unroll
                    for (int e = 0; e < S1_KPT; ++e) {
                        const int i = i0 + e;
                        if (((eq >> e) & 1u) && ((bits[i / 32] >> (i % 32)) & 1u)) km |= 1u << e;
                    }
                }
            } else {
#pragma unroll
                for (int e = 0; e < S1_KPT; ++e) {
                    const int i = i0 + e;
                    if (i < ndoc) {
                        const uint32_t bn = lin_bin(x[e], vlo, scale);
                        if (bn > d || (bn == d && ((bits[i / 32] >> (i % 32)) & 1u))) km |= 1u << e;
                    }
                }
            }
            uint32_t pos = cnt[r * S1_WAVES + w] + lane_offset(km);
#pragma unroll
            for (int e = 0; e < S1_KPT; ++e) {
                if ((km >> e) & 1u) {
                    if (pos < (uint32_t)kdoc) dst[pos] = off + p + i0 + e;
                    ++pos;
                }
            }
        });
        return;
    }

    // ---- 3'. heavy ties: radix passes over the keys of bin d --------------
    uint32_t prefix = 0u, pmask = 0u, rr = rem;
    for (int pass = 0; pass < 3; ++pass) {
        const int shift = pass == 0 ? 21 : (pass == 1 ? 10 : 0);
        const int width = pass == 2 ? 10 : 11;
        const uint32_t dmask = (1u << width) - 1u;
        for (int i = tid; i < S1_NB; i += S1_THREADS) hist[i] = 0u;
        __syncthreads();
        s1_rows(rs, nrows, c0, [&](int r, f32x4 x) {
            const int i0 = r * S1_ROW + pos0;
#pragma unroll
            for (int e = 0; e < S1_KPT; ++e) {
                if (i0 + e < ndoc) {
                    const uint32_t k = order_key(x[e]);
                    if (lin_bin(x[e], vlo, scale) == d && (k & pmask) == prefix)
                        atomicAdd(&hist[(k >> shift) & dmask], 1u);
                }
            }
        });
        __syncthreads();
        s1_find_bin(hist, rr, wtot, &sh_d, &sh_rem, &sh_cnt);
        __syncthreads();
        prefix |= sh_d << shift;
        pmask |= dmask << shift;
        rr = sh_rem;
        __syncthreads();
    }
    const uint32_t T = prefix, need = rr;  // keep keys > T and the first `need` keys == T
    // Counts per (row, wave): keys above T in cnt, keys equal to T in eqc.
    s1_rows(rs, nrows, c0, [&](int r, f32x4 x) {
        const int i0 = r * S1_ROW + pos0;
        uint32_t um = 0u, em = 0u;
#pragma unroll
        for (int e = 0; e < S1_KPT; ++e) {
            if (i0 + e < ndoc) {
                const uint32_t k = order_key(x[e]);
                if (k > T) um |= 1u << e;
                if (k == T) em |= 1u << e;
            }
        }
        const uint32_t cu = wave_count(um), ce = wave_count(em);
        if (lane == 0) {
            cnt[r * S1_WAVES + w] = cu;
            eqc[r * S1_WAVES + w] = ce;
        }
    });
    __syncthreads();
    {
        // keys == T of each (row, wave) that are kept: those ranked below `need`
        const uint32_t e_here = tid < nslot ? eqc[tid] : 0u;
        uint32_t tot;
        const uint32_t e_before = s1_scan_excl(e_here, wtot, &tot);
        if (tid < nslot) {
            cnt[tid] += e_before >= need ? 0u : min(need - e_before, e_here);
            eqc[tid] = e_before;
        }
    }
    __syncthreads();
    s1_scan_counts(cnt, nslot, wtot);
    s1_rows(rs, nrows, c0, [&](int r, f32x4 x) {
        const int i0 = r * S1_ROW + pos0;
        uint32_t em = 0u, km = 0u;
#pragma unroll
        for (int e = 0; e < S1_KPT; ++e) {
            if (i0 + e < ndoc) {
                const uint32_t k = order_key(x[e]);
                if (k == T) em |= 1u << e;
                if (k > T) km |= 1u << e;
            }
        }
        uint32_t er = eqc[r * S1_WAVES + w] + lane_offset(em);  // rank of this lane's first key == T
#pragma unroll
        for (int e = 0; e < S1_KPT; ++e) {
            if ((em >> e) & 1u) {
                if (er < need) km |= 1u << e;
                ++er;
            }
        }
        uint32_t pos = cnt[r * S1_WAVES + w] + lane_offset(km);
#pragma unroll
        for (int e = 0; e < S1_KPT; ++e) {
            if ((km >> e) & 1u) {
                if (pos < (uint32_t)kdoc) dst[pos] = off + p + i0 + e;
                ++pos;
            }
        }
    });
}

}  // namespace

bool select_one_wg_fits(const BatchArgs& a, int max_doc) {
    for (int b = 0; b < a.batch; ++b)
        if (a.cu_seq[b + 1] - a.cu_seq[b] - a.q_len[b] - a.p_len[b] > std::min(max_doc, S1_MAX))
            return false;
    return true;
}

}  // namespace tg

// ----------------------------------------- allocation-free entry point ----
// The workspace of tg_topk_select_noalloc: one copy per GPU, resident from the
// library's load to the end of the process.  In host code this name is only a
// host-side stand-in for the symbol, never a device address: select_scratch()
// obtains each device's own address with hipGetSymbolAddress, and only that
// address is handed to kernels.
static __device__ __align__(256) unsigned char scratch[TG_SELECT_SCRATCH_BYTES];

namespace tg {

namespace {
constexpr int SCRATCH_MAX_DEVICES = 64;
std::atomic<void*> scratch_ptr[SCRATCH_MAX_DEVICES];
std::mutex scratch_mu;
}  // namespace

hipError_t select_scratch(hipStream_t st, void** out) {
    int dev = -1;
    hipError_t e = st != nullptr ? hipStreamGetDevice(st, &dev) : hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= SCRATCH_MAX_DEVICES) return hipErrorInvalidDevice;
    void* p = scratch_ptr[dev].load(std::memory_order_acquire);
    if (p == nullptr) {
        // First call on this device: look the address up with the device current.
        std::lock_guard<std::mutex> lock(scratch_mu);
        p = scratch_ptr[dev].load(std::memory_order_relaxed);
        if (p == nullptr) {
            int cur = -1;
            if ((e = hipGetDevice(&cur)) != hipSuccess) return e;
            if (cur != dev && (e = hipSetDevice(dev)) != hipSuccess) return e;
            e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
            if (cur != dev) {
                const hipError_t e2 = hipSetDevice(cur);
                if (e == hipSuccess) e = e2;
            }
            if (e != hipSuccess) return e;
            if (p == nullptr) return hipErrorInvalidSymbol;
            scratch_ptr[dev].store(p, std::memory_order_release);
        }
    }
    *out = p;
    return hipSuccess;
}

size_t select_workspace_bytes(const BatchArgs& a) {
    int dc, ac;
    chunk_plan(a, nullptr, &dc, &ac);
    return ws_layout(a.batch, dc, a.cu_seq[a.batch]).total;
}

hipError_t launch_select(const float* scores, const BatchArgs& a, int32_t* kept, int32_t* cu_dev,
                         void* ws, int path, hipStream_t st) {
    SelArgs s;
    s.batch = a.batch;
    for (int b = 0; b <= a.batch; ++b) {
        s.off[b] = a.cu_seq[b];
        s.out[b] = a.cu_kept[b];
    }
    for (int b = 0; b < a.batch; ++b) {
        s.q[b] = a.q_len[b];
        s.p[b] = a.p_len[b];
    }
    s.scores = scores;
    s.kept = kept;
    s.cu_dev = cu_dev;
    const bool one_wg = path == SELECT_ONE_WG || (path == SELECT_AUTO && select_auto_one_wg(a));
    if (one_wg) {  // every document is short enough for one workgroup
        hipLaunchKernelGGL(sel_one_kernel, dim3(a.batch), dim3(S1_THREADS), 0, st, s);
        return hipGetLastError();
    }
    int dc, ac;
    chunk_plan(a, &s, &dc, &ac);
    const WsLayout L = ws_layout(a.batch, dc, a.cu_seq[a.batch]);
    char* base = (char*)ws;
    s.hist = (uint32_t*)(base + L.hist);
    s.meta = (uint32_t*)(base + L.meta);
    s.ctr = (uint32_t*)(base + L.ctr);
    s.grp_def = (uint32_t*)(base + L.def);
    s.grp_off = (uint32_t*)(base + L.off);
    s.cand = (uint2*)(base + L.cand);
    s.rank_hist = (uint32_t*)(base + L.rank);
    s.grp_kept = (uint32_t*)(base + L.kept);
    s.big = 0;
    for (int b = 0; b < a.batch; ++b)
        if (s.doc_chunk0[b + 1] > s.doc_chunk0[b] &&
            a.cu_seq[b + 1] - a.cu_seq[b] - a.q_len[b] > BIG_DOC)
            s.big = 1;
    if (dc > 0) {
        const int n_hist = a.batch * NBIN, n_ctr = a.batch * CTR;
        const int n_rank = s.big ? a.batch * NPASS * NBIN : 0;
        const int n_kept = s.big ? s.doc_group0[a.batch] : 0;
        const int n_clear = std::max(std::max(n_hist, n_ctr), std::max(n_rank, n_kept));
        hipLaunchKernelGGL(sel_clear_kernel, dim3((n_clear + SB - 1) / SB), dim3(SB), 0, st, s.hist,
                           s.ctr, n_hist, n_ctr, s.rank_hist, n_rank, s.grp_kept, n_kept);
        const int dg = s.doc_group0[a.batch];
        hipLaunchKernelGGL(sel_hist_kernel, dim3(dg), dim3(SB), 0, st, s);
        if (s.big)
            hipLaunchKernelGGL(sel_cand_kernel<true>, dim3(dg), dim3(SB), 0, st, s);
        else
            hipLaunchKernelGGL(sel_cand_kernel<false>, dim3(dg), dim3(SB), 0, st, s);
        if (s.big) {
            for (int p = 0; p < NPASS; ++p)
                hipLaunchKernelGGL(sel_rank_kernel, dim3(RANK_WG), dim3(SB), 0, st, s, p);
            hipLaunchKernelGGL(sel_rankcount_kernel, dim3(RANK_WG), dim3(SB), 0, st, s);
        }
    }
    if (s.all_group0[a.batch] > 0)
        hipLaunchKernelGGL(sel_compact_kernel, dim3(s.all_group0[a.batch]), dim3(SB), 0, st, s);
    return hipGetLastError();
}

}  // namespace tg
