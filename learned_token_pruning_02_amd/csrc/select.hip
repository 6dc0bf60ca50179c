// Top-K selection with the question tail always kept (spke.com page,
// three-phase list, second bullet; "Seule la partie document ..." for the
// question; "Comment déployer TokenGate ?" for the max_kept_prefill_tokens
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
//   2. histogram of the top 11 key bits per chunk (LDS), summed into the
//      request's histogram with global atomics; the chunk that finishes last
//      (atomic ticket, no waiting) finds the bucket d1 holding the K_doc-th
//      best key;
//   3. per chunk, count the keys above d1, append the keys in d1 with their
//      index and histogram their next 11 key bits; the last chunk picks the
//      first digit from that histogram and ranks the candidates sharing it
//      exactly by an LDS radix select over the 52-bit composite (low 21 key
//      bits, then reversed index), which turns (key desc, index asc) into a
//      single descending order, then counts the kept tokens of every chunk and
//      scans them into output offsets;
//   4. per chunk, re-derive each key's keep flag from (d1, composite prefix)
//      and write the kept ids in index order (wave ballots + a small count
//      table per workgroup), and the question tail after them.
// Results do not depend on which workgroup finishes last.
#include <algorithm>
#include <cstdlib>

#include "tg_device.h"
#include "tg_kernels.h"

namespace tg {

namespace {

constexpr int SB = 256;                 // threads per workgroup
constexpr int SWAVES = SB / WAVE;
constexpr int SITEMS = 8;               // keys per thread
constexpr int SCHUNK = SB * SITEMS;     // 2048 keys per chunk
constexpr int NBIN = 2048;
constexpr int META = 8;                 // u32 words of per-request metadata
constexpr int CTR = 16;                 // u32 counters per request (tickets, candidate count)
constexpr int NPASS = 5;                // radix passes over the 52-bit candidate composite
constexpr int BIG_DOC = 1 << 20;        // documents above this rank their candidates with every workgroup
constexpr int RANK_WG = 512;            // workgroups of the many-workgroup candidate passes
constexpr uint32_t CAND_LDS = 8192;     // threshold-bucket candidates staged in LDS

__device__ __forceinline__ uint32_t order_key(float f) {
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7fffffffu) > 0x7f800000u) return 0u;  // NaN: lowest of all
    if (u == 0x80000000u) u = 0u;                     // -0 -> +0
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Composite rank key of a candidate inside the threshold bucket: the low 21
// key bits, then 0x7fffffff - index, so that larger = better and unique.
__device__ __forceinline__ uint64_t composite(uint32_t key, uint32_t idx) {
    return ((uint64_t)(key & 0x1fffffu) << 31) | (uint64_t)(0x7fffffffu - idx);
}

// Digit p of the composite: bit offset and width (11 + 10 + 11 + 11 + 9 = 52).
__device__ __forceinline__ int pass_shift(int p) {
    return p == 0 ? 41 : (p == 1 ? 31 : (p == 2 ? 20 : (p == 3 ? 9 : 0)));
}
__device__ __forceinline__ int pass_width(int p) { return p == 1 ? 10 : (p == 4 ? 9 : 11); }

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
    const float* scores;
    int32_t* kept;
    int32_t* cu_dev;
    uint32_t* hist;       // [B][NBIN]
    uint32_t* meta;       // [B][META]: d1, rem1, cnt1, cprefix lo/hi, cmask lo/hi, done
    uint32_t* ctr;        // [B][CTR]: hist ticket, candidate ticket, candidate count,
                          //           rank-pass tickets [4, 4+NPASS), count ticket 4+NPASS
    uint32_t* rank_hist;  // [B][NPASS][NBIN]: first-digit histogram ([b][0]), and every pass of the many-workgroup ranking
    uint32_t* chunk_kept; // [doc chunks]: kept candidates per chunk (many-workgroup ranking only)
    int32_t big;          // rank candidates with every workgroup (some document > BIG_DOC)
    uint32_t* chunk_def;  // [doc chunks]: keys above d1
    uint32_t* chunk_off;  // [doc chunks]: output offset of the chunk's first kept token
    uint2* cand;          // [T]: (key, local index), request b at off[b]
};

__device__ __forceinline__ int find_request(const int32_t* base, int batch, int blk) {
    int b = 0;
    while (b + 1 < batch && base[b + 1] <= blk) ++b;
    return b;
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
                                                       uint32_t* chunk_kept, int n_kept) {
    const int i = blockIdx.x * SB + threadIdx.x;
    if (i < n_hist) hist[i] = 0u;
    if (i < n_ctr) ctr[i] = 0u;
    if (i < n_rank) rank_hist[i] = 0u;
    if (i < n_kept) chunk_kept[i] = 0u;
}

// ------------------------------------------------------------- launch 2 ----
__global__ __launch_bounds__(SB) void sel_hist_kernel(SelArgs a) {
    __shared__ uint32_t h[NBIN];
    __shared__ uint32_t wtot[SWAVES];
    __shared__ uint32_t sh_last, sh_d, sh_gt, sh_cnt;
    const int tid = threadIdx.x;
    const int b = find_request(a.doc_chunk0, a.batch, blockIdx.x);
    const int c = blockIdx.x - a.doc_chunk0[b];
    const int nck = a.doc_chunk0[b + 1] - a.doc_chunk0[b];
    const int N = a.off[b + 1] - a.off[b];
    const int ndoc = N - a.q[b] - a.p[b];
    const int kdoc = a.out[b + 1] - a.out[b] - a.q[b] - a.p[b];
    const float* s = a.scores + a.off[b] + a.p[b];  // document tokens, indexed from 0

    for (int i = tid; i < NBIN; i += SB) h[i] = 0u;
    __syncthreads();
    uint32_t kv[SITEMS];
#pragma unroll
    for (int it = 0; it < SITEMS; ++it) {
        const int i = c * SCHUNK + it * SB + tid;
        kv[it] = i < ndoc ? order_key(s[i]) : 0u;
    }
#pragma unroll
    for (int it = 0; it < SITEMS; ++it) {
        const int i = c * SCHUNK + it * SB + tid;
        if (i < ndoc) atomicAdd(&h[kv[it] >> 21], 1u);
    }
    __syncthreads();
    uint32_t* gh = a.hist + (size_t)b * NBIN;
    for (int i = tid; i < NBIN; i += SB)
        if (h[i] != 0u) atomicAdd(&gh[i], h[i]);
    wait_own_writes();
    __syncthreads();
    if (tid == 0) sh_last = atomicAdd(&a.ctr[b * CTR + 0], 1u) == (uint32_t)(nck - 1);
    __syncthreads();
    if (!sh_last) return;
    find_bin([&](int i) { return coherent_load(&gh[i]); }, NBIN, (uint32_t)kdoc, wtot, &sh_d,
             &sh_gt, &sh_cnt);
    if (tid == 0) {
        uint32_t* m = a.meta + b * META;
        m[0] = sh_d;
        m[1] = (uint32_t)kdoc - sh_gt;
        m[2] = sh_cnt;
    }
}

// ------------------------------------------------------------- launch 3 ----
__global__ __launch_bounds__(SB) void sel_cand_kernel(SelArgs a) {
    __shared__ uint32_t wtot[SWAVES];
    __shared__ uint32_t sh_base, sh_last, sh_d, sh_gt, sh_cnt, sh_total;
    __shared__ uint32_t h[NBIN];
    __shared__ uint2 cl[CAND_LDS];
    const int tid = threadIdx.x;
    const int b = find_request(a.doc_chunk0, a.batch, blockIdx.x);
    const int c = blockIdx.x - a.doc_chunk0[b];
    const int nck = a.doc_chunk0[b + 1] - a.doc_chunk0[b];
    const int N = a.off[b + 1] - a.off[b];
    const int ndoc = N - a.q[b] - a.p[b];
    const float* s = a.scores + a.off[b] + a.p[b];  // document tokens, indexed from 0
    uint32_t* m = a.meta + b * META;
    const uint32_t d1 = m[0];
    uint2* cand = a.cand + a.off[b];

    uint32_t kv[SITEMS];
    uint32_t above = 0, ncand = 0;
#pragma unroll
    for (int it = 0; it < SITEMS; ++it) {
        const int i = c * SCHUNK + it * SB + tid;
        kv[it] = i < ndoc ? order_key(s[i]) : 0u;
        if (i < ndoc) {
            above += (kv[it] >> 21) > d1;
            ncand += (kv[it] >> 21) == d1;
        }
    }
    uint32_t tot_above;
    block_incl_scan(above, wtot, &tot_above);
    uint32_t tot_cand;
    const uint32_t incl = block_incl_scan(ncand, wtot, &tot_cand);
    if (tid == 0) {
        coherent_store(&a.chunk_def[a.doc_chunk0[b] + c], tot_above);
        sh_base = tot_cand ? atomicAdd(&a.ctr[b * CTR + 2], tot_cand) : 0u;
    }
    __syncthreads();
    uint32_t pos = sh_base + incl - ncand;
#pragma unroll
    for (int it = 0; it < SITEMS; ++it) {
        const int i = c * SCHUNK + it * SB + tid;
        if (i < ndoc && (kv[it] >> 21) == d1) coherent_store2(&cand[pos++], make_uint2(kv[it], (uint32_t)i));
    }
    if (!a.big && tot_cand != 0u) {
        // The first ranking digit of the candidates (key bits 10-20) is
        // histogrammed here by every chunk, so that the last chunk starts
        // from the request's histogram instead of a pass over all of them.
        for (int i = tid; i < NBIN; i += SB) h[i] = 0u;
        __syncthreads();
#pragma unroll
        for (int it = 0; it < SITEMS; ++it) {
            const int i = c * SCHUNK + it * SB + tid;
            if (i < ndoc && (kv[it] >> 21) == d1) atomicAdd(&h[(kv[it] >> 10) & (NBIN - 1)], 1u);
        }
        __syncthreads();
        uint32_t* gh0 = a.rank_hist + (size_t)b * NPASS * NBIN;
        for (int i = tid; i < NBIN; i += SB)
            if (h[i] != 0u) atomicAdd(&gh0[i], h[i]);
    }
    wait_own_writes();
    __syncthreads();
    if (tid == 0) sh_last = atomicAdd(&a.ctr[b * CTR + 1], 1u) == (uint32_t)(nck - 1);
    __syncthreads();
    if (!sh_last) return;

    if (a.big) {
        // Ranking is left to the many-workgroup passes (sel_rank_kernel).
        if (tid == 0) {
            m[3] = m[4] = m[5] = m[6] = 0u;
            m[7] = 0u;
        }
        return;
    }

    // ---- the last chunk: exact rank inside bucket d1 ----------------------
    // The first digit comes from the histogram the chunks built; only the
    // candidates sharing it (usually a handful) go on, staged in LDS when
    // they fit (a degenerate bucket of heavy ties is read from global memory
    // on every pass instead), through the remaining radix passes.
    const uint32_t cnt1 = m[2];
    uint32_t rem = m[1];
    uint64_t cprefix = 0, cmask = 0;
    {
        const uint32_t* gh0 = a.rank_hist + (size_t)b * NPASS * NBIN;
        find_bin([&](int i) { return coherent_load(&gh0[i]); }, NBIN, rem, wtot, &sh_d, &sh_gt,
                 &sh_cnt);
        rem -= sh_gt;
        cprefix = (uint64_t)sh_d << pass_shift(0);
        cmask = (uint64_t)(NBIN - 1) << pass_shift(0);
    }
    const uint32_t cnt0 = sh_cnt;  // candidates sharing the first digit
    const bool in_lds = cnt0 <= CAND_LDS;
    if (tid == 0) sh_total = 0u;
    __syncthreads();
    if (cnt0 != rem && in_lds) {
        for (uint32_t j = tid; j < cnt1; j += SB) {
            const uint2 e = coherent_load2(&cand[j]);
            if ((composite(e.x, e.y) & cmask) == cprefix) cl[atomicAdd(&sh_total, 1u)] = e;
        }
    }
    __syncthreads();
    const uint32_t nlist = in_lds ? cnt0 : cnt1;
    auto cand_at = [&](uint32_t j) { return in_lds ? cl[j] : coherent_load2(&cand[j]); };
#pragma unroll 1
    for (int p = 1; p < NPASS && cnt0 != rem; ++p) {
        const int sh = pass_shift(p);
        const int wd = pass_width(p);
        const int nb = 1 << wd;
        for (int i = tid; i < NBIN; i += SB) h[i] = 0u;
        __syncthreads();
        for (uint32_t j = tid; j < nlist; j += SB) {
            const uint2 e = cand_at(j);
            const uint64_t cp = composite(e.x, e.y);
            if ((cp & cmask) == cprefix) atomicAdd(&h[(cp >> sh) & (uint64_t)(nb - 1)], 1u);
        }
        __syncthreads();
        find_bin([&](int i) { return h[i]; }, nb, rem, wtot, &sh_d, &sh_gt, &sh_cnt);
        rem -= sh_gt;
        cprefix |= (uint64_t)sh_d << sh;
        cmask |= (uint64_t)(nb - 1) << sh;
        const uint32_t cnt = sh_cnt;
        __syncthreads();
        if (cnt == rem) break;  // every composite with this prefix is kept
    }

    // Kept candidates per chunk, then exclusive offsets of all chunks.
    uint32_t* ccnt = h;  // reuse: up to NBIN chunks handled per round
    const uint32_t* def = a.chunk_def + a.doc_chunk0[b];
    uint32_t* coff = a.chunk_off + a.doc_chunk0[b];
    uint32_t carry = 0;
    for (int c0 = 0; c0 < nck; c0 += NBIN) {
        for (int i = tid; i < NBIN; i += SB) h[i] = 0u;
        __syncthreads();
        for (uint32_t j = tid; j < cnt1; j += SB) {
            const uint2 e = coherent_load2(&cand[j]);
            const int ch = (int)(e.y / SCHUNK) - c0;
            if (ch >= 0 && ch < NBIN && (composite(e.x, e.y) & cmask) >= cprefix)
                atomicAdd(&ccnt[ch], 1u);
        }
        __syncthreads();
        // each thread owns NBIN/SB consecutive chunks
        const int per = NBIN / SB;
        uint32_t v[NBIN / SB];
        uint32_t sum = 0;
        for (int j = 0; j < per; ++j) {
            const int ch = c0 + tid * per + j;
            v[j] = ch < nck ? ccnt[tid * per + j] + coherent_load(&def[ch]) : 0u;
            sum += v[j];
        }
        const uint32_t incl2 = block_incl_scan(sum, wtot, &sh_total);
        uint32_t run = carry + incl2 - sum;
        for (int j = 0; j < per; ++j) {
            const int ch = c0 + tid * per + j;
            if (ch < nck) coff[ch] = run;
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
}

// ------------------------------------ large documents: ranking by all ----
// The same radix passes over the candidate composite as the last chunk runs
// above, with the candidate list of every selecting request spread over
// RANK_WG workgroups: each histograms its share of the candidates that match
// the prefix fixed so far (LDS, then global atomics), and the workgroup that
// finishes last picks the digit and updates the request's prefix.  Launched
// once per pass; a request whose rank is already fixed is skipped.
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
        const uint64_t cprefix = (uint64_t)m[3] | ((uint64_t)m[4] << 32);
        const uint64_t cmask = (uint64_t)m[5] | ((uint64_t)m[6] << 32);
        const uint2* cand = a.cand + a.off[b];
        for (int i = tid; i < nb; i += SB) h[i] = 0u;
        __syncthreads();
        for (uint32_t j = blockIdx.x * SB + tid; j < cnt1; j += RANK_WG * SB) {
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
        if (tid == 0) sh_last = atomicAdd(&a.ctr[b * CTR + 4 + p], 1u) == (uint32_t)(RANK_WG - 1);
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

// Kept candidates per chunk (global atomics over all workgroups), then the
// workgroup finishing last scans every chunk's kept count into its output
// offset, as the last chunk of sel_cand does for small documents.
__global__ __launch_bounds__(SB) void sel_rankcount_kernel(SelArgs a) {
    __shared__ uint32_t wtot[SWAVES];
    __shared__ uint32_t sh_last, sh_total;
    const int tid = threadIdx.x;
    for (int b = 0; b < a.batch; ++b) {
        if (a.doc_chunk0[b + 1] == a.doc_chunk0[b]) continue;
        const uint32_t* m = a.meta + b * META;
        const uint32_t cnt1 = m[2];
        const uint64_t cprefix = (uint64_t)m[3] | ((uint64_t)m[4] << 32);
        const uint64_t cmask = (uint64_t)m[5] | ((uint64_t)m[6] << 32);
        const uint2* cand = a.cand + a.off[b];
        uint32_t* kc = a.chunk_kept + a.doc_chunk0[b];
        for (uint32_t j = blockIdx.x * SB + tid; j < cnt1; j += RANK_WG * SB) {
            const uint2 e = cand[j];
            if ((composite(e.x, e.y) & cmask) >= cprefix) atomicAdd(&kc[e.y / SCHUNK], 1u);
        }
        wait_own_writes();
        __syncthreads();
        if (tid == 0) sh_last = atomicAdd(&a.ctr[b * CTR + 4 + NPASS], 1u) == (uint32_t)(RANK_WG - 1);
        __syncthreads();
        if (!sh_last) continue;
        const int nck = a.doc_chunk0[b + 1] - a.doc_chunk0[b];
        const uint32_t* def = a.chunk_def + a.doc_chunk0[b];
        uint32_t* coff = a.chunk_off + a.doc_chunk0[b];
        uint32_t carry = 0;
        constexpr int per = NBIN / SB;
        for (int c0 = 0; c0 < nck; c0 += NBIN) {
            uint32_t v[per];
            uint32_t sum = 0;
            for (int j = 0; j < per; ++j) {
                const int ch = c0 + tid * per + j;
                v[j] = ch < nck ? coherent_load(&kc[ch]) + coherent_load(&def[ch]) : 0u;
                sum += v[j];
            }
            const uint32_t incl = block_incl_scan(sum, wtot, &sh_total);
            uint32_t run = carry + incl - sum;
            for (int j = 0; j < per; ++j) {
                const int ch = c0 + tid * per + j;
                if (ch < nck) coff[ch] = run;
                run += v[j];
            }
            carry += sh_total;
            __syncthreads();
        }
    }
}

// ------------------------------------------------------------- launch 4 ----
__global__ __launch_bounds__(SB) void sel_compact_kernel(SelArgs a) {
    __shared__ uint32_t tab[SITEMS * SWAVES];
    const int tid = threadIdx.x, lane = lane_id(), w = tid / WAVE;
    const int b = find_request(a.all_chunk0, a.batch, blockIdx.x);
    const int c = blockIdx.x - a.all_chunk0[b];
    if (blockIdx.x == 0 && a.cu_dev != nullptr)
        for (int i = tid; i <= a.batch; i += SB) a.cu_dev[i] = a.out[i];
    const int off = a.off[b];
    const int N = a.off[b + 1] - off;
    const int q = a.q[b];
    const int pf = a.p[b];
    const int out = a.out[b];
    const int keep = a.out[b + 1] - out;
    const int lo = c * SCHUNK;
    const int hi = min(lo + SCHUNK, N);
    if (keep >= N) {
        for (int i = lo + tid; i < hi; i += SB) a.kept[out + i] = off + i;
        return;
    }
    const int ndoc = N - q - pf;
    const int kdoc = keep - q - pf;
    // The always-kept tokens, prefix then question, as one list of pf + q <= N
    // entries shared out by chunk: prefix token f goes to output f, question
    // token f - pf after the prefix and the kept document tokens.
    for (int f = lo + tid; f < min(lo + SCHUNK, pf + q); f += SB) {
        const int i = f < pf ? f : N - q + (f - pf);
        a.kept[out + (f < pf ? f : pf + kdoc + (f - pf))] = off + i;
    }
    // Chunk c of the document: document tokens [lo, lo + SCHUNK), at request
    // positions pf + i, written after the prefix.
    if (kdoc <= 0 || lo >= ndoc) return;

    const uint32_t* m = a.meta + b * META;
    const uint32_t d1 = m[0];
    const uint64_t cprefix = (uint64_t)m[3] | ((uint64_t)m[4] << 32);
    const uint64_t cmask = (uint64_t)m[5] | ((uint64_t)m[6] << 32);
    const uint32_t base = a.chunk_off[a.doc_chunk0[b] + c];
    const float* s = a.scores + off + pf;

    uint64_t km[SITEMS];
#pragma unroll
    for (int it = 0; it < SITEMS; ++it) {
        const int i = lo + it * SB + tid;
        bool k = false;
        if (i < ndoc) {
            const uint32_t key = order_key(s[i]);
            const uint32_t dg = key >> 21;
            k = dg > d1 || (dg == d1 && (composite(key, (uint32_t)i) & cmask) >= cprefix);
        }
        km[it] = __ballot(k);
        if (lane == 0) tab[it * SWAVES + w] = (uint32_t)__popcll(km[it]);
    }
    __syncthreads();
    if (w == 0) {  // exclusive scan of the SITEMS*SWAVES = 32 counts
        uint32_t v = lane < SITEMS * SWAVES ? tab[lane] : 0u;
        uint32_t incl = v;
#pragma unroll
        for (int o = 1; o < WAVE; o <<= 1) {
            const uint32_t n = __shfl_up(incl, o, WAVE);
            if (lane >= o) incl += n;
        }
        if (lane < SITEMS * SWAVES) tab[lane] = incl - v;
    }
    __syncthreads();
#pragma unroll
    for (int it = 0; it < SITEMS; ++it) {
        if ((km[it] >> lane) & 1ull) {
            const int i = lo + it * SB + tid;
            const uint32_t pos = base + tab[it * SWAVES + w] + lanes_below(km[it]);
            if (pos < (uint32_t)kdoc) a.kept[out + pf + pos] = off + pf + i;
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
    L.def = p;  p = align256(p + (size_t)doc_chunks * 4);
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
    }
    *doc_chunks = dc;
    *all_chunks = ac;
}

// ------------------------------------------------ one-workgroup path ----
// When every document of the batch is short enough, each request is selected
// by one 1024-thread workgroup in a single launch: thread t holds the keys of
// the document positions [t*IT, (t+1)*IT) in registers, three histogram
// passes (11, 11, 10 key bits; one private 2048-bin LDS histogram per wave,
// so atomics only contend within a wave -- gate scores crowd a few dozen
// top-bit bins) find the exact K_doc-th best key T and how many keys equal
// to T are kept, and one ordered compaction (block scans of the keys equal
// to T in index order, then of the kept tokens) writes the kept ids.  No
// workspace, no global atomics.
constexpr int SM_THREADS = 1024;
constexpr int SM_WAVES = SM_THREADS / WAVE;
constexpr int SM_IT = 32;                       // keys per thread at most
constexpr int SM_MAX = SM_THREADS * SM_IT;      // 32768 document tokens per request

// Exclusive block scan over 1024 threads; *total gets the sum.
__device__ __forceinline__ uint32_t scan1024_excl(uint32_t v, uint32_t* wtot, uint32_t* total) {
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
    for (int i = 0; i < SM_WAVES; ++i) {
        if (i < w) before += wtot[i];
        all += wtot[i];
    }
    __syncthreads();
    *total = all;
    return x - v + before;
}

__global__ __launch_bounds__(SM_THREADS) void sel_small_kernel(SelArgs a) {
    __shared__ uint32_t whist[SM_WAVES][NBIN];   // 128 KiB: one histogram per wave
    __shared__ uint32_t wtot[SM_WAVES];
    __shared__ uint32_t sh_d, sh_rem;

    const int b = blockIdx.x, tid = threadIdx.x, w = tid / WAVE, lane = lane_id();
    if (b == 0 && a.cu_dev != nullptr)
        for (int i = tid; i <= a.batch; i += SM_THREADS) a.cu_dev[i] = a.out[i];
    const int off = a.off[b], N = a.off[b + 1] - off;
    const int out = a.out[b], K = a.out[b + 1] - out;
    int32_t* kept = a.kept + out;
    if (K >= N) {  // the budget covers the request
        for (int i = tid; i < N; i += SM_THREADS) kept[i] = off + i;
        return;
    }
    const int q = a.q[b], p = a.p[b];
    const int ndoc = N - q - p, kdoc = K - q - p;
    for (int i = tid; i < p; i += SM_THREADS) kept[i] = off + i;
    for (int i = tid; i < q; i += SM_THREADS) kept[p + kdoc + i] = off + N - q + i;

    const int IT = (ndoc + SM_THREADS - 1) / SM_THREADS;
    const int i0 = min(ndoc, tid * IT), i1 = min(ndoc, i0 + IT);
    const int nmine = i1 - i0;
    uint32_t kr[SM_IT];
    const float* s = a.scores + off + p + i0;
#pragma unroll
    for (int j = 0; j < SM_IT; ++j) kr[j] = j < nmine ? order_key(s[j]) : 0u;

    // Threshold key T (the kdoc-th best key) and `need`, the number of keys
    // equal to T that are kept (the lowest-indexed ones).  kdoc == 0 keeps
    // nothing: T above every key.
    uint32_t thr = 0xffffffffu, need = 0;
    if (kdoc > 0) {
        uint32_t prefix = 0, pmask = 0, rem = (uint32_t)kdoc;
        uint32_t* hw = whist[w];
        for (int pass = 0; pass < 3; ++pass) {
            const int shift = pass == 0 ? 21 : (pass == 1 ? 10 : 0);
            const int width = pass == 2 ? 10 : 11;
            const uint32_t dmask = (1u << width) - 1u;
            for (int i = lane; i < NBIN; i += WAVE) hw[i] = 0;
            __syncthreads();
#pragma unroll
            for (int j = 0; j < SM_IT; ++j)
                if (j < nmine && (kr[j] & pmask) == prefix) atomicAdd(&hw[(kr[j] >> shift) & dmask], 1u);
            __syncthreads();
            // Thread t owns bins 2047-2t and 2046-2t (descending order in thread order).
            const int hi = NBIN - 1 - 2 * tid;
            uint32_t c0 = 0, c1 = 0;
#pragma unroll
            for (int ww = 0; ww < SM_WAVES; ++ww) {
                c0 += whist[ww][hi];
                c1 += whist[ww][hi - 1];
            }
            uint32_t tot;
            const uint32_t above = scan1024_excl(c0 + c1, wtot, &tot);  // keys in higher bins
            if (above < rem && rem <= above + c0) {
                sh_d = (uint32_t)hi;
                sh_rem = rem - above;
            } else if (above + c0 < rem && rem <= above + c0 + c1) {
                sh_d = (uint32_t)(hi - 1);
                sh_rem = rem - above - c0;
            }
            __syncthreads();
            prefix |= sh_d << shift;
            pmask |= dmask << shift;
            rem = sh_rem;
            __syncthreads();
        }
        thr = prefix;
        need = rem;
    }

    // Ordered compaction over this thread's positions [i0, i1).
    uint32_t eq = 0;
#pragma unroll
    for (int j = 0; j < SM_IT; ++j) eq += (j < nmine && kr[j] == thr) ? 1u : 0u;
    uint32_t tot;
    const uint32_t eq_before = scan1024_excl(eq, wtot, &tot);
    uint32_t nk = 0, e = eq_before;
#pragma unroll
    for (int j = 0; j < SM_IT; ++j) {
        const bool t_eq = j < nmine && kr[j] == thr;
        nk += (j < nmine && kr[j] > thr) || (t_eq && e < need);
        e += t_eq;
    }
    uint32_t pos = scan1024_excl(nk, wtot, &tot);
    int32_t* dst = kept + p;
    e = eq_before;
#pragma unroll
    for (int j = 0; j < SM_IT; ++j) {
        const bool t_eq = j < nmine && kr[j] == thr;
        if ((j < nmine && kr[j] > thr) || (t_eq && e < need)) dst[pos++] = off + p + i0 + j;
        e += t_eq;
    }
}

}  // namespace

namespace {
bool small_batch(const BatchArgs& a) {
    const char* path = std::getenv("TG_SELECT_PATH");  // "multi": always the chunked path
    if (path != nullptr && path[0] == 'm') return false;
    for (int b = 0; b < a.batch; ++b)
        if (a.cu_seq[b + 1] - a.cu_seq[b] - a.q_len[b] - a.p_len[b] > SM_MAX) return false;
    return true;
}
}  // namespace

size_t select_workspace_bytes(const BatchArgs& a) {
    int dc, ac;
    chunk_plan(a, nullptr, &dc, &ac);
    return ws_layout(a.batch, dc, a.cu_seq[a.batch]).total;
}

hipError_t launch_select(const float* scores, const BatchArgs& a, int32_t* kept, int32_t* cu_dev,
                         void* ws, hipStream_t st) {
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
    if (small_batch(a)) {  // every document fits in one workgroup's LDS
        hipLaunchKernelGGL(sel_small_kernel, dim3(a.batch), dim3(SM_THREADS), 0, st, s);
        return hipGetLastError();
    }
    int dc, ac;
    chunk_plan(a, &s, &dc, &ac);
    const WsLayout L = ws_layout(a.batch, dc, a.cu_seq[a.batch]);
    char* base = (char*)ws;
    s.hist = (uint32_t*)(base + L.hist);
    s.meta = (uint32_t*)(base + L.meta);
    s.ctr = (uint32_t*)(base + L.ctr);
    s.chunk_def = (uint32_t*)(base + L.def);
    s.chunk_off = (uint32_t*)(base + L.off);
    s.cand = (uint2*)(base + L.cand);
    s.rank_hist = (uint32_t*)(base + L.rank);
    s.chunk_kept = (uint32_t*)(base + L.kept);
    s.big = 0;
    for (int b = 0; b < a.batch; ++b)
        if (s.doc_chunk0[b + 1] > s.doc_chunk0[b] &&
            a.cu_seq[b + 1] - a.cu_seq[b] - a.q_len[b] > BIG_DOC)
            s.big = 1;
    if (dc > 0) {
        const int n_hist = a.batch * NBIN, n_ctr = a.batch * CTR;
        const int n_rank = a.batch * NPASS * NBIN, n_kept = s.big ? dc : 0;
        const int n_clear = std::max(std::max(n_hist, n_ctr), std::max(n_rank, n_kept));
        hipLaunchKernelGGL(sel_clear_kernel, dim3((n_clear + SB - 1) / SB), dim3(SB), 0, st, s.hist,
                           s.ctr, n_hist, n_ctr, s.rank_hist, n_rank, s.chunk_kept, n_kept);
        hipLaunchKernelGGL(sel_hist_kernel, dim3(dc), dim3(SB), 0, st, s);
        hipLaunchKernelGGL(sel_cand_kernel, dim3(dc), dim3(SB), 0, st, s);
        if (s.big) {
            for (int p = 0; p < NPASS; ++p)
                hipLaunchKernelGGL(sel_rank_kernel, dim3(RANK_WG), dim3(SB), 0, st, s, p);
            hipLaunchKernelGGL(sel_rankcount_kernel, dim3(RANK_WG), dim3(SB), 0, st, s);
        }
    }
    hipLaunchKernelGGL(sel_compact_kernel, dim3(ac), dim3(SB), 0, st, s);
    return hipGetLastError();
}

}  // namespace tg
