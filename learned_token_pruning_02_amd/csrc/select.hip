// Top-K selection with the question tail always kept (spke.com page,
// three-phase list, second bullet; "Seule la partie document ..." for the
// question; "Comment déployer TokenGate ?" for the max_kept_prefill_tokens
// budget).
//
// Per request b (one 1024-thread workgroup each, all requests in one launch):
//   * budget >= N_b: keep every token;
//   * otherwise keep the K_b - q_b best document tokens under the total order
//     (score descending, index ascending) plus the q_b question tokens.
//
// Scores become order-preserving u32 keys (larger key = better score; -0 and
// +0 share a key; NaN maps to 0, below -inf).  An LDS radix select over the
// key digits (11, 11 and 10 bits, most significant first) narrows the
// threshold: after each pass the digit holding the K_doc-th best key is fixed,
// and the passes stop as soon as every key sharing the fixed prefix is needed.
// The result is a prefix P (under mask M) and a count `rem` of keys with
// (key & M) == P to take.  A last pass over the document in index order keeps
// key & M > P, and the first `rem` keys equal to P in index order; wave
// ballots and a per-chunk (item, wave) count table give each kept token its
// output slot, so kept ids come out ascending without any sort.
#include "tg_device.h"
#include "tg_kernels.h"

namespace tg {

namespace {

constexpr int SEL_THREADS = 1024;
constexpr int SEL_WAVES = SEL_THREADS / WAVE;
constexpr int SEL_ITEMS = 16;                       // keys per thread per chunk
constexpr int SEL_CHUNK = SEL_THREADS * SEL_ITEMS;  // 16384 keys per chunk
constexpr int TAB = SEL_ITEMS * SEL_WAVES;          // 256 table entries

__device__ __forceinline__ uint32_t order_key(float f) {
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7fffffffu) > 0x7f800000u) return 0u;  // NaN: lowest of all
    if (u == 0x80000000u) u = 0u;                     // -0 -> +0
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Exclusive scan of TAB counters in place by wave 0 (4 per lane); returns the
// total to every lane of wave 0 and stores it in *total.
__device__ __forceinline__ void wave0_scan_table(uint32_t* tab, uint32_t* total) {
    const int lane = lane_id();
    uint32_t v[4];
    uint32_t sum = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        v[i] = tab[lane * 4 + i];
        sum += v[i];
    }
    uint32_t incl = sum;
#pragma unroll
    for (int o = 1; o < WAVE; o <<= 1) {
        const uint32_t n = __shfl_up(incl, o, WAVE);
        if (lane >= o) incl += n;
    }
    uint32_t run = incl - sum;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        tab[lane * 4 + i] = run;
        run += v[i];
    }
    if (lane == WAVE - 1) *total = incl;
}

__global__ __launch_bounds__(SEL_THREADS) void select_kernel(const float* __restrict__ scores,
                                                             BatchArgs a,
                                                             int32_t* __restrict__ kept,
                                                             int32_t* __restrict__ cu_dev) {
    const int b = blockIdx.x;
    const int tid = threadIdx.x;
    const int lane = lane_id();
    const int w = tid / WAVE;

    if (b == 0 && cu_dev != nullptr)
        for (int i = tid; i <= a.batch; i += SEL_THREADS) cu_dev[i] = a.cu_kept[i];

    const int off = a.cu_seq[b];
    const int N = a.cu_seq[b + 1] - off;
    const int q = a.q_len[b];
    const int out = a.cu_kept[b];
    const int keep = a.cu_kept[b + 1] - out;

    if (keep >= N) {
        for (int i = tid; i < N; i += SEL_THREADS) kept[out + i] = off + i;
        return;
    }
    const int ndoc = N - q;
    const int kdoc = keep - q;
    for (int i = tid; i < q; i += SEL_THREADS) kept[out + kdoc + i] = off + ndoc + i;
    if (kdoc <= 0) return;

    const float* s = scores + off;

    __shared__ uint32_t hist[2048];
    __shared__ uint32_t wsum[SEL_WAVES];
    __shared__ uint32_t sh_prefix, sh_rem, sh_cnt;
    __shared__ uint32_t tabE[TAB], tabK[TAB];
    __shared__ uint32_t totE, totK;

    // ---- radix select of the threshold ----------------------------------
    uint32_t prefix = 0, mask = 0, rem = (uint32_t)kdoc;
    for (int pass = 0; pass < 3; ++pass) {
        const int shift = pass == 0 ? 21 : (pass == 1 ? 10 : 0);
        const int nbins = pass == 2 ? 1024 : 2048;
        for (int i = tid; i < 2048; i += SEL_THREADS) hist[i] = 0;
        __syncthreads();
        for (int base = 0; base < ndoc; base += SEL_CHUNK) {
            uint32_t kv[SEL_ITEMS];
#pragma unroll
            for (int it = 0; it < SEL_ITEMS; ++it) {
                const int i = base + it * SEL_THREADS + tid;
                kv[it] = i < ndoc ? order_key(s[i]) : 0u;
            }
#pragma unroll
            for (int it = 0; it < SEL_ITEMS; ++it) {
                const int i = base + it * SEL_THREADS + tid;
                if (i < ndoc && (kv[it] & mask) == prefix)
                    atomicAdd(&hist[(kv[it] >> shift) & (uint32_t)(nbins - 1)], 1u);
            }
        }
        __syncthreads();

        // Suffix counts: thread tid owns bin group g = SEL_THREADS-1-tid, so
        // an inclusive scan in thread order runs from the highest bins down.
        const int per = nbins / SEL_THREADS;
        const int g = SEL_THREADS - 1 - tid;
        uint32_t gs = 0;
        for (int j = 0; j < per; ++j) gs += hist[g * per + j];
        uint32_t incl = gs;
#pragma unroll
        for (int o = 1; o < WAVE; o <<= 1) {
            const uint32_t n = __shfl_up(incl, o, WAVE);
            if (lane >= o) incl += n;
        }
        if (lane == WAVE - 1) wsum[w] = incl;
        __syncthreads();
        uint32_t before = 0;
        for (int i = 0; i < w; ++i) before += wsum[i];
        uint32_t ge = before + incl - gs;  // keys whose digit is above this group
        for (int j = per - 1; j >= 0; --j) {
            const int bin = g * per + j;
            const uint32_t gt = ge;
            ge += hist[bin];
            if (gt < rem && rem <= ge) {
                sh_prefix = prefix | ((uint32_t)bin << shift);
                sh_rem = rem - gt;
                sh_cnt = hist[bin];
            }
        }
        __syncthreads();
        prefix = sh_prefix;
        mask |= (uint32_t)(nbins - 1) << shift;
        rem = sh_rem;
        const uint32_t cnt = sh_cnt;
        __syncthreads();
        if (cnt == rem) break;  // every key with this prefix is kept
    }

    // ---- ordered compaction of the document ------------------------------
    uint32_t eq_carry = 0, keep_carry = 0;
    for (int base = 0; base < ndoc && keep_carry < (uint32_t)kdoc; base += SEL_CHUNK) {
        uint32_t kv[SEL_ITEMS];
        uint64_t em[SEL_ITEMS];
#pragma unroll
        for (int it = 0; it < SEL_ITEMS; ++it) {
            const int i = base + it * SEL_THREADS + tid;
            kv[it] = i < ndoc ? order_key(s[i]) : 0u;
        }
#pragma unroll
        for (int it = 0; it < SEL_ITEMS; ++it) {
            const int i = base + it * SEL_THREADS + tid;
            const bool e = i < ndoc && (kv[it] & mask) == prefix;
            em[it] = __ballot(e);
            if (lane == 0) tabE[it * SEL_WAVES + w] = (uint32_t)__popcll(em[it]);
        }
        __syncthreads();
        if (w == 0) wave0_scan_table(tabE, &totE);
        __syncthreads();
        uint64_t km[SEL_ITEMS];
#pragma unroll
        for (int it = 0; it < SEL_ITEMS; ++it) {
            const int i = base + it * SEL_THREADS + tid;
            const bool e = (em[it] >> lane) & 1ull;
            const uint32_t rank = eq_carry + tabE[it * SEL_WAVES + w] + lanes_below(em[it]);
            const bool k = i < ndoc && ((kv[it] & mask) > prefix || (e && rank < rem));
            km[it] = __ballot(k);
            if (lane == 0) tabK[it * SEL_WAVES + w] = (uint32_t)__popcll(km[it]);
        }
        __syncthreads();
        if (w == 0) wave0_scan_table(tabK, &totK);
        __syncthreads();
#pragma unroll
        for (int it = 0; it < SEL_ITEMS; ++it) {
            if ((km[it] >> lane) & 1ull) {
                const int i = base + it * SEL_THREADS + tid;
                const uint32_t pos = keep_carry + tabK[it * SEL_WAVES + w] + lanes_below(km[it]);
                if (pos < (uint32_t)kdoc) kept[out + pos] = off + i;
            }
        }
        eq_carry += totE;
        keep_carry += totK;
        __syncthreads();
    }
}

}  // namespace

hipError_t launch_select(const float* scores, const BatchArgs& a, int32_t* kept, int32_t* cu_dev,
                         hipStream_t st) {
    hipLaunchKernelGGL(select_kernel, dim3(a.batch), dim3(SEL_THREADS), 0, st, scores, a, kept,
                       cu_dev);
    return hipGetLastError();
}

}  // namespace tg
