// C ABI of the TokenGate pruned-prefill library: argument validation on the
// host, then one launch per call on the caller's stream.  Nothing here
// allocates, frees or synchronises, and every check runs before any launch,
// so an error status means nothing was enqueued.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>
#include <cstring>

#include "tg_kernels.h"
#include "tokengate.h"

namespace {

constexpr int64_t I32_LIMIT = (int64_t)1 << 31;

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }
bool aligned4(const void* p) { return ((uintptr_t)p & 3u) == 0; }

bool overlap(const void* a, int64_t abytes, const void* b, int64_t bbytes) {
    if (a == nullptr || b == nullptr || abytes <= 0 || bbytes <= 0) return false;
    const uintptr_t a0 = (uintptr_t)a, b0 = (uintptr_t)b;
    return a0 < b0 + (uintptr_t)bbytes && b0 < a0 + (uintptr_t)abytes;
}

int64_t elt_bytes(tg_dtype dt) { return dt == TG_F32 ? 4 : 2; }

bool valid_dtype(int dt) { return dt == TG_F32 || dt == TG_BF16; }

tg_status launched(hipError_t e) { return e == hipSuccess ? TG_OK : TG_ERR_LAUNCH; }

// Shared by the plan and select calls; prefix_len may be NULL (no prefix).
tg_status plan_batch_arrays(int32_t batch, const int32_t* seq_len, const int32_t* q_len,
                            const int32_t* budget, const int32_t* prefix_len,
                            tg::BatchArgs* out) {
    if (batch < 1 || batch > TG_MAX_BATCH) return TG_ERR_BAD_SHAPE;
    if (seq_len == nullptr || q_len == nullptr || budget == nullptr) return TG_ERR_NULL_PTR;
    int64_t tok = 0, kept = 0;
    out->batch = batch;
    out->cu_seq[0] = 0;
    out->cu_kept[0] = 0;
    for (int i = 0; i < batch; ++i) {
        const int64_t n = seq_len[i], q = q_len[i], k = budget[i];
        const int64_t p = prefix_len != nullptr ? prefix_len[i] : 0;
        const int64_t keep = k < n ? k : n;
        if (n < 1 || q < 0 || q > n || k < 1 || p < 0 || p + q > keep) return TG_ERR_BAD_BUDGET;
        tok += n;
        kept += keep;
        if (tok >= I32_LIMIT) return TG_ERR_BAD_SHAPE;
        out->cu_seq[i + 1] = (int32_t)tok;
        out->cu_kept[i + 1] = (int32_t)kept;
        out->q_len[i] = (int32_t)q;
        out->p_len[i] = (int32_t)p;
    }
    return TG_OK;
}

tg_status plan_batch(const tg_batch* b, tg::BatchArgs* out) {
    if (b == nullptr) return TG_ERR_NULL_PTR;
    return plan_batch_arrays(b->batch, b->seq_len, b->q_len, b->budget, nullptr, out);
}

tg_status plan_batch(const tg_batch_prefix* b, tg::BatchArgs* out) {
    if (b == nullptr) return TG_ERR_NULL_PTR;
    return plan_batch_arrays(b->batch, b->seq_len, b->q_len, b->budget, b->prefix_len, out);
}

tg_status plan_out(const tg::BatchArgs& a, int32_t* cu_seqlens, int32_t* cu_kept,
                   size_t* topk_ws_bytes) {
    if (cu_seqlens != nullptr) std::memcpy(cu_seqlens, a.cu_seq, sizeof(int32_t) * (a.batch + 1));
    if (cu_kept != nullptr) std::memcpy(cu_kept, a.cu_kept, sizeof(int32_t) * (a.batch + 1));
    if (topk_ws_bytes != nullptr) *topk_ws_bytes = tg::select_workspace_bytes(a);
    return TG_OK;
}

tg_status select_checked(const float* scores, const tg::BatchArgs& a, int32_t* kept_idx,
                         int32_t* cu_kept_dev, void* ws, size_t ws_bytes, int path,
                         hipStream_t stream) {
    if (scores == nullptr || kept_idx == nullptr) return TG_ERR_NULL_PTR;
    if (path < tg::SELECT_AUTO || path > tg::SELECT_CHUNKED) return TG_ERR_BAD_SHAPE;
    if (path == tg::SELECT_ONE_WG && !tg::select_one_wg_fits(a)) return TG_ERR_UNSUPPORTED;
    const size_t need = tg::select_workspace_bytes(a);
    if (need > 0 && (ws == nullptr || ws_bytes < need)) return TG_ERR_WORKSPACE;
    if (!aligned4(scores) || !aligned4(kept_idx) || !aligned16(ws)) return TG_ERR_ALIGNMENT;
    const int64_t T = a.cu_seq[a.batch], Kt = a.cu_kept[a.batch];
    const int64_t wb = (int64_t)need;
    if (overlap(kept_idx, Kt * 4, scores, T * 4) ||
        overlap(cu_kept_dev, (a.batch + 1) * 4, scores, T * 4) ||
        overlap(cu_kept_dev, (a.batch + 1) * 4, kept_idx, Kt * 4) ||
        overlap(ws, wb, scores, T * 4) || overlap(ws, wb, kept_idx, Kt * 4) ||
        overlap(ws, wb, cu_kept_dev, (a.batch + 1) * 4))
        return TG_ERR_ALIAS;
    return launched(tg::launch_select(scores, a, kept_idx, cu_kept_dev, ws, path, stream));
}

}  // namespace

extern "C" {

const char* tg_status_str(int status) {
    switch (status) {
        case TG_OK: return "TG_OK";
        case TG_ERR_NULL_PTR: return "TG_ERR_NULL_PTR";
        case TG_ERR_BAD_SHAPE: return "TG_ERR_BAD_SHAPE";
        case TG_ERR_BAD_BUDGET: return "TG_ERR_BAD_BUDGET";
        case TG_ERR_BAD_DTYPE: return "TG_ERR_BAD_DTYPE";
        case TG_ERR_UNSUPPORTED: return "TG_ERR_UNSUPPORTED";
        case TG_ERR_ALIGNMENT: return "TG_ERR_ALIGNMENT";
        case TG_ERR_WORKSPACE: return "TG_ERR_WORKSPACE";
        case TG_ERR_LAUNCH: return "TG_ERR_LAUNCH";
        case TG_ERR_ALIAS: return "TG_ERR_ALIAS";
        default: return "TG_ERR_UNKNOWN";
    }
}

int tg_abi_version(void) { return TG_ABI_VERSION; }

tg_status tg_plan(const tg_batch* b, int32_t* cu_seqlens, int32_t* cu_kept,
                  size_t* topk_ws_bytes) {
    tg::BatchArgs a;
    const tg_status st = plan_batch(b, &a);
    if (st != TG_OK) return st;
    return plan_out(a, cu_seqlens, cu_kept, topk_ws_bytes);
}

tg_status tg_plan_prefix(const tg_batch_prefix* b, int32_t* cu_seqlens, int32_t* cu_kept,
                         size_t* topk_ws_bytes) {
    tg::BatchArgs a;
    const tg_status st = plan_batch(b, &a);
    if (st != TG_OK) return st;
    return plan_out(a, cu_seqlens, cu_kept, topk_ws_bytes);
}

tg_status tg_gate_score(tg_dtype dt, const void* hidden, int64_t T, int32_t d_model,
                        const void* w1, const void* b1, const void* w2, const void* b2,
                        int32_t d_gate, float* scores, hipStream_t stream) {
    if (!valid_dtype(dt)) return TG_ERR_BAD_DTYPE;
    if (T < 0 || T >= I32_LIMIT || d_model < 1 || d_gate < 1) return TG_ERR_BAD_SHAPE;
    if (hidden == nullptr || w1 == nullptr || w2 == nullptr || scores == nullptr)
        return TG_ERR_NULL_PTR;
    if (dt == TG_F32) {
        if (d_model % 4 != 0 || d_gate > 1024 || d_model > 16384) return TG_ERR_UNSUPPORTED;
    } else {
        if (d_model % 64 != 0 || (d_gate != 64 && d_gate != 128 && d_gate != 256))
            return TG_ERR_UNSUPPORTED;
    }
    if (!aligned16(hidden) || !aligned16(w1) || !aligned4(scores)) return TG_ERR_ALIGNMENT;
    const int64_t eb = elt_bytes(dt);
    if (overlap(scores, T * 4, hidden, T * d_model * eb) ||
        overlap(scores, T * 4, w1, (int64_t)d_gate * d_model * eb))
        return TG_ERR_ALIAS;
    if (T == 0) return TG_OK;
    if (dt == TG_F32)
        return launched(tg::launch_gate_f32((const float*)hidden, T, d_model, (const float*)w1,
                                            (const float*)b1, (const float*)w2, (const float*)b2,
                                            d_gate, scores, stream));
    return launched(
        tg::launch_gate_bf16(hidden, T, d_model, w1, b1, w2, b2, d_gate, scores, stream));
}

tg_status tg_topk_select(const float* scores, const tg_batch* b, int32_t* kept_idx,
                         int32_t* cu_kept_dev, void* ws, size_t ws_bytes, hipStream_t stream) {
    tg::BatchArgs a;
    const tg_status st = plan_batch(b, &a);
    if (st != TG_OK) return st;
    return select_checked(scores, a, kept_idx, cu_kept_dev, ws, ws_bytes, tg::SELECT_AUTO, stream);
}

tg_status tg_topk_select_noalloc(const float* scores, const tg_batch* b, int32_t* kept_idx,
                                 int32_t* cu_kept_dev, hipStream_t stream) {
    tg::BatchArgs a;
    const tg_status st = plan_batch(b, &a);
    if (st != TG_OK) return st;
    if (scores == nullptr || kept_idx == nullptr) return TG_ERR_NULL_PTR;
    // The one-workgroup path needs no workspace; the chunked path's must fit
    // the static scratch.  All of this is decided before any HIP call.
    const bool chunked = !tg::select_auto_one_wg(a);
    const size_t need = chunked ? tg::select_workspace_bytes(a) : 0;
    if (need > TG_SELECT_SCRATCH_BYTES) return TG_ERR_WORKSPACE;
    if (!aligned4(scores) || !aligned4(kept_idx) || !aligned4(cu_kept_dev)) return TG_ERR_ALIGNMENT;
    const int64_t T = a.cu_seq[a.batch], Kt = a.cu_kept[a.batch];
    if (overlap(kept_idx, Kt * 4, scores, T * 4) ||
        overlap(cu_kept_dev, (a.batch + 1) * 4, scores, T * 4) ||
        overlap(cu_kept_dev, (a.batch + 1) * 4, kept_idx, Kt * 4))
        return TG_ERR_ALIAS;
    void* ws = nullptr;
    if (need > 0 && tg::select_scratch(stream, &ws) != hipSuccess) return TG_ERR_LAUNCH;
    return launched(tg::launch_select(scores, a, kept_idx, cu_kept_dev, ws,
                                      chunked ? tg::SELECT_CHUNKED : tg::SELECT_ONE_WG, stream));
}

tg_status tg_topk_select_path(const float* scores, const tg_batch_prefix* b, int32_t* kept_idx,
                              int32_t* cu_kept_dev, void* ws, size_t ws_bytes, int path,
                              hipStream_t stream) {
    tg::BatchArgs a;
    const tg_status st = plan_batch(b, &a);
    if (st != TG_OK) return st;
    return select_checked(scores, a, kept_idx, cu_kept_dev, ws, ws_bytes, path, stream);
}

tg_status tg_topk_select_prefix(const float* scores, const tg_batch_prefix* b, int32_t* kept_idx,
                                int32_t* cu_kept_dev, void* ws, size_t ws_bytes,
                                hipStream_t stream) {
    tg::BatchArgs a;
    const tg_status st = plan_batch(b, &a);
    if (st != TG_OK) return st;
    return select_checked(scores, a, kept_idx, cu_kept_dev, ws, ws_bytes, tg::SELECT_AUTO, stream);
}

tg_status tg_gather_compact(tg_dtype dt, const void* hidden, int64_t T, int32_t d_model,
                            const float* scores, const int32_t* kept_idx, int64_t Kt,
                            void* hidden_kept, float* scores_kept, hipStream_t stream) {
    if (!valid_dtype(dt)) return TG_ERR_BAD_DTYPE;
    if (T < 0 || Kt < 0 || d_model < 1 || T >= I32_LIMIT || Kt >= I32_LIMIT)
        return TG_ERR_BAD_SHAPE;
    if (hidden == nullptr || kept_idx == nullptr || hidden_kept == nullptr)
        return TG_ERR_NULL_PTR;
    if ((scores == nullptr) != (scores_kept == nullptr)) return TG_ERR_NULL_PTR;
    const int64_t row_bytes = (int64_t)d_model * elt_bytes(dt);
    if (row_bytes % 16 != 0) return TG_ERR_UNSUPPORTED;
    if (!aligned16(hidden) || !aligned16(hidden_kept) || !aligned4(kept_idx)) return TG_ERR_ALIGNMENT;
    if (scores != nullptr && (!aligned4(scores) || !aligned4(scores_kept))) return TG_ERR_ALIGNMENT;
    if (overlap(hidden_kept, Kt * row_bytes, hidden, T * row_bytes) ||
        overlap(hidden_kept, Kt * row_bytes, kept_idx, Kt * 4) ||
        overlap(scores_kept, Kt * 4, scores, T * 4) ||
        overlap(scores_kept, Kt * 4, hidden_kept, Kt * row_bytes))
        return TG_ERR_ALIAS;
    if (Kt == 0) return TG_OK;
    return launched(tg::launch_gather(hidden, T, (int)row_bytes, scores, kept_idx, Kt, hidden_kept,
                                      scores_kept, stream));
}

namespace {
tg_status attn_prefill_checked(tg_dtype dt, const void* q, const void* k, const void* v,
                               const float* s_kept, const float* gain, const float* temp,
                               const int32_t* cu_kept_host, int32_t batch, int32_t Hq,
                               int32_t Hkv, int32_t d_head, void* out, float* lse, void* ws,
                               size_t ws_bytes, bool with_ws, hipStream_t stream) {
    if (!valid_dtype(dt)) return TG_ERR_BAD_DTYPE;
    if (q == nullptr || k == nullptr || v == nullptr || temp == nullptr || cu_kept_host == nullptr ||
        out == nullptr || (s_kept == nullptr) != (gain == nullptr))
        return TG_ERR_NULL_PTR;
    if (batch < 1 || batch > TG_MAX_BATCH || Hq < 1 || Hkv < 1 || Hq % Hkv != 0)
        return TG_ERR_BAD_SHAPE;
    if (d_head != 64 && d_head != 128) return TG_ERR_UNSUPPORTED;
    tg::AttnShape sh;
    sh.batch = batch;
    sh.Hq = Hq;
    sh.Hkv = Hkv;
    sh.d_head = d_head;
    if (cu_kept_host[0] != 0) return TG_ERR_BAD_SHAPE;
    for (int i = 0; i <= batch; ++i) {
        if (i > 0 && cu_kept_host[i] < cu_kept_host[i - 1]) return TG_ERR_BAD_SHAPE;
        sh.cu[i] = cu_kept_host[i];
    }
    sh.Kt = cu_kept_host[batch];
    if (dt == TG_BF16) {
        // The bf16 kernel addresses one request's K/V rows with 32-bit offsets.
        for (int i = 0; i < batch; ++i)
            if ((int64_t)(cu_kept_host[i + 1] - cu_kept_host[i]) * Hkv * d_head * 2 >= I32_LIMIT)
                return TG_ERR_UNSUPPORTED;
    }
    const size_t need = with_ws && dt == TG_BF16 ? tg::attn_prefill_workspace_bytes(sh) : 0;
    if (need > 0 && (ws == nullptr || ws_bytes < need)) return TG_ERR_WORKSPACE;
    if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(out) ||
        (s_kept != nullptr && (!aligned4(s_kept) || !aligned4(gain))) || !aligned4(temp) ||
        (lse != nullptr && !aligned4(lse)) || (need > 0 && !aligned16(ws)))
        return TG_ERR_ALIGNMENT;
    const int64_t eb = elt_bytes(dt);
    const int64_t qb = sh.Kt * Hq * d_head * eb, kb = sh.Kt * Hkv * d_head * eb;
    const int64_t lb = (int64_t)Hq * sh.Kt * 4, wb = (int64_t)need;
    if (overlap(out, qb, q, qb) || overlap(out, qb, k, kb) || overlap(out, qb, v, kb) ||
        overlap(out, qb, s_kept, sh.Kt * 4) || overlap(lse, lb, out, qb) ||
        overlap(lse, lb, q, qb) || overlap(lse, lb, k, kb) || overlap(lse, lb, v, kb))
        return TG_ERR_ALIAS;
    if (need > 0) {
        const void* ins[] = {q, k, v, out};
        const int64_t sz[] = {qb, kb, kb, qb};
        for (int i = 0; i < 4; ++i)
            if (overlap(ws, wb, ins[i], sz[i])) return TG_ERR_ALIAS;
        if (overlap(ws, wb, s_kept, sh.Kt * 4) || overlap(ws, wb, lse, lb) ||
            overlap(ws, wb, gain, Hq * 4) || overlap(ws, wb, temp, Hq * 4))
            return TG_ERR_ALIAS;
    }
    if (sh.Kt == 0) return TG_OK;
    if (dt == TG_F32)
        return launched(tg::launch_attn_f32((const float*)q, (const float*)k, (const float*)v,
                                            s_kept, gain, temp, sh, (float*)out, lse, stream));
    return launched(tg::launch_attn_bf16(q, k, v, s_kept, gain, temp, sh, out, lse,
                                         need > 0 ? ws : nullptr, need, stream));
}
}  // namespace

tg_status tg_gated_attn_prefill(tg_dtype dt, const void* q, const void* k, const void* v,
                                const float* s_kept, const float* gain, const float* temp,
                                const int32_t* cu_kept_host, int32_t batch, int32_t Hq,
                                int32_t Hkv, int32_t d_head, void* out, float* lse,
                                hipStream_t stream) {
    return attn_prefill_checked(dt, q, k, v, s_kept, gain, temp, cu_kept_host, batch, Hq, Hkv,
                                d_head, out, lse, nullptr, 0, false, stream);
}

tg_status tg_gated_attn_prefill_ws(tg_dtype dt, const void* q, const void* k, const void* v,
                                   const float* s_kept, const float* gain, const float* temp,
                                   const int32_t* cu_kept_host, int32_t batch, int32_t Hq,
                                   int32_t Hkv, int32_t d_head, void* out, float* lse, void* ws,
                                   size_t ws_bytes, hipStream_t stream) {
    return attn_prefill_checked(dt, q, k, v, s_kept, gain, temp, cu_kept_host, batch, Hq, Hkv,
                                d_head, out, lse, ws, ws_bytes, true, stream);
}

namespace {
tg_status attn_shape(const int32_t* cu_kept_host, int32_t batch, int32_t Hq, int32_t Hkv,
                     int32_t d_head, tg::AttnShape* sh) {
    if (cu_kept_host == nullptr) return TG_ERR_NULL_PTR;
    if (batch < 1 || batch > TG_MAX_BATCH || Hq < 1 || Hkv < 1 || Hq % Hkv != 0)
        return TG_ERR_BAD_SHAPE;
    if (cu_kept_host[0] != 0) return TG_ERR_BAD_SHAPE;
    sh->batch = batch;
    sh->Hq = Hq;
    sh->Hkv = Hkv;
    sh->d_head = d_head;
    for (int i = 0; i <= batch; ++i) {
        if (i > 0 && cu_kept_host[i] < cu_kept_host[i - 1]) return TG_ERR_BAD_SHAPE;
        sh->cu[i] = cu_kept_host[i];
    }
    sh->Kt = cu_kept_host[batch];
    return TG_OK;
}
}  // namespace

tg_status tg_attn_prefill_plan(tg_dtype dt, const int32_t* cu_kept_host, int32_t batch,
                               int32_t Hq, int32_t Hkv, int32_t d_head, size_t* ws_bytes) {
    if (ws_bytes == nullptr) return TG_ERR_NULL_PTR;
    if (!valid_dtype(dt)) return TG_ERR_BAD_DTYPE;
    if (d_head != 64 && d_head != 128) return TG_ERR_UNSUPPORTED;
    tg::AttnShape sh;
    const tg_status st = attn_shape(cu_kept_host, batch, Hq, Hkv, d_head, &sh);
    if (st != TG_OK) return st;
    *ws_bytes = dt == TG_BF16 ? tg::attn_prefill_workspace_bytes(sh) : 0;
    return TG_OK;
}

tg_status tg_attn_backward_plan(const int32_t* cu_kept_host, int32_t batch, int32_t Hq, int32_t Hkv,
                                size_t* ws_bytes) {
    if (ws_bytes == nullptr) return TG_ERR_NULL_PTR;
    tg::AttnShape sh;
    const tg_status st = attn_shape(cu_kept_host, batch, Hq, Hkv, 128, &sh);
    if (st != TG_OK) return st;
    *ws_bytes = tg::attn_bwd_workspace_bytes(sh);
    return TG_OK;
}

tg_status tg_gated_attn_backward(tg_dtype dt, const void* q, const void* k, const void* v,
                                 const float* s_kept, const float* gain, const float* temp,
                                 const void* out, const float* lse, const void* dout,
                                 const int32_t* cu_kept_host, int32_t batch, int32_t Hq,
                                 int32_t Hkv, int32_t d_head, void* dq, void* dk, void* dv,
                                 float* ds, float* dgain, float* dtemp, void* ws, size_t ws_bytes,
                                 hipStream_t stream) {
    if (!valid_dtype(dt)) return TG_ERR_BAD_DTYPE;
    if (q == nullptr || k == nullptr || v == nullptr || temp == nullptr || out == nullptr ||
        lse == nullptr || dout == nullptr || dq == nullptr || dk == nullptr || dv == nullptr ||
        dtemp == nullptr)
        return TG_ERR_NULL_PTR;
    const bool bias = s_kept != nullptr;
    if ((gain != nullptr) != bias || (ds != nullptr) != bias || (dgain != nullptr) != bias)
        return TG_ERR_NULL_PTR;
    tg::AttnShape sh;
    const tg_status st = attn_shape(cu_kept_host, batch, Hq, Hkv, d_head, &sh);
    if (st != TG_OK) return st;
    if (dt != TG_BF16 || (d_head != 64 && d_head != 128) || Hq / Hkv > 64) return TG_ERR_UNSUPPORTED;
    for (int i = 0; i < batch; ++i)
        if ((int64_t)(cu_kept_host[i + 1] - cu_kept_host[i]) * Hq * d_head * 2 >= I32_LIMIT)
            return TG_ERR_UNSUPPORTED;
    const size_t need = tg::attn_bwd_workspace_bytes(sh);
    if (ws == nullptr || ws_bytes < need) return TG_ERR_WORKSPACE;
    const void* a16[] = {q, k, v, out, dout, dq, dk, dv, ws};
    for (const void* p : a16)
        if (!aligned16(p)) return TG_ERR_ALIGNMENT;
    const void* a4[] = {s_kept, gain, temp, lse, ds, dgain, dtemp};
    for (const void* p : a4)
        if (p != nullptr && !aligned4(p)) return TG_ERR_ALIGNMENT;
    const int64_t Kt = sh.Kt;
    const int64_t qb = Kt * Hq * d_head * 2, kb = Kt * Hkv * d_head * 2;
    const void* ins[] = {q, k, v, s_kept, gain, temp, out, lse, dout};
    const int64_t inb[] = {qb, kb, kb, Kt * 4, Hq * 4, Hq * 4, qb, Kt * Hq * 4, qb};
    void* outs[] = {dq, dk, dv, ds, dgain, dtemp, ws};
    const int64_t outb[] = {qb, kb, kb, Kt * 4, Hq * 4, Hq * 4, (int64_t)need};
    for (int o = 0; o < 7; ++o) {
        for (int i = 0; i < 9; ++i)
            if (overlap(outs[o], outb[o], ins[i], inb[i])) return TG_ERR_ALIAS;
        for (int o2 = o + 1; o2 < 7; ++o2)
            if (overlap(outs[o], outb[o], outs[o2], outb[o2])) return TG_ERR_ALIAS;
    }
    if (Kt == 0) return TG_OK;
    return launched(tg::launch_attn_bwd(sh, q, k, v, s_kept, gain, temp, out, lse, dout, dq, dk, dv,
                                        ds, dgain, dtemp, ws, stream));
}

namespace {
tg_status gate_bwd_shape(tg_dtype dt, int64_t Kt, int32_t d, int32_t dg) {
    if (!valid_dtype(dt)) return TG_ERR_BAD_DTYPE;
    if (Kt < 0 || Kt >= I32_LIMIT || d < 1 || dg < 1) return TG_ERR_BAD_SHAPE;
    const int m = dt == TG_BF16 ? 64 : 4;
    if (d % m != 0 || dg % m != 0) return TG_ERR_UNSUPPORTED;
    return TG_OK;
}
}  // namespace

tg_status tg_gate_backward_plan(tg_dtype dt, int64_t Kt, int32_t d_model, int32_t d_gate,
                                size_t* ws_bytes) {
    if (ws_bytes == nullptr) return TG_ERR_NULL_PTR;
    const tg_status st = gate_bwd_shape(dt, Kt, d_model, d_gate);
    if (st != TG_OK) return st;
    *ws_bytes = tg::gate_bwd_workspace_bytes(dt, Kt, d_model, d_gate);
    return TG_OK;
}

tg_status tg_gate_backward(tg_dtype dt, const void* hidden_kept, int64_t Kt, int32_t d_model,
                           const void* w1, const void* b1, const void* w2, int32_t d_gate,
                           const float* ds_kept, void* dhidden_kept, void* dw1, float* db1,
                           float* dw2, float* db2, void* ws, size_t ws_bytes, hipStream_t stream) {
    if (!valid_dtype(dt)) return TG_ERR_BAD_DTYPE;
    if (hidden_kept == nullptr || w1 == nullptr || w2 == nullptr || ds_kept == nullptr ||
        dhidden_kept == nullptr || dw1 == nullptr || dw2 == nullptr || db2 == nullptr ||
        (b1 == nullptr) != (db1 == nullptr))
        return TG_ERR_NULL_PTR;
    const tg_status st = gate_bwd_shape(dt, Kt, d_model, d_gate);
    if (st != TG_OK) return st;
    const size_t need = tg::gate_bwd_workspace_bytes(dt, Kt, d_model, d_gate);
    if (ws == nullptr || ws_bytes < need) return TG_ERR_WORKSPACE;
    const void* a16[] = {hidden_kept, w1, b1, w2, dhidden_kept, dw1, ws};
    for (const void* p : a16)
        if (p != nullptr && !aligned16(p)) return TG_ERR_ALIGNMENT;
    const void* a4[] = {ds_kept, db1, dw2, db2};
    for (const void* p : a4)
        if (p != nullptr && !aligned4(p)) return TG_ERR_ALIGNMENT;
    const int64_t eb = elt_bytes(dt);
    const int64_t xb = Kt * d_model * eb, wb = (int64_t)d_gate * d_model * eb, vb = d_gate * eb;
    const void* ins[] = {hidden_kept, w1, b1, w2, ds_kept};
    const int64_t inb[] = {xb, wb, vb, vb, Kt * 4};
    void* outs[] = {dhidden_kept, dw1, db1, dw2, db2, ws};
    const int64_t outb[] = {xb, wb, (int64_t)d_gate * 4, (int64_t)d_gate * 4, 4, (int64_t)need};
    for (int o = 0; o < 6; ++o) {
        for (int i = 0; i < 5; ++i)
            if (overlap(outs[o], outb[o], ins[i], inb[i])) return TG_ERR_ALIAS;
        for (int o2 = o + 1; o2 < 6; ++o2)
            if (overlap(outs[o], outb[o], outs[o2], outb[o2])) return TG_ERR_ALIAS;
    }
    if (Kt == 0) return TG_OK;
    return launched(tg::launch_gate_bwd(dt, hidden_kept, Kt, d_model, w1, b1, w2, d_gate, ds_kept,
                                        dhidden_kept, dw1, db1, dw2, db2, ws, stream));
}

tg_status tg_decode_plan(int32_t batch, int32_t Hq, int32_t d_head, int32_t max_len,
                         size_t* ws_bytes) {
    if (ws_bytes == nullptr) return TG_ERR_NULL_PTR;
    if (batch < 1 || batch > TG_DECODE_MAX_BATCH || Hq < 1 || max_len < 0) return TG_ERR_BAD_SHAPE;
    if (d_head != 64 && d_head != 128) return TG_ERR_UNSUPPORTED;
    *ws_bytes = tg::decode_workspace_bytes(batch, Hq, d_head, max_len);
    return TG_OK;
}

tg_status tg_gated_attn_decode(tg_dtype dt, const void* q, const void* k, const void* v,
                               const float* s, int64_t cache_rows, const int64_t* row_off,
                               const int32_t* cache_len, int32_t batch, int32_t max_len,
                               const float* gain, const float* temp, int32_t Hq, int32_t Hkv,
                               int32_t d_head, void* out, float* lse, void* ws, size_t ws_bytes,
                               hipStream_t stream) {
    if (!valid_dtype(dt)) return TG_ERR_BAD_DTYPE;
    if (q == nullptr || k == nullptr || v == nullptr || row_off == nullptr ||
        cache_len == nullptr || temp == nullptr || out == nullptr || (s == nullptr) != (gain == nullptr))
        return TG_ERR_NULL_PTR;
    if (batch < 1 || batch > TG_DECODE_MAX_BATCH || Hq < 1 || Hkv < 1 || Hq % Hkv != 0 ||
        cache_rows < 0 || max_len < 0)
        return TG_ERR_BAD_SHAPE;
    if (d_head != 64 && d_head != 128) return TG_ERR_UNSUPPORTED;
    if (Hq / Hkv > 8) return TG_ERR_UNSUPPORTED;
    const size_t need = tg::decode_workspace_bytes(batch, Hq, d_head, max_len);
    if (need > 0 && (ws == nullptr || ws_bytes < need)) return TG_ERR_WORKSPACE;
    if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(out) ||
        (need > 0 && !aligned16(ws)) || (s != nullptr && (!aligned4(s) || !aligned4(gain))) ||
        !aligned4(temp) || (lse != nullptr && !aligned4(lse)) || ((uintptr_t)row_off & 7u) != 0 ||
        !aligned4(cache_len))
        return TG_ERR_ALIGNMENT;
    const int64_t eb = elt_bytes(dt);
    const int64_t qb = (int64_t)batch * Hq * d_head * eb, kb = cache_rows * Hkv * d_head * eb;
    const int64_t sb = cache_rows * 4, lb = (int64_t)batch * Hq * 4, wb = (int64_t)need;
    const void* ins[] = {q, k, v, s, row_off, cache_len, gain, temp};
    const int64_t inb[] = {qb, kb, kb, sb, (int64_t)batch * 8, (int64_t)batch * 4, (int64_t)Hq * 4,
                           (int64_t)Hq * 4};
    for (int i = 0; i < 8; ++i)
        if (overlap(out, qb, ins[i], inb[i]) || overlap(lse, lb, ins[i], inb[i]) ||
            (need > 0 && overlap(ws, wb, ins[i], inb[i])))
            return TG_ERR_ALIAS;
    if (overlap(out, qb, lse, lb) || (need > 0 && (overlap(ws, wb, out, qb) || overlap(ws, wb, lse, lb))))
        return TG_ERR_ALIAS;
    tg::DecodeShape sh;
    sh.batch = batch;
    sh.Hq = Hq;
    sh.Hkv = Hkv;
    sh.d_head = d_head;
    sh.max_len = max_len;
    sh.rows = cache_rows;
    return launched(tg::launch_decode(dt, sh, q, k, v, s, row_off, cache_len, gain, temp, out, lse,
                                      ws, stream));
}

tg_status tg_rmsnorm(tg_dtype dt, const void* x, const void* w, float eps, int64_t M, int32_t d,
                     void* y, hipStream_t stream) {
    if (!valid_dtype(dt)) return TG_ERR_BAD_DTYPE;
    if (x == nullptr || w == nullptr || y == nullptr) return TG_ERR_NULL_PTR;
    if (M < 0 || d < 1 || !(eps >= 0.0f) || !std::isfinite(eps)) return TG_ERR_BAD_SHAPE;
    const int64_t eb = elt_bytes(dt);
    if ((int64_t)d * eb % 16 != 0) return TG_ERR_UNSUPPORTED;
    if (!aligned16(x) || !aligned16(w) || !aligned16(y)) return TG_ERR_ALIGNMENT;
    const int64_t xb = M * d * eb;
    if ((y != x && overlap(y, xb, x, xb)) || overlap(y, xb, w, d * eb)) return TG_ERR_ALIAS;
    if (M == 0) return TG_OK;
    return launched(tg::launch_rmsnorm(dt, x, w, eps, M, d, y, stream));
}

tg_status tg_kept_positions(const int32_t* kept_idx, const int32_t* cu_seqlens_host,
                            const int32_t* cu_kept_host, int32_t batch, int32_t* pos,
                            hipStream_t stream) {
    if (kept_idx == nullptr || cu_seqlens_host == nullptr || cu_kept_host == nullptr ||
        pos == nullptr)
        return TG_ERR_NULL_PTR;
    if (batch < 1 || batch > TG_MAX_BATCH) return TG_ERR_BAD_SHAPE;
    tg::BatchArgs a{};
    a.batch = batch;
    if (cu_seqlens_host[0] != 0 || cu_kept_host[0] != 0) return TG_ERR_BAD_SHAPE;
    for (int i = 0; i <= batch; ++i) {
        if (i > 0 && (cu_seqlens_host[i] < cu_seqlens_host[i - 1] || cu_kept_host[i] < cu_kept_host[i - 1]))
            return TG_ERR_BAD_SHAPE;
        a.cu_seq[i] = cu_seqlens_host[i];
        a.cu_kept[i] = cu_kept_host[i];
    }
    const int64_t Kt = cu_kept_host[batch];
    if (!aligned4(kept_idx) || !aligned4(pos)) return TG_ERR_ALIGNMENT;
    if (overlap(pos, Kt * 4, kept_idx, Kt * 4)) return TG_ERR_ALIAS;
    if (Kt == 0) return TG_OK;
    return launched(tg::launch_kept_positions(kept_idx, Kt, a, pos, stream));
}

tg_status tg_qk_norm_rope(tg_dtype dt, void* q, void* k, const void* q_norm_w, const void* k_norm_w,
                          const int32_t* pos, int64_t M, int32_t Hq, int32_t Hkv, int32_t d_head,
                          float theta, float eps, hipStream_t stream) {
    if (!valid_dtype(dt)) return TG_ERR_BAD_DTYPE;
    if (q == nullptr || k == nullptr || pos == nullptr) return TG_ERR_NULL_PTR;
    if (M < 0 || Hq < 1 || Hkv < 1 || !(theta > 0.0f) || !std::isfinite(theta) || !(eps >= 0.0f) ||
        !std::isfinite(eps))
        return TG_ERR_BAD_SHAPE;
    if (d_head != 64 && d_head != 128) return TG_ERR_UNSUPPORTED;
    if (!aligned16(q) || !aligned16(k) || (q_norm_w != nullptr && !aligned16(q_norm_w)) ||
        (k_norm_w != nullptr && !aligned16(k_norm_w)) || !aligned4(pos))
        return TG_ERR_ALIGNMENT;
    const int64_t eb = elt_bytes(dt);
    const int64_t qb = M * Hq * d_head * eb, kb = M * Hkv * d_head * eb, wb = d_head * eb;
    if (overlap(q, qb, k, kb) || overlap(q, qb, pos, M * 4) || overlap(k, kb, pos, M * 4) ||
        overlap(q, qb, q_norm_w, wb) || overlap(q, qb, k_norm_w, wb) || overlap(k, kb, q_norm_w, wb) ||
        overlap(k, kb, k_norm_w, wb))
        return TG_ERR_ALIAS;
    if (M == 0) return TG_OK;
    return launched(tg::launch_qk_norm_rope(dt, q, k, q_norm_w, k_norm_w, pos, M, Hq, Hkv, d_head,
                                            theta, eps, stream));
}

tg_status tg_silu_mul(tg_dtype dt, const void* gu, int64_t M, int32_t F, void* out,
                      hipStream_t stream) {
    if (!valid_dtype(dt)) return TG_ERR_BAD_DTYPE;
    if (gu == nullptr || out == nullptr) return TG_ERR_NULL_PTR;
    if (M < 0 || F < 1) return TG_ERR_BAD_SHAPE;
    const int64_t eb = elt_bytes(dt);
    if ((int64_t)F * eb % 16 != 0) return TG_ERR_UNSUPPORTED;
    if (!aligned16(gu) || !aligned16(out)) return TG_ERR_ALIGNMENT;
    if (overlap(out, M * F * eb, gu, M * 2 * F * eb)) return TG_ERR_ALIAS;
    if (M == 0) return TG_OK;
    return launched(tg::launch_silu_mul(dt, gu, M, F, out, stream));
}

namespace {
tg_status linear_checked(tg_dtype dt, const void* x, const void* w, void* y, int64_t M, int32_t N,
                         int32_t K, int accumulate, int tile, hipStream_t stream) {
    if (!valid_dtype(dt)) return TG_ERR_BAD_DTYPE;
    if (M < 0 || N < 1 || K < 1 || M >= I32_LIMIT || tile < 0 || tile > 3) return TG_ERR_BAD_SHAPE;
    if (x == nullptr || w == nullptr || y == nullptr) return TG_ERR_NULL_PTR;
    if (dt == TG_BF16 && (N % 64 != 0 || K % 64 != 0)) return TG_ERR_UNSUPPORTED;
    if (!aligned16(x) || !aligned16(w) || !aligned16(y)) return TG_ERR_ALIGNMENT;
    const int64_t eb = elt_bytes(dt);
    if (overlap(y, M * N * eb, x, M * K * eb) || overlap(y, M * N * eb, w, (int64_t)N * K * eb))
        return TG_ERR_ALIAS;
    if (M == 0) return TG_OK;
    if (dt == TG_F32)
        return launched(tg::launch_linear_f32((const float*)x, (const float*)w, (float*)y, M, N, K,
                                              accumulate, stream));
    return launched(tg::launch_linear_bf16(x, w, y, M, N, K, accumulate, tile, stream));
}
}  // namespace

tg_status tg_linear(tg_dtype dt, const void* x, const void* w, void* y, int64_t M, int32_t N,
                    int32_t K, int accumulate, hipStream_t stream) {
    return linear_checked(dt, x, w, y, M, N, K, accumulate, 0, stream);
}

tg_status tg_linear_tile(tg_dtype dt, const void* x, const void* w, void* y, int64_t M, int32_t N,
                         int32_t K, int accumulate, int tile, hipStream_t stream) {
    return linear_checked(dt, x, w, y, M, N, K, accumulate, tile, stream);
}

tg_status tg_linear_swiglu(tg_dtype dt, const void* x, const void* w_gu, void* out, int64_t M,
                           int32_t F, int32_t K, int tile, hipStream_t stream) {
    if (!valid_dtype(dt)) return TG_ERR_BAD_DTYPE;
    if (M < 0 || F < 1 || K < 1 || M >= I32_LIMIT || F >= I32_LIMIT / 2 || tile < 0 || tile > 3)
        return TG_ERR_BAD_SHAPE;
    if (x == nullptr || w_gu == nullptr || out == nullptr) return TG_ERR_NULL_PTR;
    if (dt != TG_BF16 || F % 128 != 0 || K % 64 != 0) return TG_ERR_UNSUPPORTED;
    if (!aligned16(x) || !aligned16(w_gu) || !aligned16(out)) return TG_ERR_ALIGNMENT;
    const int64_t ob = M * F * 2;
    if (overlap(out, ob, x, M * K * 2) || overlap(out, ob, w_gu, 2 * (int64_t)F * K * 2))
        return TG_ERR_ALIAS;
    if (M == 0) return TG_OK;
    return launched(tg::launch_linear_bf16_swiglu(x, w_gu, out, M, F, K, tile, stream));
}

tg_status tg_linear_multi(tg_dtype dt, const void* x, int32_t nseg, const void* const* w,
                          void* const* y, const int32_t* n, int64_t M, int32_t K, int accumulate,
                          int tile, hipStream_t stream) {
    if (!valid_dtype(dt)) return TG_ERR_BAD_DTYPE;
    if (nseg < 1 || nseg > TG_LINEAR_MAX_SEG || M < 0 || K < 1 || M >= I32_LIMIT || tile < 0 ||
        tile > 3)
        return TG_ERR_BAD_SHAPE;
    if (x == nullptr || w == nullptr || y == nullptr || n == nullptr) return TG_ERR_NULL_PTR;
    int64_t total = 0;
    for (int i = 0; i < nseg; ++i) {
        if (w[i] == nullptr || y[i] == nullptr) return TG_ERR_NULL_PTR;
        if (n[i] < 1) return TG_ERR_BAD_SHAPE;
        total += n[i];
    }
    if (total >= I32_LIMIT) return TG_ERR_BAD_SHAPE;
    if (dt == TG_BF16) {
        if (K % 64 != 0) return TG_ERR_UNSUPPORTED;
        for (int i = 0; i < nseg; ++i)
            if (n[i] % (nseg > 1 ? 256 : 64) != 0) return TG_ERR_UNSUPPORTED;
    }
    if (!aligned16(x)) return TG_ERR_ALIGNMENT;
    for (int i = 0; i < nseg; ++i)
        if (!aligned16(w[i]) || !aligned16(y[i])) return TG_ERR_ALIGNMENT;
    const int64_t eb = elt_bytes(dt);
    for (int i = 0; i < nseg; ++i) {
        const int64_t yb = M * n[i] * eb;
        if (overlap(y[i], yb, x, M * K * eb)) return TG_ERR_ALIAS;
        for (int j = 0; j < nseg; ++j) {
            if (overlap(y[i], yb, w[j], (int64_t)n[j] * K * eb)) return TG_ERR_ALIAS;
            if (j != i && overlap(y[i], yb, y[j], M * n[j] * eb)) return TG_ERR_ALIAS;
        }
    }
    if (M == 0) return TG_OK;
    if (dt == TG_F32) {
        for (int i = 0; i < nseg; ++i) {
            const hipError_t e = tg::launch_linear_f32((const float*)x, (const float*)w[i],
                                                       (float*)y[i], M, n[i], K, accumulate, stream);
            if (e != hipSuccess) return launched(e);
        }
        return TG_OK;
    }
    int nn[TG_LINEAR_MAX_SEG];
    for (int i = 0; i < nseg; ++i) nn[i] = n[i];
    return launched(tg::launch_linear_bf16_multi(x, nseg, w, y, nn, M, K, accumulate, tile, stream));
}

}  // extern "C"
