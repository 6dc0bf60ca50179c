/*
 * tokengate.h -- C ABI of the TokenGate pruned-prefill hot path on MI355X (gfx950).
 *
 * TokenGate (MarkTechPost article, French rendering on spke.com, section
 * "Comment TokenGate a-t-il appris le fonctionnement de la réduction des
 * tokens ?") splits prefill in three phases: layers up to the gate layer L see
 * all N tokens; at L a small MLP scores every token from its post-attention
 * residual and a top-K selector keeps the best ones; layers above L see only
 * the K kept tokens and never create KV for the pruned ones.  Only the
 * document part of the prompt may be pruned, the question never is.  In the
 * layers above L the score of each kept token is a bias on the attention
 * logits, with a learnable per-head gain and temperature (same page, "Qu'est-ce
 * que l'attention gérée par des tokens ?").  `generate` takes a
 * max_kept_prefill_tokens budget (same page, "Comment déployer TokenGate ?").
 *
 * The four calls below are those steps.  The pages sketch the bias only; the
 * attention here computes, for query row i and key j <= i of one request,
 *     l_ij = tau_h * (q_i . k_j) / sqrt(d_head) + g_h * s_j
 * and softmax over j.
 *
 * Conventions shared by every call
 *  - Tensors are DEVICE pointers owned by the caller, row-major, contiguous and
 *    16-byte aligned.  Batch metadata (tg_batch, cu_kept_host) is HOST memory,
 *    read during the call only.
 *  - The library never allocates, frees or synchronises.  Work is enqueued on
 *    `stream` (a hipStream_t; NULL = the default stream).  Pointers must stay
 *    valid until that work completes.
 *  - Output buffers must not overlap input buffers (TG_ERR_ALIAS where the
 *    extents are known on the host).
 *  - Every argument is validated on the host before anything is launched; on
 *    an error status nothing is launched and no output is written.
 *    TG_ERR_LAUNCH reports a launch failure returned by the HIP runtime.
 *    Faults inside a kernel surface at the caller's next synchronisation.
 *  - No exceptions cross the ABI.  The library keeps no mutable global state:
 *    calls on different streams are independent.
 *  - Scores, gains and temperatures are always fp32.  Hidden states and
 *    q/k/v/out are fp32 (TG_F32) or bf16 (TG_BF16); bf16 results are rounded
 *    to nearest even from fp32 accumulators.
 */
#ifndef TOKENGATE_H
#define TOKENGATE_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define TG_ABI_VERSION 1

/* Largest number of requests in one packed batch. */
#define TG_MAX_BATCH 64

typedef enum {
    TG_OK = 0,
    TG_ERR_NULL_PTR = 1,     /* a required pointer is NULL                         */
    TG_ERR_BAD_SHAPE = 2,    /* a size is negative, zero where it may not be, or
                                sizes disagree with each other                      */
    TG_ERR_BAD_BUDGET = 3,   /* a request violates N_b >= 1, 0 <= q_b <= N_b,
                                budget_b >= 1 or q_b <= min(budget_b, N_b)          */
    TG_ERR_BAD_DTYPE = 4,    /* dtype is not TG_F32 / TG_BF16                       */
    TG_ERR_UNSUPPORTED = 5,  /* valid but outside what the kernels implement        */
    TG_ERR_ALIGNMENT = 6,    /* a tensor pointer is not 16-byte aligned             */
    TG_ERR_WORKSPACE = 7,    /* workspace NULL or smaller than tg_plan reported     */
    TG_ERR_LAUNCH = 8,       /* the HIP runtime rejected a launch                   */
    TG_ERR_ALIAS = 9         /* an output buffer overlaps an input buffer           */
} tg_status;

typedef enum { TG_F32 = 0, TG_BF16 = 1 } tg_dtype;

/* A packed batch of B requests laid out back to back in the token dimension.
 * Request b owns global tokens [cu_seqlens[b], cu_seqlens[b+1]); its last
 * q_len[b] tokens are the question (never pruned), the rest is the document.
 * budget[b] is max_kept_prefill_tokens for that request and COUNTS the
 * question: min(budget[b], seq_len[b]) tokens are kept.  All three arrays are
 * host memory of length `batch` (1 <= batch <= TG_MAX_BATCH). */
typedef struct {
    int32_t batch;
    const int32_t *seq_len;
    const int32_t *q_len;
    const int32_t *budget;
} tg_batch;

/* Human-readable name of a status code (never NULL). */
const char *tg_status_str(int status);

/* TG_ABI_VERSION of the loaded library. */
int tg_abi_version(void);

/*
 * tg_plan -- host only, launches nothing.
 * Validates `b` and writes cu_seqlens[B+1] and cu_kept[B+1] (exclusive prefix
 * sums of seq_len and of K_b = min(budget_b, seq_len_b)) and the workspace
 * size tg_topk_select needs.  Any output pointer may be NULL to skip it.
 * Errors: TG_ERR_NULL_PTR (b or its arrays), TG_ERR_BAD_SHAPE (batch outside
 * [1, TG_MAX_BATCH], total tokens >= 2^31), TG_ERR_BAD_BUDGET.
 */
tg_status tg_plan(const tg_batch *b, int32_t *cu_seqlens, int32_t *cu_kept,
                  size_t *topk_ws_bytes);

/*
 * tg_gate_score -- the gate MLP (spke.com page, three-phase list, second
 * bullet: an MLP scores every token from its post-attention residual at L).
 *     s_t = w2 . GELU(W1 x_t + b1) + b2,   GELU(z) = z * Phi(z) (erf form)
 * hidden : [T][d_model] in dt            (the layer-L post-attention residual)
 * w1     : [d_gate][d_model] in dt       (torch Linear layout)
 * b1     : [d_gate] in dt, or NULL for no bias
 * w2     : [d_gate] in dt
 * b2     : [1] in dt (device scalar), or NULL for no bias
 * scores : [T] fp32 output, one score per token, question tokens included.
 * Supported: TG_F32 with d_model % 4 == 0 and d_gate <= 1024;
 *            TG_BF16 with d_model % 64 == 0 and d_gate in {64, 128, 256}.
 * T == 0 is a no-op.  Errors: TG_ERR_NULL_PTR, TG_ERR_BAD_SHAPE,
 * TG_ERR_BAD_DTYPE, TG_ERR_UNSUPPORTED, TG_ERR_ALIGNMENT, TG_ERR_LAUNCH.
 */
tg_status tg_gate_score(tg_dtype dt, const void *hidden, int64_t T, int32_t d_model,
                        const void *w1, const void *b1, const void *w2, const void *b2,
                        int32_t d_gate, float *scores, hipStream_t stream);

/*
 * tg_topk_select -- the top-K selector (spke.com page, second bullet; the
 * question is never pruned; the budget is max_kept_prefill_tokens).
 * For each request: if budget_b >= N_b every token is kept; otherwise the
 * K_b - q_b best DOCUMENT tokens under the total order
 *     (score descending, token index ascending)
 * are kept together with the whole question tail.  For ordering, -0 equals +0
 * and NaN ranks below -inf.
 * scores      : [T] fp32 (T = sum of seq_len), device
 * kept_idx    : [sum K_b] int32 output: global token ids, ascending within each
 *               request, requests in batch order (request b fills
 *               [cu_kept[b], cu_kept[b+1]))
 * cu_kept_dev : [B+1] int32 output copy of cu_kept, or NULL
 * ws/ws_bytes : device workspace of at least tg_plan's topk_ws_bytes bytes,
 *               16-byte aligned (may be NULL when that size is 0).  Its
 *               contents on entry do not matter; calls that share one
 *               workspace must not run concurrently.
 * Two implementations give identical results: when every request's document
 * has at most 32768 tokens, one 1024-thread workgroup per request selects in
 * a single launch for the whole batch (the workspace is then unused);
 * otherwise the documents are cut into chunks over many workgroups
 * (tg_topk_select_path forces either).
 * Errors: those of tg_plan, TG_ERR_NULL_PTR, TG_ERR_WORKSPACE, TG_ERR_LAUNCH.
 */
tg_status tg_topk_select(const float *scores, const tg_batch *b, int32_t *kept_idx,
                         int32_t *cu_kept_dev, void *ws, size_t ws_bytes,
                         hipStream_t stream);

/* A packed batch whose requests also start with a template prefix that is
 * never pruned (spke.com page, "Comment déployer TokenGate ?": a placeholder
 * in the prompt template marks the document that may be pruned; the template
 * text around it stays).  Request b is [prefix | document | question]:
 * prefix_len[b] leading tokens and q_len[b] trailing tokens are always kept,
 * the document is the span between them.  prefix_len is host memory of length
 * `batch`, or NULL for no prefix (then this is tg_batch). */
typedef struct {
    int32_t batch;
    const int32_t *seq_len;
    const int32_t *q_len;
    const int32_t *budget;
    const int32_t *prefix_len;
} tg_batch_prefix;

/*
 * tg_plan_prefix -- tg_plan for a tg_batch_prefix.  A request must also have
 * prefix_len[b] >= 0 and prefix_len[b] + q_len[b] <= min(budget[b],
 * seq_len[b]), else TG_ERR_BAD_BUDGET.
 */
tg_status tg_plan_prefix(const tg_batch_prefix *b, int32_t *cu_seqlens, int32_t *cu_kept,
                         size_t *topk_ws_bytes);

/*
 * tg_topk_select_prefix -- tg_topk_select for a tg_batch_prefix: when the
 * budget does not cover the request, the K_b - p_b - q_b best document tokens
 * (same order as tg_topk_select, document span [p_b, N_b - q_b)) are kept with
 * the whole prefix and the whole question; kept ids ascend within a request.
 * The workspace size comes from tg_plan_prefix.  Errors: those of
 * tg_plan_prefix and of tg_topk_select.
 *
 * Random-K selection (same page, benchmarks: even a random choice of K
 * tokens scores well on the co-adapted backbone) is this selector, or
 * tg_topk_select, run on random keys in place of the gate scores: the caller
 * draws them (the library draws no random numbers) and passes them as
 * `scores`; ties go to the lower index as always.
 */
tg_status tg_topk_select_prefix(const float *scores, const tg_batch_prefix *b, int32_t *kept_idx,
                                int32_t *cu_kept_dev, void *ws, size_t ws_bytes,
                                hipStream_t stream);

/* Size of the device scratch array behind tg_topk_select_noalloc. */
#define TG_SELECT_SCRATCH_BYTES ((size_t)8 << 20)

/*
 * tg_topk_select_noalloc -- tg_topk_select for callers that cannot allocate
 * device memory: code under HIP graph capture, tight serving loops, harnesses
 * that forbid hipMalloc.  The selector's workspace is a file-scope device
 * array of TG_SELECT_SCRATCH_BYTES (8 MiB) inside the library; every GPU the
 * library runs on holds its own copy until the process ends.  The call
 * allocates and frees nothing; the caller still owns scores, kept_idx and
 * cu_kept_dev.  Arguments and results as tg_topk_select.
 * Limit: a batch that tg_topk_select runs on the one-workgroup path (every
 * document at most 32768 tokens) uses no scratch; any other batch must need at most
 * TG_SELECT_SCRATCH_BYTES of workspace (tg_plan's topk_ws_bytes; a single
 * request of up to about 900k tokens), else TG_ERR_WORKSPACE and nothing is
 * launched.
 * Every call on one GPU shares that GPU's scratch, which keeps the previous
 * call's contents (the call clears what must start at zero itself): calls
 * that overlap in time on one GPU (two streams, two host threads) race, and
 * the caller must serialise them.
 * Errors: those of tg_topk_select (TG_ERR_WORKSPACE as above), and
 * TG_ERR_LAUNCH when the scratch address cannot be obtained.
 */
tg_status tg_topk_select_noalloc(const float *scores, const tg_batch *b, int32_t *kept_idx,
                                 int32_t *cu_kept_dev, hipStream_t stream);

/*
 * tg_topk_select_path -- tg_topk_select_prefix with the implementation chosen
 * by the caller (for testing that both give the same kept ids; prefix_len may
 * be NULL, which is tg_topk_select): path 0 chooses as tg_topk_select does,
 * 1 forces the one-workgroup path (TG_ERR_UNSUPPORTED when a document has
 * more than 65536 tokens), 2 forces the chunked path.  Any other path is
 * TG_ERR_BAD_SHAPE.  Other arguments and errors as tg_topk_select_prefix.
 */
tg_status tg_topk_select_path(const float *scores, const tg_batch_prefix *b, int32_t *kept_idx,
                              int32_t *cu_kept_dev, void *ws, size_t ws_bytes, int path,
                              hipStream_t stream);

/*
 * tg_gather_compact -- compaction (spke.com page, third bullet: layers above L
 * process only the kept tokens).
 *     hidden_kept[r] = hidden[kept_idx[r]]   (bit for bit)
 *     scores_kept[r] = scores[kept_idx[r]]   (when both pointers are given)
 * hidden      : [T][d_model] in dt;  kept_idx : [Kt] int32 in [0, T)
 * hidden_kept : [Kt][d_model] in dt output
 * scores, scores_kept : [T] / [Kt] fp32, both NULL or both non-NULL
 * An index outside [0, T) is not dereferenced: its output row is left as is
 * and its score is set to NaN.
 * Supported: d_model * sizeof(dt) % 16 == 0.  Kt == 0 is a no-op.
 */
tg_status tg_gather_compact(tg_dtype dt, const void *hidden, int64_t T, int32_t d_model,
                            const float *scores, const int32_t *kept_idx, int64_t Kt,
                            void *hidden_kept, float *scores_kept, hipStream_t stream);

/*
 * tg_gated_attn_prefill -- causal GQA token-gated attention over the kept
 * tokens (spke.com page, "Qu'est-ce que l'attention gérée par des tokens ?").
 * For request b (rows [cu_kept_host[b], cu_kept_host[b+1])), query head h,
 * KV head h / (Hq / Hkv), local query row i and local key j <= i:
 *     l_ij = temp[h] * (q_i . k_j) / sqrt(d_head) + gain[h] * s_kept[j]
 *     out_i = sum_j softmax_j(l_ij) v_j,   lse_i = ln sum_j exp(l_ij)
 * Requests never attend to each other.
 * q   : [Kt][Hq][d_head] in dt       k, v : [Kt][Hkv][d_head] in dt
 * s_kept : [Kt] fp32                 gain, temp : [Hq] fp32
 * s_kept and gain may both be NULL: the bias term is then zero (plain causal
 * GQA attention with the per-head temperature; the kernel is built without
 * the bias stage).  Exactly one of them NULL is TG_ERR_NULL_PTR.
 * cu_kept_host : [batch+1] HOST int32, cu_kept_host[0] == 0, non-decreasing
 * out : [Kt][Hq][d_head] in dt output
 * lse : [Hq][Kt] fp32 output, or NULL
 * Supported: d_head in {64, 128}, Hq % Hkv == 0, 1 <= batch <= TG_MAX_BATCH;
 * for TG_BF16 the K (and V) rows of one request span less than 2 GiB,
 * (cu_kept_host[b+1] - cu_kept_host[b]) * Hkv * d_head * 2 < 2^31, else
 * TG_ERR_UNSUPPORTED.
 * Only K/V rows of kept tokens exist: nothing of size N is read or written.
 * Errors: TG_ERR_BAD_DTYPE, TG_ERR_NULL_PTR, TG_ERR_BAD_SHAPE (batch, heads,
 * cu_kept_host), TG_ERR_UNSUPPORTED, TG_ERR_ALIGNMENT, TG_ERR_ALIAS,
 * TG_ERR_LAUNCH.
 */
tg_status tg_gated_attn_prefill(tg_dtype dt, const void *q, const void *k, const void *v,
                                const float *s_kept, const float *gain, const float *temp,
                                const int32_t *cu_kept_host, int32_t batch, int32_t Hq,
                                int32_t Hkv, int32_t d_head, void *out, float *lse,
                                hipStream_t stream);

/*
 * tg_attn_prefill_plan -- workspace bytes of tg_gated_attn_prefill_ws for this
 * packed batch (arguments as for tg_gated_attn_prefill).  Nonzero only for
 * TG_BF16, a single request, two or more query heads per KV head, a request
 * too short to give every CU two workgroups with whole query tiles (fewer
 * than 512 four-wave workgroups), and a longest query tile of more than 18
 * key tiles of 64; *ws_bytes = 0 otherwise.  Errors: TG_ERR_NULL_PTR,
 * TG_ERR_BAD_DTYPE, TG_ERR_BAD_SHAPE, TG_ERR_UNSUPPORTED (d_head).
 */
tg_status tg_attn_prefill_plan(tg_dtype dt, const int32_t *cu_kept_host, int32_t batch,
                               int32_t Hq, int32_t Hkv, int32_t d_head, size_t *ws_bytes);

/*
 * tg_gated_attn_prefill_ws -- tg_gated_attn_prefill with a caller workspace
 * (the same attention: spke.com page, "Qu'est-ce que l'attention gérée par
 * des tokens ?").  When tg_attn_prefill_plan gives nonzero bytes, each query
 * tile is cut into pieces of near-equal length, at most 24 key tiles of 64
 * (at most 16 when the request's longest tile has 19 to 24), one
 * workgroup each, so that the short causal tiles of one request spread over
 * the whole chip.  Each piece leaves its unnormalised output, exponent base
 * and row sum in fp32 in ws; the last piece of a tile to finish combines the
 * pieces in piece order (the result does not depend on which finishes last)
 * and writes out and lse.  The result equals tg_gated_attn_prefill's within
 * the rounding of the bf16 probabilities and the fp32 sums (the bf16 outputs
 * may differ in the last bits).
 * ws : at least tg_attn_prefill_plan bytes, caller-owned, 16-byte aligned;
 *      may be NULL when that size is 0.  Its first 2048 bytes are per-tile
 *      counters that must be zero before the first call: zero-fill the
 *      workspace once when it is allocated.  Every call that completes leaves
 *      them zero again, so the workspace serves any later call (of any shape)
 *      without clearing.  Calls that share one workspace must not run
 *      concurrently.
 * Errors: those of tg_gated_attn_prefill, and TG_ERR_WORKSPACE.
 */
tg_status tg_gated_attn_prefill_ws(tg_dtype dt, const void *q, const void *k, const void *v,
                                   const float *s_kept, const float *gain, const float *temp,
                                   const int32_t *cu_kept_host, int32_t batch, int32_t Hq,
                                   int32_t Hkv, int32_t d_head, void *out, float *lse, void *ws,
                                   size_t ws_bytes, hipStream_t stream);

/*
 * tg_attn_backward_plan -- workspace bytes of tg_gated_attn_backward for this
 * packed batch (cu_kept_host as for tg_gated_attn_prefill).  Errors:
 * TG_ERR_NULL_PTR, TG_ERR_BAD_SHAPE (batch, heads, cu_kept_host).
 */
tg_status tg_attn_backward_plan(const int32_t *cu_kept_host, int32_t batch, int32_t Hq,
                                int32_t Hkv, size_t *ws_bytes);

/*
 * tg_gated_attn_backward -- gradients of the token-gated attention.  The
 * score bias is the path by which the gate receives a gradient (spke.com
 * page, "Qu'est-ce que l'attention gérée par des tokens ?"; the top-K choice
 * itself has none).  For the forward of tg_gated_attn_prefill on the same
 * inputs, with out and lse as it returned them and an upstream gradient dout
 * of the loss with respect to out, with l_ij = temp[h] r_ij + gain[h] s_j,
 * r_ij = q_i.k_j / sqrt(d_head), P = softmax_j(l), D_i = dout_i . out_i,
 * dL_ij = P_ij (dout_i . v_j - D_i):
 *     dq_i = temp[h]/sqrt(d_head) sum_j dL_ij k_j
 *     dk_j = sum_h temp[h]/sqrt(d_head) sum_i dL_ij q_i     (h over the group)
 *     dv_j = sum_h sum_i P_ij dout_i
 *     ds_j = sum_h gain[h] sum_i dL_ij,  dgain[h] = sum_ij dL_ij s_j,
 *     dtemp[h] = sum_ij dL_ij r_ij
 * Layouts as in tg_gated_attn_prefill: q, out, dout, dq [Kt][Hq][d_head];
 * k, v, dk, dv [Kt][Hkv][d_head]; lse [Hq][Kt] fp32; s_kept, ds [Kt] fp32;
 * gain, temp, dgain, dtemp [Hq] fp32.  s_kept, gain, ds and dgain are all
 * NULL (no bias term) or all non-NULL.  Every gradient is overwritten.
 * ws: tg_attn_backward_plan bytes, caller-owned, 16-byte aligned, no
 * initialisation needed.  Deterministic: no floating-point atomics.
 * Supported: TG_BF16 only, d_head in {64, 128}, Hq % Hkv == 0 with
 * Hq / Hkv <= 64, per-request K/V spans below 2 GiB; else TG_ERR_UNSUPPORTED.
 * Errors: TG_ERR_BAD_DTYPE, TG_ERR_NULL_PTR, TG_ERR_BAD_SHAPE,
 * TG_ERR_UNSUPPORTED, TG_ERR_ALIGNMENT, TG_ERR_WORKSPACE, TG_ERR_ALIAS,
 * TG_ERR_LAUNCH.
 */
tg_status tg_gated_attn_backward(tg_dtype dt, const void *q, const void *k, const void *v,
                                 const float *s_kept, const float *gain, const float *temp,
                                 const void *out, const float *lse, const void *dout,
                                 const int32_t *cu_kept_host, int32_t batch, int32_t Hq,
                                 int32_t Hkv, int32_t d_head, void *dq, void *dk, void *dv,
                                 float *ds, float *dgain, float *dtemp, void *ws,
                                 size_t ws_bytes, hipStream_t stream);

/*
 * tg_gate_backward_plan -- workspace bytes of tg_gate_backward.  Errors:
 * TG_ERR_NULL_PTR, TG_ERR_BAD_DTYPE, TG_ERR_BAD_SHAPE.
 */
tg_status tg_gate_backward_plan(tg_dtype dt, int64_t Kt, int32_t d_model, int32_t d_gate,
                                size_t *ws_bytes);

/*
 * tg_gate_backward -- gradients of the gate MLP over the kept rows.  The gate
 * is trained through the score bias of the attention above it (spke.com page,
 * "Comment TokenGate a-t-il appris ..."); the top-K choice has no gradient, so
 * only kept tokens receive one.  With z_t = W1 x_t + b1,
 * s_t = w2 . GELU(z_t) + b2 and the score gradient ds (for instance ds of
 * tg_gated_attn_backward), over the Kt given rows:
 *     dz_t = ds_t * w2 * GELU'(z_t),   GELU'(z) = Phi(z) + z phi(z)
 *     dhidden_t = W1^T dz_t,  dw1 = sum_t dz_t x_t^T,  db1 = sum_t dz_t,
 *     dw2 = sum_t ds_t GELU(z_t),  db2 = sum_t ds_t
 * hidden_kept : [Kt][d_model] in dt (the gathered kept rows; a pruned token's
 * gradient is zero and its row need not be passed);  w1 [d_gate][d_model],
 * b1 [d_gate] (nullable), w2 [d_gate] in dt;  ds_kept [Kt] fp32.
 * dhidden_kept [Kt][d_model] and dw1 [d_gate][d_model] in dt; db1 (NULL iff
 * b1 is NULL), dw2 [d_gate] and db2 [1] fp32.  All overwritten.
 * ws: tg_gate_backward_plan bytes, caller-owned, 16-byte aligned.
 * The products run on the tg_linear kernels with fp32 accumulation.  For
 * TG_BF16 the two products with few output tiles are split over their
 * contraction into fp32 partials summed in a fixed order: z (over d_model;
 * z is not rounded before GELU') and dw1 (over the kept rows); dz and the
 * outputs are rounded once to dt.  For TG_F32, z, dz and the outputs are
 * fp32.  The column sums are fixed-order reductions.
 * Supported: TG_BF16 with d_model and d_gate multiples of 64, TG_F32 with
 * multiples of 4.  Kt == 0 is a no-op.  Errors: TG_ERR_BAD_DTYPE,
 * TG_ERR_NULL_PTR, TG_ERR_BAD_SHAPE, TG_ERR_UNSUPPORTED, TG_ERR_ALIGNMENT,
 * TG_ERR_WORKSPACE, TG_ERR_ALIAS, TG_ERR_LAUNCH.
 */
tg_status tg_gate_backward(tg_dtype dt, const void *hidden_kept, int64_t Kt, int32_t d_model,
                           const void *w1, const void *b1, const void *w2, int32_t d_gate,
                           const float *ds_kept, void *dhidden_kept, void *dw1, float *db1,
                           float *dw2, float *db2, void *ws, size_t ws_bytes,
                           hipStream_t stream);

/* Cached rows per split of tg_gated_attn_decode; its workspace is sized in
 * these. */
#define TG_DECODE_CHUNK 128
/* Largest batch of tg_gated_attn_decode (one grid dimension per request). */
#define TG_DECODE_MAX_BATCH 65535

/*
 * tg_decode_plan -- workspace bytes for tg_gated_attn_decode with this batch,
 * query-head count, head size and largest cache length (host only; 0 bytes
 * when max_len == 0).  Errors: TG_ERR_NULL_PTR (ws_bytes), TG_ERR_BAD_SHAPE
 * (batch outside [1, TG_DECODE_MAX_BATCH], Hq < 1, max_len < 0),
 * TG_ERR_UNSUPPORTED (d_head not 64 or 128).
 */
tg_status tg_decode_plan(int32_t batch, int32_t Hq, int32_t d_head, int32_t max_len,
                         size_t *ws_bytes);

/*
 * tg_gated_attn_decode -- one generation step of token-gated attention over
 * the kept-only KV cache.  Pruned tokens never get a KV record (spke.com page,
 * three-phase list, third bullet), so after a pruned prefill the cache holds
 * the kept rows, each with its gate score, and generation runs on them (page
 * "Comment déployer TokenGate ?").  The pages do not say whether the score
 * bias applies while generating; here it does, with the prefill's logit.
 * For request b, query head h and KV head h / (Hq / Hkv), over the
 * n_b = min(cache_len[b], max_len) cached rows r_j = row_off[b] + j, j < n_b
 * (the new token's own row already appended, so no causal mask):
 *     l_j = temp[h] * (q_bh . k[r_j]) / sqrt(d_head) + gain[h] * s[r_j]
 *     out_bh = sum_j softmax_j(l_j) v[r_j],   lse_bh = ln sum_j exp(l_j)
 * q    : [batch][Hq][d_head] in dt      out : same shape, dt output
 * k, v : [cache_rows][Hkv][d_head] in dt, the row pool of every request
 *        (packed back to back, padded per request, or anything in between)
 * s    : [cache_rows] fp32; s and gain may both be NULL (no bias term)
 * gain, temp : [Hq] fp32           lse : [batch][Hq] fp32 output or NULL
 * row_off   : [batch] DEVICE int64 first pool row of each request
 * cache_len : [batch] DEVICE int32 cached rows of each request
 *   Both are read on the device, so a decode loop needs no host round trip.
 *   A row outside [0, cache_rows) counts as absent and is never read; a
 *   request with no row present gets out = 0 and lse = -inf.
 * ws   : tg_decode_plan bytes of device memory, caller-owned, 16-byte
 *        aligned, no initialisation needed (NULL allowed when 0 bytes).
 * Supported: d_head in {64, 128}, Hq % Hkv == 0 with Hq / Hkv <= 8, else
 * TG_ERR_UNSUPPORTED.  Two kernels on `stream`: per (chunk of
 * TG_DECODE_CHUNK rows, KV head, request) softmax partials, then their merge.
 * Errors: TG_ERR_BAD_DTYPE, TG_ERR_NULL_PTR, TG_ERR_BAD_SHAPE,
 * TG_ERR_UNSUPPORTED, TG_ERR_ALIGNMENT, TG_ERR_WORKSPACE, TG_ERR_ALIAS,
 * TG_ERR_LAUNCH.
 */
tg_status tg_gated_attn_decode(tg_dtype dt, const void *q, const void *k, const void *v,
                               const float *s, int64_t cache_rows, const int64_t *row_off,
                               const int32_t *cache_len, int32_t batch, int32_t max_len,
                               const float *gain, const float *temp, int32_t Hq, int32_t Hkv,
                               int32_t d_head, void *out, float *lse, void *ws,
                               size_t ws_bytes, hipStream_t stream);

/* ---- The rest of a pruned decoder layer on the kept rows ----------------
 * Layers above the gate run on the kept tokens only (spke.com page,
 * three-phase list, third bullet).  The pages name the Qwen3-1.7B backbone
 * but not its layer; these calls are the pieces of the published Qwen3
 * decoder layer that are not projections (tg_linear) or attention:
 *   x  -> tg_rmsnorm -> tg_linear (q, k, v) -> tg_qk_norm_rope
 *      -> tg_gated_attn_prefill -> tg_linear (o, accumulate into x)
 *      -> tg_rmsnorm -> tg_linear (gate|up) -> tg_silu_mul
 *      -> tg_linear (down, accumulate into x)
 * All run on the caller's stream, allocate nothing and compute in fp32 with
 * one rounding at each store. */

/*
 * tg_rmsnorm -- y[m] = x[m] / sqrt(mean_j x[m][j]^2 + eps) * w, rows of d.
 * x, y : [M][d] in dt (y == x allowed: in place; other overlaps are
 * TG_ERR_ALIAS);  w : [d] in dt.  Supported: d * sizeof(dt) % 16 == 0.
 * M == 0 is a no-op.  Errors: TG_ERR_BAD_DTYPE, TG_ERR_NULL_PTR,
 * TG_ERR_BAD_SHAPE (M < 0, d < 1, eps < 0 or not finite), TG_ERR_UNSUPPORTED,
 * TG_ERR_ALIGNMENT, TG_ERR_ALIAS, TG_ERR_LAUNCH.
 */
tg_status tg_rmsnorm(tg_dtype dt, const void *x, const void *w, float eps, int64_t M, int32_t d,
                     void *y, hipStream_t stream);

/*
 * tg_kept_positions -- the original position of each kept row inside its
 * request: pos[r] = kept_idx[r] - cu_seqlens_host[b] for the request b with
 * cu_kept_host[b] <= r < cu_kept_host[b+1].  A kept token keeps the position
 * it had in the full prompt (the rotary embedding of the layers above the
 * gate uses it).  kept_idx, pos : [Kt] DEVICE int32, Kt = cu_kept_host[batch];
 * cu_seqlens_host, cu_kept_host : [batch+1] HOST int32 as returned by tg_plan.
 * Errors: TG_ERR_NULL_PTR, TG_ERR_BAD_SHAPE (batch, offsets not starting at 0
 * or decreasing), TG_ERR_ALIGNMENT, TG_ERR_ALIAS, TG_ERR_LAUNCH.
 */
tg_status tg_kept_positions(const int32_t *kept_idx, const int32_t *cu_seqlens_host,
                            const int32_t *cu_kept_host, int32_t batch, int32_t *pos,
                            hipStream_t stream);

/*
 * tg_qk_norm_rope -- in place on q [M][Hq][d_head] and k [M][Hkv][d_head]
 * (dt): each head vector is RMS-normalised over d_head with its weight
 * (q_norm_w / k_norm_w, [d_head] in dt; NULL skips that normalisation), then
 * rotated (rotary embedding, RoFormer, half-split pairing): for i < d_head/2
 * and a = pos[m] * theta^(-2i/d_head),
 *     x'_i = x_i cos a - x_{i+d/2} sin a,   x'_{i+d/2} = x_{i+d/2} cos a + x_i sin a.
 * pos : [M] DEVICE int32 (tg_kept_positions).  The angle is formed and reduced
 * modulo 2 pi in double precision; sin and cos in fp32.
 * Supported: d_head in {64, 128}.  M == 0 is a no-op.  Errors:
 * TG_ERR_BAD_DTYPE, TG_ERR_NULL_PTR (q, k, pos), TG_ERR_BAD_SHAPE (M < 0,
 * heads < 1, theta <= 0, eps < 0), TG_ERR_UNSUPPORTED, TG_ERR_ALIGNMENT,
 * TG_ERR_ALIAS, TG_ERR_LAUNCH.
 */
tg_status tg_qk_norm_rope(tg_dtype dt, void *q, void *k, const void *q_norm_w,
                          const void *k_norm_w, const int32_t *pos, int64_t M, int32_t Hq,
                          int32_t Hkv, int32_t d_head, float theta, float eps,
                          hipStream_t stream);

/*
 * tg_silu_mul -- the SwiGLU product: out[m][j] = silu(gu[m][j]) * gu[m][F+j]
 * with silu(z) = z / (1 + e^-z); gu : [M][2F] in dt (the gate and up
 * projections side by side, as one tg_linear with the two weights stacked),
 * out : [M][F] in dt.  Supported: F * sizeof(dt) % 16 == 0.  M == 0 is a
 * no-op.  Errors: TG_ERR_BAD_DTYPE, TG_ERR_NULL_PTR, TG_ERR_BAD_SHAPE,
 * TG_ERR_UNSUPPORTED, TG_ERR_ALIGNMENT, TG_ERR_ALIAS, TG_ERR_LAUNCH.
 */
tg_status tg_silu_mul(tg_dtype dt, const void *gu, int64_t M, int32_t F, void *out,
                      hipStream_t stream);

/*
 * tg_linear -- auxiliary projection for layers above the gate, run on the
 * kept rows only (spke.com page, third bullet).
 *     y[M][N] = x[M][K] . w[N][K]^T            (accumulate == 0)
 *     y[M][N] = y[M][N] + x[M][K] . w[N][K]^T  (accumulate != 0; residual add)
 * fp32 accumulation, one rounding to dt at the store.
 * Supported: TG_BF16 with N % 64 == 0 and K % 64 == 0; TG_F32 any N, K with
 * K % 4 == 0.  M == 0 is a no-op.  The bf16 output tile (128x128, 256x128 or
 * 256x256 rows x columns per workgroup) is the largest that still gives every
 * compute unit work.  Errors: TG_ERR_BAD_DTYPE, TG_ERR_BAD_SHAPE,
 * TG_ERR_NULL_PTR, TG_ERR_UNSUPPORTED, TG_ERR_ALIGNMENT, TG_ERR_ALIAS,
 * TG_ERR_LAUNCH.
 */
tg_status tg_linear(tg_dtype dt, const void *x, const void *w, void *y, int64_t M,
                    int32_t N, int32_t K, int accumulate, hipStream_t stream);

/*
 * tg_linear_tile -- tg_linear with the bf16 output tile chosen by the caller
 * (for testing every tile on the same shapes): tile 0 chooses as tg_linear
 * does, 1 forces 128x128, 2 forces 256x128, 3 forces 256x256; any other tile
 * is TG_ERR_BAD_SHAPE.  The fp32 path ignores it.  Other arguments and errors
 * as tg_linear.
 */
tg_status tg_linear_tile(tg_dtype dt, const void *x, const void *w, void *y, int64_t M,
                         int32_t N, int32_t K, int accumulate, int tile, hipStream_t stream);

/*
 * tg_linear_swiglu -- the gate and up projections of the feed-forward block
 * of a layer above the gate with the SwiGLU product in their epilogue, on
 * the kept rows only (spke.com page, three-phase list, third bullet):
 *     out[M][F] = silu(x . w_gu[0:F]^T) * (x . w_gu[F:2F]^T),
 * silu(z) = z / (1 + e^-z), from the fp32 accumulators, one rounding to bf16
 * at the store (tg_linear followed by tg_silu_mul rounds both products to
 * bf16 first).  x : [M][K], w_gu : [2F][K] (gate rows, then up rows),
 * out : [M][F], bf16, device.  tile as in tg_linear_tile (0 chooses from M
 * and 2F).  Supported: TG_BF16 with F % 128 == 0 and K % 64 == 0, else
 * TG_ERR_UNSUPPORTED.  M == 0 is a no-op.  Errors: TG_ERR_BAD_DTYPE,
 * TG_ERR_BAD_SHAPE, TG_ERR_NULL_PTR, TG_ERR_UNSUPPORTED, TG_ERR_ALIGNMENT,
 * TG_ERR_ALIAS, TG_ERR_LAUNCH.
 */
tg_status tg_linear_swiglu(tg_dtype dt, const void *x, const void *w_gu, void *out, int64_t M,
                           int32_t F, int32_t K, int tile, hipStream_t stream);

/* Most products of one tg_linear_multi call. */
#define TG_LINEAR_MAX_SEG 3

/*
 * tg_linear_multi -- several projections of the same rows in one launch:
 * the q, k and v projections of a layer above the gate, run on the kept
 * rows only (spke.com page, three-phase list, third bullet).  For i < nseg:
 *     y_i[M][n_i] (+)= x[M][K] . w_i[n_i][K]^T
 * with accumulate as for tg_linear, fp32 accumulation and one rounding to dt
 * at the store.  x : [M][K] device; w, y : HOST arrays of nseg device
 * pointers (w_i [n_i][K], y_i [M][n_i], each contiguous); n : HOST array of
 * the nseg sizes; 1 <= nseg <= TG_LINEAR_MAX_SEG.  The bf16 products share
 * one grid whose output tile is chosen from M and the sum of the n_i as
 * tg_linear chooses it (tile: 0, or 1-3 to force one as in tg_linear_tile);
 * each y_i is bit-identical to tg_linear_tile of the same product with that
 * tile.  TG_F32 runs the products one after another.
 * Supported: TG_BF16 with K % 64 == 0 and every n_i a multiple of 256 (of
 * 64 when nseg == 1); TG_F32 with K % 4 == 0.  M == 0 is a no-op.
 * Errors: TG_ERR_BAD_DTYPE, TG_ERR_BAD_SHAPE (nseg, M, K, n_i, tile),
 * TG_ERR_NULL_PTR, TG_ERR_UNSUPPORTED, TG_ERR_ALIGNMENT, TG_ERR_ALIAS (an
 * output overlapping x, a weight or another output), TG_ERR_LAUNCH.
 */
tg_status tg_linear_multi(tg_dtype dt, const void *x, int32_t nseg, const void *const *w,
                          void *const *y, const int32_t *n, int64_t M, int32_t K, int accumulate,
                          int tile, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* TOKENGATE_H */
