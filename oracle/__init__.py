"""CPU oracle for the TokenGate pruned-prefill path -- TEST INFRASTRUCTURE ONLY.

Only the test-suite, the package's smoke check and the benchmark's CPU-baseline
leg may import this module.  The product path (the HIP library and its Python
binding) never calls it and shares no code with it.

Every function is the plain definition of one step, in float64 on the CPU,
with library primitives (matmul, erf, exp, a stable lexicographic sort) as the
only building blocks and no blocking, fusion or reordering.  The steps follow
the three-phase forward pass and the token-gated attention described on the
MarkTechPost article as rendered in French on spke.com ("Comment TokenGate
a-t-il appris le fonctionnement de la réduction des tokens ?" and "Qu'est-ce que
l'attention gérée par des tokens ?"):

* a small MLP scores every token from its post-attention residual at the gate
  layer L                                               -> ``gate_score``
* a top-K selector keeps the best-scoring tokens; only the document part of
  the prompt may be dropped, the question is always kept -> ``topk_select``
* layers above L process only the K kept tokens and create no KV for the
  dropped ones                                           -> ``gather_compact``
* each kept token's score becomes a bias on the attention logits, with a
  learnable per-head gain and a per-head temperature     -> ``gated_attention``
* generation then reads a KV cache that holds the kept tokens only, each row
  with its score; a new token attends to every cached row with the same bias
                                                         -> ``gated_decode_attention``

The pages only sketch the bias.  The exact logit used here is
``tau_h * (q_i . k_j) / sqrt(d_head) + g_h * s_j`` over causal ``j <= i``.

Pins (tests/test_oracle_pins.py): the gate against torch's own Linear+GELU and
textbook values of the normal CDF; the selector against brute force (Python
``sorted`` and an O(N^2) rank count) and its invariants; the attention against
torch's scaled_dot_product_attention (plain causal when gains are 0 and
temperatures 1, with an explicit additive mask otherwise) and closed forms (row
0, shift invariance, a dominant key); the decode attention against SDPA with
a float mask, against the last row of the prefill attention, and closed forms
(one cached row, empty cache, layout independence); the layer stack against an
independent float64 composition; the rest of the pruned layer against torch's
rms_norm, rotary embedding written as complex multiplication, torch's silu,
and an independent composition of the whole layer.  Nothing here is "parity unpinned" except what the pages
themselves leave open: fidelity to the authors' unpublished kernels.
"""
from __future__ import annotations

import bisect
import math
from typing import Dict, List, Optional, Sequence, Tuple

import numpy as np
import torch

__all__ = [
    "gelu_erf",
    "gate_score",
    "plan",
    "topk_select",
    "gather_compact",
    "gated_attention",
    "gated_attention_rows",
    "gated_decode_attention",
    "linear",
    "stack_forward",
    "rms_norm",
    "rope",
    "silu",
    "swiglu",
    "kept_positions",
    "decoder_layer",
    "gated_attention_backward",
    "gate_backward",
]


# --------------------------------------------------------------------------
# Gate MLP (spke.com page, three-phase list, second bullet: an MLP scores each
# token from its post-attention residual at layer L).
# The activation is GELU in its exact (erf) form; the score is the raw MLP
# output, with no squashing: the selector only needs an order, and the bias
# uses the score itself.
# --------------------------------------------------------------------------
def gelu_erf(z: torch.Tensor) -> torch.Tensor:
    """GELU(z) = z * Phi(z) = z/2 * (1 + erf(z / sqrt 2)), float64."""
    z = z.double()
    return 0.5 * z * (1.0 + torch.erf(z / math.sqrt(2.0)))


def gate_score(hidden: torch.Tensor, w1: torch.Tensor, b1: Optional[torch.Tensor],
               w2: torch.Tensor, b2: Optional[torch.Tensor]) -> torch.Tensor:
    """s_t = w2 . GELU(W1 x_t + b1) + b2 for every token t, returned as fp32.

    hidden[T][d], w1[d_gate][d] (Linear layout), b1[d_gate] or None,
    w2[d_gate], b2[1] or None.  Computed in float64 from the stored values,
    rounded once to fp32 (round to nearest even).
    """
    x = hidden.double()
    z = x @ w1.double().t()
    if b1 is not None:
        z = z + b1.double()
    h = gelu_erf(z)
    s = h @ w2.double()
    if b2 is not None:
        s = s + b2.double().reshape(())
    return s.float()


# --------------------------------------------------------------------------
# Top-K selection (spke.com page: the top-K selector keeps the best-scoring
# tokens; only the document may be pruned, the question never is; `generate`
# takes a max_kept_prefill_tokens budget, "Comment déployer TokenGate ?").
# Readings: the budget counts the question tail; the question is the tail of
# each request; ties go to the lower token index; -0 equals +0; NaN ranks below
# -inf; the kept ids come out ascending.
# --------------------------------------------------------------------------
def plan(seq_len: Sequence[int], q_len: Sequence[int], budget: Sequence[int],
         prefix_len: Optional[Sequence[int]] = None) -> Tuple[List[int], List[int]]:
    """Validate a batch and return (cu_seqlens, cu_kept), each of length B+1.

    Kept per request is min(budget_b, N_b).  Raises ValueError when N_b < 1,
    q_b outside [0, N_b], budget_b < 1, p_b < 0 (template prefix, default 0)
    or p_b + q_b > min(budget_b, N_b).
    """
    if prefix_len is None:
        prefix_len = [0] * len(seq_len)
    if not (len(seq_len) == len(q_len) == len(budget) == len(prefix_len)) or len(seq_len) < 1:
        raise ValueError("batch arrays must have one equal, non-zero length")
    cu_s, cu_k = [0], [0]
    for n, q, k, p in zip(seq_len, q_len, budget, prefix_len):
        n, q, k, p = int(n), int(q), int(k), int(p)
        if n < 1 or q < 0 or q > n or k < 1 or p < 0 or p + q > min(k, n):
            raise ValueError(f"bad request: seq_len={n} q_len={q} budget={k} prefix_len={p}")
        cu_s.append(cu_s[-1] + n)
        cu_k.append(cu_k[-1] + min(k, n))
    return cu_s, cu_k


def topk_select(scores: torch.Tensor, seq_len: Sequence[int], q_len: Sequence[int],
                budget: Sequence[int], prefix_len: Optional[Sequence[int]] = None
                ) -> Tuple[torch.Tensor, List[int]]:
    """Kept global token ids (int32, ascending within each request) and cu_kept.

    Per request: if the budget covers the request, keep it all; otherwise keep
    the K_b - p_b - q_b best document tokens under (score descending, index
    ascending) plus the whole question tail and the whole template prefix.
    The document is the span between them: [p_b, N_b - q_b) (spke.com page,
    "Comment déployer TokenGate ?": a placeholder in the prompt template
    marks the prunable document; the template text around it stays).
    """
    if prefix_len is None:
        prefix_len = [0] * len(seq_len)
    cu_s, cu_k = plan(seq_len, q_len, budget, prefix_len)
    s_all = scores.detach().cpu().double().numpy()
    kept = []
    for b in range(len(seq_len)):
        lo, n, q, p = cu_s[b], int(seq_len[b]), int(q_len[b]), int(prefix_len[b])
        keep = min(int(budget[b]), n)
        if keep >= n:
            ids = np.arange(n)
        else:
            ndoc = n - q - p
            sd = s_all[lo + p: lo + p + ndoc]
            nan = np.isnan(sd)
            val = np.where(nan, 0.0, sd) + 0.0          # -0 -> +0
            cls = np.where(nan, 0, 1)                   # NaN below every number
            idx = np.arange(ndoc)
            order = np.lexsort((idx, -val, -cls))       # cls desc, val desc, idx asc
            ids = np.sort(np.concatenate([np.arange(p), p + order[: keep - q - p],
                                          np.arange(n - q, n)]))
        kept.append(ids + lo)
    out = np.concatenate(kept).astype(np.int32) if kept else np.zeros(0, np.int32)
    return torch.from_numpy(out), cu_k


# --------------------------------------------------------------------------
# Gather / compaction (spke.com page, third bullet: layers above L process only
# the K kept tokens and never create KV entries for the pruned ones).
# --------------------------------------------------------------------------
def gather_compact(hidden: torch.Tensor, scores: Optional[torch.Tensor],
                   kept_idx: torch.Tensor):
    """hidden_kept[r] = hidden[kept_idx[r]] (bit for bit), s_kept[r] = s[kept_idx[r]]."""
    idx = kept_idx.long()
    hk = hidden[idx].clone()
    sk = scores[idx].clone() if scores is not None else None
    return hk, sk


# --------------------------------------------------------------------------
# Token-gated attention (spke.com page, "Qu'est-ce que l'attention gérée par des
# tokens ?": the score of each kept token becomes a bias on the attention
# logits above L; a learnable per-head gain and a per-head temperature, the
# latter correcting for each query seeing fewer keys).
# Exact form: l_ij = tau_h (q_i . k_j) / sqrt(d_head) + g_h s_j, j <= i,
# softmax over j, GQA head h reads KV head h // (Hq / Hkv).
# --------------------------------------------------------------------------
def _head_logits(Q, Kb, s, gain_h, temp_h, dh):
    return temp_h * (Q @ Kb.t()) / math.sqrt(dh) + gain_h * s[None, :]


def gated_attention(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor,
                    s_kept: torch.Tensor, gain: torch.Tensor, temp: torch.Tensor,
                    cu_kept: Sequence[int]) -> Tuple[torch.Tensor, torch.Tensor]:
    """out[Kt][Hq][dh] (float64) and lse[Hq][Kt] (float64, natural log).

    q[Kt][Hq][dh], k,v[Kt][Hkv][dh]; requests are the row ranges of cu_kept and
    never attend to each other.
    """
    Kt, Hq, dh = q.shape
    Hkv = k.shape[1]
    group = Hq // Hkv
    out = torch.zeros(Kt, Hq, dh, dtype=torch.float64)
    lse = torch.zeros(Hq, Kt, dtype=torch.float64)
    s64 = s_kept.double()
    g64, t64 = gain.double(), temp.double()
    for b in range(len(cu_kept) - 1):
        lo, hi = int(cu_kept[b]), int(cu_kept[b + 1])
        n = hi - lo
        if n == 0:
            continue
        future = torch.triu(torch.ones(n, n, dtype=torch.bool), diagonal=1)
        for h in range(Hq):
            kv = h // group
            Q = q[lo:hi, h].double()
            Kb = k[lo:hi, kv].double()
            V = v[lo:hi, kv].double()
            logits = _head_logits(Q, Kb, s64[lo:hi], g64[h], t64[h], dh)
            logits = logits.masked_fill(future, -math.inf)
            m = logits.max(dim=1).values
            p = torch.exp(logits - m[:, None])
            denom = p.sum(dim=1)
            out[lo:hi, h] = (p @ V) / denom[:, None]
            lse[h, lo:hi] = m + torch.log(denom)
    return out, lse


def gated_attention_rows(q, k, v, s_kept, gain, temp, cu_kept: Sequence[int],
                         rows: Sequence[int]) -> Tuple[torch.Tensor, torch.Tensor]:
    """The same definition evaluated only at the given global query rows.

    Returns out[len(rows)][Hq][dh] and lse[Hq][len(rows)], float64.
    """
    Kt, Hq, dh = q.shape
    group = Hq // k.shape[1]
    cu = list(int(c) for c in cu_kept)
    out = torch.zeros(len(rows), Hq, dh, dtype=torch.float64)
    lse = torch.zeros(Hq, len(rows), dtype=torch.float64)
    s64 = s_kept.double()
    for r_i, r in enumerate(rows):
        if not 0 <= r < cu[-1]:
            raise IndexError(r)
        lo = cu[bisect.bisect_right(cu, r) - 1]
        for h in range(Hq):
            kv = h // group
            Qr = q[r:r + 1, h].double()
            Kb = k[lo:r + 1, kv].double()
            V = v[lo:r + 1, kv].double()
            logits = _head_logits(Qr, Kb, s64[lo:r + 1], float(gain[h]), float(temp[h]), dh)[0]
            m = logits.max()
            p = torch.exp(logits - m)
            denom = p.sum()
            out[r_i, h] = (p @ V) / denom
            lse[h, r_i] = m + torch.log(denom)
    return out, lse


# --------------------------------------------------------------------------
# Decode over the kept-only KV cache (spke.com page, three-phase list, third
# bullet: no KV record is created for a pruned token; "Comment déployer
# TokenGate ?": generation runs on the pruned prompt).  The pages do not say
# whether the score bias still applies when generating; it is read as yes,
# with each cached row carrying its own gate score.
# --------------------------------------------------------------------------
def gated_decode_attention(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor,
                           s: torch.Tensor, row_off: Sequence[int], cache_len: Sequence[int],
                           gain: torch.Tensor, temp: torch.Tensor
                           ) -> Tuple[torch.Tensor, torch.Tensor]:
    """One new query per request against its cached rows.

    q[B][Hq][dh]; k, v[R][Hkv][dh] and s[R] hold cache rows; request b owns
    rows row_off[b] .. row_off[b] + cache_len[b] - 1 (the new token's own row
    already appended).  Logit l_j = tau_h (q . k_j) / sqrt(dh) + g_h s_j over
    every cached row (no causal mask: the query is the newest position).
    Returns out[B][Hq][dh] and lse[B][Hq] (float64, natural log); an empty
    cache gives a zero output and lse = -inf.
    """
    B, Hq, dh = q.shape
    group = Hq // k.shape[1]
    out = torch.zeros(B, Hq, dh, dtype=torch.float64)
    lse = torch.full((B, Hq), -math.inf, dtype=torch.float64)
    s64 = s.double()
    for b in range(B):
        lo, n = int(row_off[b]), int(cache_len[b])
        if n == 0:
            continue
        for h in range(Hq):
            kv = h // group
            Qr = q[b:b + 1, h].double()
            logits = _head_logits(Qr, k[lo:lo + n, kv].double(), s64[lo:lo + n],
                                  float(gain[h]), float(temp[h]), dh)[0]
            m = logits.max()
            p = torch.exp(logits - m)
            denom = p.sum()
            out[b, h] = (p @ v[lo:lo + n, kv].double()) / denom
            lse[b, h] = m + torch.log(denom)
    return out, lse


# --------------------------------------------------------------------------
# Layers above the gate on the kept tokens only (spke.com page, third bullet).
# The pages give no layer detail; this stack is the attention sub-layer alone:
# q|k|v = x W^T, then x <- x + attn W_o^T, with the gated attention above.
# Each stored tensor is rounded to the storage dtype where a GPU pipeline
# stores it (q, k, v, attention output, updated residual).
# --------------------------------------------------------------------------
def linear(x: torch.Tensor, w: torch.Tensor) -> torch.Tensor:
    """y = x W^T in float64 (W in Linear layout [out][in])."""
    return x.double() @ w.double().t()


def stack_forward(x_kept: torch.Tensor, s_kept: torch.Tensor, layers: List[Dict[str, torch.Tensor]],
                  cu_kept: Sequence[int], n_q_heads: int, n_kv_heads: int, d_head: int,
                  store_dtype: Optional[torch.dtype] = None) -> torch.Tensor:
    """Run the attention stack over the compacted rows; returns the residual.

    store_dtype=None keeps everything in float64 (for pinning); otherwise each
    stored tensor is rounded to that dtype.
    """
    def store(t):
        return t if store_dtype is None else t.to(store_dtype)

    Kt = x_kept.shape[0]
    x = x_kept.double() if store_dtype is None else x_kept.to(store_dtype)
    for L in layers:
        q = store(linear(x, L["wq"])).reshape(Kt, n_q_heads, d_head)
        k = store(linear(x, L["wk"])).reshape(Kt, n_kv_heads, d_head)
        v = store(linear(x, L["wv"])).reshape(Kt, n_kv_heads, d_head)
        a, _ = gated_attention(q, k, v, s_kept, L["gain"], L["temp"], cu_kept)
        a = store(a).reshape(Kt, n_q_heads * d_head)
        x = store(x.double() + linear(a, L["wo"]))
    return x


# --------------------------------------------------------------------------
# The rest of a pruned decoder layer (spke.com page, three-phase list, third
# bullet: the layers above L run on the kept tokens only).  The pages name the
# backbone (Qwen3-1.7B) but not its layer; this is the published Qwen3 decoder
# layer: RMSNorm before attention and before the FFN, a per-head RMSNorm of q
# and k, rotary position embedding (RoFormer, Su et al.) with the half-split
# pairing (element i turns with element i + d_head/2), a SwiGLU FFN, no
# projection biases.  The attention in it is the token-gated attention above.
# A kept token keeps its original position inside its request.
# --------------------------------------------------------------------------
def rms_norm(x: torch.Tensor, w: torch.Tensor, eps: float) -> torch.Tensor:
    """x / sqrt(mean(x^2) + eps) * w over the last dimension, float64."""
    x = x.double()
    return x / torch.sqrt((x * x).mean(dim=-1, keepdim=True) + eps) * w.double()


def rope(x: torch.Tensor, pos: torch.Tensor, theta: float) -> torch.Tensor:
    """Rotate x[M][H][dh]: the pair (x_i, x_{i+dh/2}) turns by the angle
    pos_m * theta^(-2i/dh), i < dh/2 (float64)."""
    dh = x.shape[-1]
    half = dh // 2
    i = torch.arange(half, dtype=torch.float64)
    inv_freq = float(theta) ** (-2.0 * i / dh)
    ang = pos.double()[:, None] * inv_freq[None, :]
    c = torch.cos(ang)[:, None, :]
    s = torch.sin(ang)[:, None, :]
    x1, x2 = x[..., :half].double(), x[..., half:].double()
    return torch.cat([x1 * c - x2 * s, x2 * c + x1 * s], dim=-1)


def silu(z: torch.Tensor) -> torch.Tensor:
    """z * sigmoid(z) = z / (1 + e^-z), float64."""
    z = z.double()
    return z / (1.0 + torch.exp(-z))


def swiglu(x: torch.Tensor, wg: torch.Tensor, wu: torch.Tensor, wd: torch.Tensor) -> torch.Tensor:
    """(silu(x Wg^T) * (x Wu^T)) Wd^T, float64."""
    return linear(silu(linear(x, wg)) * linear(x, wu), wd)


def kept_positions(kept_idx: torch.Tensor, cu_seqlens: Sequence[int],
                   cu_kept: Sequence[int]) -> torch.Tensor:
    """Original position of each kept row inside its request:
    kept_idx[r] - cu_seqlens[b] for the request b that owns row r (int32)."""
    pos = torch.empty(len(kept_idx), dtype=torch.int32)
    for b in range(len(cu_kept) - 1):
        lo, hi = int(cu_kept[b]), int(cu_kept[b + 1])
        pos[lo:hi] = kept_idx[lo:hi] - int(cu_seqlens[b])
    return pos


def decoder_layer(x_kept: torch.Tensor, s_kept: torch.Tensor, pos: torch.Tensor,
                  cu_kept: Sequence[int], L: Dict[str, torch.Tensor], n_q_heads: int,
                  n_kv_heads: int, d_head: int, theta: float, eps: float,
                  store_dtype: Optional[torch.dtype] = None) -> Dict[str, torch.Tensor]:
    """One decoder layer over the kept rows; returns every stored tensor.

    L holds in_norm[d], wq[Hq*dh][d], wk, wv[Hkv*dh][d], q_norm, k_norm[dh],
    wo[d][Hq*dh], gain, temp[Hq], post_norm[d], wg, wu[F][d], wd[d][F].
    store_dtype=None keeps float64 throughout; otherwise each tensor is rounded
    where a GPU pipeline stores it: xn, q, k, v, q and k after norm + rotation,
    the attention output, h, xn2, the gate/up products, their SwiGLU product,
    and the layer output.
    """
    def store(t):
        return t if store_dtype is None else t.to(store_dtype)

    Kt = x_kept.shape[0]
    x = x_kept.double() if store_dtype is None else x_kept.to(store_dtype)
    r = {}
    r["xn"] = store(rms_norm(x, L["in_norm"], eps))
    q = store(linear(r["xn"], L["wq"])).reshape(Kt, n_q_heads, d_head)
    k = store(linear(r["xn"], L["wk"])).reshape(Kt, n_kv_heads, d_head)
    r["v"] = store(linear(r["xn"], L["wv"])).reshape(Kt, n_kv_heads, d_head)
    r["q_proj"], r["k_proj"] = q, k
    r["q"] = store(rope(rms_norm(q, L["q_norm"], eps), pos, theta))
    r["k"] = store(rope(rms_norm(k, L["k_norm"], eps), pos, theta))
    a, _ = gated_attention(r["q"], r["k"], r["v"], s_kept, L["gain"], L["temp"], cu_kept)
    r["attn"] = store(a).reshape(Kt, n_q_heads * d_head)
    r["h"] = store(x.double() + linear(r["attn"], L["wo"]))
    r["xn2"] = store(rms_norm(r["h"], L["post_norm"], eps))
    r["g"] = store(linear(r["xn2"], L["wg"]))
    r["u"] = store(linear(r["xn2"], L["wu"]))
    r["m"] = store(silu(r["g"]) * r["u"].double())
    r["out"] = store(r["h"].double() + linear(r["m"], L["wd"]))
    return r


# --------------------------------------------------------------------------
# Backward of the token-gated attention (spke.com page, "Qu'est-ce que
# l'attention gérée par des tokens ?": the score bias is what carries a
# gradient back to the gate, since the top-K choice itself has none).  With
# l_ij = tau_h r_ij + g_h s_j, r_ij = (q_i . k_j) / sqrt(dh), P = softmax_j l,
# O_i = sum_j P_ij v_j and an upstream gradient dO:
#   D_i = dO_i . O_i,  dP_ij = dO_i . v_j,  dL_ij = P_ij (dP_ij - D_i)
#   dq_i = tau_h / sqrt(dh) sum_j dL_ij k_j,   dk_j = tau_h / sqrt(dh) sum_i dL_ij q_i
#   dv_j = sum_i P_ij dO_i,   ds_j = sum_h g_h sum_i dL_ij
#   dg_h = sum_ij dL_ij s_j,  dtau_h = sum_ij dL_ij r_ij
# (GQA: a KV head collects dk, dv from every query head of its group.)
# --------------------------------------------------------------------------
def gated_attention_backward(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor,
                             s_kept: torch.Tensor, gain: torch.Tensor, temp: torch.Tensor,
                             cu_kept: Sequence[int], dout: torch.Tensor,
                             out_stored: Optional[torch.Tensor] = None) -> Dict[str, torch.Tensor]:
    """Gradients of sum(dout * gated_attention(...).out) w.r.t. q, k, v,
    s_kept, gain and temp, float64.

    out_stored: the forward output as a caller stored it (for instance in
    bf16); D_i = dO_i . O_i is then evaluated on it, as an entry point that
    takes the stored output does.  None uses the exact output."""
    Kt, Hq, dh = q.shape
    Hkv = k.shape[1]
    group = Hq // Hkv
    out, lse = gated_attention(q, k, v, s_kept, gain, temp, cu_kept)
    if out_stored is not None:
        out = out_stored.double()
    g = {"dq": torch.zeros(Kt, Hq, dh, dtype=torch.float64),
         "dk": torch.zeros(Kt, Hkv, dh, dtype=torch.float64),
         "dv": torch.zeros(Kt, Hkv, dh, dtype=torch.float64),
         "ds": torch.zeros(Kt, dtype=torch.float64),
         "dgain": torch.zeros(Hq, dtype=torch.float64),
         "dtemp": torch.zeros(Hq, dtype=torch.float64)}
    s64 = s_kept.double()
    scale = 1.0 / math.sqrt(dh)
    for b in range(len(cu_kept) - 1):
        lo, hi = int(cu_kept[b]), int(cu_kept[b + 1])
        n = hi - lo
        if n == 0:
            continue
        future = torch.triu(torch.ones(n, n, dtype=torch.bool), diagonal=1)
        for h in range(Hq):
            kv = h // group
            Q, Kb, V = q[lo:hi, h].double(), k[lo:hi, kv].double(), v[lo:hi, kv].double()
            dO, O = dout[lo:hi, h].double(), out[lo:hi, h]
            r = (Q @ Kb.t()) * scale
            P = torch.exp(float(temp[h]) * r + float(gain[h]) * s64[lo:hi][None, :] - lse[h, lo:hi][:, None])
            P = P.masked_fill(future, 0.0)
            D = (dO * O).sum(dim=1)
            dL = P * (dO @ V.t() - D[:, None])
            g["dq"][lo:hi, h] = float(temp[h]) * scale * (dL @ Kb)
            g["dk"][lo:hi, kv] += float(temp[h]) * scale * (dL.t() @ Q)
            g["dv"][lo:hi, kv] += P.t() @ dO
            col = dL.sum(dim=0)
            g["ds"][lo:hi] += float(gain[h]) * col
            g["dgain"][h] += (col * s64[lo:hi]).sum()
            g["dtemp"][h] += (dL * r).sum()
    return g


# --------------------------------------------------------------------------
# Backward of the gate MLP (spke.com page, "Comment TokenGate a-t-il appris
# ...": the gate is trained through the score bias; the top-K choice carries
# no gradient, so only kept tokens receive one).  For a kept token with
# z = W1 x + b1 and s = w2 . GELU(z) + b2, an upstream gradient ds gives
#   dz = ds * w2 * GELU'(z),  GELU'(z) = Phi(z) + z phi(z)
#   dW1 = sum_t dz_t x_t^T,  db1 = sum_t dz_t,  dw2 = sum_t ds_t GELU(z_t),
#   db2 = sum_t ds_t,  dx_t = W1^T dz_t
# --------------------------------------------------------------------------
def gate_backward(hidden_kept: torch.Tensor, w1: torch.Tensor, b1: Optional[torch.Tensor],
                  w2: torch.Tensor, ds: torch.Tensor) -> Dict[str, torch.Tensor]:
    """Gradients of sum_t ds_t s_t over the given (kept) rows, float64:
    dhidden[Kt][d], dw1[d_gate][d], db1[d_gate], dw2[d_gate], db2[1]."""
    x = hidden_kept.double()
    W1 = w1.double()
    z = x @ W1.t()
    if b1 is not None:
        z = z + b1.double()
    phi = torch.exp(-0.5 * z * z) / math.sqrt(2.0 * math.pi)
    Phi = 0.5 * (1.0 + torch.erf(z / math.sqrt(2.0)))
    d64 = ds.double()
    dz = d64[:, None] * w2.double()[None, :] * (Phi + z * phi)
    return {"dhidden": dz @ W1, "dw1": dz.t() @ x, "db1": dz.sum(dim=0),
            "dw2": gelu_erf(z).t() @ d64, "db2": d64.sum().reshape(1)}
