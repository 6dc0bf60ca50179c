"""The pruned-prefill hot path composed from the C-ABI calls.

One gated layer (MarkTechPost article on TokenGate, French rendering on
spke.com, three-phase list): score every token with the gate MLP, keep the
top-K document tokens plus the question, compact the kept rows, run token-gated
attention over the kept tokens only.  ``GatedLayer`` owns its output buffers so
repeated calls allocate nothing; every step is one library call on the current
stream.
"""
from __future__ import annotations

from typing import Dict, List, Optional, Sequence

import torch

from . import (tg_attn_prefill_plan, tg_gate_score, tg_gated_attn_prefill, tg_gather_compact,
               tg_kept_positions, tg_linear, tg_linear_multi, tg_linear_swiglu, tg_plan,
               tg_qk_norm_rope, tg_rmsnorm, tg_silu_mul, tg_topk_select)


def swiglu_projection(xn, wgu, gu, m):
    """m = silu(xn wg^T) * (xn wu^T) with wgu = [wg; wu]: one launch with the
    product in the projection's epilogue when F is a multiple of 128 (bf16),
    else the gate|up projection into gu and the product as a second launch."""
    if xn.dtype == torch.bfloat16 and (wgu.shape[0] // 2) % 128 == 0:
        tg_linear_swiglu(xn, wgu, out=m)
    else:
        tg_linear(xn, wgu, y=gu)
        tg_silu_mul(gu, out=m)


def qkv_projections(x, wq, wk, wv, yq, yk, yv):
    """yq, yk, yv = x wq^T, x wk^T, x wv^T: one launch when every output width
    is a multiple of 256 (the three products then share one grid that fills
    the chip), else three."""
    if x.dtype == torch.bfloat16 and all(w.shape[0] % 256 == 0 for w in (wq, wk, wv)):
        tg_linear_multi(x, [wq, wk, wv], ys=[yq, yk, yv])
    else:
        tg_linear(x, wq, y=yq)
        tg_linear(x, wk, y=yk)
        tg_linear(x, wv, y=yv)


class _AttnWorkspace:
    """The attention's optional workspace per kept-row layout, allocated (and
    zero-filled, as its counters require) on the first call with that layout,
    so that later calls, and HIP graphs captured after it, allocate nothing."""

    def __init__(self, Hq: int, Hkv: int, d_head: int, dtype: torch.dtype, device):
        self.Hq, self.Hkv, self.dh, self.dtype, self.device = Hq, Hkv, d_head, dtype, device
        self.bufs: Dict[tuple, Optional[torch.Tensor]] = {}

    def get(self, cu_kept: Sequence[int]) -> Optional[torch.Tensor]:
        key = tuple(cu_kept)
        if key not in self.bufs:
            n = tg_attn_prefill_plan(list(cu_kept), self.Hq, self.Hkv, self.dh, self.dtype)
            self.bufs[key] = torch.zeros(n, dtype=torch.uint8, device=self.device) if n else None
        return self.bufs[key]


class GatedLayer:
    """Buffers and calls of one gated layer for a fixed batch layout."""

    def __init__(self, T: int, d_model: int, n_q_heads: int, d_head: int, seq_len: Sequence[int],
                 q_len: Sequence[int], budget: Sequence[int], dtype: torch.dtype,
                 device="cuda", want_lse: bool = False, n_kv_heads: Optional[int] = None):
        self.seq_len, self.q_len, self.budget = list(seq_len), list(q_len), list(budget)
        self.cu_seq, self.cu_kept, ws = tg_plan(self.seq_len, self.q_len, self.budget)
        if self.cu_seq[-1] != T:
            raise ValueError("sum(seq_len) must equal the number of hidden rows")
        Kt = self.cu_kept[-1]
        self.Kt = Kt
        self.scores = torch.empty(T, dtype=torch.float32, device=device)
        self.kept = torch.empty(Kt, dtype=torch.int32, device=device)
        self.cu_kept_dev = torch.empty(len(self.cu_kept), dtype=torch.int32, device=device)
        self.workspace = torch.empty(ws, dtype=torch.uint8, device=device) if ws else None
        self.hidden_kept = torch.empty(Kt, d_model, dtype=dtype, device=device)
        self.s_kept = torch.empty(Kt, dtype=torch.float32, device=device)
        self.out = torch.empty(Kt, n_q_heads, d_head, dtype=dtype, device=device)
        self.lse = torch.empty(n_q_heads, Kt, dtype=torch.float32, device=device) if want_lse else None
        # With the KV head count known, the attention gets its workspace,
        # zero-filled once (a short single request then splits its query
        # tiles over more workgroups).
        self.attn_ws = None
        if n_kv_heads is not None and Kt > 0:
            n = tg_attn_prefill_plan(self.cu_kept, n_q_heads, n_kv_heads, d_head, dtype)
            self.attn_ws = torch.zeros(n, dtype=torch.uint8, device=device) if n else None

    def gate(self, hidden, w1, b1, w2, b2):
        return tg_gate_score(hidden, w1, b1, w2, b2, scores=self.scores)

    def select(self):
        return tg_topk_select(self.scores, self.seq_len, self.q_len, self.budget,
                              kept_idx=self.kept, cu_kept_dev=self.cu_kept_dev,
                              workspace=self.workspace)[0]

    def gather(self, hidden):
        return tg_gather_compact(hidden, self.kept, self.scores, hidden_kept=self.hidden_kept,
                                 scores_kept=self.s_kept)

    def attend(self, q, k, v, gain, temp):
        return tg_gated_attn_prefill(q, k, v, self.s_kept, gain, temp, self.cu_kept, out=self.out,
                                     lse=self.lse, workspace=self.attn_ws)[0]

    def __call__(self, hidden, w1, b1, w2, b2, q, k, v, gain, temp):
        """gate -> select -> gather -> gated attention; returns the attention output."""
        self.gate(hidden, w1, b1, w2, b2)
        self.select()
        self.gather(hidden)
        return self.attend(q, k, v, gain, temp)


class AttentionStack:
    """Layers above the gate on the kept rows only: per layer q|k|v = x W^T
    (one launch for the three products), token-gated attention,
    x += attn W_o^T (the residual updated in place)."""

    def __init__(self, Kt: int, d_model: int, n_q_heads: int, n_kv_heads: int, d_head: int,
                 dtype: torch.dtype, device="cuda"):
        self.Hq, self.Hkv, self.dh = n_q_heads, n_kv_heads, d_head
        self.q = torch.empty(Kt, n_q_heads * d_head, dtype=dtype, device=device)
        self.k = torch.empty(Kt, n_kv_heads * d_head, dtype=dtype, device=device)
        self.v = torch.empty(Kt, n_kv_heads * d_head, dtype=dtype, device=device)
        self.attn = torch.empty(Kt, n_q_heads, d_head, dtype=dtype, device=device)
        self.attn_ws = _AttnWorkspace(n_q_heads, n_kv_heads, d_head, dtype, device)

    def __call__(self, x, s_kept, cu_kept: Sequence[int], layers: List[Dict[str, torch.Tensor]]):
        Kt = x.shape[0]
        for L in layers:
            qkv_projections(x, L["wq"], L["wk"], L["wv"], self.q, self.k, self.v)
            tg_gated_attn_prefill(self.q.view(Kt, self.Hq, self.dh), self.k.view(Kt, self.Hkv, self.dh),
                                  self.v.view(Kt, self.Hkv, self.dh), s_kept, L["gain"], L["temp"],
                                  cu_kept, out=self.attn, workspace=self.attn_ws.get(cu_kept))
            tg_linear(self.attn.view(Kt, self.Hq * self.dh), L["wo"], y=x, accumulate=True)
        return x


class DecoderLayer:
    """A whole decoder layer above the gate on the kept rows (the published
    Qwen3 layer the pages' backbone uses), the residual updated in place:

        xn = rmsnorm(x);  q, k, v = xn Wq^T, xn Wk^T, xn Wv^T
        q, k <- rotary(rmsnorm_head(q)), rotary(rmsnorm_head(k))  at original positions
        x += gated_attention(q, k, v; s_kept) Wo^T
        xn = rmsnorm(x);  x += (silu(xn Wg^T) * (xn Wu^T)) Wd^T   (q|k|v and gate|up*silu one launch each)

    Weights: in_norm[d], wq[Hq*dh][d], wk, wv[Hkv*dh][d], q_norm, k_norm[dh],
    wo[d][Hq*dh], gain, temp[Hq], post_norm[d], wgu[2F][d] (gate rows then up
    rows), wd[d][F].  Every step is one library call; buffers are owned here
    so repeated calls allocate nothing.
    """

    def __init__(self, Kt: int, d_model: int, n_q_heads: int, n_kv_heads: int, d_head: int,
                 d_ffn: int, dtype: torch.dtype, theta: float = 1e6, eps: float = 1e-6,
                 device="cuda"):
        self.Hq, self.Hkv, self.dh, self.F = n_q_heads, n_kv_heads, d_head, d_ffn
        self.theta, self.eps = theta, eps
        e = dict(dtype=dtype, device=device)
        self.xn = torch.empty(Kt, d_model, **e)
        self.q = torch.empty(Kt, n_q_heads, d_head, **e)
        self.k = torch.empty(Kt, n_kv_heads, d_head, **e)
        self.v = torch.empty(Kt, n_kv_heads, d_head, **e)
        self.attn = torch.empty(Kt, n_q_heads, d_head, **e)
        self.gu = torch.empty(Kt, 2 * d_ffn, **e)
        self.m = torch.empty(Kt, d_ffn, **e)
        self.pos = torch.empty(Kt, dtype=torch.int32, device=device)
        self.attn_ws = _AttnWorkspace(n_q_heads, n_kv_heads, d_head, dtype, device)

    def positions(self, kept_idx, cu_seqlens: Sequence[int], cu_kept: Sequence[int]):
        return tg_kept_positions(kept_idx, cu_seqlens, cu_kept, pos=self.pos)

    def __call__(self, x, s_kept, cu_kept: Sequence[int], L: Dict[str, torch.Tensor]):
        """x[Kt][d] is updated in place; self.pos must hold the positions."""
        Kt = x.shape[0]
        tg_rmsnorm(x, L["in_norm"], self.eps, y=self.xn)
        qkv_projections(self.xn, L["wq"], L["wk"], L["wv"], self.q.view(Kt, -1), self.k.view(Kt, -1),
                        self.v.view(Kt, -1))
        tg_qk_norm_rope(self.q, self.k, L["q_norm"], L["k_norm"], self.pos, self.theta, self.eps)
        tg_gated_attn_prefill(self.q, self.k, self.v, s_kept, L["gain"], L["temp"], cu_kept,
                              out=self.attn, workspace=self.attn_ws.get(cu_kept))
        tg_linear(self.attn.view(Kt, -1), L["wo"], y=x, accumulate=True)
        tg_rmsnorm(x, L["post_norm"], self.eps, y=self.xn)
        swiglu_projection(self.xn, L["wgu"], self.gu, self.m)
        tg_linear(self.m, L["wd"], y=x, accumulate=True)
        return x
