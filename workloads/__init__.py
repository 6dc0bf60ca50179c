"""Seeded synthetic workloads for the TokenGate pruned-prefill path.

This module only draws inputs.  It holds none of the method's arithmetic (no
gate, no selection, no attention), so both the CPU oracle and the HIP path can
consume the exact same bytes from it.

Shapes follow the workloads the TokenGate write-ups describe: a Qwen3-1.7B
backbone (d_model 2048, 16 query heads, 8 KV heads, head dim 128) with the gate
at a low layer, contexts of 16k-128k tokens, batch 1, a question tail that is
never pruned and needle-in-a-haystack style inputs (MarkTechPost/spke.com page,
"TL;DR", "Comment TokenGate a-t-il appris ..." and the benchmark list).  The
pages publish no datasets or trained gates, so every tensor here is random:

* the layer-L residual ``hidden`` is N(0, 1);
* gate and projection weights and biases are N(0, 1/fan_in);
* per-head gains are U(0.5, 1.5) and per-head temperatures U(0.8, 1.2);
* q/k/v of the single-layer workloads are N(0, 1).

Floating point draws are fp32 and, for bf16 workloads, rounded to bf16 once
(round-to-nearest-even, via torch's own conversion).  Every tensor has its own
CPU generator seeded with ``base_seed * 1000 + tensor_id``.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field
from typing import Dict, List, Optional

import torch

__all__ = [
    "LayerShape",
    "Workload",
    "WORKLOADS",
    "get",
    "gate_inputs",
    "attn_inputs",
    "stack_weights",
    "random_scores",
    "DecodeWorkload",
    "DECODE_WORKLOADS",
    "decode_inputs",
    "QWEN3_1P7B_FFN",
    "layer_weights",
    "kept_layout",
]


@dataclass(frozen=True)
class LayerShape:
    d_model: int
    n_q_heads: int
    n_kv_heads: int
    d_head: int
    d_gate: int
    dtype: torch.dtype


@dataclass
class Workload:
    name: str
    shape: LayerShape
    seq_len: List[int]
    q_len: List[int]
    budget: List[int]
    n_needles: int = 0
    stack_layers: int = 0
    description: str = ""

    @property
    def batch(self) -> int:
        return len(self.seq_len)

    @property
    def total_tokens(self) -> int:
        return int(sum(self.seq_len))

    @property
    def kept_per_request(self) -> List[int]:
        return [min(k, n) for k, n in zip(self.budget, self.seq_len)]

    @property
    def total_kept(self) -> int:
        return int(sum(self.kept_per_request))


QWEN3_1P7B = dict(d_model=2048, n_q_heads=16, n_kv_heads=8, d_head=128, d_gate=256)


def _varlen_draws(seed: int):
    """Packed batch of four requests: budgets ~ floor(U(0.05, 0.30) * N_b) and
    question tails ~ U{64..256} (inclusive), seeded."""
    lens = [8192, 24576, 65536, 16384]
    g = torch.Generator().manual_seed(seed * 1000 + 900)
    r = torch.rand(len(lens), generator=g, dtype=torch.float64) * 0.25 + 0.05
    q = torch.randint(64, 257, (len(lens),), generator=g)
    budget = [int(math.floor(float(rb) * n)) for rb, n in zip(r, lens)]
    return lens, [int(x) for x in q], budget


def _build(seed: int = 0) -> Dict[str, Workload]:
    bf = LayerShape(dtype=torch.bfloat16, **QWEN3_1P7B)
    lens5, q5, b5 = _varlen_draws(seed)
    return {
        "tiny_fp32": Workload(
            "tiny_fp32",
            LayerShape(256, 4, 2, 64, 64, torch.float32),
            [512], [32], [128],
            description="tiny fp32 gated layer: N=512 (480 document + 32 question), "
                        "d_model=256, 4/2 heads, d_head=64, gate 256->64->1, K=128",
        ),
        "qwen3_1p7b_16k": Workload(
            "qwen3_1p7b_16k", bf, [16384], [128], [2048],
            description="Qwen3-1.7B-shaped gated layer, bf16, N=16384 (128 question), K=2048",
        ),
        "qwen3_1p7b_32k_stack4": Workload(
            "qwen3_1p7b_32k_stack4", bf, [32768], [128], [4096], stack_layers=4,
            description="Qwen3-1.7B-shaped, bf16, N=32768 (128 question), K=4096, plus a "
                        "4-layer QKV/O stack above the gate on the kept tokens",
        ),
        "qwen3_1p7b_128k_niah": Workload(
            "qwen3_1p7b_128k_niah", bf, [131072], [128], [8192], n_needles=64,
            description="Qwen3-1.7B-shaped gated layer, bf16, N=131072 (128 question), "
                        "K=8192, 64 planted high-norm needles",
        ),
        "qwen3_1p7b_varlen4": Workload(
            "qwen3_1p7b_varlen4", bf, lens5, q5, b5,
            description="packed varlen batch of 4 requests, bf16, N={8192,24576,65536,16384}, "
                        "budget U(5%,30%) of N, question tail U{64..256}",
        ),
    }


WORKLOADS: Dict[str, Workload] = _build(0)


def get(name: str, seed: int = 0) -> Workload:
    if seed == 0:
        return WORKLOADS[name]
    return _build(seed)[name]


def _gen(seed: int, tid: int) -> torch.Generator:
    return torch.Generator().manual_seed(seed * 1000 + tid)


def _normal(shape, std: float, seed: int, tid: int, dtype: torch.dtype) -> torch.Tensor:
    t = torch.randn(*shape, generator=_gen(seed, tid), dtype=torch.float32)
    if std != 1.0:
        t.mul_(std)
    return t.to(dtype)


def _uniform(n: int, lo: float, hi: float, seed: int, tid: int) -> torch.Tensor:
    return torch.rand(n, generator=_gen(seed, tid), dtype=torch.float32) * (hi - lo) + lo


def needle_positions(w: Workload, seed: int = 0) -> torch.Tensor:
    """Global token ids of the planted needles: distinct, inside the document
    span of the first request, sorted."""
    if w.n_needles == 0:
        return torch.zeros(0, dtype=torch.int64)
    ndoc = w.seq_len[0] - w.q_len[0]
    perm = torch.randperm(ndoc, generator=_gen(seed, 7))
    return torch.sort(perm[: w.n_needles]).values


def gate_inputs(w: Workload, seed: int = 0, with_bias: bool = True) -> Dict[str, torch.Tensor]:
    """hidden[T][d], w1[d_gate][d] (torch Linear layout), b1[d_gate], w2[d_gate],
    b2[1], all in the workload's storage dtype, on the CPU.

    Needles: ``x_p + sqrt(15 d) * u`` with ``u`` the unit vector along
    ``W1^T max(w2, 0)`` (computed in float64 from the stored weights), then
    rounded once to the storage dtype.  A typical row has squared norm ~d, so a
    needle has squared norm ~16 d: four times the norm of an ordinary token,
    pointed where the random gate rises.
    """
    s = w.shape
    T, d, dg = w.total_tokens, s.d_model, s.d_gate
    hidden32 = torch.randn(T, d, generator=_gen(seed, 1), dtype=torch.float32)
    w1 = _normal((dg, d), 1.0 / math.sqrt(d), seed, 2, s.dtype)
    w2 = _normal((dg,), 1.0 / math.sqrt(dg), seed, 4, s.dtype)
    if with_bias:
        b1 = _normal((dg,), 1.0 / math.sqrt(d), seed, 3, s.dtype)
        b2 = _normal((1,), 1.0 / math.sqrt(dg), seed, 5, s.dtype)
    else:
        b1 = b2 = None
    if w.n_needles:
        pos = needle_positions(w, seed)
        direction = w1.double().t() @ w2.double().clamp_min(0.0)
        direction = direction / direction.norm()
        hidden32[pos] = (hidden32[pos].double() + math.sqrt(15.0 * d) * direction).float()
    hidden = hidden32.to(s.dtype)
    del hidden32
    return dict(hidden=hidden, w1=w1, b1=b1, w2=w2, b2=b2)


def attn_inputs(w: Workload, seed: int = 0, total_kept: Optional[int] = None) -> Dict[str, torch.Tensor]:
    """q[Kt][Hq][dh], k,v[Kt][Hkv][dh] in the storage dtype; gain[Hq], temp[Hq] fp32."""
    s = w.shape
    Kt = w.total_kept if total_kept is None else total_kept
    return dict(
        q=_normal((Kt, s.n_q_heads, s.d_head), 1.0, seed, 10, s.dtype),
        k=_normal((Kt, s.n_kv_heads, s.d_head), 1.0, seed, 11, s.dtype),
        v=_normal((Kt, s.n_kv_heads, s.d_head), 1.0, seed, 12, s.dtype),
        gain=_uniform(s.n_q_heads, 0.5, 1.5, seed, 13),
        temp=_uniform(s.n_q_heads, 0.8, 1.2, seed, 14),
    )


def stack_weights(w: Workload, seed: int = 0) -> List[Dict[str, torch.Tensor]]:
    """Per stack layer: wq[Hq*dh][d], wk,wv[Hkv*dh][d], wo[d][Hq*dh] (torch Linear
    layout, N(0, 1/fan_in)), gain[Hq] ~ U(0.5,1.5), temp[Hq] ~ U(0.8,1.2)."""
    s = w.shape
    d, hq, hkv = s.d_model, s.n_q_heads * s.d_head, s.n_kv_heads * s.d_head
    out = []
    for layer in range(w.stack_layers):
        base = 100 + 10 * layer
        out.append(dict(
            wq=_normal((hq, d), 1.0 / math.sqrt(d), seed, base + 0, s.dtype),
            wk=_normal((hkv, d), 1.0 / math.sqrt(d), seed, base + 1, s.dtype),
            wv=_normal((hkv, d), 1.0 / math.sqrt(d), seed, base + 2, s.dtype),
            wo=_normal((d, hq), 1.0 / math.sqrt(hq), seed, base + 3, s.dtype),
            gain=_uniform(s.n_q_heads, 0.5, 1.5, seed, base + 4),
            temp=_uniform(s.n_q_heads, 0.8, 1.2, seed, base + 5),
        ))
    return out


def random_scores(n: int, seed: int = 0, ties: int = 0) -> torch.Tensor:
    """fp32 N(0,1) scores; with ``ties`` > 0, values are drawn from a grid of
    ``ties`` distinct levels so that equal keys are common."""
    g = _gen(seed, 20)
    if ties > 0:
        return torch.randint(0, ties, (n,), generator=g).float() / ties - 0.5
    return torch.randn(n, generator=g, dtype=torch.float32)


# ------------------------------------------------------------------ decode ----
@dataclass(frozen=True)
class DecodeWorkload:
    """One generation step over kept-only KV caches: request b has cache_len[b]
    cached rows (its kept prefill rows plus the new token's own row)."""
    name: str
    shape: LayerShape
    cache_len: List[int]

    @property
    def batch(self) -> int:
        return len(self.cache_len)


# After a pruned 128k prefill each request caches its 8192 kept rows; the
# generated token adds row 8193.  32 such requests decode together.
DECODE_WORKLOADS: Dict[str, DecodeWorkload] = {
    "qwen3_1p7b_128k_decode_b32": DecodeWorkload(
        "qwen3_1p7b_128k_decode_b32",
        LayerShape(dtype=torch.bfloat16, **QWEN3_1P7B), [8192 + 1] * 32),
}


def decode_inputs(shape: LayerShape, cache_len: List[int], seed: int = 0, gap: int = 0,
                  with_bias: bool = True) -> Dict[str, torch.Tensor]:
    """q[B][Hq][dh]; a row pool k, v[R][Hkv][dh] and s[R]; row_off[B] (int64),
    cache_len[B] (int32); gain[Hq], temp[Hq].

    Requests sit back to back in the pool with `gap` unused rows (random data)
    in front of each.  Cached scores are N(0, 1) fp32 (they stand in for gate
    scores), q/k/v N(0, 1) in the storage dtype."""
    row_off, r = [], 0
    for n in cache_len:
        r += gap
        row_off.append(r)
        r += n
    R = r
    B, hq, hkv, dh = len(cache_len), shape.n_q_heads, shape.n_kv_heads, shape.d_head
    return dict(
        q=_normal((B, hq, dh), 1.0, seed, 30, shape.dtype),
        k=_normal((R, hkv, dh), 1.0, seed, 31, shape.dtype),
        v=_normal((R, hkv, dh), 1.0, seed, 32, shape.dtype),
        s=torch.randn(R, generator=_gen(seed, 33), dtype=torch.float32) if with_bias else None,
        row_off=torch.tensor(row_off, dtype=torch.int64),
        cache_len=torch.tensor(cache_len, dtype=torch.int32),
        gain=_uniform(hq, 0.5, 1.5, seed, 34) if with_bias else None,
        temp=_uniform(hq, 0.8, 1.2, seed, 35),
    )


# ------------------------------------------------- rest of the pruned layer ----
QWEN3_1P7B_FFN = 6144      # Qwen3-1.7B intermediate size


def layer_weights(shape: LayerShape, d_ffn: int, seed: int = 0, tid0: int = 200) -> Dict[str, torch.Tensor]:
    """One decoder layer: projections N(0, 1/fan_in) in Linear layout, norm
    weights 1 + N(0, 0.1^2) (so that they matter), gain U(0.5, 1.5), temp
    U(0.8, 1.2).  wgu stacks the gate rows over the up rows ([2F][d])."""
    d, hq, hkv, dh = shape.d_model, shape.n_q_heads, shape.n_kv_heads, shape.d_head
    dt = shape.dtype

    def norm_w(n, tid):
        return (1.0 + 0.1 * torch.randn(n, generator=_gen(seed, tid), dtype=torch.float32)).to(dt)

    wg = _normal((d_ffn, d), 1.0 / math.sqrt(d), seed, tid0 + 8, dt)
    wu = _normal((d_ffn, d), 1.0 / math.sqrt(d), seed, tid0 + 9, dt)
    return dict(
        in_norm=norm_w(d, tid0 + 0),
        wq=_normal((hq * dh, d), 1.0 / math.sqrt(d), seed, tid0 + 1, dt),
        wk=_normal((hkv * dh, d), 1.0 / math.sqrt(d), seed, tid0 + 2, dt),
        wv=_normal((hkv * dh, d), 1.0 / math.sqrt(d), seed, tid0 + 3, dt),
        q_norm=norm_w(dh, tid0 + 4),
        k_norm=norm_w(dh, tid0 + 5),
        wo=_normal((d, hq * dh), 1.0 / math.sqrt(hq * dh), seed, tid0 + 6, dt),
        post_norm=norm_w(d, tid0 + 7),
        wg=wg, wu=wu, wgu=torch.cat([wg, wu], dim=0),
        wd=_normal((d, d_ffn), 1.0 / math.sqrt(d_ffn), seed, tid0 + 10, dt),
        gain=_uniform(hq, 0.5, 1.5, seed, tid0 + 11),
        temp=_uniform(hq, 0.8, 1.2, seed, tid0 + 12),
    )


def kept_layout(seq_len: List[int], q_len: List[int], budget: List[int], seed: int = 0):
    """A plausible kept-id layout without running a gate: per request, the
    question tail plus a uniformly random sorted subset of the document.
    Returns (kept ids int32, cu_seqlens, cu_kept)."""
    g = _gen(seed, 40)
    ids, cu_s, cu_k = [], [0], [0]
    for n, q, k in zip(seq_len, q_len, budget):
        k = min(k, n)
        doc = torch.sort(torch.randperm(n - q, generator=g)[: k - q]).values
        ids.append(torch.cat([doc, torch.arange(n - q, n)]) + cu_s[-1])
        cu_s.append(cu_s[-1] + n)
        cu_k.append(cu_k[-1] + k)
    return torch.cat(ids).to(torch.int32), cu_s, cu_k
