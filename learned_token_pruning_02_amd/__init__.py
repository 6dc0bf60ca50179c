"""TokenGate pruned-prefill hot path on MI355X: Python binding of libtokengate.so.

The binding only marshals arguments: it checks that tensors live on the GPU
with the right dtype and layout, allocates outputs with ``torch.empty`` when
the caller gives none, and calls the C ABI (``include/tokengate.h``) on the
current HIP stream.  Every step runs in the library's gfx950 kernels; there is
no fallback of any kind.  If the library is not built, every call raises.

Steps (MarkTechPost article on TokenGate, French rendering on spke.com):
  tg_gate_score          gate MLP score per token          (three-phase list, 2nd bullet)
  tg_topk_select         top-K of the document + question  (same bullet; question never pruned)
  tg_gather_compact      kept rows compacted               (3rd bullet)
  tg_gated_attn_prefill  causal GQA attention with a per-key score bias, per-head gain and
                         temperature                       ("attention gérée par des tokens")
  tg_linear              projection on the kept rows (layers above the gate)
"""
from __future__ import annotations

import ctypes
import os
from typing import List, Optional, Sequence, Tuple

__all__ = [
    "TokenGateError",
    "lib",
    "library_path",
    "TG_F32",
    "TG_BF16",
    "TG_MAX_BATCH",
    "tg_plan",
    "tg_gate_score",
    "tg_topk_select",
    "tg_topk_select_noalloc",
    "tg_gather_compact",
    "tg_gated_attn_prefill",
    "tg_attn_prefill_plan",
    "tg_attn_backward_plan",
    "tg_gate_backward_plan",
    "tg_gate_backward",
    "tg_gated_attn_backward",
    "tg_decode_plan",
    "tg_gated_attn_decode",
    "tg_rmsnorm",
    "tg_linear_multi",
    "tg_linear_swiglu",
    "tg_kept_positions",
    "tg_qk_norm_rope",
    "tg_silu_mul",
    "tg_linear",
]

_PKG = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_PKG, "libtokengate.so")

TG_F32 = 0
TG_BF16 = 1
TG_MAX_BATCH = 64

STATUS = {
    0: "TG_OK", 1: "TG_ERR_NULL_PTR", 2: "TG_ERR_BAD_SHAPE", 3: "TG_ERR_BAD_BUDGET",
    4: "TG_ERR_BAD_DTYPE", 5: "TG_ERR_UNSUPPORTED", 6: "TG_ERR_ALIGNMENT",
    7: "TG_ERR_WORKSPACE", 8: "TG_ERR_LAUNCH", 9: "TG_ERR_ALIAS",
}


class TokenGateError(RuntimeError):
    def __init__(self, fn: str, status: int):
        self.status = status
        super().__init__(f"{fn} failed: {STATUS.get(status, status)}")


class _Batch(ctypes.Structure):
    _fields_ = [
        ("batch", ctypes.c_int32),
        ("seq_len", ctypes.POINTER(ctypes.c_int32)),
        ("q_len", ctypes.POINTER(ctypes.c_int32)),
        ("budget", ctypes.POINTER(ctypes.c_int32)),
    ]


class _BatchPrefix(ctypes.Structure):
    _fields_ = [
        ("batch", ctypes.c_int32),
        ("seq_len", ctypes.POINTER(ctypes.c_int32)),
        ("q_len", ctypes.POINTER(ctypes.c_int32)),
        ("budget", ctypes.POINTER(ctypes.c_int32)),
        ("prefix_len", ctypes.POINTER(ctypes.c_int32)),
    ]


_lib = None


def library_path() -> str:
    return _LIB_PATH


def lib() -> ctypes.CDLL:
    """The loaded libtokengate.so (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        raise RuntimeError(
            f"{_LIB_PATH} is missing: build it with `python -m learned_token_pruning_02_amd.build` "
            "(there is no fallback implementation)")
    L = ctypes.CDLL(_LIB_PATH)
    vp, i32, i64, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
    p_i32 = ctypes.POINTER(ctypes.c_int32)
    L.tg_status_str.restype = ctypes.c_char_p
    L.tg_status_str.argtypes = [ctypes.c_int]
    L.tg_abi_version.restype = ctypes.c_int
    L.tg_abi_version.argtypes = []
    L.tg_plan.restype = ctypes.c_int
    L.tg_plan.argtypes = [ctypes.POINTER(_Batch), p_i32, p_i32, ctypes.POINTER(sz)]
    L.tg_gate_score.restype = ctypes.c_int
    L.tg_gate_score.argtypes = [ctypes.c_int, vp, i64, i32, vp, vp, vp, vp, i32, vp, vp]
    L.tg_topk_select.restype = ctypes.c_int
    L.tg_topk_select.argtypes = [vp, ctypes.POINTER(_Batch), vp, vp, vp, sz, vp]
    L.tg_topk_select_noalloc.restype = ctypes.c_int
    L.tg_topk_select_noalloc.argtypes = [vp, ctypes.POINTER(_Batch), vp, vp, vp]
    L.tg_topk_select_path.restype = ctypes.c_int
    L.tg_topk_select_path.argtypes = [vp, ctypes.POINTER(_BatchPrefix), vp, vp, vp, sz, ctypes.c_int, vp]
    L.tg_plan_prefix.restype = ctypes.c_int
    L.tg_plan_prefix.argtypes = [ctypes.POINTER(_BatchPrefix), p_i32, p_i32, ctypes.POINTER(sz)]
    L.tg_topk_select_prefix.restype = ctypes.c_int
    L.tg_topk_select_prefix.argtypes = [vp, ctypes.POINTER(_BatchPrefix), vp, vp, vp, sz, vp]
    L.tg_gather_compact.restype = ctypes.c_int
    L.tg_gather_compact.argtypes = [ctypes.c_int, vp, i64, i32, vp, vp, i64, vp, vp, vp]
    L.tg_gated_attn_prefill.restype = ctypes.c_int
    L.tg_gated_attn_prefill.argtypes = [ctypes.c_int, vp, vp, vp, vp, vp, vp, p_i32, i32, i32,
                                        i32, i32, vp, vp, vp]
    L.tg_attn_prefill_plan.restype = ctypes.c_int
    L.tg_attn_prefill_plan.argtypes = [ctypes.c_int, p_i32, i32, i32, i32, i32, ctypes.POINTER(sz)]
    L.tg_gated_attn_prefill_ws.restype = ctypes.c_int
    L.tg_gated_attn_prefill_ws.argtypes = [ctypes.c_int, vp, vp, vp, vp, vp, vp, p_i32, i32, i32,
                                           i32, i32, vp, vp, vp, sz, vp]
    L.tg_attn_backward_plan.restype = ctypes.c_int
    L.tg_attn_backward_plan.argtypes = [p_i32, i32, i32, i32, ctypes.POINTER(sz)]
    L.tg_gated_attn_backward.restype = ctypes.c_int
    L.tg_gated_attn_backward.argtypes = [ctypes.c_int, vp, vp, vp, vp, vp, vp, vp, vp, vp, p_i32, i32,
                                         i32, i32, i32, vp, vp, vp, vp, vp, vp, vp, sz, vp]
    L.tg_gate_backward_plan.restype = ctypes.c_int
    L.tg_gate_backward_plan.argtypes = [ctypes.c_int, i64, i32, i32, ctypes.POINTER(sz)]
    L.tg_gate_backward.restype = ctypes.c_int
    L.tg_gate_backward.argtypes = [ctypes.c_int, vp, i64, i32, vp, vp, vp, i32, vp, vp, vp, vp, vp,
                                   vp, vp, sz, vp]
    L.tg_decode_plan.restype = ctypes.c_int
    L.tg_decode_plan.argtypes = [i32, i32, i32, i32, ctypes.POINTER(sz)]
    L.tg_gated_attn_decode.restype = ctypes.c_int
    L.tg_gated_attn_decode.argtypes = [ctypes.c_int, vp, vp, vp, vp, i64, vp, vp, i32, i32, vp, vp,
                                       i32, i32, i32, vp, vp, vp, sz, vp]
    f32 = ctypes.c_float
    L.tg_rmsnorm.restype = ctypes.c_int
    L.tg_rmsnorm.argtypes = [ctypes.c_int, vp, vp, f32, i64, i32, vp, vp]
    L.tg_kept_positions.restype = ctypes.c_int
    L.tg_kept_positions.argtypes = [vp, p_i32, p_i32, i32, vp, vp]
    L.tg_qk_norm_rope.restype = ctypes.c_int
    L.tg_qk_norm_rope.argtypes = [ctypes.c_int, vp, vp, vp, vp, vp, i64, i32, i32, i32, f32, f32, vp]
    L.tg_silu_mul.restype = ctypes.c_int
    L.tg_silu_mul.argtypes = [ctypes.c_int, vp, i64, i32, vp, vp]
    L.tg_linear.restype = ctypes.c_int
    L.tg_linear.argtypes = [ctypes.c_int, vp, vp, vp, i64, i32, i32, ctypes.c_int, vp]
    L.tg_linear_tile.restype = ctypes.c_int
    L.tg_linear_tile.argtypes = [ctypes.c_int, vp, vp, vp, i64, i32, i32, ctypes.c_int, ctypes.c_int, vp]
    L.tg_linear_swiglu.restype = ctypes.c_int
    L.tg_linear_swiglu.argtypes = [ctypes.c_int, vp, vp, vp, i64, i32, i32, ctypes.c_int, vp]
    L.tg_linear_multi.restype = ctypes.c_int
    L.tg_linear_multi.argtypes = [ctypes.c_int, vp, i32, ctypes.POINTER(vp), ctypes.POINTER(vp), p_i32,
                                  i64, i32, ctypes.c_int, ctypes.c_int, vp]
    _lib = L
    return L


# ------------------------------------------------------------- helpers ----
def _torch():
    import torch
    return torch


def _check(fn: str, status: int):
    if status != 0:
        raise TokenGateError(fn, status)


def _stream(stream):
    torch = _torch()
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream))


def _dt(t) -> int:
    torch = _torch()
    if t.dtype == torch.float32:
        return TG_F32
    if t.dtype == torch.bfloat16:
        return TG_BF16
    raise TypeError(f"unsupported dtype {t.dtype} (float32 or bfloat16)")


def _dev(t, name: str, dtype=None):
    """Device pointer of a contiguous GPU tensor (None passes through)."""
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    return ctypes.c_void_p(t.data_ptr())


def _shape(t, name: str, shape) -> None:
    """Raise ValueError unless tensor t (skipped when None) has exactly `shape`.

    The C ABI receives bare pointers and sizes, so a tensor smaller than the
    sizes passed with it would be read or written out of bounds on the GPU;
    every wrapper checks its tensors here before any pointer is taken."""
    if t is not None and tuple(t.shape) != tuple(int(x) for x in shape):
        raise ValueError(f"{name} must have shape {tuple(int(x) for x in shape)}, got {tuple(t.shape)}")


def _numel(t, name: str, n: int) -> None:
    """Raise ValueError unless tensor t (skipped when None) has n elements."""
    if t is not None and t.numel() != int(n):
        raise ValueError(f"{name} must have {int(n)} elements, got {t.numel()}")


def _ndim(t, name: str, nd: int) -> None:
    if t.dim() != nd:
        raise ValueError(f"{name} must be {nd}-D, got shape {tuple(t.shape)}")


def _nbytes(t) -> int:
    return 0 if t is None else t.numel() * t.element_size()


def _i32_array(vals: Sequence[int]):
    arr = (ctypes.c_int32 * max(1, len(vals)))(*[int(v) for v in vals])
    return arr


def _batch(seq_len, q_len, budget, prefix_len=None):
    """tg_batch (prefix_len None) or tg_batch_prefix, and the arrays it points to."""
    n = len(seq_len)
    if not (len(q_len) == len(budget) == n) or (prefix_len is not None and len(prefix_len) != n):
        raise ValueError("seq_len, q_len, budget (and prefix_len) must have the same length")
    s, q, b = _i32_array(seq_len), _i32_array(q_len), _i32_array(budget)
    ptr = lambda a: ctypes.cast(a, ctypes.POINTER(ctypes.c_int32))
    if prefix_len is None:
        return _Batch(n, ptr(s), ptr(q), ptr(b)), (s, q, b)
    p = _i32_array(prefix_len)
    return _BatchPrefix(n, ptr(s), ptr(q), ptr(b), ptr(p)), (s, q, b, p)


# ----------------------------------------------------------------- API ----
def tg_plan(seq_len: Sequence[int], q_len: Sequence[int], budget: Sequence[int],
            prefix_len: Optional[Sequence[int]] = None) -> Tuple[List[int], List[int], int]:
    """Host-only plan: (cu_seqlens, cu_kept, select workspace bytes).  With
    prefix_len, each request also keeps that many leading template tokens
    (tg_plan_prefix)."""
    L = lib()
    bt, keep = _batch(seq_len, q_len, budget, prefix_len)
    n = len(seq_len)
    cu_s = (ctypes.c_int32 * (n + 1))()
    cu_k = (ctypes.c_int32 * (n + 1))()
    ws = ctypes.c_size_t(0)
    fn, name = (L.tg_plan, "tg_plan") if prefix_len is None else (L.tg_plan_prefix, "tg_plan_prefix")
    _check(name, fn(ctypes.byref(bt), cu_s, cu_k, ctypes.byref(ws)))
    return list(cu_s), list(cu_k), int(ws.value)


def tg_gate_score(hidden, w1, b1, w2, b2, scores=None, stream=None):
    """scores[T] (fp32) = w2 . GELU(W1 x_t + b1) + b2 for every row x_t of hidden."""
    torch = _torch()
    _ndim(hidden, "hidden", 2)
    _ndim(w1, "w1", 2)
    T, d = hidden.shape
    dg = w1.shape[0]
    _shape(w1, "w1", (dg, d))
    _numel(b1, "b1", dg)
    _numel(w2, "w2", dg)
    _numel(b2, "b2", 1)
    _numel(scores, "scores", T)
    dt = _dt(hidden)
    if scores is None:
        scores = torch.empty(T, dtype=torch.float32, device=hidden.device)
    _check("tg_gate_score", lib().tg_gate_score(
        dt, _dev(hidden, "hidden"), T, d, _dev(w1, "w1", hidden.dtype),
        _dev(b1, "b1", hidden.dtype), _dev(w2, "w2", hidden.dtype), _dev(b2, "b2", hidden.dtype),
        dg, _dev(scores, "scores", torch.float32), _stream(stream)))
    return scores


def tg_topk_select(scores, seq_len: Sequence[int], q_len: Sequence[int], budget: Sequence[int],
                   kept_idx=None, cu_kept_dev=None, workspace=None, stream=None, prefix_len=None,
                   path: int = 0):
    """Kept global token ids (int32, ascending per request) and the host cu_kept list.
    With prefix_len, each request also keeps that many leading template tokens
    and selects from the span between them and the question
    (tg_topk_select_prefix).  Random-K selection is this call on random keys
    drawn by the caller in place of the scores.  path (testing only): 1
    forces the one-workgroup implementation, 2 the chunked one
    (tg_topk_select_path); 0 lets the library choose."""
    torch = _torch()
    cu_s, cu_k, ws_bytes = tg_plan(seq_len, q_len, budget, prefix_len)
    _numel(scores, "scores", cu_s[-1])
    _numel(kept_idx, "kept_idx", cu_k[-1])
    _numel(cu_kept_dev, "cu_kept_dev", len(cu_k))
    if workspace is not None and _nbytes(workspace) < ws_bytes:
        raise ValueError(f"workspace must hold {ws_bytes} bytes, got {_nbytes(workspace)}")
    if kept_idx is None:
        kept_idx = torch.empty(cu_k[-1], dtype=torch.int32, device=scores.device)
    if ws_bytes and workspace is None:
        workspace = torch.empty(ws_bytes, dtype=torch.uint8, device=scores.device)
    if path:
        # tg_topk_select_path takes a tg_batch_prefix (prefix_len NULL: none).
        bt, keep = _batch(seq_len, q_len, budget, prefix_len if prefix_len is not None else [0] * len(seq_len))
    else:
        bt, keep = _batch(seq_len, q_len, budget, prefix_len)
    args = (_dev(scores, "scores", torch.float32), ctypes.byref(bt),
            _dev(kept_idx, "kept_idx", torch.int32), _dev(cu_kept_dev, "cu_kept_dev", torch.int32),
            _dev(workspace, "workspace"), ws_bytes if workspace is None else _nbytes(workspace))
    if path:
        _check("tg_topk_select_path", lib().tg_topk_select_path(*args, int(path), _stream(stream)))
    elif prefix_len is not None:
        _check("tg_topk_select_prefix", lib().tg_topk_select_prefix(*args, _stream(stream)))
    else:
        _check("tg_topk_select", lib().tg_topk_select(*args, _stream(stream)))
    return kept_idx, cu_k


def tg_topk_select_noalloc(scores, seq_len: Sequence[int], q_len: Sequence[int],
                           budget: Sequence[int], kept_idx, cu_kept_dev=None, stream=None):
    """tg_topk_select with the workspace in the library's static device scratch:
    the call allocates nothing (kept_idx must be given).  Returns the host
    cu_kept list."""
    torch = _torch()
    cu_s, cu_k, _ = tg_plan(seq_len, q_len, budget)
    _numel(scores, "scores", cu_s[-1])
    _numel(kept_idx, "kept_idx", cu_k[-1])
    _numel(cu_kept_dev, "cu_kept_dev", len(cu_k))
    bt, keep = _batch(seq_len, q_len, budget)
    _check("tg_topk_select_noalloc", lib().tg_topk_select_noalloc(
        _dev(scores, "scores", torch.float32), ctypes.byref(bt),
        _dev(kept_idx, "kept_idx", torch.int32), _dev(cu_kept_dev, "cu_kept_dev", torch.int32),
        _stream(stream)))
    return cu_k


def tg_gather_compact(hidden, kept_idx, scores=None, hidden_kept=None, scores_kept=None,
                      stream=None):
    """hidden_kept[r] = hidden[kept_idx[r]]; scores_kept[r] = scores[kept_idx[r]]."""
    torch = _torch()
    _ndim(hidden, "hidden", 2)
    T, d = hidden.shape
    Kt = kept_idx.numel()
    _numel(scores, "scores", T)
    _shape(hidden_kept, "hidden_kept", (Kt, d))
    _numel(scores_kept, "scores_kept", Kt)
    if hidden_kept is None:
        hidden_kept = torch.empty(Kt, d, dtype=hidden.dtype, device=hidden.device)
    if scores is not None and scores_kept is None:
        scores_kept = torch.empty(Kt, dtype=torch.float32, device=hidden.device)
    _check("tg_gather_compact", lib().tg_gather_compact(
        _dt(hidden), _dev(hidden, "hidden"), T, d, _dev(scores, "scores", torch.float32),
        _dev(kept_idx, "kept_idx", torch.int32), Kt, _dev(hidden_kept, "hidden_kept", hidden.dtype),
        _dev(scores_kept, "scores_kept", torch.float32), _stream(stream)))
    return hidden_kept, scores_kept


def _attn_shapes(q, k, v, s_kept, gain, temp, cu_kept) -> None:
    """Shape checks shared by the attention forward and backward wrappers."""
    Kt, Hq, dh = q.shape
    Hkv = k.shape[1]
    if len(cu_kept) < 2 or int(cu_kept[-1]) != Kt:
        raise ValueError(f"cu_kept[-1] must equal the {Kt} rows of q, got {list(cu_kept)[-1:]}")
    if Hkv < 1 or Hq % Hkv != 0:
        raise ValueError(f"query heads ({Hq}) must be a multiple of KV heads ({Hkv})")
    _shape(k, "k", (Kt, Hkv, dh))
    _shape(v, "v", (Kt, Hkv, dh))
    _numel(s_kept, "s_kept", Kt)
    _numel(gain, "gain", Hq)
    _numel(temp, "temp", Hq)


def tg_attn_prefill_plan(cu_kept: Sequence[int], Hq: int, Hkv: int, d_head: int,
                         dtype=None) -> int:
    """Workspace bytes of tg_gated_attn_prefill with a workspace (bf16 unless
    dtype is torch.float32); 0 when the shape does not split its tiles."""
    torch = _torch()
    ws = ctypes.c_size_t(0)
    cu = _i32_array(cu_kept)
    dt = TG_F32 if dtype == torch.float32 else TG_BF16
    _check("tg_attn_prefill_plan", lib().tg_attn_prefill_plan(
        dt, ctypes.cast(cu, ctypes.POINTER(ctypes.c_int32)), len(cu_kept) - 1, Hq, Hkv, d_head,
        ctypes.byref(ws)))
    return ws.value


def tg_gated_attn_prefill(q, k, v, s_kept, gain, temp, cu_kept: Sequence[int], out=None,
                          lse=None, want_lse: bool = False, stream=None, workspace=None):
    """Causal GQA token-gated attention over packed kept rows; returns (out, lse or None).

    s_kept=None and gain=None drop the bias term (plain causal attention with
    the per-head temperature).  With a workspace (tg_attn_prefill_plan bytes,
    zero-filled before its first use) the call is tg_gated_attn_prefill_ws,
    which cuts the query tiles of a short single request into pieces of at
    most 8 key tiles, one workgroup each."""
    torch = _torch()
    _ndim(q, "q", 3)
    _ndim(k, "k", 3)
    Kt, Hq, dh = q.shape
    Hkv = k.shape[1]
    _attn_shapes(q, k, v, s_kept, gain, temp, cu_kept)
    _shape(out, "out", q.shape)
    _shape(lse, "lse", (Hq, Kt))
    if out is None:
        out = torch.empty_like(q)
    if want_lse and lse is None:
        lse = torch.empty(Hq, Kt, dtype=torch.float32, device=q.device)
    cu = _i32_array(cu_kept)
    L = lib()
    args = (_dt(q), _dev(q, "q"), _dev(k, "k", q.dtype), _dev(v, "v", q.dtype),
            _dev(s_kept, "s_kept", torch.float32), _dev(gain, "gain", torch.float32),
            _dev(temp, "temp", torch.float32), ctypes.cast(cu, ctypes.POINTER(ctypes.c_int32)),
            len(cu_kept) - 1, Hq, Hkv, dh, _dev(out, "out", q.dtype),
            _dev(lse, "lse", torch.float32))
    if workspace is None:
        _check("tg_gated_attn_prefill", L.tg_gated_attn_prefill(*args, _stream(stream)))
    else:
        _check("tg_gated_attn_prefill_ws", L.tg_gated_attn_prefill_ws(
            *args, _dev(workspace, "workspace"), _nbytes(workspace), _stream(stream)))
    return out, lse


def tg_attn_backward_plan(cu_kept: Sequence[int], Hq: int, Hkv: int) -> int:
    """Workspace bytes of tg_gated_attn_backward."""
    ws = ctypes.c_size_t(0)
    cu = _i32_array(cu_kept)
    _check("tg_attn_backward_plan", lib().tg_attn_backward_plan(
        ctypes.cast(cu, ctypes.POINTER(ctypes.c_int32)), len(cu_kept) - 1, Hq, Hkv, ctypes.byref(ws)))
    return ws.value


def tg_gated_attn_backward(q, k, v, s_kept, gain, temp, out, lse, dout, cu_kept: Sequence[int],
                           grads=None, workspace=None, stream=None):
    """Gradients of the token-gated attention; returns a dict with dq, dk, dv
    (bf16) and ds, dgain (fp32; None without the bias) and dtemp (fp32)."""
    torch = _torch()
    _ndim(q, "q", 3)
    _ndim(k, "k", 3)
    Kt, Hq, dh = q.shape
    Hkv = k.shape[1]
    _attn_shapes(q, k, v, s_kept, gain, temp, cu_kept)
    _shape(out, "out", q.shape)
    _shape(dout, "dout", q.shape)
    _shape(lse, "lse", (Hq, Kt))
    if grads is not None:
        _shape(grads["dq"], "dq", q.shape)
        _shape(grads["dk"], "dk", k.shape)
        _shape(grads["dv"], "dv", k.shape)
        _numel(grads.get("ds"), "ds", Kt)
        _numel(grads.get("dgain"), "dgain", Hq)
        _numel(grads["dtemp"], "dtemp", Hq)
    if workspace is not None and _nbytes(workspace) < tg_attn_backward_plan(cu_kept, Hq, Hkv):
        raise ValueError("workspace is smaller than tg_attn_backward_plan reports")
    if grads is None:
        f32 = dict(dtype=torch.float32, device=q.device)
        grads = {"dq": torch.empty_like(q), "dk": torch.empty_like(k), "dv": torch.empty_like(v),
                 "ds": torch.empty(Kt, **f32) if s_kept is not None else None,
                 "dgain": torch.empty(Hq, **f32) if s_kept is not None else None,
                 "dtemp": torch.empty(Hq, **f32)}
    if workspace is None:
        workspace = torch.empty(tg_attn_backward_plan(cu_kept, Hq, Hkv), dtype=torch.uint8,
                                device=q.device)
    cu = _i32_array(cu_kept)
    f32t = torch.float32
    _check("tg_gated_attn_backward", lib().tg_gated_attn_backward(
        _dt(q), _dev(q, "q"), _dev(k, "k", q.dtype), _dev(v, "v", q.dtype),
        _dev(s_kept, "s_kept", f32t), _dev(gain, "gain", f32t), _dev(temp, "temp", f32t),
        _dev(out, "out", q.dtype), _dev(lse, "lse", f32t), _dev(dout, "dout", q.dtype),
        ctypes.cast(cu, ctypes.POINTER(ctypes.c_int32)), len(cu_kept) - 1, Hq, Hkv, dh,
        _dev(grads["dq"], "dq", q.dtype), _dev(grads["dk"], "dk", q.dtype),
        _dev(grads["dv"], "dv", q.dtype), _dev(grads["ds"], "ds", f32t),
        _dev(grads["dgain"], "dgain", f32t), _dev(grads["dtemp"], "dtemp", f32t),
        _dev(workspace, "workspace"), workspace.numel() * workspace.element_size(), _stream(stream)))
    return grads


def tg_gate_backward_plan(dtype, Kt: int, d_model: int, d_gate: int) -> int:
    """Workspace bytes of tg_gate_backward (dtype: a torch dtype)."""
    ws = ctypes.c_size_t(0)
    dt = TG_BF16 if dtype == _torch().bfloat16 else TG_F32
    _check("tg_gate_backward_plan", lib().tg_gate_backward_plan(dt, Kt, d_model, d_gate, ctypes.byref(ws)))
    return ws.value


def tg_gate_backward(hidden_kept, w1, b1, w2, ds_kept, grads=None, workspace=None, stream=None):
    """Gradients of the gate MLP over the kept rows; returns a dict with
    dhidden, dw1 (in the input dtype) and db1 (None without b1), dw2, db2 (fp32)."""
    torch = _torch()
    _ndim(hidden_kept, "hidden_kept", 2)
    _ndim(w1, "w1", 2)
    Kt, d = hidden_kept.shape
    dg = w1.shape[0]
    _shape(w1, "w1", (dg, d))
    _numel(b1, "b1", dg)
    _numel(w2, "w2", dg)
    _numel(ds_kept, "ds_kept", Kt)
    if grads is not None:
        _shape(grads["dhidden"], "dhidden", (Kt, d))
        _shape(grads["dw1"], "dw1", (dg, d))
        _numel(grads.get("db1"), "db1", dg)
        _numel(grads["dw2"], "dw2", dg)
        _numel(grads["db2"], "db2", 1)
        if (grads.get("db1") is None) != (b1 is None):
            raise ValueError("db1 must be given exactly when b1 is")
    if workspace is not None and _nbytes(workspace) < tg_gate_backward_plan(hidden_kept.dtype, Kt, d, dg):
        raise ValueError("workspace is smaller than tg_gate_backward_plan reports")
    f32 = dict(dtype=torch.float32, device=hidden_kept.device)
    if grads is None:
        grads = {"dhidden": torch.empty_like(hidden_kept), "dw1": torch.empty_like(w1),
                 "db1": torch.empty(dg, **f32) if b1 is not None else None,
                 "dw2": torch.empty(dg, **f32), "db2": torch.empty(1, **f32)}
    if workspace is None:
        workspace = torch.empty(max(1, tg_gate_backward_plan(hidden_kept.dtype, Kt, d, dg)),
                                dtype=torch.uint8, device=hidden_kept.device)
    x = hidden_kept
    _check("tg_gate_backward", lib().tg_gate_backward(
        _dt(x), _dev(x, "hidden_kept"), Kt, d, _dev(w1, "w1", x.dtype), _dev(b1, "b1", x.dtype),
        _dev(w2, "w2", x.dtype), dg, _dev(ds_kept, "ds_kept", torch.float32),
        _dev(grads["dhidden"], "dhidden", x.dtype), _dev(grads["dw1"], "dw1", x.dtype),
        _dev(grads["db1"], "db1", torch.float32), _dev(grads["dw2"], "dw2", torch.float32),
        _dev(grads["db2"], "db2", torch.float32), _dev(workspace, "workspace"),
        workspace.numel() * workspace.element_size(), _stream(stream)))
    return grads


def tg_decode_plan(batch: int, Hq: int, d_head: int, max_len: int) -> int:
    """Workspace bytes of tg_gated_attn_decode."""
    ws = ctypes.c_size_t(0)
    _check("tg_decode_plan", lib().tg_decode_plan(batch, Hq, d_head, max_len, ctypes.byref(ws)))
    return ws.value


def tg_gated_attn_decode(q, k, v, s, row_off, cache_len, gain, temp, max_len: int, out=None,
                         lse=None, want_lse: bool = False, workspace=None, stream=None):
    """One decode step over the kept-only KV cache; returns (out, lse or None).

    q[B][Hq][dh]; k, v[R][Hkv][dh] and s[R] form the row pool; row_off (int64)
    and cache_len (int32) are device tensors of length B.  s=None and
    gain=None drop the bias term."""
    torch = _torch()
    _ndim(q, "q", 3)
    _ndim(k, "k", 3)
    B, Hq, dh = q.shape
    R, Hkv = k.shape[0], k.shape[1]
    if Hkv < 1 or Hq % Hkv != 0:
        raise ValueError(f"query heads ({Hq}) must be a multiple of KV heads ({Hkv})")
    _shape(k, "k", (R, Hkv, dh))
    _shape(v, "v", (R, Hkv, dh))
    _numel(s, "s", R)
    _numel(row_off, "row_off", B)
    _numel(cache_len, "cache_len", B)
    _numel(gain, "gain", Hq)
    _numel(temp, "temp", Hq)
    _shape(out, "out", q.shape)
    _shape(lse, "lse", (B, Hq))
    need = tg_decode_plan(B, Hq, dh, max_len)
    if workspace is not None and _nbytes(workspace) < need:
        raise ValueError(f"workspace must hold {need} bytes, got {_nbytes(workspace)}")
    if out is None:
        out = torch.empty_like(q)
    if want_lse and lse is None:
        lse = torch.empty(B, Hq, dtype=torch.float32, device=q.device)
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    _check("tg_gated_attn_decode", lib().tg_gated_attn_decode(
        _dt(q), _dev(q, "q"), _dev(k, "k", q.dtype), _dev(v, "v", q.dtype),
        _dev(s, "s", torch.float32), R, _dev(row_off, "row_off", torch.int64),
        _dev(cache_len, "cache_len", torch.int32), B, max_len, _dev(gain, "gain", torch.float32),
        _dev(temp, "temp", torch.float32), Hq, Hkv, dh, _dev(out, "out", q.dtype),
        _dev(lse, "lse", torch.float32), _dev(workspace, "workspace"),
        0 if workspace is None else workspace.numel() * workspace.element_size(), _stream(stream)))
    return out, lse


def tg_rmsnorm(x, w, eps: float, y=None, stream=None):
    """y = x / sqrt(mean(x^2) + eps) * w over the last dimension of x[M][d];
    y=x runs in place."""
    torch = _torch()
    d = x.shape[-1]
    M = x.numel() // d if d else 0
    _numel(w, "w", d)
    _shape(y, "y", x.shape)
    if y is None:
        y = torch.empty_like(x)
    _check("tg_rmsnorm", lib().tg_rmsnorm(_dt(x), _dev(x, "x"), _dev(w, "w", x.dtype), eps, M, d,
                                          _dev(y, "y", x.dtype), _stream(stream)))
    return y


def tg_kept_positions(kept_idx, cu_seqlens: Sequence[int], cu_kept: Sequence[int], pos=None,
                      stream=None):
    """Original in-request position of every kept row (int32 device tensor)."""
    torch = _torch()
    if len(cu_seqlens) != len(cu_kept):
        raise ValueError("cu_seqlens and cu_kept must have the same length")
    _numel(kept_idx, "kept_idx", int(cu_kept[-1]))
    _numel(pos, "pos", int(cu_kept[-1]))
    if pos is None:
        pos = torch.empty(int(cu_kept[-1]), dtype=torch.int32, device=kept_idx.device)
    cs, ck = _i32_array(cu_seqlens), _i32_array(cu_kept)
    P = ctypes.POINTER(ctypes.c_int32)
    _check("tg_kept_positions", lib().tg_kept_positions(
        _dev(kept_idx, "kept_idx", torch.int32), ctypes.cast(cs, P), ctypes.cast(ck, P),
        len(cu_kept) - 1, _dev(pos, "pos", torch.int32), _stream(stream)))
    return pos


def tg_qk_norm_rope(q, k, q_norm_w, k_norm_w, pos, theta: float, eps: float, stream=None):
    """In place: per-head RMSNorm of q[M][Hq][dh] and k[M][Hkv][dh] (weights may
    be None), then the rotary embedding at positions pos[M]."""
    torch = _torch()
    _ndim(q, "q", 3)
    _ndim(k, "k", 3)
    M, Hq, dh = q.shape
    _shape(k, "k", (M, k.shape[1], dh))
    _numel(q_norm_w, "q_norm_w", dh)
    _numel(k_norm_w, "k_norm_w", dh)
    _numel(pos, "pos", M)
    _check("tg_qk_norm_rope", lib().tg_qk_norm_rope(
        _dt(q), _dev(q, "q"), _dev(k, "k", q.dtype), _dev(q_norm_w, "q_norm_w", q.dtype),
        _dev(k_norm_w, "k_norm_w", q.dtype), _dev(pos, "pos", torch.int32), M, Hq, k.shape[1], dh,
        theta, eps, _stream(stream)))
    return q, k


def tg_silu_mul(gu, out=None, stream=None):
    """out[M][F] = silu(gu[:, :F]) * gu[:, F:] for gu[M][2F]."""
    torch = _torch()
    _ndim(gu, "gu", 2)
    M, F2 = gu.shape
    if F2 % 2 != 0:
        raise ValueError(f"gu must have an even number of columns, got {F2}")
    _shape(out, "out", (M, F2 // 2))
    if out is None:
        out = torch.empty(M, F2 // 2, dtype=gu.dtype, device=gu.device)
    _check("tg_silu_mul", lib().tg_silu_mul(_dt(gu), _dev(gu, "gu"), M, F2 // 2,
                                            _dev(out, "out", gu.dtype), _stream(stream)))
    return out


def tg_linear(x, w, y=None, accumulate: bool = False, stream=None, tile: int = 0):
    """y = x w^T, or y += x w^T with accumulate=True (w in Linear layout [N][K]).
    tile (testing only): 1, 2, 3 force the 128x128, 256x128, 256x256 bf16
    output tile (tg_linear_tile); 0 lets the library choose."""
    torch = _torch()
    _ndim(x, "x", 2)
    _ndim(w, "w", 2)
    M, K = x.shape
    N = w.shape[0]
    _shape(w, "w", (N, K))
    _shape(y, "y", (M, N))
    if y is None:
        if accumulate:
            raise ValueError("accumulate=True needs y")
        y = torch.empty(M, N, dtype=x.dtype, device=x.device)
    args = (_dt(x), _dev(x, "x"), _dev(w, "w", x.dtype), _dev(y, "y", x.dtype), M, N, K,
            1 if accumulate else 0)
    if tile:
        _check("tg_linear_tile", lib().tg_linear_tile(*args, int(tile), _stream(stream)))
    else:
        _check("tg_linear", lib().tg_linear(*args, _stream(stream)))
    return y


def tg_linear_multi(x, ws, ys=None, accumulate: bool = False, stream=None, tile: int = 0):
    """ys[i] = x ws[i]^T (or += with accumulate=True) for up to three weights
    in Linear layout [N_i][K], in one launch (the q, k and v projections).
    Returns the list of outputs.  tile as in tg_linear."""
    torch = _torch()
    _ndim(x, "x", 2)
    M, K = x.shape
    ws = list(ws)
    if not 1 <= len(ws) <= 3:
        raise ValueError(f"tg_linear_multi takes 1 to 3 weights, got {len(ws)}")
    ns = []
    for i, w in enumerate(ws):
        _ndim(w, f"w[{i}]", 2)
        _shape(w, f"w[{i}]", (w.shape[0], K))
        ns.append(w.shape[0])
    if ys is None:
        if accumulate:
            raise ValueError("accumulate=True needs ys")
        ys = [torch.empty(M, n, dtype=x.dtype, device=x.device) for n in ns]
    ys = list(ys)
    if len(ys) != len(ws):
        raise ValueError(f"{len(ys)} outputs for {len(ws)} weights")
    for i, (y, n) in enumerate(zip(ys, ns)):
        _shape(y, f"y[{i}]", (M, n))
    wp = (ctypes.c_void_p * len(ws))(*[_dev(w, f"w[{i}]", x.dtype) for i, w in enumerate(ws)])
    yp = (ctypes.c_void_p * len(ys))(*[_dev(y, f"y[{i}]", x.dtype) for i, y in enumerate(ys)])
    na = _i32_array(ns)
    _check("tg_linear_multi", lib().tg_linear_multi(
        _dt(x), _dev(x, "x"), len(ws), wp, yp, ctypes.cast(na, ctypes.POINTER(ctypes.c_int32)), M, K,
        1 if accumulate else 0, int(tile), _stream(stream)))
    return ys


def tg_linear_swiglu(x, w_gu, out=None, stream=None, tile: int = 0):
    """out = silu(x w_gu[:F]^T) * (x w_gu[F:]^T) in one launch; w_gu is [2F][K]
    (gate rows then up rows), out [M][F].  tile as in tg_linear."""
    torch = _torch()
    _ndim(x, "x", 2)
    _ndim(w_gu, "w_gu", 2)
    M, K = x.shape
    if w_gu.shape[0] % 2 != 0:
        raise ValueError(f"w_gu has {w_gu.shape[0]} rows; it stacks F gate rows and F up rows")
    F = w_gu.shape[0] // 2
    _shape(w_gu, "w_gu", (2 * F, K))
    _shape(out, "out", (M, F))
    if out is None:
        out = torch.empty(M, F, dtype=x.dtype, device=x.device)
    _check("tg_linear_swiglu", lib().tg_linear_swiglu(
        _dt(x), _dev(x, "x"), _dev(w_gu, "w_gu", x.dtype), _dev(out, "out", x.dtype), M, F, K,
        int(tile), _stream(stream)))
    return out
