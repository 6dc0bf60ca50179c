"""The C ABI without a GPU: the library loads, exports every symbol the header
declares, plans batches exactly like the oracle, and rejects every invalid
argument on the host before anything is launched."""
import ctypes
import os
import re

import pytest

import learned_token_pruning_02_amd as tg
import oracle

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "tokengate.h")

# Fake but aligned, non-null device addresses: validation fails before use.
A = 1 << 20
B = 2 << 20
C = 3 << 20
D = 4 << 20
E = 5 << 20
F = 6 << 20
G = 7 << 20
H = 8 << 20


def header_symbols():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(tg_[a-z0-9_]+)\s*\(", text)))


def test_library_exports_every_declared_symbol():
    L = tg.lib()
    syms = header_symbols()
    assert {"tg_plan", "tg_gate_score", "tg_topk_select", "tg_gather_compact",
            "tg_gated_attn_prefill", "tg_linear", "tg_status_str", "tg_abi_version"} <= set(syms)
    for s in syms:
        assert hasattr(L, s), s
    assert L.tg_abi_version() == 1
    for code, name in tg.STATUS.items():
        assert L.tg_status_str(code).decode() == name
    assert L.tg_status_str(77).decode() == "TG_ERR_UNKNOWN"


@pytest.mark.parametrize("case", [
    ([512], [32], [128]),
    ([16384], [128], [2048]),
    ([8192, 24576, 65536, 16384], [203, 203, 87, 235], [812, 3733, 19152, 4727]),
    ([5, 1, 9], [0, 1, 9], [100, 1, 9]),
    ([7], [3], [3]),
])
def test_plan_matches_oracle(case):
    cu_s, cu_k, ws = tg.tg_plan(*case)
    o_s, o_k = oracle.plan(*case)
    assert cu_s == o_s and cu_k == o_k and ws > 0


@pytest.mark.parametrize("seq,q,bud", [
    ([0], [0], [1]),          # empty request
    ([10], [-1], [5]),        # negative question
    ([10], [11], [12]),       # question longer than the request
    ([10], [4], [0]),         # zero budget
    ([10], [4], [3]),         # budget below the question
])
def test_plan_rejects_bad_budgets(seq, q, bud):
    with pytest.raises(tg.TokenGateError) as e:
        tg.tg_plan(seq, q, bud)
    assert e.value.status == 3


def test_plan_rejects_bad_batch():
    with pytest.raises(tg.TokenGateError) as e:
        tg.tg_plan([], [], [])
    assert e.value.status == 2
    n = tg.TG_MAX_BATCH + 1
    with pytest.raises(tg.TokenGateError) as e:
        tg.tg_plan([4] * n, [1] * n, [2] * n)
    assert e.value.status == 2
    with pytest.raises(tg.TokenGateError) as e:
        tg.tg_plan([2 ** 30, 2 ** 30], [0, 0], [5, 5])       # 2^31 tokens
    assert e.value.status == 2
    L = tg.lib()
    assert L.tg_plan(None, None, None, None) == 1


def _batch(seq, q, bud, pre=None):
    return tg._batch(seq, q, bud, pre)


def test_gate_validation():
    L = tg.lib()
    f = L.tg_gate_score
    assert f(7, A, 10, 2048, B, None, C, None, 256, D, None) == 4              # dtype
    assert f(1, A, -1, 2048, B, None, C, None, 256, D, None) == 2              # T < 0
    assert f(1, A, 10, 0, B, None, C, None, 256, D, None) == 2                 # d_model
    assert f(1, None, 10, 2048, B, None, C, None, 256, D, None) == 1           # hidden
    assert f(1, A, 10, 2048, None, None, C, None, 256, D, None) == 1           # w1
    assert f(1, A, 10, 2048, B, None, None, None, 256, D, None) == 1           # w2
    assert f(1, A, 10, 2048, B, None, C, None, 256, None, None) == 1           # scores
    assert f(1, A, 10, 2000, B, None, C, None, 256, D, None) == 5              # d % 64
    assert f(1, A, 10, 2048, B, None, C, None, 192, D, None) == 5              # d_gate
    assert f(0, A, 10, 250, B, None, C, None, 64, D, None) == 5                # fp32 d % 4
    assert f(0, A, 10, 256, B, None, C, None, 2048, D, None) == 5              # fp32 d_gate
    assert f(1, A + 8, 10, 2048, B, None, C, None, 256, D, None) == 6          # misaligned
    assert f(1, A, 10, 2048, B, None, C, None, 256, A + 64, None) == 9         # scores in hidden
    assert f(1, A, 0, 2048, B, None, C, None, 256, D, None) == 0               # T == 0: no-op


def test_select_validation():
    L = tg.lib()
    bt, keep = _batch([100], [10], [20])
    ws = tg.tg_plan([100], [10], [20])[2]
    assert ws > 0
    f = L.tg_topk_select
    assert f(None, ctypes.byref(bt), B, None, C, ws, None) == 1
    assert f(A, ctypes.byref(bt), None, None, C, ws, None) == 1
    assert f(A, None, B, None, C, ws, None) == 1
    assert f(A, ctypes.byref(bt), B, None, None, ws, None) == 7          # no workspace
    assert f(A, ctypes.byref(bt), B, None, C, ws - 1, None) == 7         # too small
    assert f(A + 2, ctypes.byref(bt), B, None, C, ws, None) == 6
    assert f(A, ctypes.byref(bt), B, None, C + 8, ws, None) == 6         # workspace alignment
    assert f(A, ctypes.byref(bt), A + 40, None, C, ws, None) == 9
    assert f(A, ctypes.byref(bt), B, None, A, ws, None) == 9             # workspace over scores
    bad, keep2 = _batch([100], [10], [5])
    assert f(A, ctypes.byref(bad), B, None, C, ws, None) == 3


@pytest.mark.parametrize("case", [
    ([512], [32], [128], [16]),
    ([8192, 24576, 65536, 16384], [203, 203, 87, 235], [812, 3733, 19152, 4727], [40, 0, 300, 17]),
    ([5, 1, 9], [0, 1, 0], [100, 1, 9], [2, 0, 9]),
    ([50], [10], [25], [15]),
])
def test_plan_prefix_matches_oracle(case):
    seq, q, bud, pre = case
    cu_s, cu_k, ws = tg.tg_plan(seq, q, bud, pre)
    o_s, o_k = oracle.plan(seq, q, bud, pre)
    assert cu_s == o_s and cu_k == o_k and ws > 0


def test_select_prefix_validation():
    L = tg.lib()
    ws = tg.tg_plan([100], [10], [40], [20])[2]
    f = L.tg_topk_select_prefix
    bt, keep = _batch([100], [10], [40], [20])
    assert f(A, None, B, None, C, ws, None) == 1
    assert f(None, ctypes.byref(bt), B, None, C, ws, None) == 1
    assert f(A, ctypes.byref(bt), B, None, None, ws, None) == 7
    for pre, bud in ((31, 40), (-1, 40), (0, 9), (95, 200)):           # p + q > kept, p < 0
        bad, keep2 = _batch([100], [10], [bud], [pre])
        assert L.tg_plan_prefix(ctypes.byref(bad), None, None, None) == 3, (pre, bud)
        assert f(A, ctypes.byref(bad), B, None, C, ws, None) == 3, (pre, bud)
    nul, keep3 = _batch([100], [10], [40], [0])
    nul.prefix_len = ctypes.cast(None, ctypes.POINTER(ctypes.c_int32))  # NULL prefix: no prefix
    assert L.tg_plan_prefix(ctypes.byref(nul), None, None, None) == 0


def test_select_workspace_grows_with_tokens_and_requests():
    w1 = tg.tg_plan([1000], [10], [100])[2]
    w2 = tg.tg_plan([100000], [10], [100])[2]
    w3 = tg.tg_plan([1000] * 8, [10] * 8, [100] * 8)[2]
    assert w2 > w1 and w3 > w1
    assert w2 >= 100000 * 8                                               # candidate buffer


def test_gather_validation():
    L = tg.lib()
    f = L.tg_gather_compact
    assert f(3, A, 100, 2048, None, B, 10, C, None, None) == 4
    assert f(1, A, -1, 2048, None, B, 10, C, None, None) == 2
    assert f(1, A, 100, 2048, None, B, -1, C, None, None) == 2
    assert f(1, None, 100, 2048, None, B, 10, C, None, None) == 1
    assert f(1, A, 100, 2048, D, B, 10, C, None, None) == 1                   # scores w/o out
    assert f(1, A, 100, 2044, None, B, 10, C, None, None) == 5                # row bytes % 16
    assert f(1, A, 100, 2048, None, B, 10, C + 4, None, None) == 6
    assert f(1, A, 100, 2048, None, B, 10, A + 4096, None, None) == 9         # out inside hidden
    assert f(1, A, 100, 2048, None, B, 0, C, None, None) == 0                 # Kt == 0: no-op


def test_attention_validation():
    L = tg.lib()
    f = L.tg_gated_attn_prefill
    cu = tg._i32_array([0, 100])
    cu_p = ctypes.cast(cu, ctypes.POINTER(ctypes.c_int32))
    ok = [1, A, B, C, D, E, F, cu_p, 1, 16, 8, 128, G, None, None]

    def call(**kw):
        args = list(ok)
        names = ["dt", "q", "k", "v", "s", "gain", "temp", "cu", "batch", "Hq", "Hkv", "dh",
                 "out", "lse", "stream"]
        for k, v in kw.items():
            args[names.index(k)] = v
        return f(*args)

    assert call(dt=5) == 4
    assert call(q=None) == 1
    assert call(temp=None) == 1
    assert call(s=None) == 1             # s_kept and gain are NULL together or not at all
    assert call(gain=None) == 1
    assert call(cu=None) == 1
    assert call(batch=0) == 2
    assert call(batch=tg.TG_MAX_BATCH + 1) == 2
    assert call(Hq=12) == 2              # Hq % Hkv
    assert call(dh=96) == 5
    bad = tg._i32_array([3, 100])
    assert call(cu=ctypes.cast(bad, ctypes.POINTER(ctypes.c_int32))) == 2
    dec = tg._i32_array([0, 50, 40])
    assert call(cu=ctypes.cast(dec, ctypes.POINTER(ctypes.c_int32)), batch=2) == 2
    assert call(out=G + 8) == 6
    assert call(out=A + 256) == 9        # out overlaps q
    assert call(lse=B + 4) == 9          # lse overlaps k
    zero = tg._i32_array([0, 0])
    assert call(cu=ctypes.cast(zero, ctypes.POINTER(ctypes.c_int32))) == 0    # no rows: no-op
    # bf16 K/V rows of one request must span < 2 GiB: 2^20 rows x 8 x 128 x 2 B = 2^31
    big = tg._i32_array([0, 1 << 20])
    assert call(cu=ctypes.cast(big, ctypes.POINTER(ctypes.c_int32))) == 5


# Key split plan: a fixed 2 KiB region of per-tile counters (the split serves
# fewer than 512 query tiles x head groups), then one slot per workgroup: 4
# waves x 64 lanes x (d_head / 2 + 2) floats.  Query tiles are cut into
# ceil(nkv / 24) pieces, or ceil(nkv / 16) when the longest tile has 19 to
# 24 key tiles.  16k layer: 32 query tiles of 1..32 key tiles, sum of
# ceil((t + 1) / 24) = 40 pieces per head group, 8 head groups.
SLOT128 = 4 * 64 * (128 // 2 + 2) * 4
SLOT64 = 4 * 64 * (64 // 2 + 2) * 4


@pytest.mark.parametrize("cu,Hq,Hkv,dh,dt,expect", [
    ([0, 2048], 16, 8, 128, 1, 2048 + 320 * SLOT128),     # 16k layer's kept rows: split
    ([0, 4096], 16, 8, 128, 1, 0),                         # 32k: two whole tiles per CU already
    ([0, 1600], 8, 2, 64, 1, 2048 + 104 * SLOT64),         # four heads per workgroup, 32-row tiles
    ([0, 1537], 16, 8, 128, 1, 2048 + 208 * SLOT128),      # 25 key tiles: the shortest split
    ([0, 1536], 16, 8, 128, 1, 2048 + 256 * SLOT128),      # 24 key tiles: pieces of 16 (16 + 2 x 8 per group)
    ([0, 1153], 16, 8, 128, 1, 2048 + 176 * SLOT128),      # 19 key tiles: the shortest split into pieces of 16
    ([0, 1152], 16, 8, 128, 1, 0),                         # 18 key tiles: no split
    ([0, 13000], 2, 1, 64, 1, 2048 + 972 * SLOT64),        # one head group, up to 9 pieces
    ([0, 8192], 16, 8, 128, 1, 0),                         # eight-wave grid fills the chip
    ([0, 1000, 2048], 16, 8, 128, 1, 0),                   # two requests
    ([0, 2048], 16, 16, 128, 1, 0),                        # one head per workgroup
    ([0, 2048], 16, 8, 128, 0, 0),                         # fp32 path
])
def test_attn_prefill_plan(cu, Hq, Hkv, dh, dt, expect):
    """The key split is host logic: which shapes get a workspace, and its size."""
    L = tg.lib()
    ws = ctypes.c_size_t(123)
    arr = tg._i32_array(cu)
    assert L.tg_attn_prefill_plan(dt, ctypes.cast(arr, ctypes.POINTER(ctypes.c_int32)), len(cu) - 1,
                                  Hq, Hkv, dh, ctypes.byref(ws)) == 0
    assert ws.value == expect


def test_attn_prefill_ws_validation():
    L = tg.lib()
    f = L.tg_gated_attn_prefill_ws
    cu = tg._i32_array([0, 2048])
    cu_p = ctypes.cast(cu, ctypes.POINTER(ctypes.c_int32))
    need = 2048 + 320 * SLOT128
    W = 1 << 30
    ok = [1, A, B, C, D, E, F, cu_p, 1, 16, 8, 128, 1 << 28, None, W, need, None]
    names = ["dt", "q", "k", "v", "s", "gain", "temp", "cu", "batch", "Hq", "Hkv", "dh",
             "out", "lse", "ws", "ws_bytes", "stream"]

    def call(**kw):
        args = list(ok)
        for k, v in kw.items():
            args[names.index(k)] = v
        return f(*args)

    assert call(ws=None) == 7                       # the shape splits: a workspace is required
    assert call(ws_bytes=need - 1) == 7
    assert call(ws=W + 8) == 6                      # 16-byte alignment
    assert call(ws=A) == 9                          # workspace overlaps q
    assert call(ws=(1 << 28) - 4096) == 9           # workspace overlaps out
    assert call(dt=5) == 4
    assert L.tg_attn_prefill_plan(1, cu_p, 1, 16, 8, 128, None) == 1
    short = tg._i32_array([0, 100])                 # no split: no workspace needed
    assert call(cu=ctypes.cast(short, ctypes.POINTER(ctypes.c_int32)), ws=None, ws_bytes=0,
                q=None) == 1                        # (then the usual checks apply)


def test_decode_plan():
    L = tg.lib()
    ws = ctypes.c_size_t(0)
    assert L.tg_decode_plan(1, 16, 128, 8192, ctypes.byref(ws)) == 0
    nch = 8192 // 128
    assert ws.value >= 16 * nch * (128 + 2) * 4
    assert L.tg_decode_plan(1, 16, 128, 0, ctypes.byref(ws)) == 0 and ws.value == 0
    assert L.tg_decode_plan(0, 16, 128, 10, ctypes.byref(ws)) == 2
    assert L.tg_decode_plan(65536, 16, 128, 10, ctypes.byref(ws)) == 2
    assert L.tg_decode_plan(1, 16, 128, -1, ctypes.byref(ws)) == 2
    assert L.tg_decode_plan(1, 16, 80, 10, ctypes.byref(ws)) == 5
    assert L.tg_decode_plan(1, 16, 128, 10, None) == 1
    assert tg.tg_decode_plan(4, 16, 64, 1000) > tg.tg_decode_plan(4, 16, 64, 100)


def test_decode_validation():
    L = tg.lib()
    f = L.tg_gated_attn_decode
    ws = tg.tg_decode_plan(1, 16, 128, 100)
    W = H + 4096
    ok = [1, A, B, C, D, 100, E, E + 64, 1, 100, F, F + 64, 16, 8, 128, G, H, W, ws, None]
    names = ["dt", "q", "k", "v", "s", "rows", "off", "len", "batch", "max_len", "gain", "temp",
             "Hq", "Hkv", "dh", "out", "lse", "ws", "ws_bytes", "stream"]

    def call(**kw):
        args = list(ok)
        for k, v in kw.items():
            args[names.index(k)] = v
        return f(*args)

    assert call(dt=3) == 4
    for name in ("q", "k", "v", "off", "len", "temp", "out"):
        assert call(**{name: None}) == 1, name
    assert call(s=None) == 1 and call(gain=None) == 1      # NULL together or not at all
    assert call(batch=0) == 2 and call(batch=65536) == 2
    assert call(Hq=12) == 2 and call(rows=-1) == 2 and call(max_len=-1) == 2
    assert call(dh=96) == 5
    assert call(Hq=72, Hkv=8) == 5                          # group of 9 query heads
    assert call(ws=None) == 7 and call(ws_bytes=ws - 1) == 7
    assert call(q=A + 8) == 6 and call(out=G + 4) == 6 and call(ws=W + 8) == 6
    assert call(off=E + 4) == 6 and call(s=D + 2) == 6
    assert call(out=A + 512) == 9                           # out overlaps q
    assert call(lse=B + 64) == 9                            # lse overlaps k
    assert call(ws=C + 1024) == 9                           # workspace overlaps v
    assert call(ws=G) == 9                                  # workspace overlaps out
    assert call(lse=G + 1024) == 9                          # lse overlaps out


def test_layer_piece_validation():
    L = tg.lib()
    rn = L.tg_rmsnorm
    assert rn(3, A, B, 1e-6, 10, 2048, C, None) == 4
    assert rn(1, None, B, 1e-6, 10, 2048, C, None) == 1 and rn(1, A, None, 1e-6, 10, 2048, C, None) == 1
    assert rn(1, A, B, 1e-6, -1, 2048, C, None) == 2 and rn(1, A, B, -1.0, 10, 2048, C, None) == 2
    assert rn(1, A, B, float("nan"), 10, 2048, C, None) == 2
    assert rn(1, A, B, 1e-6, 10, 2044, C, None) == 5                    # bf16 rows of 16-byte multiples
    assert rn(1, A + 2, B, 1e-6, 10, 2048, C, None) == 6
    assert rn(1, A, B, 1e-6, 10, 2048, A + 4096, None) == 9             # partial overlap
    assert rn(1, A, B, 1e-6, 10, 2048, B, None) == 9                    # y over w
    assert rn(1, A, B, 1e-6, 0, 2048, A, None) == 0                     # in place, M == 0
    qr = L.tg_qk_norm_rope
    ok = [1, A, B, C, D, E, 100, 16, 8, 128, 1e6, 1e-6, None]

    def q(**kw):
        names = ["dt", "q", "k", "qw", "kw", "pos", "M", "Hq", "Hkv", "dh", "theta", "eps", "st"]
        args = list(ok)
        for k, v in kw.items():
            args[names.index(k)] = v
        return qr(*args)

    assert q(dt=2) == 4 and q(q=None) == 1 and q(k=None) == 1 and q(pos=None) == 1
    assert q(M=-1) == 2 and q(Hq=0) == 2 and q(theta=0.0) == 2 and q(eps=-1.0) == 2
    assert q(dh=96) == 5 and q(q=A + 4) == 6 and q(pos=E + 2) == 6
    assert q(k=A + 1024) == 9 and q(qw=A + 512) == 9 and q(pos=B + 64) == 9
    assert q(M=0) == 0
    sm = L.tg_silu_mul
    assert sm(2, A, 10, 64, B, None) == 4 and sm(1, None, 10, 64, B, None) == 1
    assert sm(1, A, -1, 64, B, None) == 2 and sm(1, A, 10, 0, B, None) == 2
    assert sm(1, A, 10, 60, B, None) == 5 and sm(1, A, 10, 64, B + 8, None) == 6
    assert sm(1, A, 10, 64, A + 1024, None) == 9 and sm(1, A, 0, 64, B, None) == 0
    kp = L.tg_kept_positions
    P = ctypes.POINTER(ctypes.c_int32)
    cs, ck = tg._i32_array([0, 100, 150]), tg._i32_array([0, 30, 60])
    cs_p, ck_p = ctypes.cast(cs, P), ctypes.cast(ck, P)
    assert kp(None, cs_p, ck_p, 2, B, None) == 1 and kp(A, None, ck_p, 2, B, None) == 1
    assert kp(A, cs_p, ck_p, 0, B, None) == 2 and kp(A, cs_p, ck_p, 65, B, None) == 2
    bad = tg._i32_array([0, 40, 30])
    assert kp(A, cs_p, ctypes.cast(bad, P), 2, B, None) == 2
    assert kp(A + 2, cs_p, ck_p, 2, B, None) == 6 and kp(A, cs_p, ck_p, 2, A + 8, None) == 9


def test_attention_backward_validation():
    L = tg.lib()
    cu = tg._i32_array([0, 100])
    P = ctypes.POINTER(ctypes.c_int32)
    cu_p = ctypes.cast(cu, P)
    ws = ctypes.c_size_t(0)
    assert L.tg_attn_backward_plan(cu_p, 1, 16, 8, ctypes.byref(ws)) == 0 and ws.value > 0
    assert L.tg_attn_backward_plan(cu_p, 1, 12, 8, ctypes.byref(ws)) == 2
    assert L.tg_attn_backward_plan(None, 1, 16, 8, ctypes.byref(ws)) == 1
    W = 64 << 20
    X = [(9 + i) << 20 for i in range(8)]  # q k v out dout dq dk dv regions
    small = [(20 << 20) + 4096 * i for i in range(8)]  # s gain temp lse ds dgain dtemp
    ok = [1, X[0], X[1], X[2], small[0], small[1], small[2], X[3], small[3], X[4], cu_p, 1, 16, 8,
          128, X[5], X[6], X[7], small[4], small[5], small[6], W, ws.value, None]
    names = ["dt", "q", "k", "v", "s", "gain", "temp", "out", "lse", "dout", "cu", "batch", "Hq",
             "Hkv", "dh", "dq", "dk", "dv", "ds", "dgain", "dtemp", "ws", "wsb", "st"]

    def call(**kw):
        args = list(ok)
        for k, v in kw.items():
            args[names.index(k)] = v
        return L.tg_gated_attn_backward(*args)

    assert call(dt=4) == 4
    for nm in ("q", "k", "v", "temp", "out", "lse", "dout", "dq", "dk", "dv", "dtemp", "cu"):
        assert call(**{nm: None}) == 1, nm
    assert call(s=None) == 1 and call(ds=None) == 1 and call(dgain=None) == 1   # bias set all or none
    assert call(batch=0) == 2 and call(Hq=12) == 2
    assert call(dt=0) == 5 and call(dh=96) == 5                                  # fp32, d_head
    assert call(ws=None) == 7 and call(wsb=ws.value - 1) == 7
    assert call(q=X[0] + 8) == 6 and call(ws=W + 8) == 6 and call(lse=small[3] + 2) == 6
    assert call(dq=X[0]) == 9 and call(dk=X[5]) == 9 and call(ws=X[2]) == 9 and call(ds=small[0]) == 9
    zero = tg._i32_array([0, 0])
    assert call(cu=ctypes.cast(zero, P)) == 0                                    # no rows: no-op


def test_gate_backward_validation():
    L = tg.lib()
    ws = ctypes.c_size_t(0)
    assert L.tg_gate_backward_plan(1, 777, 2048, 256, ctypes.byref(ws)) == 0 and ws.value > 0
    assert L.tg_gate_backward_plan(1, 777, 2000, 256, ctypes.byref(ws)) == 5
    assert L.tg_gate_backward_plan(1, -1, 2048, 256, ctypes.byref(ws)) == 2
    assert L.tg_gate_backward_plan(3, 7, 2048, 256, ctypes.byref(ws)) == 4
    assert L.tg_gate_backward_plan(1, 100, 2048, 256, ctypes.byref(ws)) == 0   # the shape called below
    W = 96 << 20
    f = L.tg_gate_backward
    ok = [1, A, 100, 2048, B, C, D, 256, E, F, G, H, H + 1024, H + 2048, W, ws.value, None]
    names = ["dt", "x", "Kt", "d", "w1", "b1", "w2", "dg", "ds", "dx", "dw1", "db1", "dw2", "db2",
             "ws", "wsb", "st"]

    def call(**kw):
        args = list(ok)
        for k, v in kw.items():
            args[names.index(k)] = v
        return f(*args)

    assert call(dt=9) == 4
    for nm in ("x", "w1", "w2", "ds", "dx", "dw1", "dw2", "db2"):
        assert call(**{nm: None}) == 1, nm
    assert call(b1=None) == 1 and call(db1=None) == 1                 # NULL together or not at all
    assert call(Kt=-1) == 2 and call(d=0) == 2 and call(dg=100) == 5
    assert call(ws=None) == 7 and call(wsb=ws.value - 1) == 7
    assert call(x=A + 8) == 6 and call(db2=H + 2050) == 6
    assert call(dx=A + 64) == 9 and call(dw1=B) == 9 and call(ws=F) == 9 and call(dw2=H) == 9
    assert call(Kt=0) == 0


def test_linear_validation():
    L = tg.lib()
    f = L.tg_linear
    assert f(2, A, B, C, 10, 128, 128, 0, None) == 4
    assert f(1, A, B, C, -1, 128, 128, 0, None) == 2
    assert f(1, A, B, C, 10, 0, 128, 0, None) == 2
    assert f(1, None, B, C, 10, 128, 128, 0, None) == 1
    assert f(1, A, B, C, 10, 96, 128, 0, None) == 5
    assert f(1, A, B, C, 10, 128, 100, 0, None) == 5
    assert f(1, A, B, C + 2, 10, 128, 128, 0, None) == 6
    assert f(1, A, B, A + 16, 10, 128, 128, 1, None) == 9
    assert f(1, A, B, C, 0, 128, 128, 0, None) == 0


def test_missing_library_fails_loudly():
    """Without the built library every entry point raises: there is no
    fallback implementation of any step."""
    import subprocess
    import sys
    code = (
        "import torch, learned_token_pruning_02_amd as tg\n"
        "tg._LIB_PATH = '/nonexistent/libtokengate.so'\n"
        "try:\n"
        "    tg.lib()\n"
        "except RuntimeError as e:\n"
        "    assert 'missing' in str(e)\n"
        "else:\n"
        "    raise SystemExit('lib() did not raise')\n"
        "try:\n"
        "    tg.tg_gate_score(torch.zeros(4, 64), torch.zeros(64, 64), None, torch.zeros(64), None)\n"
        "except RuntimeError:\n"
        "    print('raised')\n"
        "q, k = torch.zeros(8, 2, 64), torch.zeros(8, 1, 64)\n"
        "for ws in (None, torch.zeros(64, dtype=torch.uint8)):\n"
        "    try:\n"
        "        tg.tg_gated_attn_prefill(q, k, k, None, None, torch.ones(2), [0, 8], workspace=ws)\n"
        "    except RuntimeError:\n"
        "        print('attention raised')\n"
    )
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    r = subprocess.run([sys.executable, "-c", code], cwd=root, capture_output=True, text=True, timeout=240)
    assert r.returncode == 0 and "raised" in r.stdout, (r.returncode, r.stdout, r.stderr)
    assert r.stdout.count("attention raised") == 2, (r.stdout, r.stderr)


def test_select_path_validation():
    """tg_topk_select_path: an unknown path is rejected, and the one-workgroup
    path refuses a document longer than it can hold."""
    L = tg.lib()
    ws = tg.tg_plan([100], [10], [20])[2]
    bt, keep = _batch([100], [10], [20], [0])
    f = L.tg_topk_select_path
    assert f(A, ctypes.byref(bt), B, None, C, ws, 3, None) == 2
    assert f(A, ctypes.byref(bt), B, None, C, ws, -1, None) == 2
    assert f(None, ctypes.byref(bt), B, None, C, ws, 2, None) == 1
    n = 65536 + 11
    ws2 = tg.tg_plan([n], [10], [20])[2]
    bt2, keep2 = _batch([n], [10], [20], [0])
    assert f(A, ctypes.byref(bt2), B, None, C, ws2, 1, None) == 5
    # a tg_batch_prefix whose prefix_len is NULL is a plain batch
    bt3 = tg._BatchPrefix(1, keep2[0], keep2[1], keep2[2], None)
    assert f(None, ctypes.byref(bt3), B, None, C, ws2, 2, None) == 1
    assert f(A, ctypes.byref(bt3), B, None, C, ws2, 1, None) == 5


def test_linear_tile_validation():
    L = tg.lib()
    f = L.tg_linear_tile
    assert f(1, A, B, C, 10, 128, 128, 0, 4, None) == 2
    assert f(1, A, B, C, 10, 128, 128, 0, -1, None) == 2
    assert f(1, A, B, C, 10, 96, 128, 0, 1, None) == 5
    assert f(1, A, B, C, 0, 128, 128, 0, 3, None) == 0


def test_linear_multi_validation():
    L = tg.lib()
    f = L.tg_linear_multi
    vp = ctypes.c_void_p
    two = lambda a, b: (vp * 2)(a, b)
    n = lambda *v: (ctypes.c_int32 * len(v))(*v)
    W, Y = two(B, B + 4096), two(C, C + (1 << 20))
    assert f(7, A, 2, W, Y, n(256, 256), 10, 128, 0, 0, None) == 4        # dtype
    assert f(1, A, 0, W, Y, n(256, 256), 10, 128, 0, 0, None) == 2        # nseg 0
    assert f(1, A, 4, W, Y, n(256, 256), 10, 128, 0, 0, None) == 2        # nseg > 3
    assert f(1, A, 2, W, Y, n(256, 256), 10, 128, 0, 4, None) == 2        # tile
    assert f(1, A, 2, W, Y, n(256, 0), 10, 128, 0, 0, None) == 2          # a zero width
    assert f(1, None, 2, W, Y, n(256, 256), 10, 128, 0, 0, None) == 1
    assert f(1, A, 2, None, Y, n(256, 256), 10, 128, 0, 0, None) == 1
    assert f(1, A, 2, two(B, None), Y, n(256, 256), 10, 128, 0, 0, None) == 1
    assert f(1, A, 2, W, Y, None, 10, 128, 0, 0, None) == 1
    assert f(1, A, 2, W, Y, n(256, 192), 10, 128, 0, 0, None) == 5        # width not a multiple of 256
    assert f(1, A, 2, W, Y, n(256, 256), 10, 96, 0, 0, None) == 5         # K % 64
    assert f(1, A, 2, two(B, B + 8), Y, n(256, 256), 10, 128, 0, 0, None) == 6  # alignment
    assert f(1, A, 2, W, two(C, C + 512), n(256, 256), 10, 128, 0, 0, None) == 9  # outputs overlap
    assert f(1, A, 2, W, two(A, C), n(256, 256), 10, 128, 0, 0, None) == 9     # an output over x
    assert f(1, A, 2, W, Y, n(256, 256), 0, 128, 0, 0, None) == 0             # M == 0: no-op


def test_linear_swiglu_validation():
    L = tg.lib()
    f = L.tg_linear_swiglu
    assert f(7, A, B, C, 10, 128, 128, 0, None) == 4          # dtype
    assert f(1, A, B, C, -1, 128, 128, 0, None) == 2          # M
    assert f(1, A, B, C, 10, 0, 128, 0, None) == 2            # F
    assert f(1, A, B, C, 10, 128, 128, 4, None) == 2          # tile
    assert f(1, None, B, C, 10, 128, 128, 0, None) == 1
    assert f(1, A, None, C, 10, 128, 128, 0, None) == 1
    assert f(1, A, B, None, 10, 128, 128, 0, None) == 1
    assert f(0, A, B, C, 10, 128, 128, 0, None) == 5          # fp32 not built
    assert f(1, A, B, C, 10, 192, 128, 0, None) == 5          # F % 128
    assert f(1, A, B, C, 10, 128, 96, 0, None) == 5           # K % 64
    assert f(1, A + 8, B, C, 10, 128, 128, 0, None) == 6
    assert f(1, A, B, A, 10, 128, 128, 0, None) == 9          # out over x
    assert f(1, A, B, B, 10, 128, 128, 0, None) == 9          # out over the weights
    assert f(1, A, B, C, 0, 128, 128, 0, None) == 0           # M == 0: no-op


# ------------------------------------------- binding size checks (no GPU) ----
def _meta(*shape, dtype=None):
    import torch
    return torch.empty(*shape, dtype=dtype or torch.bfloat16, device="meta")


def _raises_size(fn, *args, match=None, **kw):
    """The wrapper must reject the sizes itself (ValueError naming the size
    problem), before it looks at where the tensors live."""
    with pytest.raises(ValueError) as e:
        fn(*args, **kw)
    msg = str(e.value)
    assert "GPU tensor" not in msg, msg
    if match is not None:
        assert match in msg, msg


def test_binding_checks_gate_sizes():
    import torch
    h, w1, w2 = _meta(100, 256), _meta(64, 256), _meta(64)
    _raises_size(tg.tg_gate_score, h, _meta(64, 128), None, w2, None, match="w1")
    _raises_size(tg.tg_gate_score, h, w1, _meta(32), w2, None, match="b1")
    _raises_size(tg.tg_gate_score, h, w1, None, _meta(63), None, match="w2")
    _raises_size(tg.tg_gate_score, h, w1, None, w2, _meta(2), match="b2")
    _raises_size(tg.tg_gate_score, h, w1, None, w2, None, scores=_meta(99, dtype=torch.float32),
                 match="scores")
    _raises_size(tg.tg_gate_score, _meta(100, 256, 1), w1, None, w2, None, match="hidden")


def test_binding_checks_select_sizes():
    import torch
    f32, i32 = torch.float32, torch.int32
    seq, q, bud = [300, 200], [10, 20], [50, 60]
    s = _meta(500, dtype=f32)
    _raises_size(tg.tg_topk_select, _meta(499, dtype=f32), seq, q, bud, match="scores")
    _raises_size(tg.tg_topk_select, s, seq, q, bud, kept_idx=_meta(109, dtype=i32), match="kept_idx")
    _raises_size(tg.tg_topk_select, s, seq, q, bud, cu_kept_dev=_meta(2, dtype=i32), match="cu_kept_dev")
    ws = tg.tg_plan(seq, q, bud)[2]
    # the workspace is counted in bytes whatever its element type
    _raises_size(tg.tg_topk_select, s, seq, q, bud, workspace=_meta(ws // 4 - 1, dtype=i32),
                 match="workspace")


def test_binding_checks_gather_sizes():
    import torch
    h, kept = _meta(100, 64), _meta(20, dtype=torch.int32)
    _raises_size(tg.tg_gather_compact, h, kept, scores=_meta(99, dtype=torch.float32), match="scores")
    _raises_size(tg.tg_gather_compact, h, kept, hidden_kept=_meta(21, 64), match="hidden_kept")
    _raises_size(tg.tg_gather_compact, h, kept, scores=_meta(100, dtype=torch.float32),
                 scores_kept=_meta(19, dtype=torch.float32), match="scores_kept")


def test_binding_checks_attention_sizes():
    import torch
    f32 = torch.float32
    Kt, Hq, Hkv, dh = 96, 4, 2, 64
    q, k, v = _meta(Kt, Hq, dh), _meta(Kt, Hkv, dh), _meta(Kt, Hkv, dh)
    s, g, t = _meta(Kt, dtype=f32), _meta(Hq, dtype=f32), _meta(Hq, dtype=f32)
    cu = [0, 40, Kt]
    f = tg.tg_gated_attn_prefill
    _raises_size(f, q, k, v, s, g, t, [0, 40, Kt - 1], match="cu_kept")
    _raises_size(f, q, k, v, s, g, t, [0, 40, Kt + 1], match="cu_kept")
    _raises_size(f, q, _meta(Kt - 1, Hkv, dh), v, s, g, t, cu, match="k")
    _raises_size(f, q, k, _meta(Kt, Hkv, dh - 8), s, g, t, cu, match="v")
    _raises_size(f, q, _meta(Kt, 3, dh), _meta(Kt, 3, dh), s, g, t, cu, match="multiple")
    _raises_size(f, q, k, v, _meta(Kt - 1, dtype=f32), g, t, cu, match="s_kept")
    _raises_size(f, q, k, v, s, _meta(Hq - 1, dtype=f32), t, cu, match="gain")
    _raises_size(f, q, k, v, s, g, _meta(Hq + 1, dtype=f32), cu, match="temp")
    _raises_size(f, q, k, v, s, g, t, cu, out=_meta(Kt, Hq, dh - 1), match="out")
    _raises_size(f, q, k, v, s, g, t, cu, lse=_meta(Kt, Hq, dtype=f32), match="lse")
    # backward: the same checks plus the gradient buffers
    fb = tg.tg_gated_attn_backward
    o, lse = _meta(Kt, Hq, dh), _meta(Hq, Kt, dtype=f32)
    _raises_size(fb, q, k, v, s, g, t, o, lse, _meta(Kt, Hq, dh + 1), cu, match="dout")
    _raises_size(fb, q, k, v, s, g, t, o, _meta(Hq, Kt - 1, dtype=f32), o, cu, match="lse")
    grads = {"dq": _meta(Kt, Hq, dh), "dk": _meta(Kt, Hkv, dh), "dv": _meta(Kt, Hkv, dh - 1),
             "ds": _meta(Kt, dtype=f32), "dgain": _meta(Hq, dtype=f32), "dtemp": _meta(Hq, dtype=f32)}
    _raises_size(fb, q, k, v, s, g, t, o, lse, o, cu, grads=grads, match="dv")


def test_binding_checks_other_sizes():
    import torch
    f32, i32 = torch.float32, torch.int32
    # gate backward
    x, w1, w2 = _meta(50, 128), _meta(64, 128), _meta(64)
    _raises_size(tg.tg_gate_backward, x, w1, None, w2, _meta(49, dtype=f32), match="ds_kept")
    _raises_size(tg.tg_gate_backward, x, _meta(64, 127), None, w2, _meta(50, dtype=f32), match="w1")
    # decode
    B, Hq, Hkv, dh, R = 3, 4, 2, 64, 40
    qd, kd = _meta(B, Hq, dh), _meta(R, Hkv, dh)
    args = (qd, kd, kd, _meta(R, dtype=f32), _meta(B, dtype=torch.int64), _meta(B, dtype=i32),
            _meta(Hq, dtype=f32), _meta(Hq, dtype=f32), 16)
    _raises_size(tg.tg_gated_attn_decode, qd, kd, _meta(R - 1, Hkv, dh), *args[3:], match="v")
    _raises_size(tg.tg_gated_attn_decode, *args[:4], _meta(B + 1, dtype=torch.int64), *args[5:],
                 match="row_off")
    _raises_size(tg.tg_gated_attn_decode, *args, out=_meta(B, Hq, dh + 1), match="out")
    # layer pieces and the projection
    _raises_size(tg.tg_rmsnorm, _meta(10, 64), _meta(63), 1e-6, match="w")
    _raises_size(tg.tg_rmsnorm, _meta(10, 64), _meta(64), 1e-6, y=_meta(9, 64), match="y")
    _raises_size(tg.tg_qk_norm_rope, _meta(10, 4, 64), _meta(9, 2, 64), None, None,
                 _meta(10, dtype=i32), 1e6, 1e-6, match="k")
    _raises_size(tg.tg_qk_norm_rope, _meta(10, 4, 64), _meta(10, 2, 64), None, None,
                 _meta(11, dtype=i32), 1e6, 1e-6, match="pos")
    _raises_size(tg.tg_silu_mul, _meta(10, 128), out=_meta(10, 65), match="out")
    _raises_size(tg.tg_kept_positions, _meta(10, dtype=i32), [0, 100], [0, 11], match="kept_idx")
    _raises_size(tg.tg_linear, _meta(10, 128), _meta(64, 127), match="w")
    _raises_size(tg.tg_linear, _meta(10, 128), _meta(64, 128), y=_meta(10, 63), match="y")


def test_select_noalloc_validation():
    """tg_topk_select_noalloc decides on the host, before any HIP call, that a
    batch needs more than the library's static scratch, and checks pointers
    like tg_topk_select."""
    L = tg.lib()
    f = L.tg_topk_select_noalloc
    bt, keep = _batch([100], [10], [20])
    assert f(None, ctypes.byref(bt), B, None, None) == 1
    assert f(A, ctypes.byref(bt), None, None, None) == 1
    assert f(A, None, B, None, None) == 1
    assert f(A + 2, ctypes.byref(bt), B, None, None) == 6
    assert f(A, ctypes.byref(bt), A + 40, None, None) == 9        # kept ids inside the scores
    bad, keep_b = _batch([10], [4], [3])
    assert f(A, ctypes.byref(bad), B, None, None) == 3
    # a chunked-path batch whose workspace exceeds the scratch
    big = 1_200_000
    assert tg.tg_plan([big], [128], [8192])[2] > 8 << 20
    bt2, keep2 = _batch([big], [128], [8192])
    assert f(A, ctypes.byref(bt2), B, None, None) == 7
