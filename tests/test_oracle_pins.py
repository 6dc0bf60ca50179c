"""Pins of the CPU oracle to things other than itself (no GPU needed).

Each test checks one oracle function against a library routine it does not
use, brute force, a closed form, a textbook value or an invariant the
TokenGate pages state, chosen so that a plausible slip (dropped bias, wrong
sign, transposed weight, wrong GQA mapping, bias on the query instead of the
key, anti-causal mask, wrong softmax scale, wrong tie-break) fails at least
one of them.
"""
import math
import os

import numpy as np
import pytest
import torch
import torch.nn.functional as F
from hypothesis import given, settings, strategies as st

import oracle
import workloads

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# ----------------------------------------------------------------- gate ----
@pytest.mark.parametrize("with_bias", [True, False])
def test_gate_matches_torch_linear_gelu(with_bias):
    g = torch.Generator().manual_seed(1)
    T, d, dg = 37, 48, 16                   # non-square W1 catches a transpose
    x = torch.randn(T, d, generator=g)
    w1 = torch.randn(dg, d, generator=g) / math.sqrt(d)
    w2 = torch.randn(dg, generator=g) / math.sqrt(dg)
    b1 = torch.randn(dg, generator=g) if with_bias else None
    b2 = torch.randn(1, generator=g) if with_bias else None
    got = oracle.gate_score(x, w1, b1, w2, b2)
    h = F.gelu(F.linear(x.double(), w1.double(), None if b1 is None else b1.double()),
               approximate="none")
    want = F.linear(h, w2.double()[None, :], None if b2 is None else b2.double())[:, 0]
    assert got.dtype == torch.float32 and got.shape == (T,)
    torch.testing.assert_close(got.double(), want.float().double(), rtol=2e-7, atol=1e-9)


def _normal_cdf_table():
    rows = []
    with open(os.path.join(GOLDEN, "normal_cdf.txt")) as f:
        for line in f:
            line = line.strip()
            if line and not line.startswith("#"):
                x, p = line.split()
                rows.append((float(x), float(p)))
    return rows


def test_gate_gelu_textbook_points():
    """W1 = 0 makes every score w2 . GELU(b1) + b2, and GELU(x) = x Phi(x)."""
    rows = _normal_cdf_table()
    pts = [x for x, _ in rows] + [-x for x, _ in rows if x > 0]
    phi = {x: p for x, p in rows}
    phi.update({-x: 1.0 - p for x, p in rows if x > 0})
    dg, d, T = len(pts), 8, 3
    b1 = torch.tensor(pts, dtype=torch.float64)
    w1 = torch.zeros(dg, d, dtype=torch.float64)
    x = torch.randn(T, d, dtype=torch.float64)
    for u, xv in enumerate(pts):
        w2 = torch.zeros(dg, dtype=torch.float64)
        w2[u] = 1.0
        s = oracle.gate_score(x, w1, b1, w2, torch.tensor([0.25], dtype=torch.float64))
        want = xv * phi[xv] + 0.25
        assert torch.allclose(s.double(), torch.full((T,), want, dtype=torch.float64),
                              rtol=1e-7, atol=2e-10), (xv, s, want)


def test_gate_constant_when_w1_zero_all_ties():
    """All-equal scores are a degenerate case the selector must handle."""
    w1 = torch.zeros(4, 6)
    b1 = torch.tensor([0.3, -0.2, 1.0, 0.0])
    w2 = torch.tensor([0.5, -1.0, 0.25, 2.0])
    s = oracle.gate_score(torch.randn(9, 6), w1, b1, w2, torch.tensor([0.1]))
    assert torch.all(s == s[0])


# --------------------------------------------------------------- select ----
def _brute_sorted(scores, seq_len, q_len, budget, prefix_len=None):
    """Kept ids by a full Python sort with an explicit comparison key."""
    out, lo = [], 0
    prefix_len = prefix_len or [0] * len(seq_len)
    for n, q, k, p in zip(seq_len, q_len, budget, prefix_len):
        keep = min(k, n)
        if keep >= n:
            ids = list(range(n))
        else:
            def key(i):
                v = float(scores[lo + i])
                if math.isnan(v):
                    return (1, 0.0, i)
                return (0, -(v + 0.0), i)
            doc = sorted(range(p, n - q), key=key)[: keep - q - p]
            ids = sorted(list(range(p)) + doc + list(range(n - q, n)))
        out += [lo + i for i in ids]
        lo += n
    return out


def _brute_rank(scores, seq_len, q_len, budget, prefix_len=None):
    """Kept ids by counting, for every document token, how many beat it."""
    def beats(a, ia, b, ib):            # does (a, ia) come before (b, ib)?
        na, nb = math.isnan(a), math.isnan(b)
        if na != nb:
            return nb
        if not na and a != b:
            return a > b
        return ia < ib

    out, lo = [], 0
    prefix_len = prefix_len or [0] * len(seq_len)
    for n, q, k, p in zip(seq_len, q_len, budget, prefix_len):
        keep = min(k, n)
        for i in range(n):
            if keep >= n or i >= n - q or i < p:
                out.append(lo + i)
                continue
            vi = float(scores[lo + i])
            rank = sum(beats(float(scores[lo + j]), j, vi, i) for j in range(p, n - q) if j != i)
            if rank < keep - q - p:
                out.append(lo + i)
        lo += n
    return out


SPECIALS = [0.0, -0.0, float("inf"), float("-inf"), float("nan"), 1.0, -1.0, 1e-30, -1e-30]


@pytest.mark.parametrize("case", range(12))
def test_select_matches_brute_force(case):
    g = torch.Generator().manual_seed(100 + case)
    B = 1 + case % 3
    seq_len = torch.randint(1, 60, (B,), generator=g).tolist()
    q_len = [int(torch.randint(0, n + 1, (1,), generator=g)) for n in seq_len]
    budget = [max(1, q + int(torch.randint(0, n + 3, (1,), generator=g))) for q, n in zip(q_len, seq_len)]
    budget = [max(b, 1) for b in budget]
    T = sum(seq_len)
    if case % 2:
        s = (torch.randint(0, 5, (T,), generator=g).float() - 2.0) / 2.0   # heavy ties
    else:
        s = torch.randn(T, generator=g)
    if case % 4 == 3:
        pos = torch.randint(0, T, (min(T, 8),), generator=g)
        for j, p in enumerate(pos.tolist()):
            s[p] = SPECIALS[(j + case) % len(SPECIALS)]
    kept, cu = oracle.topk_select(s, seq_len, q_len, budget)
    assert kept.tolist() == _brute_sorted(s, seq_len, q_len, budget)
    assert kept.tolist() == _brute_rank(s, seq_len, q_len, budget)
    assert cu[-1] == len(kept)


@settings(max_examples=60, deadline=None)
@given(st.lists(st.sampled_from(SPECIALS + [0.5, 0.25, -2.0]), min_size=1, max_size=40),
       st.integers(0, 40), st.integers(1, 45))
def test_select_invariants(vals, q, budget):
    n = len(vals)
    q = min(q, n)
    budget = max(budget, q) if q > 0 else budget
    s = torch.tensor(vals, dtype=torch.float32)
    kept, cu = oracle.topk_select(s, [n], [q], [budget])
    k = kept.tolist()
    assert len(k) == min(budget, n) == cu[1]
    assert k == sorted(set(k))                          # ascending, unique
    assert set(range(n - q, n)) <= set(k)               # question tail always kept
    doc = [i for i in range(n - q)]
    kept_doc = [i for i in doc if i in set(k)]
    drop_doc = [i for i in doc if i not in set(k)]

    def key(i):
        v = float(s[i])
        return (-math.inf, 0) if math.isnan(v) else (v + 0.0, 1)

    for i in kept_doc:                                  # threshold property
        for j in drop_doc:
            ki, kj = key(i), key(j)
            assert ki[0] > kj[0] or (ki[0] == kj[0] and (ki[1] > kj[1] or (ki[1] == kj[1] and i < j)))


@pytest.mark.parametrize("case", range(12))
def test_select_with_template_prefix_matches_brute_force(case):
    """Always-kept template prefix in front of the document span."""
    g = torch.Generator().manual_seed(300 + case)
    B = 1 + case % 3
    seq_len = torch.randint(1, 60, (B,), generator=g).tolist()
    q_len, p_len, budget = [], [], []
    for n in seq_len:
        q = int(torch.randint(0, n + 1, (1,), generator=g))
        p = int(torch.randint(0, n - q + 1, (1,), generator=g))
        q_len.append(q)
        p_len.append(p)
        budget.append(max(1, p + q + int(torch.randint(0, n + 3, (1,), generator=g))))
    T = sum(seq_len)
    if case % 2:
        s = (torch.randint(0, 5, (T,), generator=g).float() - 2.0) / 2.0   # heavy ties
    else:
        s = torch.randn(T, generator=g)
    if case % 4 == 3:
        pos = torch.randint(0, T, (min(T, 8),), generator=g)
        for j, p in enumerate(pos.tolist()):
            s[p] = SPECIALS[(j + case) % len(SPECIALS)]
    kept, cu = oracle.topk_select(s, seq_len, q_len, budget, p_len)
    assert kept.tolist() == _brute_sorted(s, seq_len, q_len, budget, p_len)
    assert kept.tolist() == _brute_rank(s, seq_len, q_len, budget, p_len)
    assert cu[-1] == len(kept)


def test_select_prefix_special_cases():
    s = torch.randn(50)
    kept, _ = oracle.topk_select(s, [50], [10], [25], [15])    # budget == prefix + tail
    assert kept.tolist() == list(range(15)) + list(range(40, 50))
    kept, _ = oracle.topk_select(s, [50], [10], [20], [0])     # prefix 0: the plain selector
    assert kept.tolist() == oracle.topk_select(s, [50], [10], [20])[0].tolist()
    kept, _ = oracle.topk_select(torch.full((50,), 0.75), [50], [5], [12], [3])   # all ties
    assert kept.tolist() == list(range(7)) + list(range(45, 50))
    with pytest.raises(ValueError):
        oracle.topk_select(s, [50], [10], [24], [15])          # budget below prefix + tail
    with pytest.raises(ValueError):
        oracle.topk_select(s, [50], [10], [30], [-1])


def test_select_special_budgets():
    s = torch.randn(50)
    kept, _ = oracle.topk_select(s, [50], [10], [10])          # budget == tail
    assert kept.tolist() == list(range(40, 50))
    kept, _ = oracle.topk_select(s, [50], [10], [500])         # budget >= N
    assert kept.tolist() == list(range(50))
    kept, _ = oracle.topk_select(torch.full((50,), 0.75), [50], [5], [12])   # all ties
    assert kept.tolist() == list(range(7)) + list(range(45, 50))
    with pytest.raises(ValueError):
        oracle.topk_select(s, [50], [10], [9])                 # budget below tail
    with pytest.raises(ValueError):
        oracle.topk_select(s, [50], [51], [60])


def test_select_nan_zero_inf_order():
    s = torch.tensor([float("nan"), -0.0, 0.0, float("-inf"), float("inf"), 1.0, float("nan"), -1.0])
    kept, _ = oracle.topk_select(s, [8], [0], [4])
    assert kept.tolist() == [1, 2, 4, 5]                       # inf, 1, then -0/+0 tie by index
    kept, _ = oracle.topk_select(s, [8], [0], [7])
    assert kept.tolist() == [0, 1, 2, 3, 4, 5, 7]              # first NaN beats the second by index


# --------------------------------------------------------------- gather ----
def test_gather_bitwise():
    h = torch.randn(20, 7).to(torch.bfloat16)
    s = torch.randn(20)
    idx = torch.tensor([0, 3, 4, 19], dtype=torch.int32)
    hk, sk = oracle.gather_compact(h, s, idx)
    for r, i in enumerate(idx.tolist()):
        assert torch.equal(hk[r].view(torch.int16), h[i].view(torch.int16))
        assert sk[r].item() == s[i].item()


# ------------------------------------------------------------ attention ----
def _attn_case(seed, lens=(5, 17, 33), Hq=4, Hkv=2, dh=16):
    g = torch.Generator().manual_seed(seed)
    Kt = sum(lens)
    cu = [0]
    for n in lens:
        cu.append(cu[-1] + n)
    q = torch.randn(Kt, Hq, dh, generator=g, dtype=torch.float64)
    k = torch.randn(Kt, Hkv, dh, generator=g, dtype=torch.float64)
    v = torch.randn(Kt, Hkv, dh, generator=g, dtype=torch.float64)
    s = torch.randn(Kt, generator=g, dtype=torch.float64)
    gain = torch.rand(Hq, generator=g, dtype=torch.float64) + 0.5
    temp = torch.rand(Hq, generator=g, dtype=torch.float64) * 0.4 + 0.8
    return q, k, v, s, gain, temp, cu


def _sdpa_reference(q, k, v, s, gain, temp, cu):
    """torch SDPA (float64): queries scaled by tau_h, float mask g_h s_j plus causal."""
    Kt, Hq, dh = q.shape
    rep = Hq // k.shape[1]
    out = torch.zeros_like(q)
    for b in range(len(cu) - 1):
        lo, hi = cu[b], cu[b + 1]
        n = hi - lo
        Q = (q[lo:hi].permute(1, 0, 2) * temp[:, None, None])          # [Hq][n][dh]
        K = k[lo:hi].permute(1, 0, 2).repeat_interleave(rep, dim=0).contiguous()
        V = v[lo:hi].permute(1, 0, 2).repeat_interleave(rep, dim=0).contiguous()
        mask = gain[:, None, None] * s[lo:hi][None, None, :].expand(Hq, n, n)
        mask = mask.masked_fill(torch.ones(n, n, dtype=torch.bool).triu(1), -math.inf)
        o = F.scaled_dot_product_attention(Q[None], K[None], V[None], attn_mask=mask[None])
        out[lo:hi] = o[0].permute(1, 0, 2)
    return out


def test_attention_plain_causal_when_gain0_temp1():
    q, k, v, s, _, _, cu = _attn_case(3)
    Hq = q.shape[1]
    out, _ = oracle.gated_attention(q, k, v, s, torch.zeros(Hq), torch.ones(Hq), cu)
    rep = Hq // k.shape[1]
    for b in range(len(cu) - 1):
        lo, hi = cu[b], cu[b + 1]
        Q = q[lo:hi].permute(1, 0, 2)[None]
        K = k[lo:hi].permute(1, 0, 2).repeat_interleave(rep, dim=0)[None].contiguous()
        V = v[lo:hi].permute(1, 0, 2).repeat_interleave(rep, dim=0)[None].contiguous()
        want = F.scaled_dot_product_attention(Q, K, V, is_causal=True)[0].permute(1, 0, 2)
        torch.testing.assert_close(out[lo:hi], want, rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("seed", [4, 5])
def test_attention_general_matches_sdpa_with_mask(seed):
    q, k, v, s, gain, temp, cu = _attn_case(seed)
    out, _ = oracle.gated_attention(q, k, v, s, gain, temp, cu)
    torch.testing.assert_close(out, _sdpa_reference(q, k, v, s, gain, temp, cu), rtol=1e-12, atol=1e-12)


def test_attention_lse_from_sdpa_probabilities():
    """With V = identity, SDPA returns the probability matrix; p_i0 = exp(l_i0 - lse_i)."""
    n, Hq, dh = 9, 2, 9
    g = torch.Generator().manual_seed(8)
    q = torch.randn(n, Hq, dh, generator=g, dtype=torch.float64)
    k = torch.randn(n, 1, dh, generator=g, dtype=torch.float64)
    v = torch.eye(n, dtype=torch.float64)[:, None, :]
    s = torch.randn(n, generator=g, dtype=torch.float64)
    gain = torch.tensor([0.7, 1.3], dtype=torch.float64)
    temp = torch.tensor([0.9, 1.1], dtype=torch.float64)
    out, lse = oracle.gated_attention(q, k, v, s, gain, temp, [0, n])
    P = _sdpa_reference(q, k, v, s, gain, temp, [0, n])        # [n][Hq][n] = probabilities
    torch.testing.assert_close(out, P, rtol=1e-12, atol=1e-12)
    for h in range(Hq):
        l0 = temp[h] * (q[:, h] @ k[0, 0]) / math.sqrt(dh) + gain[h] * s[0]
        torch.testing.assert_close(lse[h], l0 - torch.log(P[:, h, 0]), rtol=1e-12, atol=1e-12)


def test_attention_closed_forms():
    q, k, v, s, gain, temp, cu = _attn_case(6, lens=(12,))
    out, lse = oracle.gated_attention(q, k, v, s, gain, temp, cu)
    Hq = q.shape[1]
    rep = Hq // k.shape[1]
    for h in range(Hq):      # row 0 sees only key 0
        assert torch.equal(out[0, h], v[0, h // rep])
        want = temp[h] * (q[0, h] @ k[0, h // rep]) / math.sqrt(q.shape[2]) + gain[h] * s[0]
        assert abs(float(lse[h, 0] - want)) < 1e-12
    # constant scores: output does not depend on the gain
    c = torch.full_like(s, 0.37)
    o1, _ = oracle.gated_attention(q, k, v, c, gain, temp, cu)
    o2, _ = oracle.gated_attention(q, k, v, c, gain * 3.0, temp, cu)
    torch.testing.assert_close(o1, o2, rtol=1e-12, atol=1e-12)
    # shifting every score leaves the output unchanged and moves lse by g_h * c
    o3, l3 = oracle.gated_attention(q, k, v, s + 2.5, gain, temp, cu)
    torch.testing.assert_close(o3, out, rtol=1e-10, atol=1e-12)
    torch.testing.assert_close(l3, lse + 2.5 * gain[:, None], rtol=1e-12, atol=1e-10)
    # one dominant KEY: every later query row collapses onto its value
    big = s.clone()
    big[4] = 1e4
    o4, _ = oracle.gated_attention(q, k, v, big, gain, temp, cu)
    for h in range(Hq):
        torch.testing.assert_close(o4[4:, h], v[4, h // rep].expand(8, -1), rtol=0, atol=1e-12)
        torch.testing.assert_close(o4[:4, h], out[:4, h], rtol=0, atol=0)


def test_attention_rows_agree_with_full():
    q, k, v, s, gain, temp, cu = _attn_case(7)
    out, lse = oracle.gated_attention(q, k, v, s, gain, temp, cu)
    rows = [0, 4, 5, 6, 21, 22, 54]
    o_r, l_r = oracle.gated_attention_rows(q, k, v, s, gain, temp, cu, rows)
    torch.testing.assert_close(o_r, out[rows], rtol=1e-12, atol=1e-12)
    torch.testing.assert_close(l_r, lse[:, rows], rtol=1e-12, atol=1e-12)


# --------------------------------------------------------------- decode ----
def _decode_case(seed, lens=(1, 7, 40, 0, 13), Hq=6, Hkv=2, dh=16, gap=5):
    """Cache rows scattered through a pool: request b starts at row_off[b],
    with `gap` unused rows (random junk) between requests."""
    g = torch.Generator().manual_seed(seed)
    row_off, r = [], gap
    for n in lens:
        row_off.append(r)
        r += n + gap
    R = r
    q = torch.randn(len(lens), Hq, dh, generator=g, dtype=torch.float64)
    k = torch.randn(R, Hkv, dh, generator=g, dtype=torch.float64)
    v = torch.randn(R, Hkv, dh, generator=g, dtype=torch.float64)
    s = torch.randn(R, generator=g, dtype=torch.float64)
    gain = torch.rand(Hq, generator=g, dtype=torch.float64) + 0.5
    temp = torch.rand(Hq, generator=g, dtype=torch.float64) * 0.4 + 0.8
    return q, k, v, s, row_off, list(lens), gain, temp


def test_decode_matches_sdpa_with_mask():
    """Against torch SDPA: one query row, queries scaled by tau_h, float mask
    g_h s_j over the cached rows, no causal mask."""
    q, k, v, s, off, lens, gain, temp = _decode_case(31)
    out, lse = oracle.gated_decode_attention(q, k, v, s, off, lens, gain, temp)
    Hq, rep = q.shape[1], q.shape[1] // k.shape[1]
    for b, (lo, n) in enumerate(zip(off, lens)):
        if n == 0:
            continue
        Q = (q[b][:, None, :] * temp[:, None, None])[None]                       # [1][Hq][1][dh]
        K = k[lo:lo + n].permute(1, 0, 2).repeat_interleave(rep, dim=0)[None].contiguous()
        V = v[lo:lo + n].permute(1, 0, 2).repeat_interleave(rep, dim=0)[None].contiguous()
        mask = (gain[:, None] * s[lo:lo + n][None, :])[None, :, None, :]
        want = F.scaled_dot_product_attention(Q, K, V, attn_mask=mask)[0, :, 0]
        torch.testing.assert_close(out[b], want, rtol=1e-12, atol=1e-12)
        # lse through the probabilities (V = identity over the cached rows)
        P = F.scaled_dot_product_attention(Q, K, torch.eye(n, dtype=torch.float64).expand(1, Hq, n, n),
                                           attn_mask=mask)[0, :, 0]                # [Hq][n]
        l0 = temp * (q[b] @ k[lo].repeat_interleave(rep, dim=0).t()).diagonal() / math.sqrt(q.shape[2]) \
            + gain * s[lo]
        torch.testing.assert_close(lse[b], l0 - torch.log(P[:, 0]), rtol=1e-12, atol=1e-12)


def test_decode_is_the_last_prefill_row():
    """A cache holding a request's rows 0..r, queried with row r's q, gives
    row r of the prefill attention (output and lse)."""
    q, k, v, s, gain, temp, cu = _attn_case(32, lens=(29,))
    out, lse = oracle.gated_attention(q, k, v, s, gain, temp, cu)
    for r in (0, 1, 13, 28):
        o_d, l_d = oracle.gated_decode_attention(q[r:r + 1], k, v, s, [0], [r + 1], gain, temp)
        torch.testing.assert_close(o_d[0], out[r], rtol=1e-12, atol=1e-12)
        torch.testing.assert_close(l_d[0], lse[:, r], rtol=1e-12, atol=1e-12)


def test_decode_closed_forms_and_layout():
    q, k, v, s, off, lens, gain, temp = _decode_case(33)
    out, lse = oracle.gated_decode_attention(q, k, v, s, off, lens, gain, temp)
    Hq, dh, rep = q.shape[1], q.shape[2], q.shape[1] // k.shape[1]
    for h in range(Hq):      # a single cached row returns its value; lse is its logit
        assert torch.equal(out[0, h], v[off[0], h // rep])
        want = temp[h] * (q[0, h] @ k[off[0], h // rep]) / math.sqrt(dh) + gain[h] * s[off[0]]
        assert abs(float(lse[0, h] - want)) < 1e-12
    assert torch.equal(out[3], torch.zeros_like(out[3]))          # empty cache
    assert torch.isneginf(lse[3]).all()
    # the same rows packed back to back give the same result
    idx = torch.cat([torch.arange(lo, lo + n) for lo, n in zip(off, lens)])
    packed = [0]
    for n in lens[:-1]:
        packed.append(packed[-1] + n)
    o2, l2 = oracle.gated_decode_attention(q, k[idx], v[idx], s[idx], packed, lens, gain, temp)
    assert torch.equal(o2, out) and torch.equal(l2, lse)
    # constant scores: no dependence on the gain; a dominant key takes over
    c = torch.full_like(s, -0.8)
    o3, _ = oracle.gated_decode_attention(q, k, v, c, off, lens, gain, temp)
    o4, _ = oracle.gated_decode_attention(q, k, v, c, off, lens, gain * 4, temp)
    torch.testing.assert_close(o3, o4, rtol=1e-12, atol=1e-12)
    big = s.clone()
    big[off[2] + 17] = 1e4
    o5, _ = oracle.gated_decode_attention(q, k, v, big, off, lens, gain, temp)
    for h in range(Hq):
        torch.testing.assert_close(o5[2, h], v[off[2] + 17, h // rep], rtol=0, atol=1e-12)


# ---------------------------------------------------------------- stack ----
def test_stack_matches_independent_composition():
    g = torch.Generator().manual_seed(9)
    Kt, d, Hq, Hkv, dh = 23, 32, 4, 2, 8
    cu = [0, 10, 23]
    x = torch.randn(Kt, d, generator=g, dtype=torch.float64)
    s = torch.randn(Kt, generator=g, dtype=torch.float64)
    layers = []
    for _ in range(2):
        layers.append(dict(
            wq=torch.randn(Hq * dh, d, generator=g, dtype=torch.float64) / math.sqrt(d),
            wk=torch.randn(Hkv * dh, d, generator=g, dtype=torch.float64) / math.sqrt(d),
            wv=torch.randn(Hkv * dh, d, generator=g, dtype=torch.float64) / math.sqrt(d),
            wo=torch.randn(d, Hq * dh, generator=g, dtype=torch.float64) / math.sqrt(Hq * dh),
            gain=torch.rand(Hq, generator=g, dtype=torch.float64) + 0.5,
            temp=torch.rand(Hq, generator=g, dtype=torch.float64) * 0.4 + 0.8))
    got = oracle.stack_forward(x, s, layers, cu, Hq, Hkv, dh)
    want = x.clone()
    for L in layers:
        q = F.linear(want, L["wq"]).view(Kt, Hq, dh)
        k = F.linear(want, L["wk"]).view(Kt, Hkv, dh)
        v = F.linear(want, L["wv"]).view(Kt, Hkv, dh)
        a = _sdpa_reference(q, k, v, s, L["gain"], L["temp"], cu).reshape(Kt, Hq * dh)
        want = want + F.linear(a, L["wo"])
    torch.testing.assert_close(got, want, rtol=1e-10, atol=1e-10)


# ---------------------------------------------------------------- e2e ------
def test_needles_survive_reduced_haystack():
    """Planted needles (the 128k workload's construction) survive the oracle's
    gate + top-K on a shorter haystack of the same layer shape."""
    w = workloads.Workload("needles_16k", workloads.WORKLOADS["qwen3_1p7b_128k_niah"].shape,
                           [16384], [128], [1024], n_needles=64)
    inp = workloads.gate_inputs(w, seed=0)
    s = oracle.gate_score(inp["hidden"], inp["w1"], inp["b1"], inp["w2"], inp["b2"])
    kept, _ = oracle.topk_select(s, w.seq_len, w.q_len, w.budget)
    needles = set(workloads.needle_positions(w, 0).tolist())
    assert needles <= set(kept.tolist())


# ------------------------------------------------ rest of the pruned layer ----
def test_rms_norm_matches_torch_and_closed_form():
    g = torch.Generator().manual_seed(50)
    x = torch.randn(7, 3, 48, generator=g, dtype=torch.float64) * 3
    w = torch.randn(48, generator=g, dtype=torch.float64)
    want = F.rms_norm(x, (48,), weight=w, eps=1e-6)
    torch.testing.assert_close(oracle.rms_norm(x, w, 1e-6), want, rtol=1e-13, atol=1e-13)
    c = torch.full((2, 16), -2.5, dtype=torch.float64)          # constant row: c / sqrt(c^2 + eps)
    got = oracle.rms_norm(c, torch.ones(16, dtype=torch.float64), 0.25)
    torch.testing.assert_close(got, torch.full_like(c, -2.5 / math.sqrt(6.25 + 0.25)), rtol=1e-15, atol=0)


def test_rope_is_complex_rotation():
    """The pair (x_i, x_{i+dh/2}) as the complex number x_i + j x_{i+dh/2},
    multiplied by e^{j pos theta^(-2i/dh)}."""
    g = torch.Generator().manual_seed(51)
    M, H, dh, theta = 9, 3, 16, 10000.0
    x = torch.randn(M, H, dh, generator=g, dtype=torch.float64)
    pos = torch.tensor([0, 1, 2, 7, 100, 4095, 65536, 131071, 3], dtype=torch.int32)
    half = dh // 2
    inv = theta ** (-torch.arange(0, dh, 2, dtype=torch.float64) / dh)
    ang = pos.double()[:, None] * inv[None, :]
    z = torch.complex(x[..., :half], x[..., half:]) * torch.polar(torch.ones_like(ang), ang)[:, None, :]
    want = torch.cat([z.real, z.imag], dim=-1)
    torch.testing.assert_close(oracle.rope(x, pos, theta), want, rtol=1e-12, atol=1e-12)


def test_rope_invariants_and_hand_values():
    g = torch.Generator().manual_seed(52)
    x = torch.randn(6, 2, 32, generator=g, dtype=torch.float64)
    zero = torch.zeros(6, dtype=torch.int32)
    assert torch.equal(oracle.rope(x, zero, 1e6), x)                         # position 0: identity
    pos = torch.tensor([3, 17, 900, 5, 131000, 2], dtype=torch.int32)
    r = oracle.rope(x, pos, 1e6)
    torch.testing.assert_close(r.norm(dim=-1), x.norm(dim=-1), rtol=1e-13, atol=0)
    # only the offset between two positions matters for their dot product
    qv, kv = x[0:1], x[1:2]
    for m, n, t in ((5, 2, 11), (1000, 10, 12345), (7, 7, 3)):
        a = (oracle.rope(qv, torch.tensor([m]), 1e6) * oracle.rope(kv, torch.tensor([n]), 1e6)).sum()
        b = (oracle.rope(qv, torch.tensor([m + t]), 1e6) * oracle.rope(kv, torch.tensor([n + t]), 1e6)).sum()
        assert abs(float(a - b)) < 1e-10
    # dh = 4, theta = 100, position 1: angles 1 and 0.1 rad
    e = torch.eye(4, dtype=torch.float64)[:, None, :]
    out = oracle.rope(e, torch.ones(4, dtype=torch.int32), 100.0)[:, 0]
    want = torch.tensor([[math.cos(1), 0, math.sin(1), 0], [0, math.cos(0.1), 0, math.sin(0.1)],
                         [-math.sin(1), 0, math.cos(1), 0], [0, -math.sin(0.1), 0, math.cos(0.1)]],
                        dtype=torch.float64)
    torch.testing.assert_close(out, want, rtol=0, atol=1e-15)


def test_silu_and_swiglu_match_torch():
    g = torch.Generator().manual_seed(53)
    z = torch.randn(1000, generator=g, dtype=torch.float64) * 6
    torch.testing.assert_close(oracle.silu(z), F.silu(z), rtol=1e-14, atol=1e-15)
    assert float(oracle.silu(torch.zeros(1))) == 0.0
    x = torch.randn(5, 24, generator=g, dtype=torch.float64)
    wg, wu = torch.randn(40, 24, generator=g, dtype=torch.float64), torch.randn(40, 24, generator=g, dtype=torch.float64)
    wd = torch.randn(24, 40, generator=g, dtype=torch.float64)
    want = F.linear(F.silu(F.linear(x, wg)) * F.linear(x, wu), wd)
    torch.testing.assert_close(oracle.swiglu(x, wg, wu, wd), want, rtol=1e-12, atol=1e-12)


def test_kept_positions():
    seq, q, bud = [30, 1, 50], [5, 1, 10], [12, 1, 50]
    s = torch.randn(sum(seq), generator=torch.Generator().manual_seed(54))
    kept, cu_k = oracle.topk_select(s, seq, q, bud)
    cu_s = oracle.plan(seq, q, bud)[0]
    pos = oracle.kept_positions(kept, cu_s, cu_k)
    for b in range(3):
        p = pos[cu_k[b]:cu_k[b + 1]]
        assert (p >= 0).all() and (p < seq[b]).all()
        assert torch.equal(p + cu_s[b], kept[cu_k[b]:cu_k[b + 1]])
    assert pos[cu_k[2]:].tolist() == list(range(50))                        # all kept: 0..N-1
    assert pos[cu_k[0]:cu_k[1]][-5:].tolist() == list(range(25, 30))        # the question tail


def _layer_weights(g, d, Hq, Hkv, dh, F_):
    r = lambda *s: torch.randn(*s, generator=g, dtype=torch.float64)
    return dict(in_norm=1 + 0.1 * r(d), wq=r(Hq * dh, d) / math.sqrt(d), wk=r(Hkv * dh, d) / math.sqrt(d),
                wv=r(Hkv * dh, d) / math.sqrt(d), q_norm=1 + 0.1 * r(dh), k_norm=1 + 0.1 * r(dh),
                wo=r(d, Hq * dh) / math.sqrt(Hq * dh), gain=torch.rand(Hq, generator=g, dtype=torch.float64) + 0.5,
                temp=torch.rand(Hq, generator=g, dtype=torch.float64) * 0.4 + 0.8, post_norm=1 + 0.1 * r(d),
                wg=r(F_, d) / math.sqrt(d), wu=r(F_, d) / math.sqrt(d), wd=r(d, F_) / math.sqrt(F_))


def test_decoder_layer_matches_independent_composition():
    """torch's rms_norm, rotary embedding as complex multiplication, SDPA with
    tau-scaled queries and a float mask g_h s_j plus the causal mask, torch's
    silu: the same layer composed independently, in float64."""
    g = torch.Generator().manual_seed(55)
    d, Hq, Hkv, dh, F_, theta, eps = 32, 4, 2, 8, 48, 1e6, 1e-6
    cu = [0, 6, 19]
    Kt = cu[-1]
    L = _layer_weights(g, d, Hq, Hkv, dh, F_)
    x = torch.randn(Kt, d, generator=g, dtype=torch.float64)
    s = torch.randn(Kt, generator=g, dtype=torch.float64)
    pos = torch.tensor([0, 3, 4, 9, 10, 11] + [2, 5, 8, 13, 21, 34, 55, 89, 144, 233, 377, 610, 987],
                       dtype=torch.int32)
    got = oracle.decoder_layer(x, s, pos, cu, L, Hq, Hkv, dh, theta, eps)["out"]

    def rot(t):
        half = dh // 2
        inv = theta ** (-torch.arange(0, dh, 2, dtype=torch.float64) / dh)
        ang = pos.double()[:, None] * inv[None, :]
        z = torch.complex(t[..., :half], t[..., half:]) * torch.polar(torch.ones_like(ang), ang)[:, None, :]
        return torch.cat([z.real, z.imag], dim=-1)

    xn = F.rms_norm(x, (d,), weight=L["in_norm"], eps=eps)
    q = rot(F.rms_norm(F.linear(xn, L["wq"]).view(Kt, Hq, dh), (dh,), weight=L["q_norm"], eps=eps))
    k = rot(F.rms_norm(F.linear(xn, L["wk"]).view(Kt, Hkv, dh), (dh,), weight=L["k_norm"], eps=eps))
    v = F.linear(xn, L["wv"]).view(Kt, Hkv, dh)
    a = _sdpa_reference(q, k, v, s, L["gain"], L["temp"], cu).reshape(Kt, Hq * dh)
    h = x + F.linear(a, L["wo"])
    hn = F.rms_norm(h, (d,), weight=L["post_norm"], eps=eps)
    want = h + F.linear(F.silu(F.linear(hn, L["wg"])) * F.linear(hn, L["wu"]), L["wd"])
    torch.testing.assert_close(got, want, rtol=1e-11, atol=1e-11)


# -------------------------------------------------------- attention backward ----
def _autograd_grads(q, k, v, s, gain, temp, cu, dout):
    leaves = [t.clone().requires_grad_(True) for t in (q, k, v, s, gain, temp)]
    out, _ = oracle.gated_attention(*leaves, cu)
    (out * dout).sum().backward()
    return dict(zip(["dq", "dk", "dv", "ds", "dgain", "dtemp"], [t.grad for t in leaves]))


@pytest.mark.parametrize("seed,lens,Hq,Hkv", [(70, (5, 17, 33), 4, 2), (71, (1, 40), 6, 2), (72, (24,), 3, 3)])
def test_attention_backward_matches_autograd(seed, lens, Hq, Hkv):
    """Autograd through the forward definition (gated_attention is built from
    differentiable float64 torch ops) against the hand-derived backward."""
    q, k, v, s, gain, temp, cu = _attn_case(seed, lens=lens, Hq=Hq, Hkv=Hkv)
    dout = torch.randn(q.shape, generator=torch.Generator().manual_seed(seed + 100), dtype=torch.float64)
    got = oracle.gated_attention_backward(q, k, v, s, gain, temp, cu, dout)
    want = _autograd_grads(q, k, v, s, gain, temp, cu, dout)
    for name in want:
        torch.testing.assert_close(got[name], want[name], rtol=1e-10, atol=1e-11, msg=name)


def test_attention_backward_finite_differences():
    """Central differences of L = sum(dout * out) for a few entries of every
    input, independent of any autograd."""
    q, k, v, s, gain, temp, cu = _attn_case(73, lens=(9, 14), Hq=4, Hkv=2, dh=8)
    dout = torch.randn(q.shape, generator=torch.Generator().manual_seed(173), dtype=torch.float64)
    got = oracle.gated_attention_backward(q, k, v, s, gain, temp, cu, dout)
    args = dict(q=q, k=k, v=v, s=s, gain=gain, temp=temp)

    def loss(**kw):
        a = dict(args, **kw)
        out, _ = oracle.gated_attention(a["q"], a["k"], a["v"], a["s"], a["gain"], a["temp"], cu)
        return float((out * dout).sum())

    eps = 1e-6
    picks = {"q": [(3, 1, 2), (20, 3, 7)], "k": [(0, 0, 0), (12, 1, 5)], "v": [(8, 1, 3), (22, 0, 6)],
             "s": [(0,), (4,), (15,)], "gain": [(0,), (3,)], "temp": [(1,), (2,)]}
    for name, idxs in picks.items():
        for idx in idxs:
            plus, minus = args[name].clone(), args[name].clone()
            plus[idx] += eps
            minus[idx] -= eps
            fd = (loss(**{name: plus}) - loss(**{name: minus})) / (2 * eps)
            key = "d" + name
            assert abs(fd - float(got[key][idx])) < 1e-6 * max(1.0, abs(fd)), (name, idx, fd, float(got[key][idx]))


def test_attention_backward_special_cases():
    q, k, v, s, gain, temp, cu = _attn_case(74, lens=(10,))
    dout = torch.randn(q.shape, generator=torch.Generator().manual_seed(174), dtype=torch.float64)
    g0 = oracle.gated_attention_backward(q, k, v, s, gain, temp, cu, dout)
    # row 0 attends only to key 0: its softmax is constant, so it sends no gradient to q_0
    assert float(g0["dq"][0].abs().max()) < 1e-14
    # shifting every score leaves the output unchanged: the score gradients sum to zero
    assert abs(float(g0["ds"].sum())) < 1e-12
    # dout = 0 gives zero gradients everywhere
    gz = oracle.gated_attention_backward(q, k, v, s, gain, temp, cu, torch.zeros_like(dout))
    assert all(float(t.abs().max()) == 0.0 for t in gz.values())


def test_attention_backward_stored_output():
    """Given the exact output as the stored one, nothing changes; given a
    perturbed one, only the D_i term moves: dv is untouched."""
    q, k, v, s, gain, temp, cu = _attn_case(75, lens=(7, 12))
    dout = torch.randn(q.shape, generator=torch.Generator().manual_seed(175), dtype=torch.float64)
    out, _ = oracle.gated_attention(q, k, v, s, gain, temp, cu)
    a = oracle.gated_attention_backward(q, k, v, s, gain, temp, cu, dout)
    b = oracle.gated_attention_backward(q, k, v, s, gain, temp, cu, dout, out_stored=out)
    for n in a:
        assert torch.equal(a[n], b[n]), n
    c = oracle.gated_attention_backward(q, k, v, s, gain, temp, cu, dout, out_stored=out * 1.01)
    assert torch.equal(c["dv"], a["dv"]) and not torch.equal(c["dq"], a["dq"])


# -------------------------------------------------------------- gate backward ----
@pytest.mark.parametrize("with_bias", [True, False])
def test_gate_backward_matches_autograd(with_bias):
    """Autograd through gate_score's float64 definition (before its fp32
    rounding) against the hand-derived backward."""
    g = torch.Generator().manual_seed(90)
    T, d, dg = 13, 24, 10
    x = torch.randn(T, d, generator=g, dtype=torch.float64)
    w1 = torch.randn(dg, d, generator=g, dtype=torch.float64) / math.sqrt(d)
    b1 = torch.randn(dg, generator=g, dtype=torch.float64) if with_bias else None
    w2 = torch.randn(dg, generator=g, dtype=torch.float64)
    b2 = torch.randn(1, generator=g, dtype=torch.float64)
    ds = torch.randn(T, generator=g, dtype=torch.float64)
    leaves = [t.clone().requires_grad_(True) for t in (x, w1, w2, b2)] + \
        ([b1.clone().requires_grad_(True)] if with_bias else [])
    lx, lw1, lw2, lb2 = leaves[:4]
    lb1 = leaves[4] if with_bias else None
    z = lx @ lw1.t() + (lb1 if with_bias else 0.0)
    s = oracle.gelu_erf(z) @ lw2 + lb2
    (s * ds).sum().backward()
    got = oracle.gate_backward(x, w1, b1, w2, ds)
    torch.testing.assert_close(got["dhidden"], lx.grad, rtol=1e-12, atol=1e-12)
    torch.testing.assert_close(got["dw1"], lw1.grad, rtol=1e-12, atol=1e-12)
    torch.testing.assert_close(got["dw2"], lw2.grad, rtol=1e-12, atol=1e-12)
    torch.testing.assert_close(got["db2"], lb2.grad, rtol=1e-12, atol=1e-12)
    if with_bias:
        torch.testing.assert_close(got["db1"], lb1.grad, rtol=1e-12, atol=1e-12)


def test_gate_backward_finite_differences_and_cases():
    g = torch.Generator().manual_seed(91)
    T, d, dg = 6, 8, 5
    x = torch.randn(T, d, generator=g, dtype=torch.float64)
    w1 = torch.randn(dg, d, generator=g, dtype=torch.float64)
    b1 = torch.randn(dg, generator=g, dtype=torch.float64)
    w2 = torch.randn(dg, generator=g, dtype=torch.float64)
    ds = torch.randn(T, generator=g, dtype=torch.float64)
    got = oracle.gate_backward(x, w1, b1, w2, ds)

    def loss(x=x, w1=w1, b1=b1, w2=w2):
        z = x @ w1.t() + b1
        return float((0.5 * z * (1 + torch.erf(z / math.sqrt(2))) @ w2 * ds).sum())

    eps = 1e-6
    for name, t, idx in (("dhidden", x, (2, 3)), ("dw1", w1, (4, 1)), ("db1", b1, (0,)), ("dw2", w2, (3,))):
        plus, minus = t.clone(), t.clone()
        plus[idx] += eps
        minus[idx] -= eps
        key = {"dhidden": "x", "dw1": "w1", "db1": "b1", "dw2": "w2"}[name]
        fd = (loss(**{key: plus}) - loss(**{key: minus})) / (2 * eps)
        assert abs(fd - float(got[name][idx])) < 1e-6 * max(1.0, abs(fd)), (name, fd)
    assert float(got["db2"]) == float(ds.sum())
    zero = oracle.gate_backward(x, w1, b1, w2, torch.zeros(T, dtype=torch.float64))
    assert all(float(v.abs().max()) == 0.0 for v in zero.values())
    # GELU'(0) = 1/2: with W1 = 0 and no bias, dz = ds * w2 / 2
    z0 = oracle.gate_backward(x, torch.zeros(dg, d, dtype=torch.float64), None, w2, ds)
    torch.testing.assert_close(z0["db1"], 0.5 * ds.sum() * w2, rtol=1e-14, atol=1e-14)
