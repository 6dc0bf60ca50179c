"""GPU parity of the token-gated attention backward against the oracle.

The entry point takes the forward's output and lse as inputs; here both come
from the oracle's forward (out rounded to bf16 as a forward would store it,
lse to fp32) and go to both sides, with the same bf16 q, k, v and upstream
gradient; the oracle evaluates D_i = dO_i . O_i on that stored output, as
the entry point defines it.  dq, dk, dv: P and dL enter the
matrix cores rounded to bf16 (relative error <= 2^-9 per term), and dv_j, for
instance, sums P_ij dO_i over every later query, which for a key with a high
score can be tens while the signed sum nearly cancels.  So each element is
held to the bf16 tolerance (2e-2 relative / 1e-2 absolute) plus 2^-8 times
the sum of the absolute values of its terms (twice the rounding bound).
ds, dgain and dtemp
are fp32 sums of terms that cancel (each row of dL sums to zero), so their
error is measured against the scale of the terms: |got - ref| <= 1e-4 *
(sum of |terms|) + 2e-2 |ref|; 1e-4 covers fp32 rounding of the logits (|S|
up to ~50) and of sums over up to 8192 terms with a wide margin.  A term
dL_ij = P_ij (dP_ij - D_i) is itself a difference, so its scale is
P_ij (|dP_ij| + |D_i|).
"""
import pytest
import torch

import learned_token_pruning_02_amd as tg
import oracle
from parity_util import announce, tol

pytestmark = pytest.mark.gpu


def _case(lens, hq, hkv, dh, seed, bias=True):
    g = torch.Generator().manual_seed(seed)
    Kt = sum(lens)
    cu = [0]
    for n in lens:
        cu.append(cu[-1] + n)
    r = lambda *s: torch.randn(*s, generator=g).to(torch.bfloat16)
    q, k, v = r(Kt, hq, dh), r(Kt, hkv, dh), r(Kt, hkv, dh)
    dout = r(Kt, hq, dh)
    s = torch.randn(Kt, generator=g) if bias else None
    gain = (torch.rand(hq, generator=g) + 0.5) if bias else None
    temp = torch.rand(hq, generator=g) * 0.4 + 0.8
    return q, k, v, s, gain, temp, dout, cu


def _forward_inputs(q, k, v, s, gain, temp, cu):
    """The stored forward output (bf16) and lse (fp32) from the oracle."""
    z = torch.zeros(cu[-1]) if s is None else s
    gn = torch.zeros(q.shape[1]) if gain is None else gain
    out, lse = oracle.gated_attention(q, k, v, z, gn, temp, cu)
    return out.to(torch.bfloat16), lse.float()


def _gpu(q, k, v, s, gain, temp, out, lse, dout, cu):
    c = lambda t: None if t is None else t.cuda()
    gr = tg.tg_gated_attn_backward(c(q), c(k), c(v), c(s), c(gain), c(temp), c(out), c(lse),
                                   c(dout), cu)
    torch.cuda.synchronize()
    return {n: (None if t is None else t.cpu()) for n, t in gr.items()}


def _term_scales(q, k, v, s, gain, temp, dout, cu, out_stored):
    """Sums of |terms| of every gradient (float64), the scale their rounding
    error is measured against."""
    Kt, Hq, dh = q.shape
    Hkv = k.shape[1]
    G = Hq // Hkv
    z = torch.zeros(Kt, dtype=torch.float64) if s is None else s.double()
    gn = torch.zeros(Hq) if gain is None else gain
    out, lse = oracle.gated_attention(q, k, v, z, gn, temp, cu)
    ds_sc = torch.zeros(Kt, dtype=torch.float64)
    dg_sc = torch.zeros(Hq, dtype=torch.float64)
    dt_sc = torch.zeros(Hq, dtype=torch.float64)
    dq_sc = torch.zeros(Kt, Hq, dh, dtype=torch.float64)
    dk_sc = torch.zeros(Kt, Hkv, dh, dtype=torch.float64)
    dv_sc = torch.zeros(Kt, Hkv, dh, dtype=torch.float64)
    for b in range(len(cu) - 1):
        lo, hi = cu[b], cu[b + 1]
        n = hi - lo
        fut = torch.ones(n, n, dtype=torch.bool).triu(1)
        for h in range(Hq):
            Q, K, V = q[lo:hi, h].double(), k[lo:hi, h // G].double(), v[lo:hi, h // G].double()
            r = Q @ K.t() / dh ** 0.5
            P = torch.exp(float(temp[h]) * r + float(gn[h]) * z[lo:hi][None, :] - lse[h, lo:hi][:, None])
            P = P.masked_fill(fut, 0.0)
            dO = dout[lo:hi, h].double()
            # dL = P (dP - D) is a difference: its rounding scale is P (|dP| + |D|)
            dL = P * ((dO @ V.t()).abs() + (dO * out_stored[lo:hi, h].double()).sum(1).abs()[:, None])
            ds_sc[lo:hi] += abs(float(gn[h])) * dL.sum(0)
            dg_sc[h] += (dL * z[lo:hi].abs()[None, :]).sum()
            dt_sc[h] += (dL * r.abs()).sum()
            c = float(temp[h]) / dh ** 0.5
            dq_sc[lo:hi, h] = c * (dL @ K.abs())
            dk_sc[lo:hi, h // G] += c * (dL.t() @ Q.abs())
            dv_sc[lo:hi, h // G] += P.t() @ dO.abs()
    return {"dq": dq_sc, "dk": dk_sc, "dv": dv_sc, "ds": ds_sc, "dgain": dg_sc, "dtemp": dt_sc}


def _check(got, ref, scales, what):
    rt, at = tol(torch.bfloat16)
    for n in ("dq", "dk", "dv", "ds", "dgain", "dtemp"):
        if got[n] is None:
            continue
        g = got[n].double()
        assert torch.isfinite(g).all(), f"{what} {n}: non-finite"
        err = (g - ref[n]).abs()
        if n in ("dq", "dk", "dv"):
            bound = at + rt * ref[n].abs() + 2.0 ** -8 * scales[n]
        else:
            bound = 1e-4 * scales[n] + rt * ref[n].abs() + 1e-6
        ratio = err / bound
        assert (ratio <= 1).all(), (f"{what} {n}", int((ratio > 1).sum()), float(ratio.max()))
        # normwise: a systematic error (a lost factor, a wrong head) moves the
        # whole tensor, independent rounding errors do not
        rn = float(ref[n].norm())
        if rn > 0:
            assert float((g - ref[n]).norm()) <= 1e-2 * rn, (f"{what} {n} normwise",
                                                             float((g - ref[n]).norm()) / rn)


CASES = [
    ("tiny_mixed", (5, 17, 33), 4, 2, 64, True),
    ("ragged_dh128", (1, 100, 257), 16, 8, 128, True),
    ("g1_nobias", (130, 64), 4, 4, 128, False),
    ("g4_dh64", (300,), 8, 2, 64, True),
    ("g3_odd_steps", (77, 200), 6, 2, 128, True),
    ("qwen_2k", (2048,), 16, 8, 128, True),
]


@pytest.mark.parametrize("name,lens,hq,hkv,dh,bias", CASES, ids=[c[0] for c in CASES])
def test_attention_backward_parity(name, lens, hq, hkv, dh, bias):
    announce(f"attn backward {name} lens={lens} heads={hq}/{hkv} dh={dh}")
    q, k, v, s, gain, temp, dout, cu = _case(lens, hq, hkv, dh, seed=80, bias=bias)
    out, lse = _forward_inputs(q, k, v, s, gain, temp, cu)
    got = _gpu(q, k, v, s, gain, temp, out, lse, dout, cu)
    z = torch.zeros(cu[-1]) if s is None else s
    gn = torch.zeros(hq) if gain is None else gain
    ref = oracle.gated_attention_backward(q, k, v, z, gn, temp, cu, dout, out_stored=out)
    _check(got, ref, _term_scales(q, k, v, s, gain, temp, dout, cu, out), name)


def test_attention_backward_full_size_one_group():
    """The 8192 kept rows of the pruned 128k prompt in the full launch
    configuration (16/8 heads x 128).  Gains are zero outside query heads 0
    and 1 (KV head 0), so ds comes from that group alone; every gradient of
    that group is checked against the oracle run on the group's slice."""
    Kt, hq, hkv, dh = 8192, 16, 8, 128
    q, k, v, s, gain, temp, dout, cu = _case((Kt,), hq, hkv, dh, seed=82)
    gain[2:] = 0.0
    announce(f"attn backward full size Kt={Kt}")
    sl = lambda t, n: t[:, :n].contiguous()
    q2, k1, v1, do2 = sl(q, 2), sl(k, 1), sl(v, 1), sl(dout, 2)
    out2, lse2 = _forward_inputs(q2, k1, v1, s, gain[:2], temp[:2], cu)
    out = torch.zeros(Kt, hq, dh, dtype=torch.bfloat16)
    lse = torch.zeros(hq, Kt)
    out[:, :2] = out2
    lse[:2] = lse2
    got = _gpu(q, k, v, s, gain, temp, out, lse, dout, cu)
    ref = oracle.gated_attention_backward(q2, k1, v1, s, gain[:2], temp[:2], cu, do2, out_stored=out2)
    mine = {"dq": got["dq"][:, :2], "dk": got["dk"][:, :1], "dv": got["dv"][:, :1], "ds": got["ds"],
            "dgain": got["dgain"][:2], "dtemp": got["dtemp"][:2]}
    _check(mine, ref, _term_scales(q2, k1, v1, s, gain[:2], temp[:2], do2, cu, out2), "full size")


def test_attention_backward_deterministic():
    q, k, v, s, gain, temp, dout, cu = _case((700, 300), 16, 8, 128, seed=81)
    announce("attn backward determinism")
    out, lse = _forward_inputs(q, k, v, s, gain, temp, cu)
    a = _gpu(q, k, v, s, gain, temp, out, lse, dout, cu)
    b = _gpu(q, k, v, s, gain, temp, out, lse, dout, cu)
    for n in a:
        assert torch.equal(a[n], b[n]), n
