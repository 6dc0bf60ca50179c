"""GPU parity of the gate MLP backward against the oracle.

Inputs are the gathered kept rows, the gate weights and a score gradient;
the oracle evaluates the backward in float64 from the same stored values.
The products accumulate in fp32 from values rounded once to the storage
dtype (z, dz), so each element is held to the bf16 (2e-2 relative / 1e-2
absolute) or fp32 (1e-5) tolerance plus 2^-8 (bf16) or 2^-20 (fp32) times
the sum of the absolute values of its terms, and every tensor normwise to
1e-2 (bf16) or 1e-5 (fp32).
"""
import math

import pytest
import torch

import learned_token_pruning_02_amd as tg
import oracle
from parity_util import announce, tol

pytestmark = pytest.mark.gpu


def _case(Kt, d, dg, dtype, seed, bias=True):
    g = torch.Generator().manual_seed(seed)
    x = torch.randn(Kt, d, generator=g).to(dtype)
    w1 = (torch.randn(dg, d, generator=g) / math.sqrt(d)).to(dtype)
    b1 = (torch.randn(dg, generator=g) / math.sqrt(d)).to(dtype) if bias else None
    w2 = (torch.randn(dg, generator=g) / math.sqrt(dg)).to(dtype)
    ds = torch.randn(Kt, generator=g) * 0.3
    return x, w1, b1, w2, ds


def _scales(x, w1, b1, w2, ds):
    z = x.double() @ w1.double().t() + (0.0 if b1 is None else b1.double())
    phi = torch.exp(-0.5 * z * z) / math.sqrt(2 * math.pi)
    Phi = 0.5 * (1 + torch.erf(z / math.sqrt(2)))
    adz = (ds.double()[:, None] * w2.double()[None, :] * (Phi + z * phi)).abs()
    return {"dhidden": adz @ w1.double().abs(), "dw1": adz.t() @ x.double().abs(), "db1": adz.sum(0),
            "dw2": (z * Phi).abs().t() @ ds.double().abs(), "db2": ds.double().abs().sum().reshape(1)}


def _run_check(x, w1, b1, w2, ds, what):
    c = lambda t: None if t is None else t.cuda()
    got = tg.tg_gate_backward(c(x), c(w1), c(b1), c(w2), c(ds))
    torch.cuda.synchronize()
    ref = oracle.gate_backward(x, w1, b1, w2, ds)
    sc = _scales(x, w1, b1, w2, ds)
    rt, at = tol(x.dtype)
    k, nrm = (2.0 ** -8, 1e-2) if x.dtype == torch.bfloat16 else (2.0 ** -20, 1e-5)
    for n in ("dhidden", "dw1", "db1", "dw2", "db2"):
        if got[n] is None:
            continue
        gv = got[n].cpu().double()
        assert torch.isfinite(gv).all(), f"{what} {n}"
        err = (gv - ref[n]).abs()
        bound = at + rt * ref[n].abs() + k * sc[n]
        ratio = err / bound
        assert (ratio <= 1).all(), (f"{what} {n}", int((ratio > 1).sum()), float(ratio.max()))
        rn = float(ref[n].norm())
        if rn > 0:
            assert float((gv - ref[n]).norm()) <= nrm * rn, (f"{what} {n} normwise",
                                                            float((gv - ref[n]).norm()) / rn)


CASES = [
    ("bf16_ragged", 777, 2048, 256, torch.bfloat16, True),
    ("bf16_nobias", 64, 512, 128, torch.bfloat16, False),
    ("bf16_six_slices", 3001, 1024, 192, torch.bfloat16, True),
    ("bf16_one_row", 1, 128, 64, torch.bfloat16, True),
    ("f32_small", 300, 256, 64, torch.float32, True),
]


@pytest.mark.parametrize("name,Kt,d,dg,dtype,bias", CASES, ids=[c[0] for c in CASES])
def test_gate_backward_parity(name, Kt, d, dg, dtype, bias):
    announce(f"gate backward {name} Kt={Kt} d={d} dg={dg}")
    _run_check(*_case(Kt, d, dg, dtype, seed=95, bias=bias), name)


def test_gate_backward_full_size():
    """The 8192 kept rows of the pruned 128k prompt, gate 2048 -> 256 -> 1."""
    announce("gate backward full size Kt=8192")
    _run_check(*_case(8192, 2048, 256, torch.bfloat16, seed=96), "full size")
