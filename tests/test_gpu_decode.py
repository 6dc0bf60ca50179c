"""GPU parity of the token-gated decode attention against the oracle.

Output and lse within the bf16 (2e-2 relative / 1e-2 absolute) or fp32 (1e-5)
tolerance, on identical cached rows.  Covers every query-group size the
kernel instantiates (1, 2, 4, 8 and a padded 3), both head sizes, chunk
boundaries (127/128/129 rows), empty caches, lengths clamped by max_len, rows
outside the pool, the full-size 32-request workload, and replays of a
captured HIP graph whose cache lengths change between replays.
"""
import pytest
import torch

import learned_token_pruning_02_amd as tg
import oracle
import workloads
from parity_util import announce, assert_within, tol

pytestmark = pytest.mark.gpu


def _shape(hq, hkv, dh, dtype):
    return workloads.LayerShape(d_model=hq * dh, n_q_heads=hq, n_kv_heads=hkv, d_head=dh,
                                d_gate=64, dtype=dtype)


def _gpu(inp, max_len, cache_len=None, row_off=None):
    dev = {k: (v.cuda() if isinstance(v, torch.Tensor) else v) for k, v in inp.items()}
    if cache_len is not None:
        dev["cache_len"] = torch.tensor(cache_len, dtype=torch.int32, device="cuda")
    if row_off is not None:
        dev["row_off"] = torch.tensor(row_off, dtype=torch.int64, device="cuda")
    out, lse = tg.tg_gated_attn_decode(dev["q"], dev["k"], dev["v"], dev["s"], dev["row_off"],
                                       dev["cache_len"], dev["gain"], dev["temp"], max_len,
                                       want_lse=True)
    torch.cuda.synchronize()
    return out.cpu(), lse.cpu()


def _ref(inp, row_off=None, lens=None):
    row_off = inp["row_off"].tolist() if row_off is None else row_off
    lens = inp["cache_len"].tolist() if lens is None else lens
    Hq = inp["q"].shape[1]
    s = inp["s"] if inp["s"] is not None else torch.zeros(inp["k"].shape[0])
    gain = inp["gain"] if inp["gain"] is not None else torch.zeros(Hq)
    return oracle.gated_decode_attention(inp["q"], inp["k"], inp["v"], s, row_off, lens, gain,
                                         inp["temp"])


def _check(out, lse, ref, ref_lse, dtype, what):
    rtol, atol = tol(dtype)
    assert_within(out, ref, rtol, atol, f"{what} out")
    fin = torch.isfinite(ref_lse)
    assert torch.equal(torch.isfinite(lse), fin), f"{what}: lse finiteness differs"
    assert torch.equal(lse[~fin], ref_lse[~fin].float()), f"{what}: empty-cache lse"
    assert_within(lse[fin], ref_lse[fin], rtol, atol, f"{what} lse")


CASES = [
    # name, dtype, Hq, Hkv, dh, cache lengths, gap rows, bias
    ("bf16_g2_dh128_varlen", torch.bfloat16, 16, 8, 128, [1, 127, 128, 129, 3000, 257], 3, True),
    ("bf16_g4_dh64", torch.bfloat16, 8, 2, 64, [5, 300, 1000], 0, True),
    ("bf16_g1_dh128_nobias", torch.bfloat16, 4, 4, 128, [200, 33], 1, False),
    ("bf16_g8_dh128", torch.bfloat16, 16, 2, 128, [513, 64], 2, True),
    ("bf16_g3_dh64", torch.bfloat16, 6, 2, 64, [100, 250], 7, True),
    ("f32_g2_dh128", torch.float32, 4, 2, 128, [1, 129, 700], 2, True),
    ("f32_g8_dh64", torch.float32, 8, 1, 64, [300, 31], 0, True),
    ("f32_g3_dh128_nobias", torch.float32, 3, 1, 128, [256, 5], 4, False),
]


@pytest.mark.parametrize("name,dtype,hq,hkv,dh,lens,gap,bias", CASES, ids=[c[0] for c in CASES])
def test_decode_parity(name, dtype, hq, hkv, dh, lens, gap, bias):
    announce(f"decode {name} lens={lens}")
    inp = workloads.decode_inputs(_shape(hq, hkv, dh, dtype), lens, seed=40, gap=gap, with_bias=bias)
    out, lse = _gpu(inp, max(lens))
    ref, ref_lse = _ref(inp)
    _check(out, lse, ref, ref_lse, dtype, name)


def test_decode_edges():
    """Empty caches, max_len below a cache length, rows outside the pool on
    either side, and max_len == 0."""
    lens = [0, 300, 40, 129, 64]
    inp = workloads.decode_inputs(_shape(16, 8, 128, torch.bfloat16), lens, seed=41, gap=2)
    R = inp["k"].shape[0]
    off = inp["row_off"].tolist()
    announce(f"decode edges R={R} off={off}")
    # request 1 clamped to max_len 200; request 3 runs 10 rows past the pool's
    # end; request 4 starts 20 rows before row 0.
    row_off = [off[0], off[1], off[2], R - 119, -20]
    got, got_lse = _gpu(inp, 200, row_off=row_off)
    ref, ref_lse = _ref(inp, row_off=[off[0], off[1], off[2], R - 119, 0],
                        lens=[0, 200, 40, 119, 44])
    _check(got, got_lse, ref, ref_lse, torch.bfloat16, "edges")
    assert torch.equal(got[0], torch.zeros_like(got[0]))
    got0, lse0 = _gpu(inp, 0)
    assert torch.equal(got0, torch.zeros_like(got0)) and torch.isneginf(lse0).all()


def test_decode_full_workload():
    """The 32-request decode step over 8193 cached rows each (the kept cache
    of a pruned 128k prefill), every output against the oracle."""
    w = workloads.DECODE_WORKLOADS["qwen3_1p7b_128k_decode_b32"]
    announce(f"decode {w.name}")
    inp = workloads.decode_inputs(w.shape, w.cache_len, seed=42)
    out, lse = _gpu(inp, max(w.cache_len))
    ref, ref_lse = _ref(inp)
    _check(out, lse, ref, ref_lse, torch.bfloat16, w.name)


def test_decode_graph_replay_with_growing_cache():
    """Captured once, replayed as the caches grow: lengths live on the device,
    so each replay sees the new lengths; every replay matches an eager call."""
    lens = [700, 100, 1500]
    cap = 1600
    inp = workloads.decode_inputs(_shape(16, 8, 128, torch.bfloat16), [cap] * 3, seed=43)
    dev = {k: v.cuda() for k, v in inp.items()}
    cur = torch.tensor(lens, dtype=torch.int32, device="cuda")
    out = torch.empty_like(dev["q"])
    lse = torch.empty(3, 16, dtype=torch.float32, device="cuda")
    ws = torch.empty(tg.tg_decode_plan(3, 16, 128, cap), dtype=torch.uint8, device="cuda")
    args = (dev["q"], dev["k"], dev["v"], dev["s"], dev["row_off"], cur, dev["gain"], dev["temp"],
            cap)
    announce("decode graph capture")
    tg.tg_gated_attn_decode(*args, out=out, lse=lse, workspace=ws)  # warm-up outside capture
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        tg.tg_gated_attn_decode(*args, out=out, lse=lse, workspace=ws)
    torch.cuda.synchronize()
    for step in range(4):
        new = [min(cap, n + 37 * step) for n in lens]
        cur.copy_(torch.tensor(new, dtype=torch.int32))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got, got_lse = out.cpu(), lse.cpu()
        eo, el = tg.tg_gated_attn_decode(*args, want_lse=True)
        torch.cuda.synchronize()
        assert torch.equal(got, eo.cpu()) and torch.equal(got_lse, el.cpu()), f"replay {step}"
        if step in (0, 3):
            ref, ref_lse = _ref(inp, lens=new)
            _check(got, got_lse, ref, ref_lse, torch.bfloat16, f"replay {step}")
