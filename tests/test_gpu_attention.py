"""GPU parity of token-gated attention (and the projection GEMM) against the oracle.

Attention outputs and log-sum-exps: within 1e-5 (fp32) or 2e-2 relative /
1e-2 absolute (bf16) of the oracle's float64 result on the same stored
inputs.  Full-size layers are checked on sampled rows.
"""
import zlib

import pytest
import torch

import learned_token_pruning_02_amd as tg
import oracle
import workloads
from parity_util import announce, assert_within, tol

pytestmark = pytest.mark.gpu


def _inputs(lens, Hq, Hkv, dh, dtype, seed, s_scale=1.0):
    g = torch.Generator().manual_seed(seed)
    Kt = sum(lens)
    cu = [0]
    for n in lens:
        cu.append(cu[-1] + n)
    q = torch.randn(Kt, Hq, dh, generator=g).to(dtype)
    k = torch.randn(Kt, Hkv, dh, generator=g).to(dtype)
    v = torch.randn(Kt, Hkv, dh, generator=g).to(dtype)
    s = torch.randn(Kt, generator=g) * s_scale
    gain = torch.rand(Hq, generator=g) + 0.5
    temp = torch.rand(Hq, generator=g) * 0.4 + 0.8
    return q, k, v, s, gain, temp, cu


def _run(q, k, v, s, gain, temp, cu):
    out, lse = tg.tg_gated_attn_prefill(q.cuda(), k.cuda(), v.cuda(), s.cuda(), gain.cuda(),
                                        temp.cuda(), cu, want_lse=True)
    torch.cuda.synchronize()
    return out.cpu(), lse.cpu()


CASES = [
    ("fp32_tiny", [128], 4, 2, 64, torch.float32),
    ("fp32_varlen", [1, 5, 64, 130], 2, 1, 128, torch.float32),
    ("bf16_qwen_heads_varlen", [1, 37, 200, 700], 16, 8, 128, torch.bfloat16),
    ("bf16_dh64_pairs", [129, 64, 63], 4, 2, 64, torch.bfloat16),
    ("bf16_group4", [300], 8, 2, 128, torch.bfloat16),
    ("bf16_mha", [150, 90], 3, 3, 64, torch.bfloat16),
    ("bf16_16k_layer_kept", [2048], 16, 8, 128, torch.bfloat16),
]


@pytest.mark.parametrize("name,lens,Hq,Hkv,dh,dtype", CASES, ids=[c[0] for c in CASES])
def test_attention_parity(name, lens, Hq, Hkv, dh, dtype):
    announce(f"attn {name} lens={lens} Hq={Hq} Hkv={Hkv} dh={dh}")
    q, k, v, s, gain, temp, cu = _inputs(lens, Hq, Hkv, dh, dtype, seed=zlib.crc32(name.encode()) % 1000)
    out, lse = _run(q, k, v, s, gain, temp, cu)
    ref, ref_lse = oracle.gated_attention(q, k, v, s, gain, temp, cu)
    rtol, atol = tol(dtype)
    assert_within(out, ref, rtol, atol, f"{name} out")
    assert_within(lse, ref_lse, rtol, atol, f"{name} lse")


@pytest.mark.parametrize("lens,Hq,Hkv,dh,dtype", [
    ([0, 100, 0, 700, 0], 16, 8, 128, torch.bfloat16),   # empty requests around ragged ones
    ([0, 0, 65], 4, 2, 64, torch.bfloat16),
    ([0, 33, 0], 4, 2, 64, torch.float32),
    ([1] * 64, 16, 8, 128, torch.bfloat16),               # the largest batch of one-row requests
])
def test_attention_empty_and_tiny_requests(lens, Hq, Hkv, dh, dtype):
    """Requests with no kept rows inside a batch take no work and leave the
    other requests' rows exact; one-row requests attend only to themselves."""
    announce(f"attn empty/tiny lens={lens[:6]} Hq={Hq} Hkv={Hkv} dh={dh} {dtype}")
    q, k, v, s, gain, temp, cu = _inputs(lens, Hq, Hkv, dh, dtype, seed=41)
    out, lse = _run(q, k, v, s, gain, temp, cu)
    ref, ref_lse = oracle.gated_attention(q, k, v, s, gain, temp, cu)
    rtol, atol = tol(dtype)
    assert_within(out, ref, rtol, atol, "empty/tiny out")
    assert_within(lse, ref_lse, rtol, atol, "empty/tiny lse")
    if all(n == 1 for n in lens):
        # a lone key: the output is its value row, the lse its logit
        vv = v.float().repeat_interleave(Hq // Hkv, dim=1)
        assert_within(out.float(), vv, rtol, atol, "one-row requests")


def test_attention_gain0_temp1_is_plain_causal():
    q, k, v, s, _, _, cu = _inputs([333, 77], 16, 8, 128, torch.bfloat16, seed=21)
    Hq = q.shape[1]
    gain, temp = torch.zeros(Hq), torch.ones(Hq)
    out, _ = _run(q, k, v, s, gain, temp, cu)
    ref, _ = oracle.gated_attention(q, k, v, torch.zeros_like(s), gain, temp, cu)
    assert_within(out, ref, 2e-2, 1e-2, "gain0/temp1")


@pytest.mark.parametrize("lens,Hq,Hkv,dh", [([333, 77], 16, 8, 128), ([8192], 16, 8, 128), ([200, 129], 4, 2, 64)])
def test_attention_without_bias(lens, Hq, Hkv, dh):
    """s_kept = gain = NULL: the bias-free build equals the definition with a
    zero bias (checked on sampled rows for the larger case)."""
    announce(f"attn no-bias lens={lens} Hq={Hq} Hkv={Hkv} dh={dh}")
    q, k, v, s, gain, temp, cu = _inputs(lens, Hq, Hkv, dh, torch.bfloat16, seed=31)
    out, lse = tg.tg_gated_attn_prefill(q.cuda(), k.cuda(), v.cuda(), None, None, temp.cuda(), cu,
                                        want_lse=True)
    out, lse = out.cpu(), lse.cpu()
    zero = torch.zeros_like(s)
    if sum(lens) > 4096:
        rows = _sampled_rows(cu, 16, seed=7)
        ref, ref_lse = oracle.gated_attention_rows(q, k, v, zero, gain, temp, cu, rows)
        out, lse = out[rows], lse[:, rows]
    else:
        ref, ref_lse = oracle.gated_attention(q, k, v, zero, gain, temp, cu)
    assert_within(out, ref, 2e-2, 1e-2, "no-bias out")
    assert_within(lse, ref_lse, 2e-2, 1e-2, "no-bias lse")


def test_attention_fp32_without_bias():
    q, k, v, s, gain, temp, cu = _inputs([100, 30], 4, 2, 64, torch.float32, seed=32)
    out, lse = tg.tg_gated_attn_prefill(q.cuda(), k.cuda(), v.cuda(), None, None, temp.cuda(), cu,
                                        want_lse=True)
    ref, ref_lse = oracle.gated_attention(q, k, v, torch.zeros_like(s), gain, temp, cu)
    assert_within(out.cpu(), ref, 1e-5, 1e-5, "fp32 no-bias out")
    assert_within(lse.cpu(), ref_lse, 1e-5, 1e-5, "fp32 no-bias lse")


def test_attention_large_bias_range():
    """Scores spread over +-40: the bias dominates the logits."""
    q, k, v, s, gain, temp, cu = _inputs([513], 16, 8, 128, torch.bfloat16, seed=22, s_scale=20.0)
    out, lse = _run(q, k, v, s, gain, temp, cu)
    ref, ref_lse = oracle.gated_attention(q, k, v, s, gain, temp, cu)
    assert_within(out, ref, 2e-2, 1e-2, "large bias out")
    assert_within(lse, ref_lse, 2e-2, 1e-2, "large bias lse")


def _score_pattern(kind, Kt, g):
    """Gate scores that move a row's exponent base: a step far above the
    base (past the limit of the optimistic exponentials), a steady climb
    (the base moves on most tiles), a first tile far below the rest, and a
    descent (the base never moves)."""
    j = torch.arange(Kt, dtype=torch.float32)
    if kind == "step_up":
        return torch.where(j % 700 >= 200, 100.0, 0.0) + torch.randn(Kt, generator=g)
    if kind == "climb":
        return 0.4 * (j % 700) + torch.randn(Kt, generator=g)
    if kind == "low_first_tile":
        return torch.where(j % 700 < 64, -400.0, 0.0) + torch.randn(Kt, generator=g)
    if kind == "descent":
        return -0.4 * (j % 700) + torch.randn(Kt, generator=g)
    raise ValueError(kind)


BASE_KINDS = ["step_up", "climb", "low_first_tile", "descent"]


@pytest.mark.parametrize("kind", BASE_KINDS)
def test_attention_base_moves(kind):
    """Rows whose logits jump, climb or start far below the rest, in the
    four-wave kernel (all rows) and the eight-wave kernel (sampled rows)."""
    announce(f"attn base moves {kind}")
    q, k, v, _, gain, temp, cu = _inputs([700, 130], 16, 8, 128, torch.bfloat16, seed=31)
    s = _score_pattern(kind, cu[-1], torch.Generator().manual_seed(32))
    out, lse = _run(q, k, v, s, gain, temp, cu)
    ref, ref_lse = oracle.gated_attention(q, k, v, s, gain, temp, cu)
    assert_within(out, ref, 2e-2, 1e-2, f"{kind} out")
    assert_within(lse, ref_lse, 2e-2, 1e-2, f"{kind} lse")

    q, k, v, _, gain, temp, cu = _inputs([8192], 16, 8, 128, torch.bfloat16, seed=33)
    s = _score_pattern(kind, cu[-1], torch.Generator().manual_seed(34))
    out, lse = _run(q, k, v, s, gain, temp, cu)
    rows = _sampled_rows(cu, 24, seed=35) + [190, 200, 201, 260, 700, 900, 4000]
    rows = sorted(set(rows))
    ref, ref_lse = oracle.gated_attention_rows(q, k, v, s, gain, temp, cu, rows)
    assert_within(out[rows], ref, 2e-2, 1e-2, f"{kind} eight-wave out")
    assert_within(lse[:, rows], ref_lse, 2e-2, 1e-2, f"{kind} eight-wave lse")


def test_attention_high_temperature():
    """Temperatures of 6-10: the QK part alone spans tens of log2 units."""
    q, k, v, s, gain, temp, cu = _inputs([600], 16, 8, 128, torch.bfloat16, seed=36)
    temp = temp * 8.0
    out, lse = _run(q, k, v, s, gain, temp, cu)
    ref, ref_lse = oracle.gated_attention(q, k, v, s, gain, temp, cu)
    assert_within(out, ref, 2e-2, 1e-2, "high temperature out")
    assert_within(lse, ref_lse, 2e-2, 1e-2, "high temperature lse")


def test_attention_deterministic():
    q, k, v, s, gain, temp, cu = _inputs([1000, 24], 16, 8, 128, torch.bfloat16, seed=23)
    a, _ = _run(q, k, v, s, gain, temp, cu)
    b, _ = _run(q, k, v, s, gain, temp, cu)
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))


def _sampled_rows(cu, per_req, seed):
    g = torch.Generator().manual_seed(seed)
    rows = []
    for b in range(len(cu) - 1):
        lo, hi = cu[b], cu[b + 1]
        n = hi - lo
        fixed = [0, 1, 63, 64, 65, 127, 128, n - 2, n - 1]
        rows += [lo + r for r in fixed if 0 <= r < n]
        rows += (lo + torch.randint(0, n, (per_req,), generator=g)).tolist()
    return sorted(set(rows))


SPLIT_CASES = [
    # (name, lens, Hq, Hkv, d_head, score kind): one request short enough that
    # its query tiles are cut into pieces of at most 24 key tiles (the plan
    # gives a workspace), checked against the oracle and against the unsplit
    # call.
    ("16k_kept", [2048], 16, 8, 128, "random"),
    ("16k_kept_step_up", [2048], 16, 8, 128, "step_up"),
    ("ragged_tail", [1800], 16, 8, 128, "random"),
    ("group4_dh64", [1600], 8, 2, 64, "climb"),
    ("shortest_split", [1537], 16, 8, 128, "low_first_tile"),
    ("short_pieces", [1500], 16, 8, 128, "random"),
    ("shortest_short_pieces", [1153], 16, 8, 128, "climb"),
    ("three_pieces", [4000], 16, 8, 128, "random"),
    ("nine_pieces_one_group", [13000], 2, 1, 64, "descent"),
]


@pytest.mark.parametrize("name,lens,Hq,Hkv,dh,kind", SPLIT_CASES, ids=[c[0] for c in SPLIT_CASES])
def test_attention_key_split(name, lens, Hq, Hkv, dh, kind):
    announce(f"attn key split {name} lens={lens} Hq={Hq} Hkv={Hkv} dh={dh} scores={kind}")
    q, k, v, s, gain, temp, cu = _inputs(lens, Hq, Hkv, dh, torch.bfloat16, seed=zlib.crc32(name.encode()) % 1000)
    if kind != "random":
        s = _score_pattern(kind, cu[-1], torch.Generator().manual_seed(5))
    nbytes = tg.tg_attn_prefill_plan(cu, Hq, Hkv, dh)
    assert nbytes > 0
    ws = torch.zeros(nbytes, dtype=torch.uint8, device="cuda")
    gq, gk, gv, gs, gg, gt = (x.cuda() for x in (q, k, v, s, gain, temp))
    out, lse = tg.tg_gated_attn_prefill(gq, gk, gv, gs, gg, gt, cu, want_lse=True, workspace=ws)
    out2, lse2 = tg.tg_gated_attn_prefill(gq, gk, gv, gs, gg, gt, cu, want_lse=True)
    # The same workspace again: its counters were left at zero, and the
    # pieces are combined in a fixed order, so the result repeats bit for bit.
    out3, lse3 = tg.tg_gated_attn_prefill(gq, gk, gv, gs, gg, gt, cu, want_lse=True, workspace=ws)
    torch.cuda.synchronize()
    assert torch.equal(out3, out) and torch.equal(lse3, lse)
    assert int(ws[:2048].count_nonzero().item()) == 0
    out, lse, out2, lse2 = out.cpu(), lse.cpu(), out2.cpu(), lse2.cpu()
    if cu[-1] > 2048:
        rows = _sampled_rows(cu, 32, seed=9) + list(range(cu[-1] - 70, cu[-1]))
        rows = sorted(set(rows))
        ref, ref_lse = oracle.gated_attention_rows(q, k, v, s, gain, temp, cu, rows)
        got, got_lse = out[rows], lse[:, rows]
    else:
        ref, ref_lse = oracle.gated_attention(q, k, v, s, gain, temp, cu)
        got, got_lse = out, lse
    assert_within(got, ref, 2e-2, 1e-2, f"{name} out")
    assert_within(got_lse, ref_lse, 2e-2, 1e-2, f"{name} lse")
    # Against the unsplit call: each piece takes its bf16 probabilities
    # against its own exponent base, so they round differently (2^-9 relative
    # each); a row dominated by one key moves its sum, hence its lse, by up to
    # that.
    assert (out.float() - out2.float()).abs().max().item() <= 2 ** -6 * max(1.0, out2.float().abs().max().item())
    assert (lse - lse2).abs().max().item() <= 2 ** -7


@pytest.mark.parametrize("lens,Hq,Hkv,dh", [([2048], 16, 8, 128), ([1600], 8, 2, 64)])
def test_attention_key_split_without_bias(lens, Hq, Hkv, dh):
    """The key split of the bias-free build (s_kept = gain = NULL) equals the
    definition with a zero bias, and the unsplit call within the rounding of
    each piece's probabilities."""
    announce(f"attn key split no-bias lens={lens} Hq={Hq} Hkv={Hkv} dh={dh}")
    q, k, v, s, gain, temp, cu = _inputs(lens, Hq, Hkv, dh, torch.bfloat16, seed=33)
    nbytes = tg.tg_attn_prefill_plan(cu, Hq, Hkv, dh)
    assert nbytes > 0
    ws = torch.zeros(nbytes, dtype=torch.uint8, device="cuda")
    gq, gk, gv, gt = (x.cuda() for x in (q, k, v, temp))
    out, lse = tg.tg_gated_attn_prefill(gq, gk, gv, None, None, gt, cu, want_lse=True, workspace=ws)
    out2, lse2 = tg.tg_gated_attn_prefill(gq, gk, gv, None, None, gt, cu, want_lse=True)
    torch.cuda.synchronize()
    assert int(ws[:2048].count_nonzero().item()) == 0
    out, lse, out2, lse2 = out.cpu(), lse.cpu(), out2.cpu(), lse2.cpu()
    ref, ref_lse = oracle.gated_attention(q, k, v, torch.zeros_like(s), gain, temp, cu)
    assert_within(out, ref, 2e-2, 1e-2, "split no-bias out")
    assert_within(lse, ref_lse, 2e-2, 1e-2, "split no-bias lse")
    assert (out.float() - out2.float()).abs().max().item() <= 2 ** -6 * max(1.0, out2.float().abs().max().item())
    assert (lse - lse2).abs().max().item() <= 2 ** -7


def test_attention_key_split_workspace_reuse():
    """One workspace serves calls of different shapes in turn (each call
    leaves its counters at zero): every result equals that of the same call
    on a fresh zeroed workspace, bit for bit."""
    shapes = [[2048], [1500], [1800], [1537], [4000], [1153], [2048]]
    announce(f"attn key split workspace reuse: rows {[s[0] for s in shapes]}")
    big = max(tg.tg_attn_prefill_plan([0, n[0]], 16, 8, 128) for n in shapes)
    shared = torch.zeros(big, dtype=torch.uint8, device="cuda")
    for i, lens in enumerate(shapes):
        q, k, v, s, gain, temp, cu = _inputs(lens, 16, 8, 128, torch.bfloat16, seed=40 + i)
        g = [x.cuda() for x in (q, k, v, s, gain, temp)]
        need = tg.tg_attn_prefill_plan(cu, 16, 8, 128)
        assert need > 0
        fresh = torch.zeros(need, dtype=torch.uint8, device="cuda")
        o1, l1 = tg.tg_gated_attn_prefill(*g, cu, want_lse=True, workspace=shared)
        o2, l2 = tg.tg_gated_attn_prefill(*g, cu, want_lse=True, workspace=fresh)
        torch.cuda.synchronize()
        assert torch.equal(o1, o2) and torch.equal(l1, l2), lens
    assert int(shared[:2048].count_nonzero().item()) == 0


@pytest.mark.parametrize("wname", ["qwen3_1p7b_128k_niah", "qwen3_1p7b_varlen4", "qwen3_1p7b_32k_stack4"])
def test_attention_full_size_sampled(wname):
    """Workload-size attention (kept rows only) in the benchmark's launch
    configuration; the oracle evaluates sampled query rows, all heads."""
    w = workloads.WORKLOADS[wname]
    announce(f"attn full-size {wname} Kt={w.total_kept}")
    a = workloads.attn_inputs(w, seed=1)
    s = workloads.random_scores(w.total_kept, seed=2)
    cu = oracle.plan(w.seq_len, w.q_len, w.budget)[1]
    out, lse = _run(a["q"], a["k"], a["v"], s, a["gain"], a["temp"], cu)
    rows = _sampled_rows(cu, 24, seed=3)
    ref, ref_lse = oracle.gated_attention_rows(a["q"], a["k"], a["v"], s, a["gain"], a["temp"], cu, rows)
    assert_within(out[rows], ref, 2e-2, 1e-2, f"{wname} out")
    assert_within(lse[:, rows], ref_lse, 2e-2, 1e-2, f"{wname} lse")


EIGHT_WAVE = [
    # (name, lens, Hq, Hkv, d_head): sized so that the eight-wave kernel runs
    # (at least 512 workgroups of 256/HPB query rows per head group).
    ("dh64_mha", [8192], 16, 16, 64),
    ("dh128_group4", [8192], 16, 4, 128),
    ("dh64_group2_varlen", [3000, 9000, 5000], 16, 8, 64),
    # Paired workgroups (two query tiles each) whose first tile is the
    # partial last tile of a request, with waves past the request's end.
    ("dh128_group2_varlen_partial", [5000, 7000, 3333], 16, 8, 128),
]


@pytest.mark.parametrize("name,lens,Hq,Hkv,dh", EIGHT_WAVE, ids=[c[0] for c in EIGHT_WAVE])
def test_attention_eight_wave_sampled(name, lens, Hq, Hkv, dh):
    """The eight-wave kernel's other instantiations (one and four query heads
    per KV head, d_head 64), checked on sampled rows, all heads."""
    announce(f"attn eight-wave {name} lens={lens} Hq={Hq} Hkv={Hkv} dh={dh}")
    q, k, v, s, gain, temp, cu = _inputs(lens, Hq, Hkv, dh, torch.bfloat16,
                                         seed=zlib.crc32(name.encode()) % 1000)
    out, lse = _run(q, k, v, s, gain, temp, cu)
    rows = _sampled_rows(cu, 16, seed=5)
    ref, ref_lse = oracle.gated_attention_rows(q, k, v, s, gain, temp, cu, rows)
    assert_within(out[rows], ref, 2e-2, 1e-2, f"{name} out")
    assert_within(lse[:, rows], ref_lse, 2e-2, 1e-2, f"{name} lse")


# ---------------------------------------------------------------- linear ----
@pytest.mark.parametrize("tile", [1, 2, 3])
def test_linear_every_tiling(tile):
    """Each workgroup tiling (128x128, 256x128, 256x256; the launcher picks
    one by output size, tg_linear_tile forces it) on ragged m and n, with odd
    (K = 192 in 64-wide chunks) and even numbers of k chunks, accumulating and
    not."""
    rt, at = tol(torch.bfloat16)
    for M, N, K, acc in ((777, 320, 2048, False), (1000, 192, 192, True), (300, 2112, 64, True)):
        announce(f"linear tile={tile} M={M} N={N} K={K} acc={acc}")
        g = torch.Generator().manual_seed(M * 7 + N)
        x = torch.randn(M, K, generator=g).to(torch.bfloat16)
        w = (torch.randn(N, K, generator=g) / K ** 0.5).to(torch.bfloat16)
        y0 = torch.randn(M, N, generator=g).to(torch.bfloat16)
        y = y0.cuda().clone()
        tg.tg_linear(x.cuda(), w.cuda(), y=y, accumulate=acc, tile=tile)
        torch.cuda.synchronize()
        ref = oracle.linear(x, w) + (y0.double() if acc else 0.0)
        assert_within(y.cpu(), ref, rt, at, f"linear {tile}")


@pytest.mark.parametrize("M,N,K,dtype,acc", [
    (300, 192, 256, torch.bfloat16, False),
    (300, 192, 256, torch.bfloat16, True),
    (1, 64, 64, torch.bfloat16, True),
    (4096, 1024, 2048, torch.bfloat16, False),
    # 256x128-tile kernel (taken when the output has >= 512 such tiles): ragged m and n
    (8192 + 77, 2048 + 64, 2048, torch.bfloat16, False),
    (8192 + 77, 2048 + 64, 2048, torch.bfloat16, True),
    (16384 + 5, 4096, 64, torch.bfloat16, True),
    (37, 50, 20, torch.float32, False),
    (37, 50, 20, torch.float32, True),
])
def test_linear_parity(M, N, K, dtype, acc):
    announce(f"linear M={M} N={N} K={K} {dtype} acc={acc}")
    g = torch.Generator().manual_seed(M + N + K)
    x = torch.randn(M, K, generator=g).to(dtype)
    w = (torch.randn(N, K, generator=g) / K ** 0.5).to(dtype)
    y0 = torch.randn(M, N, generator=g).to(dtype)
    y = y0.cuda().clone()
    tg.tg_linear(x.cuda(), w.cuda(), y=y, accumulate=acc)
    ref = oracle.linear(x, w) + (y0.double() if acc else 0.0)
    rtol, atol = tol(dtype)
    assert_within(y.cpu(), ref, rtol, atol, "linear")


@pytest.mark.parametrize("tile", [0, 1, 2, 3])
def test_linear_multi_matches_separate_products(tile):
    """Three projections of the same rows in one launch (tg_linear_multi):
    every output equal bit for bit to tg_linear_tile of the same product with
    the tile the fused grid uses, and within the bf16 bound of the oracle;
    ragged M, accumulating and not, the q/k/v widths of the 32k stack."""
    rt, at = tol(torch.bfloat16)
    for M, ns, K, acc in ((1000 + 13, (512, 256, 256), 256, False), (4096, (2048, 1024, 1024), 2048, False),
                          (777, (256, 512), 192, True)):
        announce(f"linear_multi tile={tile} M={M} N={ns} K={K} acc={acc}")
        g = torch.Generator().manual_seed(M * 3 + sum(ns) + tile)
        x = torch.randn(M, K, generator=g).to(torch.bfloat16)
        ws = [(torch.randn(n, K, generator=g) / K ** 0.5).to(torch.bfloat16) for n in ns]
        y0 = [torch.randn(M, n, generator=g).to(torch.bfloat16) for n in ns]
        ys = [t.cuda().clone() for t in y0]
        xc, wc = x.cuda(), [w.cuda() for w in ws]
        tg.tg_linear_multi(xc, wc, ys=ys, accumulate=acc, tile=tile)
        # the tile the fused grid takes for the whole width (as tg_linear chooses)
        N = sum(ns)
        t256, t128 = ((M + 255) // 256) * ((N + 255) // 256), ((M + 255) // 256) * ((N + 127) // 128)
        used = tile if tile else (3 if t256 >= 256 else 2 if t128 >= 512 else 1)
        for i, (w, n) in enumerate(zip(wc, ns)):
            sep = y0[i].cuda().clone()
            tg.tg_linear(xc, w, y=sep, accumulate=acc, tile=used)
            torch.cuda.synchronize()
            assert torch.equal(ys[i].cpu(), sep.cpu()), f"segment {i} differs from tg_linear_tile {used}"
            ref = oracle.linear(x, ws[i]) + (y0[i].double() if acc else 0.0)
            assert_within(ys[i].cpu(), ref, rt, at, f"linear_multi segment {i}")


@pytest.mark.parametrize("tile", [0, 1, 2, 3])
def test_linear_swiglu(tile):
    """Gate and up projections with the SwiGLU product in the epilogue
    (tg_linear_swiglu) against the oracle's silu(x Wg^T) * (x Wu^T), on
    ragged M, one or several k chunks and several unit blocks."""
    rt, at = tol(torch.bfloat16)
    for M, F, K in ((777, 384, 192), (300, 128, 64), (4096 + 31, 1536, 2048)):
        announce(f"linear_swiglu tile={tile} M={M} F={F} K={K}")
        g = torch.Generator().manual_seed(M + F + K + tile)
        x = torch.randn(M, K, generator=g).to(torch.bfloat16)
        w = (torch.randn(2 * F, K, generator=g) / K ** 0.5).to(torch.bfloat16)
        out = tg.tg_linear_swiglu(x.cuda(), w.cuda(), tile=tile)
        torch.cuda.synchronize()
        gu = oracle.linear(x, w)
        assert_within(out.cpu(), oracle.silu(gu[:, :F]) * gu[:, F:], rt, at, f"swiglu {tile}")
