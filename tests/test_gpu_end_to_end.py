"""The whole gated layer on the GPU against the oracle, step by step.

* gate scores within tolerance of the oracle's;
* the selector on the GPU's own scores equals the oracle's selector on those
  same scores (bit-exact), and differs from the all-oracle chain only at ids
  whose oracle score lies within the bf16 tolerance of the threshold score;
* gather and attention on the GPU's compacted rows match the oracle on those
  same rows;
* on the 128k needle workload every planted needle survives.
"""
import pytest
import torch

import learned_token_pruning_02_amd as tg
import oracle
import workloads
from learned_token_pruning_02_amd.path import AttentionStack, GatedLayer
from parity_util import announce, assert_within, tol

pytestmark = pytest.mark.gpu


def _near_threshold_only(kept_a, kept_b, s_ref, w, rtol, atol):
    """Ids in exactly one of the two kept sets must have an oracle score within
    tolerance of the K_doc-th best document score of their request."""
    a, b = set(kept_a.tolist()), set(kept_b.tolist())
    diff = a ^ b
    if not diff:
        return
    cu_s, _ = oracle.plan(w.seq_len, w.q_len, w.budget)
    for t in diff:
        r = max(i for i in range(w.batch) if cu_s[i] <= t)
        lo, n, q = cu_s[r], w.seq_len[r], w.q_len[r]
        kdoc = min(w.budget[r], n) - q
        doc = torch.sort(s_ref[lo:lo + n - q].double(), descending=True).values
        thr = float(doc[kdoc - 1])
        assert abs(float(s_ref[t]) - thr) <= atol + rtol * abs(thr), (t, float(s_ref[t]), thr)


def _oracle_scores(gi, rows_per_chunk=16384):
    """The oracle's gate scores of every token, computed in row chunks to
    bound the float64 working set."""
    T = gi["hidden"].shape[0]
    return torch.cat([oracle.gate_score(gi["hidden"][i:i + rows_per_chunk], gi["w1"], gi["b1"],
                                        gi["w2"], gi["b2"]) for i in range(0, T, rows_per_chunk)])


@pytest.mark.parametrize("wname", ["tiny_fp32", "qwen3_1p7b_16k", "qwen3_1p7b_varlen4",
                                   "qwen3_1p7b_128k_niah"])
def test_gated_layer_chain(wname):
    w = workloads.WORKLOADS[wname]
    sh = w.shape
    announce(f"chain {wname}")
    gi = workloads.gate_inputs(w, seed=0)
    ai = workloads.attn_inputs(w, seed=0)
    g = {k: v.cuda() for k, v in gi.items()}
    a = {k: v.cuda() for k, v in ai.items()}
    layer = GatedLayer(w.total_tokens, sh.d_model, sh.n_q_heads, sh.d_head, w.seq_len, w.q_len,
                       w.budget, sh.dtype, n_kv_heads=sh.n_kv_heads)
    out = layer(g["hidden"], g["w1"], g["b1"], g["w2"], g["b2"], a["q"], a["k"], a["v"],
                a["gain"], a["temp"])
    torch.cuda.synchronize()
    rtol, atol = tol(sh.dtype)

    s_gpu = layer.scores.cpu()
    s_ref = _oracle_scores(gi)
    assert_within(s_gpu, s_ref, rtol, atol, "scores")
    if w.n_needles:
        assert set(workloads.needle_positions(w, 0).tolist()) <= set(layer.kept.cpu().tolist())

    kept_gpu = layer.kept.cpu()
    kept_on_gpu_scores, cu = oracle.topk_select(s_gpu, w.seq_len, w.q_len, w.budget)
    assert torch.equal(kept_gpu, kept_on_gpu_scores)
    assert layer.cu_kept == cu and layer.cu_kept_dev.cpu().tolist() == cu
    kept_ref, _ = oracle.topk_select(s_ref, w.seq_len, w.q_len, w.budget)
    _near_threshold_only(kept_gpu, kept_ref, s_ref, w, rtol, atol)

    hk_ref, sk_ref = oracle.gather_compact(gi["hidden"], s_gpu, kept_gpu)
    bits = torch.int16 if sh.dtype == torch.bfloat16 else torch.int32
    assert torch.equal(layer.hidden_kept.cpu().view(bits), hk_ref.view(bits))
    assert torch.equal(layer.s_kept.cpu(), sk_ref)

    if w.total_kept <= 4096:
        ref, _ = oracle.gated_attention(ai["q"], ai["k"], ai["v"], sk_ref, ai["gain"], ai["temp"], cu)
        assert_within(out.cpu(), ref, rtol, atol, "attention")
    else:
        rows = sorted(set(torch.randint(0, w.total_kept, (200,), generator=torch.Generator().manual_seed(1)).tolist()
                          + [c - 1 for c in cu[1:]] + cu[:-1]))
        ref, _ = oracle.gated_attention_rows(ai["q"], ai["k"], ai["v"], sk_ref, ai["gain"], ai["temp"], cu, rows)
        assert_within(out.cpu()[rows], ref, rtol, atol, "attention rows")


def test_needles_survive_128k():
    w = workloads.WORKLOADS["qwen3_1p7b_128k_niah"]
    announce("needles 128k")
    gi = workloads.gate_inputs(w, seed=0)
    g = {k: v.cuda() for k, v in gi.items()}
    s = tg.tg_gate_score(g["hidden"], g["w1"], g["b1"], g["w2"], g["b2"])
    kept, cu = tg.tg_topk_select(s, w.seq_len, w.q_len, w.budget)
    kept = kept.cpu()
    assert kept.numel() == 8192 and cu == [0, 8192]
    assert set(workloads.needle_positions(w, 0).tolist()) <= set(kept.tolist())
    assert set(range(w.total_tokens - 128, w.total_tokens)) <= set(kept.tolist())
    assert torch.equal(kept, torch.sort(kept).values) and kept.unique().numel() == kept.numel()
    ref, _ = oracle.topk_select(s.cpu(), w.seq_len, w.q_len, w.budget)
    assert torch.equal(kept, ref)


def test_stack_reduced_step_by_step():
    """Four attention-stack layers of the Qwen3-1.7B shape on 1024 kept rows.

    The stack has no normalisation, so the residual grows layer by layer and
    the upper layers' softmax becomes nearly one-hot: a one-ulp bf16 rounding
    difference in q or k can switch the dominant key, and differences compound
    over layers.  Every sub-step of every layer is therefore checked on
    identical inputs: projections from the GPU's residual, attention from the
    GPU's q/k/v, the residual update from the GPU's attention output."""
    base = workloads.WORKLOADS["qwen3_1p7b_32k_stack4"]
    sh = base.shape
    Kt = 1024
    Hq, Hkv, dh = sh.n_q_heads, sh.n_kv_heads, sh.d_head
    announce("stack reduced")
    g = torch.Generator().manual_seed(31)
    x0 = torch.randn(Kt, sh.d_model, generator=g).to(torch.bfloat16)
    s = torch.randn(Kt, generator=g)
    layers = workloads.stack_weights(base, seed=0)
    cu = [0, Kt]
    x = x0.cuda().clone()
    stack = AttentionStack(Kt, sh.d_model, Hq, Hkv, dh, sh.dtype)
    for li, L in enumerate(layers):
        x_in = x.cpu()
        stack(x, s.cuda(), cu, [{k: v.cuda() for k, v in L.items()}])
        torch.cuda.synchronize()
        q, k, v, a = stack.q.cpu(), stack.k.cpu(), stack.v.cpu(), stack.attn.cpu()
        assert_within(q, oracle.linear(x_in, L["wq"]), 2e-2, 1e-2, f"layer {li} q")
        assert_within(k, oracle.linear(x_in, L["wk"]), 2e-2, 1e-2, f"layer {li} k")
        assert_within(v, oracle.linear(x_in, L["wv"]), 2e-2, 1e-2, f"layer {li} v")
        ref_a, _ = oracle.gated_attention(q.view(Kt, Hq, dh), k.view(Kt, Hkv, dh),
                                          v.view(Kt, Hkv, dh), s, L["gain"], L["temp"], cu)
        assert_within(a, ref_a, 2e-2, 1e-2, f"layer {li} attention")
        ref_x = x_in.double() + oracle.linear(a.view(Kt, Hq * dh), L["wo"])
        assert_within(x.cpu(), ref_x, 2e-2, 1e-2, f"layer {li} residual")


def test_stack_full_size_sampled_rows():
    """The 32k workload's four stack layers at their real size (the 4096 kept
    rows the gated layer compacts, fed the gate's own kept scores), run as
    the benchmark runs them; every sub-step of every layer is checked on
    sampled rows against the oracle on the GPU's own inputs of that step
    (projections from the GPU residual, attention from the GPU's q/k/v, the
    residual update from the GPU's attention output)."""
    w = workloads.WORKLOADS["qwen3_1p7b_32k_stack4"]
    sh = w.shape
    Hq, Hkv, dh = sh.n_q_heads, sh.n_kv_heads, sh.d_head
    announce("stack 32k full size, sampled rows")
    g = {k: v.cuda() for k, v in workloads.gate_inputs(w, seed=0).items()}
    a = {k: v.cuda() for k, v in workloads.attn_inputs(w, seed=0).items()}
    layer = GatedLayer(w.total_tokens, sh.d_model, Hq, dh, w.seq_len, w.q_len, w.budget, sh.dtype)
    layer(g["hidden"], g["w1"], g["b1"], g["w2"], g["b2"], a["q"], a["k"], a["v"], a["gain"], a["temp"])
    Kt = layer.Kt
    assert Kt == 4096
    cu = layer.cu_kept
    s = layer.s_kept.cpu()
    x = layer.hidden_kept.clone()
    stack = AttentionStack(Kt, sh.d_model, Hq, Hkv, dh, sh.dtype)
    rows = sorted(set(torch.randint(0, Kt, (96,), generator=torch.Generator().manual_seed(2)).tolist()
                      + [0, 1, 63, 64, 127, 128, Kt - 1]))
    for li, L in enumerate(workloads.stack_weights(w, 0)):
        x_in = x.cpu()
        stack(x, layer.s_kept, cu, [{k: v.cuda() for k, v in L.items()}])
        torch.cuda.synchronize()
        q, k, v, att = stack.q.cpu(), stack.k.cpu(), stack.v.cpu(), stack.attn.cpu()
        for nm, got, wt in (("q", q, L["wq"]), ("k", k, L["wk"]), ("v", v, L["wv"])):
            assert_within(got[rows], oracle.linear(x_in[rows], wt), 2e-2, 1e-2, f"layer {li} {nm}")
        ref_a, _ = oracle.gated_attention_rows(q.view(Kt, Hq, dh), k.view(Kt, Hkv, dh), v.view(Kt, Hkv, dh),
                                               s, L["gain"], L["temp"], cu, rows)
        assert_within(att[rows], ref_a, 2e-2, 1e-2, f"layer {li} attention")
        ref_x = x_in[rows].double() + oracle.linear(att.view(Kt, Hq * dh)[rows], L["wo"])
        assert_within(x.cpu()[rows], ref_x, 2e-2, 1e-2, f"layer {li} residual")


def test_gated_layer_graph_replays():
    """The gated layer captured once as a HIP graph (as the benchmark times
    it): three replays, each on new inputs written into the captured buffers,
    with eager work and host synchronisations in between, each equal bit for
    bit to an eager layer run on the same inputs."""
    w = workloads.WORKLOADS["qwen3_1p7b_16k"]
    sh = w.shape
    announce("gated layer graph replays 16k")
    g = {k: v.cuda() for k, v in workloads.gate_inputs(w, seed=0).items()}
    a = {k: v.cuda() for k, v in workloads.attn_inputs(w, seed=0).items()}
    mk = lambda: GatedLayer(w.total_tokens, sh.d_model, sh.n_q_heads, sh.d_head, w.seq_len,
                            w.q_len, w.budget, sh.dtype, n_kv_heads=sh.n_kv_heads)
    layer, eager = mk(), mk()
    run = lambda L: L(g["hidden"], g["w1"], g["b1"], g["w2"], g["b2"], a["q"], a["k"], a["v"],
                      a["gain"], a["temp"])
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        run(layer)
    torch.cuda.current_stream().wait_stream(side)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        run(layer)
    for rep in range(3):
        gen = torch.Generator(device="cuda").manual_seed(100 + rep)
        g["hidden"].copy_(torch.randn(g["hidden"].shape, generator=gen, device="cuda"))
        a["q"].copy_(torch.randn(a["q"].shape, generator=gen, device="cuda"))
        layer.out.zero_()
        layer.kept.fill_(-1)
        torch.cuda.synchronize()
        graph.replay()
        run(eager)
        torch.cuda.synchronize()
        for name in ["scores", "kept", "s_kept", "hidden_kept", "out"]:
            assert torch.equal(getattr(layer, name), getattr(eager, name)), (rep, name)
