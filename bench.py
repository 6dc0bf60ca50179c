"""Benchmark of the TokenGate pruned-prefill hot path on one MI355X.

One step is one gated layer over one batch of synthetic, HBM-resident input:
    gate MLP score (all tokens) -> top-K select (+ question tail)
    -> gather/compact -> causal GQA token-gated attention over the kept rows
(plus the four QKV/attention/O layers above the gate for the stack workload).

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME] [--graph] [--no-context]
    python bench.py --select-sweep      # selector alone, T = 2^20 .. 2^26, K = T/16
    python bench.py --layer | --backward | --decode   # the other paths, one line each

Prints ONE JSON line: whole-step throughput in tokens of context per second
(N / step time, one launch per kernel; the same step replayed as one HIP graph
is reported beside it, and is the value with --graph), the per-kernel split
(mean, median, minimum), the roofline of the dominant kernel, derived rates
(attention-only and kept-token rates, the bias overhead against the bias-free
build of the same attention kernel, attention on all N tokens without pruning,
K/V bytes kept vs full) and the CPU oracle timed on a bounded sample of the
same workload.  Each kernel is also timed cold, right after 512 MiB are
written to evict the 256 MiB Infinity Cache (labelled *_cold).  Under
"configs", every other workload (16k, 32k with the 4-layer stack, the varlen
batch, the tiny fp32 layer) gets its own step time, throughput and per-kernel
warm and cold figures; --no-configs skips them.  --no-context skips the two
context timings (for profiles that should hold the hot path only).
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0        # MI355X HBM3E, GB/s
WARM_S = 0.1                 # seconds of untimed steps before timing a non-primary workload
BF16_PEAK_TFLOPS = 2500.0    # MI355X dense bf16 MFMA, TFLOP/s
F32_PEAK_TFLOPS = 157.3      # MI355X fp32 vector, TFLOP/s


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=20)
    # The GPU idles for seconds while the host draws the inputs, and its clocks
    # take tens of milliseconds of steady work to come back up: 200 untimed
    # steps (~0.1 s at 128k) reach the steady state (5 measured 12% slower).
    p.add_argument("--warmup", type=int, default=200)
    p.add_argument("--workload", default="qwen3_1p7b_128k_niah")
    p.add_argument("--seed", type=int, default=0)
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--no-context", action="store_true",
                   help="skip the context timings (attention without bias, attention on all N "
                        "tokens), so that a profile holds the hot path's kernels only")
    p.add_argument("--graph", action="store_true",
                   help="report the HIP graph replay time of the step as the value")
    p.add_argument("--detail", default="", help="also write the JSON line, indented, to this path")
    p.add_argument("--no-configs", action="store_true",
                   help="time the named workload only (not every other workload as well)")
    p.add_argument("--copy-calibration", action="store_true",
                   help="only run a plain device copy of 512 MiB (reference for HBM byte counters)")
    p.add_argument("--select-sweep", action="store_true",
                   help="only time the selector on T = 2^20 .. 2^26 random scores, K = T/16")
    p.add_argument("--layer", action="store_true",
                   help="only time one whole decoder layer on the 8192 kept rows of the 128k prompt")
    p.add_argument("--backward", action="store_true",
                   help="only time the token-gated attention backward on the 8192 kept rows of the 128k prompt")
    p.add_argument("--decode", action="store_true",
                   help="only time one decode step over kept-only KV caches (32 requests x 8193 rows)")
    return p.parse_args()


def select_sweep(reps: int = 20):
    """Selector throughput beyond the layer sizes: one request of T random
    fp32 scores, keep K = T/16 (no question tail); one JSON line per T."""
    import torch

    import learned_token_pruning_02_amd as tg
    g = torch.Generator(device="cuda").manual_seed(0)
    for e in range(20, 27):
        T = 1 << e
        K = T // 16
        scores = torch.randn(T, generator=g, device="cuda")
        cu_s, cu_k, ws = tg.tg_plan([T], [0], [K])
        kept = torch.empty(K, dtype=torch.int32, device="cuda")
        wsb = torch.empty(ws, dtype=torch.uint8, device="cuda")
        for _ in range(50):
            tg.tg_topk_select(scores, [T], [0], [K], kept_idx=kept, workspace=wsb)
        torch.cuda.synchronize()
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(reps + 1)]
        ev[0].record()
        for i in range(reps):
            tg.tg_topk_select(scores, [T], [0], [K], kept_idx=kept, workspace=wsb)
            ev[i + 1].record()
        torch.cuda.synchronize()
        ms = sorted(ev[i].elapsed_time(ev[i + 1]) for i in range(reps))
        med = ms[reps // 2]
        print(json.dumps({"metric": "select GB/s (T*4 read + K*4 written)", "T": T, "K": K,
                          "us_median": med * 1e3, "us_min": ms[0] * 1e3,
                          "GB/s": (T * 4 + K * 4) / (med * 1e-3) / 1e9}), flush=True)
        del scores, kept, wsb


def copy_calibration():
    """A plain device-to-device copy of exactly 512 MiB, timed; run under a
    counter collector, its FETCH_SIZE / WRITE_SIZE readings give the factor
    that turns those counters into bytes."""
    import torch
    n = 512 << 20
    src = torch.empty(n, dtype=torch.uint8, device="cuda").fill_(1)
    dst = torch.empty_like(src)
    for _ in range(2):
        dst.copy_(src)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    dst.copy_(src)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1)
    print(json.dumps({"copy_bytes_read": n, "copy_bytes_written": n, "ms": ms,
                      "GB/s_read_plus_write": 2 * n / ms / 1e6}), flush=True)


def algorithmic(w, Kt_per_req):
    """Algorithmic bytes / FLOPs per launch of each kernel for workload w."""
    sh = w.shape
    eb = 2 if sh.dtype.is_floating_point and sh.dtype.itemsize == 2 else 4
    T, d, dg = w.total_tokens, sh.d_model, sh.d_gate
    Kt = sum(Kt_per_req)
    pairs = sum(k * (k + 1) // 2 for k in Kt_per_req)
    return {
        "gate": {"bytes": T * (d * eb + 4) + dg * d * eb + 2 * dg * eb,
                 "flops": 2 * T * (d * dg + dg)},
        "select": {"bytes": T * 4 + Kt * 4, "flops": 0},
        "gather": {"bytes": Kt * (2 * d * eb + 12), "flops": 0},
        "attention": {"bytes": Kt * (sh.n_q_heads * 2 + sh.n_kv_heads * 2) * sh.d_head * eb + Kt * 4,
                      "flops": 4 * sh.d_head * sh.n_q_heads * pairs},
    }


KERNEL_FRAG = {"gate": "gate_bf16_kernel", "select": "sel_cand_kernel",
               "gather": "gather_rows_kernel", "attention": "attn_bf16_kernel",
               "decode": "decode_chunk_kernel"}


def recorded_traffic_sum(workload: str, frags):
    """HBM bytes per call summed over the kernels `frags` of a committed
    counter record of this workload, or None when one is missing or its
    source changed since."""
    import glob
    import hashlib
    for f in sorted(glob.glob(os.path.join(ROOT, "profiles", "*_hbm_traffic.json"))):
        rec = json.load(open(f))
        if not rec.get("workload", "").startswith(workload):
            continue
        total = 0.0
        for frag in frags:
            k = rec.get("kernels", {}).get(frag)
            if k is None:
                return None
            with open(os.path.join(ROOT, k["source"]), "rb") as src:
                if hashlib.sha256(src.read()).hexdigest() != k["source_sha256"]:
                    return None
            total += k["read_bytes"] + k["written_bytes"]
        return total
    return None


def recorded_traffic(workload: str, kernel: str):
    """HBM bytes per launch of `kernel` from a committed counter record of this
    workload, or None when there is none or the kernel source changed since."""
    import glob
    import hashlib
    frag = KERNEL_FRAG[kernel]
    for f in sorted(glob.glob(os.path.join(ROOT, "profiles", "*_hbm_traffic.json"))):
        rec = json.load(open(f))
        if not rec.get("workload", "").startswith(workload) or frag not in rec.get("kernels", {}):
            continue
        k = rec["kernels"][frag]
        with open(os.path.join(ROOT, k["source"]), "rb") as src:
            if hashlib.sha256(src.read()).hexdigest() != k["source_sha256"]:
                return None
        return k["read_bytes"] + k["written_bytes"]
    return None


def cpu_baseline(w, gi, ai, s_gpu, kept, cu):
    """The oracle as it stands, on a bounded sample of the workload, scaled to
    the whole layer: the gate on the first 8192 tokens, the selector and the
    gather on the whole layer, attention for 2 of the query heads (one KV head)
    on all kept rows."""
    import torch

    import oracle

    sh = w.shape
    T = w.total_tokens
    t_s = min(T, 8192)
    t0 = time.perf_counter()
    oracle.gate_score(gi["hidden"][:t_s], gi["w1"], gi["b1"], gi["w2"], gi["b2"])
    t_gate = (time.perf_counter() - t0) * T / t_s
    t0 = time.perf_counter()
    oracle.topk_select(s_gpu, w.seq_len, w.q_len, w.budget)
    t_sel = time.perf_counter() - t0
    t0 = time.perf_counter()
    oracle.gather_compact(gi["hidden"], s_gpu, kept)
    t_gath = time.perf_counter() - t0
    hs = min(2, sh.n_q_heads)
    group = sh.n_q_heads // sh.n_kv_heads
    kv_need = (hs + group - 1) // group
    s_kept = s_gpu[kept.long()]
    t0 = time.perf_counter()
    oracle.gated_attention(ai["q"][:, :hs].contiguous(), ai["k"][:, :kv_need].contiguous(),
                           ai["v"][:, :kv_need].contiguous(), s_kept, ai["gain"][:hs],
                           ai["temp"][:hs], cu)
    t_attn = (time.perf_counter() - t0) * sh.n_q_heads / hs
    total = t_gate + t_sel + t_gath + t_attn
    return {
        "value": T / total,
        "unit": "tokens/s",
        "cores": torch.get_num_threads(),
        "kind": "oracle",
        "sample": (f"oracle gate on {t_s} of {T} tokens, selector and gather on the whole layer, "
                   f"attention for {hs} of {sh.n_q_heads} query heads on all {len(kept)} kept rows; "
                   "each part scaled to the whole layer"),
        "seconds_scaled": {"gate": t_gate, "select": t_sel, "gather": t_gath, "attention": t_attn},
        "cpu_model": cpu_model(),
        "affinity_cpus": len(os.sched_getaffinity(0)),
    }


def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def backward_bench(args):
    """The token-gated attention backward (all four kernels of one call) on
    the 8192 kept rows of the 128k prompt, Qwen3-1.7B heads.  Algorithmic
    work: the five matrix products of an attention backward (S, dP, dV, dK,
    dQ), 2.5 times the forward's FLOPs; this implementation also recomputes
    S and dP in its dQ pass, which the rate does not credit."""
    import torch

    import learned_token_pruning_02_amd as tg
    import workloads

    w = workloads.WORKLOADS["qwen3_1p7b_128k_niah"]
    sh = w.shape
    a = {k: v.cuda() for k, v in workloads.attn_inputs(w, seed=args.seed).items()}
    Kt = w.total_kept
    cu = [0, Kt]
    s = workloads.random_scores(Kt, seed=args.seed + 2).cuda()
    g = torch.Generator(device="cuda").manual_seed(args.seed + 3)
    dout = torch.randn(Kt, sh.n_q_heads, sh.d_head, device="cuda", generator=g).to(sh.dtype)
    out, lse = tg.tg_gated_attn_prefill(a["q"], a["k"], a["v"], s, a["gain"], a["temp"], cu, want_lse=True)
    ws = torch.empty(tg.tg_attn_backward_plan(cu, sh.n_q_heads, sh.n_kv_heads), dtype=torch.uint8,
                     device="cuda")
    grads = {"dq": torch.empty_like(a["q"]), "dk": torch.empty_like(a["k"]), "dv": torch.empty_like(a["v"]),
             "ds": torch.empty(Kt, device="cuda"), "dgain": torch.empty(sh.n_q_heads, device="cuda"),
             "dtemp": torch.empty(sh.n_q_heads, device="cuda")}
    st = torch.cuda.current_stream()

    def call():
        tg.tg_gated_attn_backward(a["q"], a["k"], a["v"], s, a["gain"], a["temp"], out, lse, dout, cu,
                                  grads=grads, workspace=ws, stream=st)

    for _ in range(args.warmup):
        call()
    torch.cuda.synchronize()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]
    t0 = time.perf_counter()
    ev[0].record(st)
    for i in range(args.steps):
        call()
        ev[i + 1].record(st)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms = [ev[i].elapsed_time(ev[i + 1]) for i in range(args.steps)]
    mean = sum(ms) / len(ms)
    flops = 2.5 * 4 * sh.d_head * sh.n_q_heads * Kt * (Kt + 1) // 2
    tf = flops / (mean * 1e-3) / 1e12

    # The gate MLP backward on the same kept rows, fed the score gradient.
    gi = workloads.gate_inputs(workloads.WORKLOADS["qwen3_1p7b_16k"], seed=args.seed)
    gw = {k: (None if v is None else v.cuda()) for k, v in gi.items() if k != "hidden"}
    gx = torch.randn(Kt, sh.d_model, device="cuda", generator=g).to(sh.dtype)
    gws = torch.empty(tg.tg_gate_backward_plan(sh.dtype, Kt, sh.d_model, sh.d_gate), dtype=torch.uint8,
                      device="cuda")
    ggr = tg.tg_gate_backward(gx, gw["w1"], gw["b1"], gw["w2"], grads["ds"], workspace=gws, stream=st)
    for _ in range(args.warmup):
        tg.tg_gate_backward(gx, gw["w1"], gw["b1"], gw["w2"], grads["ds"], grads=ggr, workspace=gws, stream=st)
    gev = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]
    gev[0].record(st)
    for i in range(args.steps):
        tg.tg_gate_backward(gx, gw["w1"], gw["b1"], gw["w2"], grads["ds"], grads=ggr, workspace=gws, stream=st)
        gev[i + 1].record(st)
    torch.cuda.synchronize()
    gms = sum(gev[i].elapsed_time(gev[i + 1]) for i in range(args.steps)) / args.steps
    gflops = 3 * 2 * Kt * sh.d_model * sh.d_gate
    rec = {
        "metric": "gated attention backward tokens/s (context tokens per layer)",
        "value": w.total_tokens / (mean * 1e-3), "unit": "tokens/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": wall * 1e3 / args.steps, "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic (seeded)",
        "config": {"workload": "qwen3_1p7b_128k_backward", "tokens": w.total_tokens, "kept": Kt,
                   "heads_q": sh.n_q_heads, "heads_kv": sh.n_kv_heads, "d_head": sh.d_head},
        "roofline": {"bound": "mfma", "achieved": tf, "peak": BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                     "frac": tf / BF16_PEAK_TFLOPS,
                     "traffic": recorded_traffic_sum(
                         "qwen3_1p7b_128k_backward",
                         ["bwd_dot_kernel", "bwd_kv_kernel", "bwd_q_kernel", "bwd_reduce_kernel"]),
                     "kernel": "attention backward (dot, KV pass, Q pass, reduce; one call)",
                     "algorithmic_flops_per_call": flops},
        "ms_call": {"mean": mean, "median": sorted(ms)[len(ms) // 2], "min": min(ms),
                    "all": [round(x, 4) for x in ms]},
        "gate_backward": {"ms": gms, "TFLOP/s": gflops / (gms * 1e-3) / 1e12,
                          "note": "gate MLP backward on the 8192 kept rows (three products on the "
                                  "projection kernel, dz and column sums), fed this call's ds"},
    }
    if not args.no_cpu_baseline:
        import oracle
        n_cpu = 2048
        qc, kc, vc = (a[x][:n_cpu, :2].cpu().contiguous() if x == "q" else a[x][:n_cpu, :1].cpu().contiguous()
                      for x in ("q", "k", "v"))
        t0 = time.perf_counter()
        oracle.gated_attention_backward(qc, kc, vc, s[:n_cpu].cpu(), a["gain"][:2].cpu(), a["temp"][:2].cpu(),
                                        [0, n_cpu], dout[:n_cpu, :2].cpu())
        t = (time.perf_counter() - t0) * (sh.n_q_heads / 2) * (Kt / n_cpu) ** 2
        rec["cpu_baseline"] = {"value": w.total_tokens / t, "unit": "tokens/s",
                               "cores": torch.get_num_threads(), "kind": "oracle",
                               "sample": (f"oracle backward for 2 of {sh.n_q_heads} heads on the first "
                                          f"{n_cpu} of {Kt} kept rows, scaled by heads and (rows)^2")}
    print(json.dumps(rec), flush=True)


def decode_bench(args):
    """One decode step (both kernels of tg_gated_attn_decode) over the kept-only
    caches of 32 requests, 8193 rows each; HBM-bound, so the roofline is the
    cached K/V/score bytes plus q and out per call over the call's time."""
    import torch

    import learned_token_pruning_02_amd as tg
    import workloads

    w = workloads.DECODE_WORKLOADS["qwen3_1p7b_128k_decode_b32"]
    sh = w.shape
    inp = workloads.decode_inputs(sh, w.cache_len, seed=args.seed)
    d = {k: v.cuda() for k, v in inp.items()}
    B, max_len = w.batch, max(w.cache_len)
    out = torch.empty_like(d["q"])
    lse = torch.empty(B, sh.n_q_heads, dtype=torch.float32, device="cuda")
    ws = torch.empty(tg.tg_decode_plan(B, sh.n_q_heads, sh.d_head, max_len), dtype=torch.uint8,
                     device="cuda")
    stream = torch.cuda.current_stream()

    def call():
        tg.tg_gated_attn_decode(d["q"], d["k"], d["v"], d["s"], d["row_off"], d["cache_len"],
                                d["gain"], d["temp"], max_len, out=out, lse=lse, workspace=ws,
                                stream=stream)

    for _ in range(args.warmup):
        call()
    torch.cuda.synchronize()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]
    t0 = time.perf_counter()
    ev[0].record(stream)
    for i in range(args.steps):
        call()
        ev[i + 1].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms = [ev[i].elapsed_time(ev[i + 1]) for i in range(args.steps)]
    mean = sum(ms) / len(ms)
    rows = sum(w.cache_len)
    eb = 2
    bytes_call = (rows * sh.n_kv_heads * sh.d_head * eb * 2 + rows * 4
                  + 2 * B * sh.n_q_heads * sh.d_head * eb + B * sh.n_q_heads * 4)
    gbs = bytes_call / (mean * 1e-3) / 1e9
    rec = {
        "metric": "gated decode tokens/s per layer", "value": B / (mean * 1e-3), "unit": "tokens/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": wall * 1e3 / args.steps,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic (seeded)",
        "config": {"workload": w.name, "requests": B, "cache_rows_per_request": max_len,
                   "heads_q": sh.n_q_heads, "heads_kv": sh.n_kv_heads, "d_head": sh.d_head},
        "roofline": {"bound": "hbm", "achieved": gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": gbs / HBM_PEAK_GBS, "traffic": recorded_traffic(w.name, "decode"),
                     "kernel": "decode (split-K chunk kernel + merge, one call)",
                     "algorithmic_bytes_per_call": bytes_call},
        "ms_call": {"mean": mean, "median": sorted(ms)[len(ms) // 2], "min": min(ms)},
    }
    if not args.no_cpu_baseline:
        import oracle
        nb = 4
        off, lens = inp["row_off"].tolist()[:nb], w.cache_len[:nb]
        t0 = time.perf_counter()
        oracle.gated_decode_attention(inp["q"][:nb], inp["k"], inp["v"], inp["s"], off, lens,
                                      inp["gain"], inp["temp"])
        t = (time.perf_counter() - t0) * B / nb
        rec["cpu_baseline"] = {"value": B / t, "unit": "tokens/s", "cores": torch.get_num_threads(),
                               "kind": "oracle",
                               "sample": f"oracle decode for {nb} of {B} requests, scaled to {B}"}
    print(json.dumps(rec), flush=True)


def layer_bench(args):
    """One whole decoder layer above the gate (RMSNorm, q/k/v projections, q/k
    norm + rotary embedding, gated attention, output projection, RMSNorm,
    SwiGLU FFN) on the 8192 kept rows of the pruned 128k prompt, Qwen3-1.7B
    shape; per-call HIP events on the library's stream."""
    import torch

    import learned_token_pruning_02_amd as tg
    import workloads
    from learned_token_pruning_02_amd.path import DecoderLayer

    w = workloads.WORKLOADS["qwen3_1p7b_128k_niah"]
    sh = w.shape
    F = workloads.QWEN3_1P7B_FFN
    L = {k: v.cuda() for k, v in workloads.layer_weights(sh, F, seed=args.seed).items()}
    kept, cu_s, cu_k = workloads.kept_layout(w.seq_len, w.q_len, w.budget, seed=args.seed)
    Kt = cu_k[-1]
    g = torch.Generator().manual_seed(args.seed * 7 + 1)
    x0 = torch.randn(Kt, sh.d_model, generator=g).to(sh.dtype).cuda()
    s = torch.randn(Kt, generator=g).cuda()
    x = x0.clone()
    layer = DecoderLayer(Kt, sh.d_model, sh.n_q_heads, sh.n_kv_heads, sh.d_head, F, sh.dtype)
    layer.positions(kept.cuda(), cu_s, cu_k)
    st = torch.cuda.current_stream()
    theta, eps = layer.theta, layer.eps
    names = ["in_norm", "qkv_proj", "qk_norm_rope", "attention", "o_proj",
             "post_norm", "gate_up_silu", "down"]
    calls = [
        lambda: tg.tg_rmsnorm(x, L["in_norm"], eps, y=layer.xn, stream=st),
        lambda: tg.tg_linear_multi(layer.xn, [L["wq"], L["wk"], L["wv"]],
                                   ys=[layer.q.view(Kt, -1), layer.k.view(Kt, -1), layer.v.view(Kt, -1)],
                                   stream=st),
        lambda: tg.tg_qk_norm_rope(layer.q, layer.k, L["q_norm"], L["k_norm"], layer.pos, theta, eps,
                                   stream=st),
        lambda: tg.tg_gated_attn_prefill(layer.q, layer.k, layer.v, s, L["gain"], L["temp"], cu_k,
                                         out=layer.attn, stream=st),
        lambda: tg.tg_linear(layer.attn.view(Kt, -1), L["wo"], y=x, accumulate=True, stream=st),
        lambda: tg.tg_rmsnorm(x, L["post_norm"], eps, y=layer.xn, stream=st),
        lambda: tg.tg_linear_swiglu(layer.xn, L["wgu"], out=layer.m, stream=st),
        lambda: tg.tg_linear(layer.m, L["wd"], y=x, accumulate=True, stream=st),
    ]
    for _ in range(args.warmup):
        for c in calls:
            c()
    torch.cuda.synchronize()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(len(calls) + 1)] for _ in range(args.steps)]
    t0 = time.perf_counter()
    for i in range(args.steps):
        evs[i][0].record(st)
        for j, c in enumerate(calls):
            c()
            evs[i][j + 1].record(st)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    per = {n: sum(e[j].elapsed_time(e[j + 1]) for e in evs) / args.steps for j, n in enumerate(names)}
    step_ms = sum(e[0].elapsed_time(e[-1]) for e in evs) / args.steps
    d, hq, hkv, dh = sh.d_model, sh.n_q_heads, sh.n_kv_heads, sh.d_head
    flops = {"qkv_proj": 2 * Kt * d * (hq + 2 * hkv) * dh,
             "o_proj": 2 * Kt * hq * dh * d, "gate_up_silu": 2 * Kt * d * 2 * F, "down": 2 * Kt * F * d,
             "attention": 4 * dh * hq * Kt * (Kt + 1) // 2}
    eb = 2
    hbm = {"in_norm": 2 * Kt * d * eb, "post_norm": 2 * Kt * d * eb,
           "qk_norm_rope": 2 * Kt * (hq + hkv) * dh * eb + Kt * 4}
    kern = {n: {"ms": per[n]} for n in names}
    for n, f in flops.items():
        kern[n]["TFLOP/s"] = f / (per[n] * 1e-3) / 1e12
        kern[n]["mfma_frac"] = kern[n]["TFLOP/s"] / BF16_PEAK_TFLOPS
    for n, b in hbm.items():
        kern[n]["GB/s"] = b / (per[n] * 1e-3) / 1e9
        kern[n]["hbm_frac"] = kern[n]["GB/s"] / HBM_PEAK_GBS
    gu = kern["gate_up_silu"]["TFLOP/s"]
    rec = {
        "metric": "pruned decoder layer tokens/s (context tokens per layer)",
        "value": w.total_tokens / (step_ms * 1e-3), "unit": "tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": wall * 1e3 / args.steps,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic (seeded; random-init Qwen3-1.7B-shaped layer)",
        "config": {"workload": "qwen3_1p7b_128k_layer", "tokens": w.total_tokens, "kept": Kt,
                   "d_model": d, "heads_q": hq, "heads_kv": hkv, "d_head": dh, "d_ffn": F},
        "roofline": {"bound": "mfma", "achieved": gu, "peak": BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                     "frac": gu / BF16_PEAK_TFLOPS, "traffic": None, "kernel": "gate|up projection with the SwiGLU product (tg_linear_swiglu)"},
        "kept_rows_per_s": Kt / (step_ms * 1e-3), "gpu_ms_per_layer": step_ms,
        "layer_TFLOP/s": sum(flops.values()) / (step_ms * 1e-3) / 1e12,
        "kernels": kern,
    }
    if not args.no_cpu_baseline:
        import oracle
        rows = 64
        Lc = {k: v.cpu() for k, v in L.items()}
        t0 = time.perf_counter()
        xn = oracle.rms_norm(x0[:rows].cpu(), Lc["in_norm"], eps)
        for nm in ("wq", "wk", "wv"):
            oracle.linear(xn, Lc[nm])
        h = oracle.linear(torch.zeros(rows, hq * dh, dtype=torch.float64), Lc["wo"])
        oracle.swiglu(oracle.rms_norm(h, Lc["post_norm"], eps), Lc["wg"], Lc["wu"], Lc["wd"])
        t_rows = (time.perf_counter() - t0) * Kt / rows
        t0 = time.perf_counter()
        q1 = layer.q[:, :2].cpu().contiguous()
        oracle.gated_attention(q1, layer.k[:, :1].cpu().contiguous(), layer.v[:, :1].cpu().contiguous(),
                               s.cpu(), Lc["gain"][:2], Lc["temp"][:2], cu_k)
        t_attn = (time.perf_counter() - t0) * hq / 2
        rec["cpu_baseline"] = {"value": w.total_tokens / (t_rows + t_attn), "unit": "tokens/s",
                               "cores": torch.get_num_threads(), "kind": "oracle",
                               "sample": (f"oracle row-wise steps on {rows} of {Kt} kept rows and "
                                          f"attention for 2 of {hq} heads, each scaled to the layer")}
    print(json.dumps(rec), flush=True)


def measure_config(w, args, dev, primary: bool):
    """One gated layer (plus the stack for the stack workload) of workload w:
    per-kernel HIP-event times over args.steps eager steps, the same step
    replayed as a HIP graph (checked bit for bit against the eager step),
    and each kernel again right after 512 MiB are written (evicting the
    256 MiB Infinity Cache).  With primary, also the context timings (the
    attention without its bias, the attention on all N tokens).  Returns the
    per-workload record and the objects the CPU baseline needs."""
    import torch

    import learned_token_pruning_02_amd as tg
    import workloads
    from learned_token_pruning_02_amd.path import AttentionStack, GatedLayer

    sh = w.shape
    gi = workloads.gate_inputs(w, seed=args.seed)
    ai = workloads.attn_inputs(w, seed=args.seed)
    g = {k: (None if v is None else v.to(dev)) for k, v in gi.items()}
    a = {k: v.to(dev) for k, v in ai.items()}
    layer = GatedLayer(w.total_tokens, sh.d_model, sh.n_q_heads, sh.d_head, w.seq_len, w.q_len,
                       w.budget, sh.dtype, device=dev, n_kv_heads=sh.n_kv_heads)
    stack = None
    if w.stack_layers:
        stack = AttentionStack(layer.Kt, sh.d_model, sh.n_q_heads, sh.n_kv_heads, sh.d_head,
                               sh.dtype, device=dev)
        sw = [{k: v.to(dev) for k, v in L.items()} for L in workloads.stack_weights(w, args.seed)]
        x_stack = torch.empty_like(layer.hidden_kept)

    names = ["gate", "select", "gather", "attention"] + (["stack"] if stack else [])

    def step(ev=None):
        if ev is not None:
            ev[0].record()
        layer.gate(g["hidden"], g["w1"], g["b1"], g["w2"], g["b2"])
        if ev is not None:
            ev[1].record()
        layer.select()
        if ev is not None:
            ev[2].record()
        layer.gather(g["hidden"])
        if ev is not None:
            ev[3].record()
        layer.attend(a["q"], a["k"], a["v"], a["gain"], a["temp"])
        if ev is not None:
            ev[4].record()
        if stack is not None:
            x_stack.copy_(layer.hidden_kept)
            stack(x_stack, layer.s_kept, layer.cu_kept, sw)
            if ev is not None:
                ev[5].record()

    # Untimed warm-up: W steps for the named workload; the other workloads,
    # whose steps are shorter, run at least WARM_S seconds of steps, so that
    # each is timed at the chip's steady clocks.
    nwarm = args.warmup
    if not primary:
        for _ in range(3):
            step()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(3):
            step()
        torch.cuda.synchronize()
        nwarm = max(args.warmup, int(WARM_S / max((time.perf_counter() - t0) / 3, 1e-6)))
    for _ in range(nwarm):
        step()
    torch.cuda.synchronize()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(len(names) + 1)]
           for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(evs[i])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    samples = {n: sorted(e[j].elapsed_time(e[j + 1]) for e in evs) for j, n in enumerate(names)}
    per = {n: sum(v) / len(v) for n, v in samples.items()}  # ms per launch (mean)
    gpu_ms = evs[0][0].elapsed_time(evs[-1][-1]) / args.steps
    ms_per_step_eager = wall * 1e3 / args.steps

    # The whole step (every shape is fixed by the host-side plan, nothing in
    # it reads back to the host or clears memory with a memset) captured once
    # as a HIP graph; K replays are timed, and every replay must reproduce
    # the eager step's outputs bit for bit.
    ref_out, ref_kept = layer.out.clone(), layer.kept.clone()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    layer.out.zero_()
    graph.replay()
    torch.cuda.synchronize()
    if not (torch.equal(layer.out, ref_out) and torch.equal(layer.kept, ref_kept)):
        raise RuntimeError(f"{w.name}: graph replay of the step does not reproduce the eager step")
    for _ in range(nwarm):  # the capture left the GPU idle: warm up again
        graph.replay()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        graph.replay()
    torch.cuda.synchronize()
    ms_per_step_graph = (time.perf_counter() - t0) * 1e3 / args.steps
    if not (torch.equal(layer.out, ref_out) and torch.equal(layer.kept, ref_kept)):
        raise RuntimeError(f"{w.name}: the timed graph replays do not reproduce the eager step")
    del graph

    # Each kernel again right after 512 MiB are written (the 256 MiB Infinity
    # Cache then holds none of its inputs), on the outputs of the last step.
    flush = torch.empty(512 << 20, dtype=torch.uint8, device=dev)
    calls = {"gate": lambda: layer.gate(g["hidden"], g["w1"], g["b1"], g["w2"], g["b2"]),
             "select": layer.select,
             "gather": lambda: layer.gather(g["hidden"]),
             "attention": lambda: layer.attend(a["q"], a["k"], a["v"], a["gain"], a["temp"])}
    cold = {}
    for n, fn in calls.items():
        ms = []
        for _ in range(5):
            flush.fill_(1)
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            fn()
            e1.record()
            torch.cuda.synchronize()
            ms.append(e0.elapsed_time(e1))
        ms.sort()
        cold[n] = {"ms_median": ms[len(ms) // 2], "ms_min": ms[0]}
    del flush

    kept_per_req = [layer.cu_kept[i + 1] - layer.cu_kept[i] for i in range(w.batch)]
    alg = algorithmic(w, kept_per_req)
    bf16 = sh.dtype == torch.bfloat16
    mfma_peak = BF16_PEAK_TFLOPS if bf16 else F32_PEAK_TFLOPS
    kernels = {}
    for n in ["gate", "select", "gather", "attention"]:
        t = per[n] * 1e-3
        tc = cold[n]["ms_median"] * 1e-3
        kernels[n] = {"ms": per[n], "ms_median": samples[n][len(samples[n]) // 2],
                      "ms_min": samples[n][0], "GB/s": alg[n]["bytes"] / t / 1e9,
                      "hbm_frac": alg[n]["bytes"] / t / 1e9 / HBM_PEAK_GBS,
                      "TFLOP/s": alg[n]["flops"] / t / 1e12,
                      "ms_cold": cold[n]["ms_median"],
                      "hbm_frac_cold": alg[n]["bytes"] / tc / 1e9 / HBM_PEAK_GBS}
        if n in ("gate", "attention"):
            kernels[n]["mfma_frac"] = kernels[n]["TFLOP/s"] / mfma_peak
    if stack is not None:
        kernels["stack"] = {"ms": per["stack"]}

    derived = None
    if primary:
        def timed(fn, reps, warm=50):
            ev = [torch.cuda.Event(enable_timing=True) for _ in range(reps + 1)]
            for _ in range(warm):
                fn()
            ev[0].record()
            for i in range(reps):
                fn()
                ev[i + 1].record()
            torch.cuda.synchronize()
            return sorted(ev[i].elapsed_time(ev[i + 1]) for i in range(reps))

        # The bias overhead: the same attention kernel built without the bias
        # stage (s_kept = gain = NULL), same inputs, same stream.
        nobias_out = torch.empty_like(layer.out)
        t_bias = timed(lambda: layer.attend(a["q"], a["k"], a["v"], a["gain"], a["temp"]), 10)
        t_nobias = t_bias if args.no_context else timed(
            lambda: tg.tg_gated_attn_prefill(a["q"], a["k"], a["v"], None, None, a["temp"],
                                             layer.cu_kept, out=nobias_out), 10)
        # Context: the same kernel on every token of the prompt without
        # pruning (no bias, temperature 1).
        t_full = [float("nan")]
        if not args.no_context:
            gfull = torch.Generator(device=dev).manual_seed(args.seed + 7)
            Tn = w.total_tokens
            qf = torch.randn(Tn, sh.n_q_heads, sh.d_head, device=dev, generator=gfull).to(sh.dtype)
            kf = torch.randn(Tn, sh.n_kv_heads, sh.d_head, device=dev, generator=gfull).to(sh.dtype)
            vf = torch.randn(Tn, sh.n_kv_heads, sh.d_head, device=dev, generator=gfull).to(sh.dtype)
            of = torch.empty_like(qf)
            ones = torch.ones(sh.n_q_heads, device=dev)
            t_full = timed(lambda: tg.tg_gated_attn_prefill(qf, kf, vf, None, None, ones, layer.cu_seq,
                                                            out=of), 3, warm=2)
            del qf, kf, vf, of
        eb = 2 if bf16 else 4
        kv_row = 2 * sh.n_kv_heads * sh.d_head * eb
        derived = {
            "attn_layer_tok_s": w.total_tokens / (per["attention"] * 1e-3),
            "kept_tok_s": layer.Kt / (per["attention"] * 1e-3),
            "bias_overhead": t_bias[len(t_bias) // 2] / t_nobias[len(t_nobias) // 2],
            "attn_ms_median_bias": t_bias[len(t_bias) // 2],
            "attn_ms_median_nobias": t_nobias[len(t_nobias) // 2],
            "kv_bytes_kept": layer.Kt * kv_row,
            "kv_bytes_full": w.total_tokens * kv_row,
            "full_prefill_attn_ms_median": t_full[len(t_full) // 2],
            "attention_saving": t_full[len(t_full) // 2] / t_bias[len(t_bias) // 2],
        }

    summary = {
        "tokens": w.total_tokens, "kept": layer.Kt, "requests": w.batch, "warmup_steps": nwarm,
        "dtype": "bf16" if bf16 else "f32", "stack_layers": w.stack_layers,
        "ms_per_step": ms_per_step_eager, "ms_per_step_graph": ms_per_step_graph,
        "tokens_per_s": w.total_tokens / (ms_per_step_eager * 1e-3),
        "tokens_per_s_graph": w.total_tokens / (ms_per_step_graph * 1e-3),
        "kernels_us": {n: round(v["ms"] * 1e3, 2) for n, v in kernels.items()},
        "kernels_us_cold": {n: round(cold[n]["ms_median"] * 1e3, 2) for n in cold},
        "gate_hbm_frac": kernels["gate"]["hbm_frac"],
        "gate_hbm_frac_cold": kernels["gate"]["hbm_frac_cold"],
        "gather_hbm_frac": kernels["gather"]["hbm_frac"],
        "gather_hbm_frac_cold": kernels["gather"]["hbm_frac_cold"],
        "attn_mfma_frac": kernels["attention"]["mfma_frac"],
        "select_us": kernels["select"]["ms"] * 1e3,
    }
    res = {"summary": summary, "kernels": kernels, "cold": cold, "derived": derived,
           "per": per, "gpu_ms": gpu_ms, "ms_per_step_eager": ms_per_step_eager,
           "ms_per_step_graph": ms_per_step_graph, "bf16": bf16, "mfma_peak": mfma_peak,
           "Kt": layer.Kt, "cu_kept": list(layer.cu_kept)}
    if primary and not args.no_cpu_baseline:
        res["cpu_inputs"] = (gi, ai, layer.scores.cpu(), layer.kept.cpu())
    del layer, stack, g, a
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    return res


def main():
    args = parse()
    if args.copy_calibration:
        copy_calibration()
        return
    if args.layer:
        if args.gpus != 1:
            print(f"bench.py runs on one GPU only; --gpus {args.gpus} is not supported", flush=True)
            sys.exit(2)
        layer_bench(args)
        return
    if args.backward:
        if args.gpus != 1:
            print(f"bench.py runs on one GPU only; --gpus {args.gpus} is not supported", flush=True)
            sys.exit(2)
        backward_bench(args)
        return
    if args.decode:
        if args.gpus != 1:
            print(f"bench.py runs on one GPU only; --gpus {args.gpus} is not supported", flush=True)
            sys.exit(2)
        decode_bench(args)
        return
    if args.select_sweep:
        select_sweep()
        return
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only; --gpus {args.gpus} is not supported "
              "(the path is single-GPU; sharding is a design note, not built)", file=sys.stderr)
        sys.exit(2)

    import torch

    import learned_token_pruning_02_amd as tg
    import workloads

    tg.lib()  # fail loudly when the library is missing
    if not torch.cuda.is_available():
        raise RuntimeError("bench.py needs a GPU")
    dev = torch.device("cuda:0")
    w = workloads.get(args.workload, args.seed)
    sh = w.shape

    main_res = measure_config(w, args, dev, primary=True)
    configs = {w.name: main_res["summary"]}
    if not args.no_configs:
        # Every other workload of the same layer shape (and the tiny fp32
        # one): per-config step time, throughput, per-kernel warm and cold
        # times and their roofline fractions.
        for name in workloads.WORKLOADS:
            if name == w.name:
                continue
            other = workloads.get(name, args.seed)
            print(f"[bench] {name}", file=sys.stderr, flush=True)
            configs[name] = measure_config(other, args, dev, primary=False)["summary"]

    per = main_res["per"]
    kernels = main_res["kernels"]
    bf16 = main_res["bf16"]
    ms_per_step = main_res["ms_per_step_eager"]
    launch = "eager (one launch per kernel)"
    if args.graph:
        ms_per_step = main_res["ms_per_step_graph"]
        launch = "hip graph (one step captured, replayed)"

    dominant = max(["gate", "select", "gather", "attention"], key=lambda n: per[n])
    if dominant == "attention":
        roof = {"bound": "mfma" if bf16 else "alu", "achieved": kernels["attention"]["TFLOP/s"],
                "peak": main_res["mfma_peak"], "unit": "TFLOP/s"}
    else:
        roof = {"bound": "hbm", "achieved": kernels[dominant]["GB/s"], "peak": HBM_PEAK_GBS,
                "unit": "GB/s"}
    roof["frac"] = roof["achieved"] / roof["peak"]
    roof["traffic"] = recorded_traffic(w.name, dominant)
    roof["kernel"] = dominant

    cpu = None
    if "cpu_inputs" in main_res:
        gi, ai, s_cpu, kept_cpu = main_res["cpu_inputs"]
        cpu = cpu_baseline(w, gi, ai, s_cpu, kept_cpu, main_res["cu_kept"])

    line = {
        "metric": "gated-prefill tokens/s per layer",
        "value": w.total_tokens / (ms_per_step * 1e-3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if bf16 else "f32",
        "data": "synthetic (seeded; random-init gate and projection weights)",
        "config": {"workload": w.name, "tokens": w.total_tokens, "kept": main_res["Kt"],
                   "requests": w.batch, "d_model": sh.d_model, "heads_q": sh.n_q_heads,
                   "heads_kv": sh.n_kv_heads, "d_head": sh.d_head, "d_gate": sh.d_gate,
                   "stack_layers": w.stack_layers},
        "roofline": roof,
        "cpu_baseline": cpu,
        "kernels": kernels,
        "derived": main_res["derived"],
        "gpu_ms_per_step": main_res["gpu_ms"],
        "launch": launch,
        "ms_per_step_eager": main_res["ms_per_step_eager"],
        "ms_per_step_graph": main_res["ms_per_step_graph"],
        "cold_after_cache_flush": main_res["cold"],
        "configs": configs,
    }
    if args.detail:
        with open(args.detail, "w") as f:
            json.dump(line, f, indent=1)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
