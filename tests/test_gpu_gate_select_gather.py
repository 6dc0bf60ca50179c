"""GPU parity of the gate, the top-K selector and the gather against the oracle.

Gate scores: within the fp32 (1e-5) or bf16 (2e-2 relative / 1e-2 absolute)
tolerance.  Selection, run on the oracle's fp32 scores: bit-exact kept ids.
Gather: bitwise.
"""
import math

import pytest
import torch

import learned_token_pruning_02_amd as tg
import oracle
import workloads
from parity_util import announce, assert_within, tol

pytestmark = pytest.mark.gpu


def _shape(d, dg, dtype, hq=4, hkv=2, dh=64):
    return workloads.LayerShape(d, hq, hkv, dh, dg, dtype)


def _wl(name, shape, seq, q, bud, needles=0):
    return workloads.Workload(name, shape, list(seq), list(q), list(bud), n_needles=needles)


# ------------------------------------------------------------------ gate ----
GATE_CASES = [
    ("tiny_fp32", None, True),
    ("tiny_fp32", None, False),
    ("fp32_T77_d64_dg200", (77, 64, 200, torch.float32), True),
    ("bf16_T3000_d2048_dg256", (3000, 2048, 256, torch.bfloat16), True),
    ("bf16_T3000_d2048_dg256_nobias", (3000, 2048, 256, torch.bfloat16), False),
    ("bf16_T700_d128_dg64", (700, 128, 64, torch.bfloat16), False),
    ("bf16_T1000_d256_dg128", (1000, 256, 128, torch.bfloat16), True),
    ("bf16_T1_d64_dg64", (1, 64, 64, torch.bfloat16), True),
    ("bf16_T16383_d2048_dg256", (16383, 2048, 256, torch.bfloat16), True),  # units split, ragged tail
    ("bf16_T16385_d2048_dg256", (16385, 2048, 256, torch.bfloat16), False), # 128-token tiles
    ("bf16_T65535_d128_dg256", (65535, 128, 256, torch.bfloat16), True),     # 128-token tiles
    ("bf16_T70001_d128_dg256", (70001, 128, 256, torch.bfloat16), True),     # 256-token tiles
    ("bf16_T65536_d192_dg256_nobias", (65536, 192, 256, torch.bfloat16), False),  # same, three k chunks
    ("bf16_T131109_d128_dg256", (131109, 128, 256, torch.bfloat16), True),   # same, ragged tail
    ("bf16_T131109_d128_dg128", (131109, 128, 128, torch.bfloat16), True),   # same, d_gate 128
    ("qwen3_1p7b_16k", None, True),
]


@pytest.mark.parametrize("name,spec,bias", GATE_CASES, ids=[c[0] + ("" if c[2] else "-nobias") for c in GATE_CASES])
def test_gate_parity(name, spec, bias):
    if spec is None:
        w = workloads.WORKLOADS[name]
    else:
        T, d, dg, dt = spec
        w = _wl(name, _shape(d, dg, dt), [T], [0], [T])
    announce(f"gate {name} bias={bias} T={w.total_tokens} d={w.shape.d_model} dg={w.shape.d_gate}")
    inp = workloads.gate_inputs(w, seed=3, with_bias=bias)
    ref = oracle.gate_score(inp["hidden"], inp["w1"], inp["b1"], inp["w2"], inp["b2"])
    g = {k: (v.cuda() if v is not None else None) for k, v in inp.items()}
    got = tg.tg_gate_score(g["hidden"], g["w1"], g["b1"], g["w2"], g["b2"])
    torch.cuda.synchronize()
    rtol, atol = tol(w.shape.dtype)
    assert_within(got, ref, rtol, atol, f"gate {name}")


def test_gate_full_128k_sampled_rows():
    """The 128k-token layer in the launch configuration the benchmark times,
    checked on sampled rows (all needles, the ends, random rows)."""
    w = workloads.WORKLOADS["qwen3_1p7b_128k_niah"]
    announce("gate 128k sampled")
    inp = workloads.gate_inputs(w, seed=0)
    g = {k: v.cuda() for k, v in inp.items()}
    got = tg.tg_gate_score(g["hidden"], g["w1"], g["b1"], g["w2"], g["b2"]).cpu()
    gen = torch.Generator().manual_seed(5)
    rows = torch.cat([torch.tensor([0, 1, 255, 256, w.total_tokens - 1]),
                      workloads.needle_positions(w, 0),
                      torch.randint(0, w.total_tokens, (3000,), generator=gen)]).unique()
    ref = oracle.gate_score(inp["hidden"][rows], inp["w1"], inp["b1"], inp["w2"], inp["b2"])
    assert_within(got[rows], ref, 2e-2, 1e-2, "gate 128k sampled")


def test_gate_deterministic():
    w = _wl("det", _shape(512, 256, torch.bfloat16), [4099], [0], [4099])
    inp = {k: v.cuda() for k, v in workloads.gate_inputs(w, seed=9).items()}
    a = tg.tg_gate_score(inp["hidden"], inp["w1"], inp["b1"], inp["w2"], inp["b2"]).clone()
    b = tg.tg_gate_score(inp["hidden"], inp["w1"], inp["b1"], inp["w2"], inp["b2"])
    assert torch.equal(a.view(torch.int32), b.view(torch.int32))


# ---------------------------------------------------------------- select ----
def _select_case(seq, q, bud, scores, prefix=None):
    """Both implementations (one workgroup per request when every document
    fits in LDS, the chunked multi-workgroup path otherwise or when forced)
    must give the oracle's kept ids bit for bit, and the device cu_kept."""
    ref, cu_ref = oracle.topk_select(scores, seq, q, bud, prefix)
    sg = scores.cuda()
    # path 0: the library's choice; 2: the chunked path forced.
    for path in (0, 2):
        announce(f"select[path {path}] B={len(seq)} T={sum(seq)} seq={seq[:4]} q={q[:4]} budget={bud[:4]}"
                 + ("" if prefix is None else f" prefix={prefix[:4]}"))
        cu_dev = torch.full((len(seq) + 1,), -1, dtype=torch.int32, device="cuda")
        got, cu = tg.tg_topk_select(sg, seq, q, bud, cu_kept_dev=cu_dev, prefix_len=prefix, path=path)
        torch.cuda.synchronize()
        assert cu == cu_ref
        assert cu_dev.cpu().tolist() == cu_ref, f"{path}: device cu_kept"
        assert torch.equal(got.cpu(), ref), f"{path}: kept ids differ"


@pytest.mark.parametrize("wname", list(workloads.WORKLOADS))
def test_select_workload_shapes_random_scores(wname):
    w = workloads.WORKLOADS[wname]
    _select_case(w.seq_len, w.q_len, w.budget, workloads.random_scores(w.total_tokens, seed=4))


def test_select_on_oracle_gate_scores_16k():
    w = workloads.WORKLOADS["qwen3_1p7b_16k"]
    inp = workloads.gate_inputs(w, seed=0)
    s = oracle.gate_score(inp["hidden"], inp["w1"], inp["b1"], inp["w2"], inp["b2"])
    _select_case(w.seq_len, w.q_len, w.budget, s)


@pytest.mark.parametrize("levels", [3, 50, 1000])
def test_select_heavy_ties(levels):
    T = 40000
    _select_case([T], [100], [5000], workloads.random_scores(T, seed=6, ties=levels))


def test_select_all_equal():
    T = 50000
    _select_case([T], [64], [7000], torch.full((T,), 0.3125))


def test_select_specials():
    g = torch.Generator().manual_seed(7)
    T = 20000
    s = torch.randn(T, generator=g)
    specials = torch.tensor([float("nan"), -0.0, 0.0, float("inf"), float("-inf")])
    pos = torch.randint(0, T - 50, (4000,), generator=g)
    s[pos] = specials[torch.randint(0, 5, (4000,), generator=g)]
    for bud in (60, 2000, 9000, 16000, 19999):
        _select_case([T], [50], [bud], s)


def test_select_budget_edges():
    g = torch.Generator().manual_seed(8)
    seq = [1, 1, 2, 5, 300, 300, 300, 4096, 17000, 9]
    q = [0, 1, 0, 5, 0, 100, 299, 128, 0, 3]
    bud = [1, 1, 1, 5, 1, 100, 400, 4096, 16999, 4]
    s = torch.randn(sum(seq), generator=g)
    _select_case(seq, q, bud, s)


def test_select_max_batch_and_large_request():
    g = torch.Generator().manual_seed(9)
    seq = [int(x) for x in torch.randint(1, 3000, (tg.TG_MAX_BATCH,), generator=g)]
    q = [min(n, int(x)) for n, x in zip(seq, torch.randint(0, 300, (len(seq),), generator=g))]
    bud = [max(qq, 1) + int(x) for qq, x in zip(q, torch.randint(0, 1500, (len(seq),), generator=g))]
    _select_case(seq, q, bud, torch.randn(sum(seq), generator=g))
    T = 1 << 20
    _select_case([T], [128], [T // 16], workloads.random_scores(T, seed=10))


def test_select_one_workgroup_limits():
    """Documents of exactly 65536 tokens (the largest the one-workgroup path
    takes), 65537 (chunked path), ties across the threshold, NaN and +-0, a
    budget of one, and a batch mixing keep-all requests."""
    g = torch.Generator().manual_seed(30)
    L = 65536
    s = workloads.random_scores(L + 64, seed=31, ties=300)
    s[torch.randint(0, L, (500,), generator=g)] = float("nan")
    s[torch.randint(0, L, (500,), generator=g)] = -0.0
    _select_case([L + 64], [64], [5000], s)
    _select_case([L + 65], [64], [5000], workloads.random_scores(L + 65, seed=32, ties=300))
    _select_case([40000], [1], [1], workloads.random_scores(40000, seed=33))
    seq = [100, 20000, 7, 32768, 513, 20000]                 # the last keeps only its question token
    _select_case(seq, [10, 100, 7, 0, 13, 1], [100, 3000, 9, 30000, 64, 1], torch.randn(sum(seq), generator=g))


def test_select_one_workgroup_bins():
    """The one-workgroup path's key range comes from a sample and its bins
    are linear in it: keys far outside the sampled range (a few huge and tiny
    scores), a threshold inside the end bins, and a threshold bin with more
    candidates than are ranked in LDS (then the radix passes rank it)."""
    g = torch.Generator().manual_seed(34)
    T = 60000
    s = torch.randn(T, generator=g)
    s[torch.randint(0, T, (7,), generator=g)] = 1e30       # outliers beyond the binned range
    s[torch.randint(0, T, (7,), generator=g)] = -1e30
    for bud in (3, 20, 30000, 59990):                       # thresholds at the ends of the range
        _select_case([T], [0], [bud], s)
    # 3000 copies of one value straddling the threshold: bin d is too big to rank in LDS
    s2 = torch.randn(T, generator=g)
    s2[torch.randint(0, T, (3000,), generator=g)] = 1.0
    n_above = int((s2 > 1.0).sum())
    _select_case([T], [10], [n_above + 1500], s2)
    # a bf16-rounded normal: many small ties, a modest candidate set
    _select_case([T], [128], [T // 8], torch.randn(T, generator=g).to(torch.bfloat16).float())


@pytest.mark.parametrize("n", [1, 2, 383, 384, 385, 1000, 9000])
def test_select_chunked_bins_candidates(n):
    """The chunked path bins linearly over the range of the document's first
    chunk.  Here that chunk holds the largest ordinary score (5.0), so the
    top bin holds exactly the n planted scores above it: n straddles the
    count the last workgroup ranks by counting (384), the LDS radix passes
    and the passes that read the candidates from global memory.  Planted
    scores equal (ranked by index alone) and distinct (by value)."""
    g = torch.Generator().manual_seed(40 + n)
    T = 100_000
    s = torch.randn(T, generator=g).clamp(-4.9, 4.9)
    s[0] = 5.0
    pos = 2048 + torch.randperm(T - 2048 - 64, generator=g)[:n]
    for distinct in (False, True):
        x = s.clone()
        x[pos] = 10.0 + (torch.randperm(n, generator=g).float() * 1e-3 if distinct else 0.0)
        _select_case([T], [64], [64 + (n + 1) // 2], x)
    if n in (1, 1000):
        # a first chunk far narrower than the rest: most keys clamp to the
        # end bins, and the threshold bin holds ~T/2 candidates
        y = torch.randn(T, generator=g)
        y[:2048] *= 1e-3
        _select_case([T], [64], [64 + 3 * n], y)


def test_select_sweep_scale():
    """The selector at the throughput sweep's scale (one request, no tail,
    K = T/16), bit-exact against the oracle."""
    T = 1 << 24
    _select_case([T], [0], [T // 16], workloads.random_scores(T, seed=11))


@pytest.mark.parametrize("levels", [0, 40, 5000])
def test_select_large_document_path(levels):
    """Documents above 2^20 tokens rank their threshold candidates with every
    workgroup; with heavy ties the passes run down to the index digits."""
    T = (1 << 21) + 5
    s = workloads.random_scores(T, seed=12, ties=levels) if levels else workloads.random_scores(T, seed=12)
    _select_case([T], [77], [T // 10], s)


def test_select_large_document_in_a_batch():
    """One large document switches the whole batch to the many-workgroup
    ranking; the small requests must come out the same."""
    seq = [(1 << 20) + 3000, 5000, 70000, 9]
    q = [100, 10, 0, 3]
    bud = [300000, 4000, 6000, 4]
    g = torch.Generator().manual_seed(13)
    s = torch.randn(sum(seq), generator=g)
    s[(1 << 20):(1 << 20) + 2000] = 0.5  # a run of equal scores near the first threshold
    _select_case(seq, q, bud, s)


def test_select_grouped_chunks():
    """Beyond 2048 chunks of 2048 keys, each workgroup of the chunked path
    takes a group of consecutive chunks (one ticket, one histogram flush and
    one candidate append per group): a batch that crosses that line, and a
    large document with heavy ties."""
    seq = [(1 << 22) + 77, 3000, 100000, 5]
    q = [0, 10, 64, 5]
    bud = [(1 << 18) + 5, 2000, 9000, 5]
    g = torch.Generator().manual_seed(14)
    s = torch.randn(sum(seq), generator=g)
    s[5000:9000] = 1.5  # a run of equal scores near the threshold of the large request
    _select_case(seq, q, bud, s)
    T = (1 << 23) + 11
    _select_case([T], [3], [T // 16], workloads.random_scores(T, seed=15, ties=40))


# ----------------------------------------------- select: template prefix ----
def _prefixes(seq, q, bud, g, cap=600):
    return [int(torch.randint(0, max(1, min(cap, min(b, n) - qq) + 1), (1,), generator=g))
            for n, qq, b in zip(seq, q, bud)]


@pytest.mark.parametrize("wname", list(workloads.WORKLOADS))
def test_select_prefix_workload_shapes(wname):
    """An always-kept template prefix in front of every document."""
    w = workloads.WORKLOADS[wname]
    g = torch.Generator().manual_seed(21)
    _select_case(w.seq_len, w.q_len, w.budget, workloads.random_scores(w.total_tokens, seed=22),
                 _prefixes(w.seq_len, w.q_len, w.budget, g))


def test_select_prefix_edges():
    """Prefix only, prefix + question filling the budget, an empty document,
    a budget covering the request, ties across the prefix boundary."""
    g = torch.Generator().manual_seed(23)
    seq = [1, 2, 300, 300, 300, 4096, 17000, 9, 5000, 777]
    q = [0, 0, 0, 100, 50, 128, 0, 3, 64, 0]
    bud = [1, 1, 120, 150, 400, 4096, 9000, 9, 700, 100]
    pre = [1, 1, 120, 50, 250, 3968, 8999, 6, 33, 0]
    s = torch.randn(sum(seq), generator=g)
    s[1000:1300] = 0.75  # equal scores straddling a prefix boundary
    _select_case(seq, q, bud, s, pre)


def test_select_prefix_specials_and_ties():
    g = torch.Generator().manual_seed(24)
    T = 30000
    s = workloads.random_scores(T, seed=25, ties=20)
    specials = torch.tensor([float("nan"), -0.0, 0.0, float("inf"), float("-inf")])
    pos = torch.randint(0, T, (3000,), generator=g)
    s[pos] = specials[torch.randint(0, 5, (3000,), generator=g)]
    for bud, pre in ((300, 200), (4000, 1), (12000, 5000), (29000, 28900)):
        _select_case([T], [100], [bud], s, [pre])


def test_select_prefix_max_batch_and_large_document():
    g = torch.Generator().manual_seed(26)
    seq = [int(x) for x in torch.randint(1, 3000, (tg.TG_MAX_BATCH,), generator=g)]
    q = [min(n, int(x)) for n, x in zip(seq, torch.randint(0, 300, (len(seq),), generator=g))]
    bud = [max(qq, 1) + int(x) for qq, x in zip(q, torch.randint(0, 1500, (len(seq),), generator=g))]
    _select_case(seq, q, bud, torch.randn(sum(seq), generator=g), _prefixes(seq, q, bud, g))
    T = (1 << 21) + 5   # the many-workgroup ranking of documents above 2^20 tokens
    _select_case([T], [77], [T // 10], workloads.random_scores(T, seed=27, ties=40), [1500])


def test_select_random_keys():
    """Random-K selection: the selector run on caller-drawn uniform keys."""
    w = workloads.WORKLOADS["qwen3_1p7b_16k"]
    keys = torch.rand(w.total_tokens, generator=torch.Generator().manual_seed(28))
    _select_case(w.seq_len, w.q_len, w.budget, keys)
    _select_case(w.seq_len, w.q_len, w.budget, keys, [16] * len(w.seq_len))


# ---------------------------------------------------------------- gather ----
@pytest.mark.parametrize("dtype,d,T,Kt", [
    (torch.bfloat16, 2048, 5000, 777),    # 4 KiB rows: one pass of four loads per lane
    (torch.bfloat16, 2048, 20000, 9000),  # the 128k layer's row size, more rows
    (torch.bfloat16, 4096, 5000, 777),    # 8 KiB rows: two passes
    (torch.float32, 2048, 3000, 1500),    # fp32 8 KiB rows
    (torch.float32, 256, 5000, 777),      # 1 KiB rows: the tail loop only
    (torch.bfloat16, 8, 5000, 777),       # 16-byte rows: one lane per row
])
def test_gather_bitwise(dtype, d, T, Kt):
    announce(f"gather {dtype} d={d} T={T} Kt={Kt}")
    g = torch.Generator().manual_seed(11)
    hidden = torch.randn(T, d, generator=g).to(dtype)
    s = torch.randn(T, generator=g)
    kept = torch.sort(torch.randperm(T, generator=g)[:Kt]).values.to(torch.int32)
    hk, sk = tg.tg_gather_compact(hidden.cuda(), kept.cuda(), s.cuda())
    rh, rs = oracle.gather_compact(hidden, s, kept)
    bits = torch.int16 if dtype == torch.bfloat16 else torch.int32
    assert torch.equal(hk.cpu().view(bits), rh.view(bits))
    assert torch.equal(sk.cpu().view(torch.int32), rs.view(torch.int32))


@pytest.mark.parametrize("d", [64, 2048])
def test_gather_out_of_range_rows_untouched(d):
    T = 100
    hidden = torch.randn(T, d).to(torch.bfloat16).cuda()
    s = torch.randn(T).cuda()
    kept = torch.tensor([3, -1, 99, 100, 7], dtype=torch.int32).cuda()
    out = torch.full((5, d), 7.0, dtype=torch.bfloat16, device="cuda")
    sk = torch.zeros(5, device="cuda")
    tg.tg_gather_compact(hidden, kept, s, hidden_kept=out, scores_kept=sk)
    out, sk = out.cpu(), sk.cpu()
    assert torch.equal(out[0], hidden[3].cpu()) and torch.equal(out[2], hidden[99].cpu())
    assert torch.equal(out[4], hidden[7].cpu())
    assert (out[1] == 7.0).all() and (out[3] == 7.0).all()
    assert math.isnan(sk[1]) and math.isnan(sk[3]) and sk[0] == s[3].cpu()
