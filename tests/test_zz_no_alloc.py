"""tg_topk_select_noalloc, the selector whose workspace is the library's static
device scratch, against tg_topk_select with a caller workspace: kept ids and
the device cu_kept bit-exact, on two calls in a row (the second on a smaller
batch, so the scratch still holds the first call's contents), and both equal
to the oracle's selection."""
import pytest
import torch

import learned_token_pruning_02_amd as tg
import oracle
from parity_util import announce

pytestmark = pytest.mark.gpu


def _scores(T, seed):
    # Scores rounded to bf16 precision, so that many of them tie.
    g = torch.Generator().manual_seed(seed)
    return torch.randn(T, generator=g).to(torch.bfloat16).float()


def _both(seq, q, bud, seed):
    s = _scores(sum(seq), seed)
    ref, cu_ref = oracle.topk_select(s, seq, q, bud)
    sg = s.cuda()
    announce(f"noalloc select B={len(seq)} T={sum(seq)} seq={seq} q={q} budget={bud}")
    kept_ws, cu_ws = tg.tg_topk_select(sg, seq, q, bud)
    kept = torch.full((cu_ref[-1],), -1, dtype=torch.int32, device="cuda")
    cu_dev = torch.full((len(seq) + 1,), -1, dtype=torch.int32, device="cuda")
    cu = tg.tg_topk_select_noalloc(sg, seq, q, bud, kept, cu_kept_dev=cu_dev)
    torch.cuda.synchronize()
    assert cu == cu_ws == cu_ref
    assert cu_dev.cpu().tolist() == cu_ref
    assert torch.equal(kept.cpu(), kept_ws.cpu()), "noalloc differs from tg_topk_select"
    assert torch.equal(kept.cpu(), ref), "noalloc differs from the oracle"


def test_noalloc_matches_select_two_calls():
    # 1: one 128k request on the chunked path (the scratch in use);
    # 2: a smaller varlen batch, also chunked (one document > 32768 tokens).
    _both([131072], [128], [8192], seed=11)
    _both([70000, 3000, 500], [64, 100, 500], [9000, 700, 600], seed=12)


def test_noalloc_small_batch_uses_no_scratch():
    # Every document takes the one-workgroup path: no scratch at all.
    _both([30000, 16384, 2048], [128, 128, 64], [3000, 2048, 256], seed=13)
