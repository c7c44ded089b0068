"""Relaxed chain verification on the GPU (eagle3_relaxed_accept through the C
ABI): accept lengths and bonus ids bit-exact against the oracle."""
import numpy as np
import pytest
import torch

import oracle
import workloads as W
from eagle_draft_head_step_amd import binding

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")


def _run(draft, logits, relaxed, topk, delta):
    B = draft.shape[0]
    acc = torch.full((B,), -7, dtype=torch.int32, device=DEV)
    bon = torch.full((B,), -7, dtype=torch.int32, device=DEV)
    binding.relaxed_accept(draft.to(DEV).contiguous(), logits.to(DEV).contiguous(),
                           None if relaxed is None else relaxed.to(DEV).contiguous(), topk, delta, acc, bon)
    torch.cuda.synchronize()
    return acc.cpu().long(), bon.cpu().long()


def _check(tag, draft, logits, relaxed, topk, delta):
    print(f"[relaxed] {tag}", flush=True)
    a, b = _run(draft, logits, relaxed, topk, delta)
    ra, rb = oracle.relaxed_accept(draft, logits, relaxed, topk, delta)
    assert torch.equal(a, ra), (tag, (a != ra).nonzero()[:5].flatten().tolist())
    assert torch.equal(b, rb), (tag, (b != rb).nonzero()[:5].flatten().tolist())
    return a


@pytest.mark.parametrize("vocab", [3000, 2999, 129280])
@pytest.mark.parametrize("seed", [0, 1])
def test_relaxed_parity_planted(vocab, seed):
    cfg = W.get_config("mla_small")
    B = 64 if vocab < 10000 else 16
    x = W.make_relaxed_inputs(cfg, seed, batch=B, vocab=vocab)
    a = _check(f"V={vocab} seed={seed}", x["draft"], x["logits"], x["relaxed"], cfg.relaxed_topk,
               cfg.relaxed_delta)
    assert len(set(a.tolist())) > 1
    _check(f"V={vocab} seed={seed} all relaxed", x["draft"], x["logits"], None, cfg.relaxed_topk,
           cfg.relaxed_delta)
    for topk, delta in ((1, 0.6), (3, 0.0), (12, 0.25), (vocab, 100.0)):
        _check(f"V={vocab} seed={seed} topk={topk} delta={delta}", x["draft"], x["logits"], x["relaxed"],
               topk, delta)


def test_relaxed_full_size_b256_g7_sampled_rows():
    """DeepseekV3 vocabulary at batch 256, gamma 7; rows are independent, so
    the oracle checks a sample of them one by one."""
    cfg = W.get_config("dsv3_mla_b256_accept")
    x = W.make_relaxed_inputs(cfg, 0, vocab=129280)
    a, b = _run(x["draft"], x["logits"], x["relaxed"], cfg.relaxed_topk, cfg.relaxed_delta)
    rows = sorted(set([0, cfg.batch - 1] + np.random.default_rng(0).choice(cfg.batch, 30, replace=False).tolist()))
    ra, rb = oracle.relaxed_accept(x["draft"][rows], x["logits"][rows], x["relaxed"][rows], cfg.relaxed_topk,
                                   cfg.relaxed_delta)
    assert torch.equal(a[rows], ra) and torch.equal(b[rows], rb)
    print(f"  accept-length histogram {torch.bincount(a, minlength=cfg.gamma + 1).tolist()}", flush=True)


def test_relaxed_edges():
    # equal logits everywhere: rank is the id
    B, g, V = 3, 2, 40
    z = torch.zeros(B, g + 1, V, dtype=torch.float32)
    draft = torch.tensor([[0, 0], [3, 0], [0, 9]], dtype=torch.int32)
    a = _check("flat", draft, z, None, 4, 0.0)
    assert a.tolist() == [2, 2, 1]
    a = _check("flat greedy", draft, z, torch.zeros(B, dtype=torch.uint8), 4, 0.0)
    assert a.tolist() == [2, 0, 1]
    # -0 and +0 are the same logit
    z2 = torch.full((1, 2, 8), -1.0)
    z2[0, :, 5] = -0.0
    z2[0, :, 6] = 0.0
    _check("signed zeros", torch.tensor([[6]], dtype=torch.int32), z2, torch.zeros(1, dtype=torch.uint8), 2, 0.0)
    _check("signed zeros relaxed", torch.tensor([[6]], dtype=torch.int32), z2, None, 2, 0.0)
    # a gap of exactly -delta (fp32 0.6) is accepted, one ulp more is not
    d32 = np.float32(0.6)
    at = np.float32(1.0) - d32
    assert float(np.float32(1.0)) - float(at) == float(d32)
    z3 = torch.full((2, 2, 16), -3.0)
    z3[:, :, 0] = 1.0
    z3[0, 0, 7] = float(at)
    z3[1, 0, 7] = float(np.nextafter(at, np.float32(-1)))
    a = _check("delta boundary", torch.tensor([[7], [7]], dtype=torch.int32), z3, None, 10, 0.6)
    assert a.tolist() == [1, 0]
    # ids outside the vocabulary are never accepted
    x = W.make_relaxed_inputs(W.get_config("mla_small"), 7, batch=8, vocab=1000)
    d = x["draft"].clone()
    d[0, 0], d[1, 1], d[2, 0] = -1, 1000, 2 ** 31 - 1
    _check("out of range", d, x["logits"], None, 1000, 100.0)
    # one row, gamma 1
    x = W.make_relaxed_inputs(W.get_config("tiny_mha_b1"), 0, batch=1, vocab=128256)
    _check("B=1 gamma=1", x["draft"], x["logits"], x["relaxed"], 10, 0.6)


def test_relaxed_workspace_reuse_and_stream():
    """The partials need no clearing: back-to-back calls on one workspace, the
    second with a smaller batch, on a side stream."""
    cfg = W.get_config("mla_small")
    big = W.make_relaxed_inputs(cfg, 11, batch=64, vocab=50000)
    small = W.make_relaxed_inputs(cfg, 12, batch=5, vocab=50000)
    ws = torch.empty(binding.relaxed_accept_workspace_size(64, cfg.gamma, 50000), dtype=torch.uint8, device=DEV)
    s = torch.cuda.Stream()
    for x in (big, small):
        B = x["draft"].shape[0]
        acc = torch.empty(B, dtype=torch.int32, device=DEV)
        bon = torch.empty(B, dtype=torch.int32, device=DEV)
        dd, zz, rr = x["draft"].to(DEV), x["logits"].to(DEV), x["relaxed"].to(DEV)
        torch.cuda.synchronize()
        binding.relaxed_accept(dd, zz, rr, 10, 0.6, acc, bon, workspace=ws, stream=s)
        s.synchronize()
        ra, rb = oracle.relaxed_accept(x["draft"], x["logits"], x["relaxed"], 10, 0.6)
        assert torch.equal(acc.cpu().long(), ra) and torch.equal(bon.cpu().long(), rb)
