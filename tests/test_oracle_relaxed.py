"""Pins of the oracle's relaxed chain verification (CPU).

Relaxed acceptance inside thinking spans (MAX-walkthrough section 10): a
draft token is accepted when it is one of the target's relaxed_topk most
likely tokens and (the reading of relaxed_delta) its log-probability is at
most relaxed_delta below the top-1's.  The pins check what that definition
fixes without the oracle's sort: brute force over every logit vector of a
4-token vocabulary (ties and both zeros included); the reductions to the
greedy rule; monotonicity in topk and delta; the closed form of the planted
workload (whose ranks and gaps are known by construction); and the identity
that makes the delta test exact, log-softmax gaps equal logit gaps.
"""
import itertools

import numpy as np
import pytest
import torch

import oracle
import workloads as W

CFG = W.get_config("mla_small")


def _inputs(seed, batch=48, vocab=3000):
    return W.make_relaxed_inputs(CFG, seed, batch=batch, vocab=vocab)


def test_brute_force_tiny_vocab():
    vals = [-1.0, -0.0, 0.0, 0.5]
    for zs in itertools.product(vals, repeat=4):
        z = torch.tensor(zs, dtype=torch.float32)
        # rank by pairwise comparison: u goes before t if its logit is larger,
        # or equal with a smaller id
        rank = [sum(1 for u in range(4) if zs[u] > zs[t] or (zs[u] == zs[t] and u < t)) for t in range(4)]
        top1 = rank.index(0)
        for t in range(4):
            draft = torch.tensor([[t]], dtype=torch.int32)
            logits = torch.stack([z, z]).unsqueeze(0)            # [1, 2, 4]
            for topk in (1, 2, 3, 4):
                for delta in (0.0, 0.5, 1.0, 2.0):
                    ok = rank[t] < topk and zs[t] - max(zs) >= -delta
                    a, b = oracle.relaxed_accept(draft, logits, None, topk, delta)
                    assert int(a[0]) == int(ok), (zs, t, topk, delta)
                    assert int(b[0]) == top1, (zs, t, topk, delta)
            a, b = oracle.relaxed_accept(draft, logits, torch.zeros(1, dtype=torch.uint8), 4, 2.0)
            assert int(a[0]) == int(rank[t] == 0) and int(b[0]) == top1


@pytest.mark.parametrize("seed", [0, 1])
def test_greedy_rows_and_topk1_are_the_greedy_rule(seed):
    x = _inputs(seed)
    tgt = x["logits"].argmax(dim=2).to(torch.int32)          # first maximum on ties
    ga, gb = oracle.greedy_accept(x["draft"], tgt)
    B = x["draft"].shape[0]
    a, b = oracle.relaxed_accept(x["draft"], x["logits"], torch.zeros(B, dtype=torch.uint8), 10, 0.6)
    assert torch.equal(a, ga) and torch.equal(b, gb)
    a, b = oracle.relaxed_accept(x["draft"], x["logits"], None, 1, 5.0)
    assert torch.equal(a, ga) and torch.equal(b, gb)


def test_monotone_in_topk_and_delta():
    x = _inputs(2)
    prev = None
    for topk in (1, 2, 5, 10, 12, 20):
        a, _ = oracle.relaxed_accept(x["draft"], x["logits"], None, topk, 0.6)
        if prev is not None:
            assert bool((a >= prev).all())
        prev = a
    prev = None
    for delta in (0.0, 0.1, 0.3, 0.6, 1.0, 100.0):
        a, _ = oracle.relaxed_accept(x["draft"], x["logits"], None, 10, delta)
        if prev is not None:
            assert bool((a >= prev).all())
        prev = a
    rel, _ = oracle.relaxed_accept(x["draft"], x["logits"], None, 10, 0.6)
    gr, _ = oracle.relaxed_accept(x["draft"], x["logits"], torch.zeros(len(rel), dtype=torch.uint8), 10, 0.6)
    assert bool((rel >= gr).all()) and bool((rel > gr).any())


def test_unbounded_candidates_accept_everything():
    x = _inputs(3, vocab=500)
    a, b = oracle.relaxed_accept(x["draft"], x["logits"], None, 500, 1e30)
    assert bool((a == CFG.gamma).all())
    assert torch.equal(b, x["logits"][:, CFG.gamma].argmax(dim=1))


@pytest.mark.parametrize("vocab", [3000, 129280])
def test_planted_closed_form(vocab):
    """The planted head fixes every decision: planted r = 2m or 2m + 1 shares
    the logit 8 - s*m with its partner, so its rank is 2m plus one if the
    partner's id is smaller; the background lies below every planted logit,
    more than any delta here away from the top."""
    x = _inputs(4, batch=24 if vocab > 10000 else 64, vocab=vocab)
    z, draft, rel, planted = x["logits"], x["draft"], x["relaxed"], x["planted"]
    B, g = draft.shape
    d32 = float(np.float32(CFG.relaxed_delta))
    exp_a = torch.zeros(B, dtype=torch.int64)
    exp_b = torch.zeros(B, dtype=torch.int64)
    for b in range(B):
        a = 0
        while a < g:
            ids = planted[b, a].tolist()
            t = int(draft[b, a])
            ok = False
            if t in ids:
                r = ids.index(t)
                m, partner = r // 2, ids[r ^ 1]
                rank = 2 * m + (1 if partner < t else 0)
                gap = float(z[b, a, t]) - float(z[b, a, ids[0]])   # both planted, exact in fp64
                ok = rank == 0 if not rel[b] else (rank < CFG.relaxed_topk and gap >= -d32)
            if not ok:
                break
            a += 1
        exp_a[b] = a
        exp_b[b] = min(planted[b, a, 0], planted[b, a, 1])
    a, bo = oracle.relaxed_accept(draft, z, rel, CFG.relaxed_topk, CFG.relaxed_delta)
    assert torch.equal(a, exp_a) and torch.equal(bo, exp_b)
    assert len(set(a.tolist())) > 1


def test_log_prob_gap_is_logit_gap():
    """The normaliser cancels: log_softmax(z)[t] - log_softmax(z)[u] = z[t] - z[u]."""
    z = _inputs(5, batch=2, vocab=129280)["logits"].to(torch.float64)
    lp = torch.log_softmax(z, dim=-1)
    top = z.argmax(dim=-1, keepdim=True)
    assert torch.allclose(lp - lp.gather(-1, top), z - z.gather(-1, top), rtol=0, atol=1e-12)
