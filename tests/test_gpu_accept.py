"""Greedy chain verification on the GPU: bit-exact against brute force and
against the closed form of the synthesised workload."""
import itertools

import pytest
import torch

import oracle
import workloads as W
from eagle_draft_head_step_amd import binding

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")


def _run(draft, target):
    B = draft.shape[0]
    acc = torch.full((B,), -7, dtype=torch.int32, device=DEV)
    bon = torch.full((B,), -7, dtype=torch.int32, device=DEV)
    binding.greedy_accept(draft.to(DEV).contiguous(), target.to(DEV).contiguous(), acc, bon)
    torch.cuda.synchronize()
    return acc.cpu(), bon.cpu()


@pytest.mark.parametrize("gamma", [1, 2, 3, 4])
def test_accept_exhaustive_tiny_vocab(gamma):
    cases = torch.tensor(list(itertools.product(range(3), repeat=2 * gamma + 1)), dtype=torch.int32)
    draft, target = cases[:, :gamma].contiguous(), cases[:, gamma:].contiguous()
    acc, bon = _run(draft, target)
    ra, rb = oracle.greedy_accept(draft, target)
    assert torch.equal(acc.long(), ra) and torch.equal(bon.long(), rb)


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_accept_synthesised_b256_g7(seed):
    cfg = W.get_config("dsv3_mla_b256_accept")
    draft = W.random_drafts(cfg, seed)
    tgt, k = W.make_accept_targets(cfg, draft, seed)
    acc, bon = _run(draft, tgt)
    assert torch.equal(acc, k)
    assert torch.equal(bon, tgt[torch.arange(cfg.batch), k.long()])


def test_accept_edges():
    B, g = 1000, 5
    d = torch.randint(0, 50, (B, g), dtype=torch.int32)
    same = torch.cat([d, torch.zeros(B, 1, dtype=torch.int32)], 1)
    acc, bon = _run(d, same)
    assert bool((acc == g).all()) and bool((bon == 0).all())
    diff = torch.cat([d + 1, torch.full((B, 1), 9, dtype=torch.int32)], 1)
    acc, bon = _run(d, diff)
    assert bool((acc == 0).all()) and torch.equal(bon, d[:, 0] + 1)
