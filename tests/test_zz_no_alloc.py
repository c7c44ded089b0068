"""eagle3_relaxed_accept_noalloc (no workspace argument: the partials live in
the library's fixed per-GPU scratch array) through the C ABI, against
eagle3_relaxed_accept with a caller workspace: accept lengths and bonus ids
bit-exact, on two calls in a row, the second with a smaller input, and the
first also against the oracle on sampled rows."""
import ctypes

import numpy as np
import pytest
import torch

import oracle
import workloads as W
from eagle_draft_head_step_amd import binding

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")
ERR_WORKSPACE = -4


def _both(x, topk, delta):
    draft = x["draft"].to(DEV).contiguous()
    logits = x["logits"].to(DEV).contiguous()
    rel = x["relaxed"].to(DEV).contiguous()
    B = draft.shape[0]
    out = []
    for fn in (binding.relaxed_accept, binding.relaxed_accept_noalloc):
        acc = torch.full((B,), -7, dtype=torch.int32, device=DEV)
        bon = torch.full((B,), -7, dtype=torch.int32, device=DEV)
        fn(draft, logits, rel, topk, delta, acc, bon)
        torch.cuda.synchronize()
        out.append((acc.cpu().long(), bon.cpu().long()))
    return out


def test_noalloc_matches_workspace_entry_point():
    cfg = W.get_config("dsv3_mla_b256_accept")
    big = W.make_relaxed_inputs(cfg, 0, vocab=129280)                      # B 256, gamma 7
    small = W.make_relaxed_inputs(W.get_config("mla_small"), 3, batch=16, vocab=2999)
    for tag, x in (("B256 g7 V129280", big), ("B16 g3 V2999", small)):
        print(f"[noalloc] {tag}", flush=True)
        (a1, b1), (a2, b2) = _both(x, cfg.relaxed_topk, cfg.relaxed_delta)
        assert torch.equal(a1, a2) and torch.equal(b1, b2), tag
        assert len(set(a2.tolist())) > 1, tag
        rows = sorted(set([0, x["draft"].shape[0] - 1] +
                          np.random.default_rng(1).choice(x["draft"].shape[0], 8, replace=False).tolist()))
        ra, rb = oracle.relaxed_accept(x["draft"][rows], x["logits"][rows], x["relaxed"][rows],
                                       cfg.relaxed_topk, cfg.relaxed_delta)
        assert torch.equal(a2[rows], ra) and torch.equal(b2[rows], rb), tag


def test_noalloc_rejects_more_than_its_scratch():
    """B * (gamma + 1) above 65536 would need more than the 1 MiB array: the
    host returns EAGLE3_ERR_WORKSPACE before anything is enqueued."""
    L = binding.lib()
    d = torch.zeros(1, dtype=torch.int32, device=DEV)
    z = torch.zeros(4, dtype=torch.float32, device=DEV)
    a = torch.zeros(1, dtype=torch.int32, device=DEV)
    need = ctypes.c_size_t(0)
    assert L.eagle3_relaxed_accept_workspace_size(40000, 1, 4096, ctypes.byref(need)) == 0
    assert need.value > (1 << 20)
    rc = L.eagle3_relaxed_accept_noalloc(d.data_ptr(), z.data_ptr(), None, 40000, 1, 4096, 10,
                                         ctypes.c_float(0.6), a.data_ptr(), a.data_ptr(), None)
    assert rc == ERR_WORKSPACE
