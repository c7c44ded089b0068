"""Parity of the HIP path (through the C ABI) with the CPU oracle.

Tolerances: hidden states and logits max-abs <= 3e-2 and relative L2 <= 1e-2
(fp32 outputs, bf16 storage, fp32 accumulation); draft ids bit-exact where the
oracle's top-1/top-2 margin exceeds 1e-2; d2t and acceptance bit-exact.
"""
import numpy as np
import pytest
import torch

import oracle
import workloads as W
from eagle_draft_head_step_amd import binding
from gpu_util import (DEV, MARGIN, assert_cache_entries, assert_close, assert_ids, cache_entry,
                      cache_keys, cache_segments, clone, dev_state, gpu_caches, gpu_chain, gpu_step, to_dev)

pytestmark = pytest.mark.gpu

SMALL = ["tiny_mha_b1", "mha_small", "mha_small_b40", "mla_small", "mla_small_b48",
         "mha_small_b100", "mla_small_b200", "mla_small_b300", "mha_small_aux2_tgt_head",
         # 260 (row, kv head) pairs: whole-row 8-wave MHA attention, no key split
         "mha_small_b130", "mha_small_hd64_b128",
         # large-batch GEMM with a stream-K gate/up (160 and 100 rows)
         "mla_small_b160_wide_mlp", "mha_small_b100_wide_mlp",
         # quantized heads (weight-only FP8 / NVFP4), small to large batch
         "mha_small_fp8", "mla_small_fp8", "mha_small_nvfp4", "mha_small_b40_nvfp4", "mla_small_b48_nvfp4",
         "mha_small_b100_fp8", "mla_small_b200_nvfp4",
         # YaRN with beta_fast = beta_slow = 1 (a one-pair ramp)
         "mla_small_beta1"]


def _setup(cfg, seed=0):
    Wt = W.make_weights(cfg)
    st = W.make_inputs(cfg, seed=seed)
    head = binding.DraftHead(cfg, to_dev(Wt))
    return Wt, st, head


@pytest.mark.parametrize("name", SMALL)
def test_step_level_parity(name):
    """Each step fed the GPU's previous hidden state and token."""
    cfg = W.get_config(name)
    print(f"[parity-step] {name}", flush=True)
    seeds = range(8) if cfg.batch == 1 else [0]
    for seed in seeds:
        Wt, st, head = _setup(cfg, seed)
        d = dev_state(cfg, st)
        ora = clone(st)
        ws = head.workspace(cfg.batch, cfg.max_ctx, cfg.gamma)
        d2t = W.make_d2t(cfg).long()
        h_gpu, tok_gpu = None, None
        for k in range(cfg.gamma):
            hout, tok, did, lg = gpu_step(head, cfg, d, ws, k, hidden_in=h_gpu, token_in=tok_gpu,
                                          use_aux=(k == 0))
            torch.cuda.synchronize()
            ref = oracle.draft_step(cfg, Wt, ora, k,
                                    hidden_in=None if h_gpu is None else h_gpu.cpu(),
                                    token_in=None if tok_gpu is None else tok_gpu.cpu())
            assert_close(f"{name} s{seed} step {k} hidden", hout, ref["hidden_out"])
            assert_close(f"{name} s{seed} step {k} logits", lg, ref["logits"])
            assert_ids(f"{name} s{seed} step {k} draft id", did, ref["draft_id"], ref["margin"])
            didc = did.cpu().long()
            assert torch.equal(tok.cpu().long(), didc + d2t[didc]), "d2t map"
            cache_now = gpu_caches(cfg, d)
            pos = [int(st["ctx_len"][b]) + k for b in range(cfg.batch)]
            assert_cache_entries(f"{name} s{seed} step {k} cache",
                                 [cache_entry(cfg, cache_now, st["block_table"], b, pos[b]) for b in range(cfg.batch)],
                                 [cache_entry(cfg, ora, st["block_table"], b, pos[b]) for b in range(cfg.batch)],
                                 cache_segments(cfg))
            h_gpu, tok_gpu = hout, tok


@pytest.mark.parametrize("name", SMALL)
def test_chain_parity_free_running(name):
    """One eagle3_draft_chain call against the oracle's own chain; where the
    oracle's margin is <= 1e-2 it adopts the GPU's token (a legitimate near
    tie must not cascade)."""
    cfg = W.get_config(name)
    print(f"[parity-chain] {name}", flush=True)
    Wt, st, head = _setup(cfg)
    d = dev_state(cfg, st)
    ws = head.workspace(cfg.batch, cfg.max_ctx, cfg.gamma)
    hid, tok, did, lg = gpu_chain(head, cfg, d, ws, cfg.gamma)
    torch.cuda.synchronize()
    ora = clone(st)
    h, t = None, None
    d2t = W.make_d2t(cfg).long()
    for k in range(cfg.gamma):
        ref = oracle.draft_step(cfg, Wt, ora, k, hidden_in=h, token_in=t)
        assert_close(f"{name} chain step {k} hidden", hid[k], ref["hidden_out"])
        assert_close(f"{name} chain step {k} logits", lg[k], ref["logits"])
        assert_ids(f"{name} chain step {k} ids", did[:, k], ref["draft_id"], ref["margin"])
        g_tok = tok[:, k].cpu().long()
        g_did = did[:, k].cpu().long()
        assert torch.equal(g_tok, g_did + d2t[g_did])
        near = ref["margin"] <= MARGIN
        t = torch.where(near, g_tok, ref["token_out"])
        h = ref["hidden_out"]


def test_chain_equals_steps():
    """A chain of gamma equals gamma single steps fed their own outputs (bitwise)."""
    cfg = W.get_config("mha_small")
    Wt, st, head = _setup(cfg)
    d1, d2 = dev_state(cfg, st), dev_state(cfg, st)
    ws = head.workspace(cfg.batch, cfg.max_ctx, cfg.gamma)
    hid, tok, did, _ = gpu_chain(head, cfg, d1, ws, cfg.gamma, logits=False)
    h, t = None, None
    for k in range(cfg.gamma):
        hout, tk, _, _ = gpu_step(head, cfg, d2, ws, k, hidden_in=h, token_in=t, use_aux=(k == 0),
                                  logits=False)
        assert torch.equal(hout, hid[k]) and torch.equal(tk, tok[:, k].contiguous())
        h, t = hout, tk
    for key in cache_keys(cfg):
        assert torch.equal(d1[key], d2[key])


@pytest.mark.parametrize("name", ["mha_small", "mla_small"])
def test_determinism(name):
    cfg = W.get_config(name)
    Wt, st, head = _setup(cfg)
    ws = head.workspace(cfg.batch, cfg.max_ctx, cfg.gamma)
    outs = []
    for _ in range(2):
        d = dev_state(cfg, st)
        outs.append(gpu_chain(head, cfg, d, ws, cfg.gamma))
    torch.cuda.synchronize()
    for a, b in zip(*outs):
        assert torch.equal(a, b)


@pytest.mark.parametrize("name", ["mha_small", "mla_small"])
def test_edge_contexts(name):
    """Empty caches, page-boundary lengths and the fullest page table.  Every
    step of the chain is compared at step level (the oracle fed the GPU's
    previous hidden state and token): hidden, logits, ids and the entry it
    wrote.  Context P - 1 crosses into a new page at step 1, and the last
    step of the longest row lands in the last slot of its last page."""
    base = W.get_config(name)
    P = base.page_size
    for ctxs in ([0] * 5, [P - 1, P, P + 1, 2 * P - base.gamma, 1]):
        cfg = base.replace(batch=len(ctxs), ctx=(0, max(ctxs)), paging="identity")
        Wt, st, head = _setup(cfg)
        st["ctx_len"] = torch.tensor(ctxs, dtype=torch.int32)
        mp = st["block_table"].shape[1]
        st["block_table"] = (torch.arange(cfg.batch).view(-1, 1) * mp
                             + torch.arange(mp).view(1, -1)).to(torch.int32)
        d = dev_state(cfg, st)
        ws = head.workspace(cfg.batch, cfg.max_ctx, cfg.gamma)
        hid, tok, did, lg = gpu_chain(head, cfg, d, ws, cfg.gamma, max_ctx=max(ctxs))
        torch.cuda.synchronize()
        after = gpu_caches(cfg, d)
        ora = clone(st)
        d2t = W.make_d2t(cfg).long()
        for k in range(cfg.gamma):
            ref = oracle.draft_step(cfg, Wt, ora, k,
                                    hidden_in=None if k == 0 else hid[k - 1].cpu(),
                                    token_in=None if k == 0 else tok[:, k - 1].cpu())
            tag = f"{name} {ctxs} step {k}"
            assert_close(f"{tag} hidden", hid[k], ref["hidden_out"])
            assert_close(f"{tag} logits", lg[k], ref["logits"])
            assert_ids(f"{tag} ids", did[:, k], ref["draft_id"], ref["margin"])
            g_did = did[:, k].cpu().long()
            assert torch.equal(tok[:, k].cpu().long(), g_did + d2t[g_did])
            pos = [c + k for c in ctxs]
            assert_cache_entries(f"{tag} cache",
                                 [cache_entry(cfg, after, st["block_table"], b, pos[b]) for b in range(cfg.batch)],
                                 [cache_entry(cfg, ora, st["block_table"], b, pos[b]) for b in range(cfg.batch)],
                                 cache_segments(cfg))
        # the last position written is the last slot of the longest row's table
        assert max(ctxs) + cfg.gamma <= mp * P


def test_batch_row_permutation():
    """Rows are independent: permuting the batch permutes the outputs."""
    cfg = W.get_config("mla_small")
    Wt, st, head = _setup(cfg)
    ws = head.workspace(cfg.batch, cfg.max_ctx, cfg.gamma)
    hid, tok, _, _ = gpu_chain(head, cfg, dev_state(cfg, st), ws, cfg.gamma, logits=False)
    perm = torch.tensor([4, 2, 0, 3, 1])
    st2 = dict(st)
    for k in ("aux", "token_in", "ctx_len", "block_table"):
        st2[k] = st[k][perm].contiguous()
    hid2, tok2, _, _ = gpu_chain(head, cfg, dev_state(cfg, st2), ws, cfg.gamma, logits=False)
    torch.cuda.synchronize()
    assert torch.equal(tok2.cpu(), tok.cpu()[perm])
    assert torch.equal(hid2.cpu(), hid.cpu()[:, perm])
