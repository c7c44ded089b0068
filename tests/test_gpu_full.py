"""Parity at the full workload sizes, in the launch configuration the bench
times (one eagle3_draft_chain call over the whole batch).  The oracle
recomputes sampled rows: the first step from the original inputs, and the
last step from the GPU's previous hidden state, token and cache (rows are
independent, so a row subset is an exact check of those rows)."""
import pytest
import torch

import oracle
import workloads as W
from eagle_draft_head_step_amd import binding
from gpu_util import (assert_cache_entry, assert_close, assert_ids, cache_entry, cache_keys,
                      cache_segments, gpu_chain, to_dev)

pytestmark = pytest.mark.gpu

_WEIGHTS = {}


def _weights(cfg):
    fam = (cfg.weight_family or cfg.name, cfg.weight_format)
    if fam not in _WEIGHTS:
        _WEIGHTS.clear()
        _WEIGHTS[fam] = W.make_weights(cfg)
    return _WEIGHTS[fam]


def _sub(st, rows, cache):
    s = {k: st[k][rows].clone() for k in ("aux", "token_in", "ctx_len", "block_table")}
    s.update({k: v.clone() for k, v in cache.items()})
    return s


@pytest.mark.parametrize("idx", [0, 1, 2, 3, 4, "llama3_8b_gqa_b32_fp8", "llama3_8b_gqa_b32_nvfp4",
                                 "dsv3_mla_b16_fp8", "dsv3_mla_b16_nvfp4"])
def test_full_size_sampled_rows(idx):
    cfg = W.get_config(idx)
    print(f"[full] {cfg.name}", flush=True)
    Wt = _weights(cfg)
    st = W.make_inputs(cfg)
    head = binding.DraftHead(cfg, to_dev(Wt))
    d = to_dev(st)
    ws = head.workspace(cfg.batch, cfg.max_ctx, cfg.gamma)
    g = cfg.gamma
    hid, tok, did, lg = gpu_chain(head, cfg, d, ws, g)
    torch.cuda.synchronize()
    B = cfg.batch
    rows = sorted({0, B // 2, B - 1})
    orig = {k: st[k] for k in cache_keys(cfg)}
    after = {k: d[k].cpu() for k in cache_keys(cfg)}
    d2t = W.make_d2t(cfg).long()
    g_did = did.cpu().long()
    assert torch.equal(tok.cpu().long(), g_did + d2t[g_did]), "d2t map"
    steps = [0] if g == 1 else [0, g - 1]
    for k in steps:
        if k == 0:
            sub = _sub(st, rows, orig)
            ref = oracle.draft_step(cfg, Wt, sub, 0)
        else:
            sub = _sub(st, rows, after)
            ref = oracle.draft_step(cfg, Wt, sub, k, hidden_in=hid[k - 1, rows].cpu(),
                                    token_in=tok[rows, k - 1].cpu())
        assert_close(f"{cfg.name} step {k} hidden", hid[k, rows], ref["hidden_out"])
        assert_close(f"{cfg.name} step {k} logits", lg[k, rows], ref["logits"])
        n = assert_ids(f"{cfg.name} step {k} ids", did[rows, k], ref["draft_id"], ref["margin"])
        print(f"  step {k}: {n}/{len(rows)} rows above the margin", flush=True)
        for i, b in enumerate(rows):
            pos = int(st["ctx_len"][b]) + k
            assert_cache_entry(f"{cfg.name} step {k} row {b} cache",
                               cache_entry(cfg, after, st["block_table"], b, pos),
                               cache_entry(cfg, {kk: sub[kk] for kk in cache_keys(cfg)},
                                           sub["block_table"], i, pos),
                               cache_segments(cfg))
    del head, d, ws, hid, lg
    torch.cuda.empty_cache()
