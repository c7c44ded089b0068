"""Parity at the full workload sizes, in the launch configuration the bench
times (one eagle3_draft_chain call over the whole batch).  The oracle
recomputes sampled rows at sampled steps: the first step from the original
inputs, later steps from the GPU's previous hidden state, token and cache
(rows are independent, so a row subset is an exact check of those rows).

Rows are chosen where the kernels change tiles or schedules: the 16- and
128-row wave-tile and row-half boundaries of the GEMMs, the shortest and
longest ragged contexts, and rows split between two workgroups of the MLA
attention's balanced schedule."""
import pytest
import torch

import oracle
import workloads as W
from eagle_draft_head_step_amd import binding
from gpu_util import (assert_cache_entries, assert_close, assert_ids, cache_entry, cache_keys,
                      cache_segments, dev_state, gpu_caches, gpu_chain, to_dev)

pytestmark = pytest.mark.gpu

_WEIGHTS = {}

MLA_WORKGROUPS = 256   # persistent workgroups the MLA attention splits a batch's tiles over
MLA_TILE = 32          # keys per MLA attention tile


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


def _split_rows(ctx, step, nblocks=MLA_WORKGROUPS):
    """Rows whose 32-key tiles at `step` straddle two workgroups' equal ranges
    of all the batch's (row, tile) pairs."""
    tiles = [(int(c) + step + 1 + MLA_TILE - 1) // MLA_TILE for c in ctx]
    total = sum(tiles)
    cuts = {(total * w) // nblocks for w in range(1, nblocks)}
    rows, start = [], 0
    for b, t in enumerate(tiles):
        if any(start < c < start + t for c in cuts):
            rows.append(b)
        start += t
    return rows


def _rows(cfg, st):
    B = cfg.batch
    if cfg.name == "dsv3_mla_b16":
        return list(range(B))                                    # every row
    rows = {0, B // 2, B - 1}
    if B >= 32:
        rows |= {15, 16}
    if B > 128:
        rows |= {127, 128}
    if cfg.ctx[0] != cfg.ctx[1]:
        ctx = st["ctx_len"].tolist()
        rows |= {min(range(B), key=lambda b: ctx[b]), max(range(B), key=lambda b: ctx[b])}
        rows |= set(_split_rows(ctx, 0)[:3])
    return sorted(rows)


def _steps(g):
    if g == 1:
        return [0]
    return sorted({0, g // 2, g - 1})


@pytest.mark.parametrize("idx", [0, 1, 2, 3, 4, "llama3_8b_gqa_b32_fp8", "llama3_8b_gqa_b32_nvfp4",
                                 "dsv3_mla_b16_fp8", "dsv3_mla_b16_nvfp4"])
def test_full_size_sampled_rows(idx):
    cfg = W.get_config(idx)
    print(f"[full] {cfg.name}", flush=True)
    Wt = _weights(cfg)
    st = W.make_inputs(cfg)
    head = binding.DraftHead(cfg, to_dev(Wt))
    d = dev_state(cfg, st)
    ws = head.workspace(cfg.batch, cfg.max_ctx, cfg.gamma)
    g = cfg.gamma
    hid, tok, did, lg = gpu_chain(head, cfg, d, ws, g)
    torch.cuda.synchronize()
    rows = _rows(cfg, st)
    print(f"  rows {rows}", flush=True)
    orig = {k: st[k] for k in cache_keys(cfg)}
    after = gpu_caches(cfg, d)
    del d
    d2t = W.make_d2t(cfg).long()
    g_did = did.cpu().long()
    assert torch.equal(tok.cpu().long(), g_did + d2t[g_did]), "d2t map"
    for k in _steps(g):
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
        assert_cache_entries(
            f"{cfg.name} step {k} cache",
            [cache_entry(cfg, after, st["block_table"], b, int(st["ctx_len"][b]) + k) for b in rows],
            [cache_entry(cfg, sub, sub["block_table"], i, int(st["ctx_len"][b]) + k) for i, b in enumerate(rows)],
            cache_segments(cfg))
    del head, ws, hid, lg
    torch.cuda.empty_cache()
