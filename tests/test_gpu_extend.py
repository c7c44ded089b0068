"""Parity of the multi-token extend (eagle3_draft_extend, through the C ABI)
with the oracle's definition: every new position runs the draft step with
the target's aux state and its token, positions of a sequence in order.

Same tolerances as the step: hidden states and logits max-abs <= 3e-2 and
relative L2 <= 1e-2; ids bit-exact where the oracle's top-1/top-2 margin
exceeds 1e-2; d2t bit-exact; cache entries within one storage step plus the
bf16-activation bound.
"""
import numpy as np
import pytest
import torch

import oracle
import workloads as W
from eagle_draft_head_step_amd import binding
from gpu_util import (DEV, assert_cache_entries, assert_close, assert_ids, cache_entry, cache_keys,
                      cache_segments, clone, dev_state, gpu_caches, kc_vc, to_dev)

pytestmark = pytest.mark.gpu


def _q_lens(cfg, seed):
    """Ragged new-token counts in [0, gamma] with both ends present."""
    rng = np.random.default_rng(1234 + seed)
    q = rng.integers(0, cfg.gamma + 1, size=cfg.batch)
    q[0] = cfg.gamma
    if cfg.batch > 1:
        q[-1] = 0
    if q.sum() == 0:
        q[0] = 1
    return q.tolist()


def gpu_extend(head, cfg, d, ex, *, logits=True, max_ctx=None):
    T = int(ex["token_in"].shape[0])
    q = (ex["cu_seqlens"][1:] - ex["cu_seqlens"][:-1]).max().item()
    max_ctx = cfg.max_ctx if max_ctx is None else max_ctx
    ws = head.extend_workspace(T, cfg.batch, max_ctx, int(q))
    hid = torch.empty(T, cfg.hidden, dtype=torch.float32, device=DEV)
    tok = torch.empty(T, dtype=torch.int32, device=DEV)
    did = torch.empty(T, dtype=torch.int32, device=DEV)
    lg = torch.empty(T, cfg.draft_vocab, dtype=torch.float32, device=DEV) if logits else None
    kc, vc = kc_vc(cfg, d)
    de = to_dev(ex)
    head.draft_extend(cu_seqlens=de["cu_seqlens"], max_q_len=int(q), aux=de["aux"].reshape(T, -1),
                      token_in=de["token_in"], k_cache=kc, v_cache=vc, block_table=d["block_table"],
                      ctx_len=d["ctx_len"], max_ctx=max_ctx, hidden_out=hid, token_out=tok, draft_id_out=did,
                      logits_out=lg, workspace=ws)
    return hid, tok, did, lg


@pytest.mark.parametrize("name", ["tiny_mha_b1", "mha_small", "mha_small_b40", "mla_small", "mla_small_b48",
                                  "mha_small_b100", "mla_small_b200", "mha_small_aux2_tgt_head",
                                  "mha_small_fp8", "mla_small_b48_nvfp4", "mha_small_b130",
                                  "mha_small_hd64_b128"])
def test_extend_parity(name):
    cfg = W.get_config(name)
    print(f"[extend] {name}", flush=True)
    for seed in (0, 1):
        Wt = W.make_weights(cfg)
        st = W.make_inputs(cfg, seed=seed)
        q = [1] if cfg.batch == 1 else _q_lens(cfg, seed)
        ex = W.make_extend_inputs(cfg, q, seed=seed)
        head = binding.DraftHead(cfg, to_dev(Wt))
        d = dev_state(cfg, st)
        hid, tok, did, lg = gpu_extend(head, cfg, d, ex)
        torch.cuda.synchronize()
        ora = clone(st)
        ref = oracle.draft_extend(cfg, Wt, ora, ex["cu_seqlens"], ex["aux"], ex["token_in"])
        assert_close(f"{name} s{seed} extend hidden", hid, ref["hidden_out"])
        assert_close(f"{name} s{seed} extend logits", lg, ref["logits"])
        assert_ids(f"{name} s{seed} extend ids", did, ref["draft_id"], ref["margin"])
        d2t = W.make_d2t(cfg).long()
        dc = did.cpu().long()
        assert torch.equal(tok.cpu().long(), dc + d2t[dc]), "d2t map"
        cache_now = gpu_caches(cfg, d)
        cu = ex["cu_seqlens"].tolist()
        new = [(b, int(st["ctx_len"][b]) + j) for b in range(cfg.batch) for j in range(cu[b + 1] - cu[b])]
        assert_cache_entries(f"{name} s{seed} extend cache",
                             [cache_entry(cfg, cache_now, st["block_table"], b, p) for b, p in new],
                             [cache_entry(cfg, ora, st["block_table"], b, p) for b, p in new], cache_segments(cfg))
        for b in range(cfg.batch):
            # the slot after the last new position is untouched
            pos = int(st["ctx_len"][b]) + cu[b + 1] - cu[b]
            if pos < st["block_table"].shape[1] * cfg.page_size:
                assert torch.equal(cache_entry(cfg, cache_now, st["block_table"], b, pos),
                                   cache_entry(cfg, st, st["block_table"], b, pos)), (name, b, "wrote past q_len")


def test_extend_one_token_matches_step():
    """q_len = 1 everywhere is one draft step: the extend and eagle3_draft_step
    each against the oracle's step (tolerances of the step), and against each
    other."""
    for name in ("mha_small", "mla_small"):
        cfg = W.get_config(name)
        Wt = W.make_weights(cfg)
        st = W.make_inputs(cfg)
        ex = W.make_extend_inputs(cfg, [1] * cfg.batch)
        head = binding.DraftHead(cfg, to_dev(Wt))
        d1, d2 = dev_state(cfg, st), dev_state(cfg, st)
        hid, tok, did, lg = gpu_extend(head, cfg, d1, ex)
        B = cfg.batch
        ws = head.workspace(B, cfg.max_ctx, 1)
        h2 = torch.empty(B, cfg.hidden, dtype=torch.float32, device=DEV)
        t2 = torch.empty(B, dtype=torch.int32, device=DEV)
        kc, vc = kc_vc(cfg, d2)
        head.draft_step(step_index=0, aux=ex["aux"].reshape(B, -1).to(DEV), hidden_in=None,
                        token_in=ex["token_in"].to(DEV), k_cache=kc, v_cache=vc, block_table=d2["block_table"],
                        ctx_len=d2["ctx_len"], max_ctx=cfg.max_ctx, hidden_out=h2, token_out=t2,
                        draft_id_out=None, logits_out=None, workspace=ws)
        torch.cuda.synchronize()
        ora = clone(st)
        ora["aux"], ora["token_in"] = ex["aux"], ex["token_in"]
        ref = oracle.draft_step(cfg, Wt, ora, 0)
        assert_close(f"{name} extend q=1 hidden vs oracle step", hid, ref["hidden_out"])
        assert_close(f"{name} extend q=1 logits vs oracle step", lg, ref["logits"])
        assert_ids(f"{name} extend q=1 ids vs oracle step", did, ref["draft_id"], ref["margin"])
        assert_close(f"{name} step hidden vs oracle step", h2, ref["hidden_out"])
        assert_close(f"{name} extend vs step hidden", hid, h2)


@pytest.mark.parametrize("name", ["llama3_8b_gqa_b32", "dsv3_mla_b16"])
def test_extend_full_size_sampled_sequences(name):
    """Full shapes, ragged q_len in [1, gamma]; the oracle checks the first and
    last sequence over all their new positions."""
    cfg = W.get_config(name)
    print(f"[extend-full] {cfg.name}", flush=True)
    Wt = W.make_weights(cfg)
    st = W.make_inputs(cfg)
    rng = np.random.default_rng(7)
    q = rng.integers(1, cfg.gamma + 1, size=cfg.batch).tolist()
    ex = W.make_extend_inputs(cfg, q)
    head = binding.DraftHead(cfg, to_dev(Wt))
    d = dev_state(cfg, st)
    hid, tok, did, lg = gpu_extend(head, cfg, d, ex, logits=True)
    torch.cuda.synchronize()
    cu = ex["cu_seqlens"].tolist()
    d2t = W.make_d2t(cfg).long()
    dc = did.cpu().long()
    assert torch.equal(tok.cpu().long(), dc + d2t[dc]), "d2t map"
    cache_now = gpu_caches(cfg, d)
    for b in (0, cfg.batch // 2, cfg.batch - 1):
        sl = slice(cu[b], cu[b + 1])
        sub = {k: v.clone() for k, v in st.items() if k in cache_keys(cfg)}
        sub["ctx_len"] = st["ctx_len"][[b]]
        sub["block_table"] = st["block_table"][[b]]
        ref = oracle.draft_extend(cfg, Wt, sub, torch.tensor([0, cu[b + 1] - cu[b]], dtype=torch.int32),
                                  ex["aux"][sl], ex["token_in"][sl])
        assert_close(f"{cfg.name} seq {b} extend hidden", hid[sl], ref["hidden_out"])
        assert_close(f"{cfg.name} seq {b} extend logits", lg[sl], ref["logits"])
        n = assert_ids(f"{cfg.name} seq {b} extend ids", did[sl], ref["draft_id"], ref["margin"])
        print(f"  seq {b}: {n}/{cu[b + 1] - cu[b]} positions above the margin", flush=True)
        pos = [int(st["ctx_len"][b]) + j for j in range(cu[b + 1] - cu[b])]
        assert_cache_entries(f"{cfg.name} seq {b} extend cache",
                             [cache_entry(cfg, cache_now, st["block_table"], b, p) for p in pos],
                             [cache_entry(cfg, sub, sub["block_table"], 0, p) for p in pos], cache_segments(cfg))
    del head, d
    torch.cuda.empty_cache()


def test_extend_more_rows_than_one_gemm_block():
    """400 new positions (two new tokens for each of 200 sequences): every GEMM
    runs as two row blocks, the top-1 reduction over two candidate blocks."""
    cfg = W.get_config("mla_small_b200")
    Wt = W.make_weights(cfg)
    st = W.make_inputs(cfg, seed=5)
    ex = W.make_extend_inputs(cfg, [2] * cfg.batch, seed=5)
    head = binding.DraftHead(cfg, to_dev(Wt))
    d = dev_state(cfg, st)
    hid, tok, did, lg = gpu_extend(head, cfg, d, ex)
    torch.cuda.synchronize()
    ref = oracle.draft_extend(cfg, Wt, clone(st), ex["cu_seqlens"], ex["aux"], ex["token_in"])
    assert hid.shape[0] == 400
    assert_close("b200 x2 extend hidden", hid, ref["hidden_out"])
    assert_close("b200 x2 extend logits", lg, ref["logits"])
    assert_ids("b200 x2 extend ids", did, ref["draft_id"], ref["margin"])
