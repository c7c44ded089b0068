"""Pins of the oracle's multi-token extend (CPU).

The extend is defined as the draft step at every new position with the
target's aux state and the given token, positions of a sequence in order
(MAX-walkthrough sections 4 and 9: the draft's prefill phase over accepted
positions returns every position's hidden state and logits).  The pins check
what that definition fixes independently of how it is evaluated: one new
token per sequence is exactly one draft step; an output never depends on a
later position of its sequence (causality) but does on earlier ones; sequences
do not interact (up to fp64 summation order); sequences with no new token
leave the cache alone.
"""
import torch

import oracle
import workloads as W

CFGS = ["mha_small", "mla_small"]


def _clone(st):
    return {k: v.clone() for k, v in st.items()}


def _cache_keys(cfg):
    return ["k_cache", "v_cache"] if cfg.attn_kind == 0 else ["kv_cache"]


def _setup(name, q_lens, seed=0):
    cfg = W.get_config(name)
    Wt = W.make_weights(cfg)
    st = W.make_inputs(cfg, seed=seed)
    ex = W.make_extend_inputs(cfg, q_lens, seed=seed)
    return cfg, Wt, st, ex


def test_extend_one_token_is_one_step():
    for name in CFGS:
        cfg = W.get_config(name)
        q = [1] * cfg.batch
        cfg, Wt, st, ex = _setup(name, q)
        a, b = _clone(st), _clone(st)
        r = oracle.draft_extend(cfg, Wt, a, ex["cu_seqlens"], ex["aux"], ex["token_in"])
        b["aux"], b["token_in"] = ex["aux"], ex["token_in"]
        s = oracle.draft_step(cfg, Wt, b, 0)
        for k in ("hidden_out", "logits", "draft_id", "token_out"):
            assert torch.equal(r[k], s[k]), (name, k)
        for k in _cache_keys(cfg):
            assert torch.equal(a[k], b[k]), (name, k)


def test_extend_is_causal():
    """Changing the last new position of a sequence changes that position's
    output and nothing before it; changing the first changes the later ones."""
    for name in CFGS:
        cfg = W.get_config(name)
        q = [3] + [2] * (cfg.batch - 1)
        cfg, Wt, st, ex = _setup(name, q, seed=1)
        base = oracle.draft_extend(cfg, Wt, _clone(st), ex["cu_seqlens"], ex["aux"], ex["token_in"])
        last, first = 2, 0                          # rows of sequence 0 (q = 3)
        aux2, tok2 = ex["aux"].clone(), ex["token_in"].clone()
        aux2[last] = -aux2[last]
        tok2[last] = (tok2[last] + 1) % cfg.target_vocab
        r = oracle.draft_extend(cfg, Wt, _clone(st), ex["cu_seqlens"], aux2, tok2)
        assert torch.equal(r["hidden_out"][:last], base["hidden_out"][:last]), name
        assert torch.equal(r["hidden_out"][last + 1:], base["hidden_out"][last + 1:]), name
        assert not torch.equal(r["hidden_out"][last], base["hidden_out"][last]), name
        aux3 = ex["aux"].clone()
        aux3[first] = -aux3[first]
        r3 = oracle.draft_extend(cfg, Wt, _clone(st), ex["cu_seqlens"], aux3, ex["token_in"])
        # position 1 of sequence 0 attends to position 0's (changed) cache entry
        assert not torch.equal(r3["hidden_out"][first + 1], base["hidden_out"][first + 1]), name
        assert torch.equal(r3["hidden_out"][3:], base["hidden_out"][3:]), name


def test_extend_sequences_are_independent():
    for name in CFGS:
        cfg = W.get_config(name)
        q = [(b % 3) + 1 for b in range(cfg.batch)]
        cfg, Wt, st, ex = _setup(name, q, seed=2)
        full = oracle.draft_extend(cfg, Wt, _clone(st), ex["cu_seqlens"], ex["aux"], ex["token_in"])
        cu = ex["cu_seqlens"].tolist()
        for b in (0, cfg.batch - 1):
            sub = _clone(st)
            sub["ctx_len"] = st["ctx_len"][[b]]
            sub["block_table"] = st["block_table"][[b]]
            sl = slice(cu[b], cu[b + 1])
            one = oracle.draft_extend(cfg, Wt, sub, torch.tensor([0, cu[b + 1] - cu[b]], dtype=torch.int32),
                                      ex["aux"][sl], ex["token_in"][sl])
            # fp64 matmuls over a different number of rows may sum in another order
            assert torch.allclose(one["hidden_out"], full["hidden_out"][sl], rtol=1e-12, atol=1e-12), (name, b)
            assert torch.allclose(one["logits"], full["logits"][sl], rtol=1e-12, atol=1e-12), (name, b)
            assert torch.equal(one["token_out"], full["token_out"][sl]), (name, b)


def test_extend_empty_sequence_writes_nothing():
    for name in CFGS:
        cfg = W.get_config(name)
        q = [0] + [1] * (cfg.batch - 1)
        cfg, Wt, st, ex = _setup(name, q, seed=3)
        a = _clone(st)
        oracle.draft_extend(cfg, Wt, a, ex["cu_seqlens"], ex["aux"], ex["token_in"])
        P = cfg.page_size
        pos = int(st["ctx_len"][0])
        page, slot = int(st["block_table"][0, pos // P]), pos % P
        for k in _cache_keys(cfg):
            assert torch.equal(a[k][page, slot], st[k][page, slot]), (name, k)
