"""Pins of the CPU oracle against what the pages and the mathematics fix.

Each test checks the oracle against something other than itself: closed
forms, invariants, brute force on tiny inputs, or structured weights whose
result is known by hand.  The page-fixed constants come from
tests/golden/page_constants.json (each entry cites its page and section).
"""
import itertools
import json
import math
import os

import numpy as np
import pytest
import torch

import oracle as O
import workloads as W
from oracle import eagle3_oracle as OE

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
F64 = torch.float64


def _cfg(name, **kw):
    return W.get_config(name).replace(**kw)


# ------------------------------------------------------------- P1 shapes

@pytest.mark.parametrize("name", ["tiny_mha_b1", "mha_small", "mla_small"])
def test_step_shapes(name):
    cfg = W.get_config(name)
    Wt, st = W.make_weights(cfg), W.make_inputs(cfg)
    r = O.draft_step(cfg, Wt, st, 0)
    B = cfg.batch
    assert Wt["fc"].shape == (cfg.hidden, 3 * cfg.hidden)        # fc: 3H -> H
    assert r["hidden_out"].shape == (B, cfg.hidden)
    assert r["logits"].shape == (B, cfg.draft_vocab)
    assert Wt["w_o"].shape[0] == cfg.hidden                        # o_proj -> H
    assert Wt["lm_head"].shape == (cfg.draft_vocab, cfg.hidden)
    if cfg.attn_kind == W.MHA:
        assert Wt["w_q"].shape[1] == 2 * cfg.hidden                # q/k/v see 2H
    else:
        assert Wt["w_qa"].shape[1] == 2 * cfg.hidden and Wt["w_kva"].shape[1] == 2 * cfg.hidden
        assert Wt["w_o"].shape[1] == cfg.n_heads * cfg.v_head_dim


def test_page_constants_fixture():
    """The MLA workloads use the draft-config defaults the API page prints."""
    with open(os.path.join(GOLDEN, "page_constants.json")) as f:
        ref = json.load(f)["dsv3_mla_draft_config"]["values"]
    for name in ("dsv3_mla_b16", "dsv3_mla_b128_ragged", "dsv3_mla_b256_accept"):
        c = W.get_config(name)
        assert c.hidden == ref["hidden_size"]
        assert c.intermediate == ref["intermediate_size"]
        assert c.n_heads == ref["num_attention_heads"]
        assert c.q_lora_rank == ref["q_lora_rank"]
        assert c.kv_lora_rank == ref["kv_lora_rank"]
        assert c.qk_rope_dim == ref["qk_rope_head_dim"]
        assert c.qk_nope_dim == ref["qk_nope_head_dim"]
        assert c.v_head_dim == ref["v_head_dim"]
        assert c.draft_vocab == ref["vocab_size"] == c.target_vocab
        assert c.rms_eps == ref["rms_norm_eps"]
        assert c.rope_theta == ref["rope_theta"]
        assert c.yarn_orig_max_pos == ref["max_position_embeddings"]


# ------------------------------------------------------------- P2 RMSNorm

def test_rmsnorm_closed_forms():
    eps = 1e-6
    H = 37
    g = torch.linspace(0.5, 1.5, H, dtype=F64)
    c = 3.25
    v = torch.full((H,), c, dtype=F64)
    np.testing.assert_allclose(O.rms_norm(v, g, eps), c * g / math.sqrt(c * c + eps), rtol=1e-15)
    a, j = -2.5, 11
    v = torch.zeros(H, dtype=F64)
    v[j] = a
    out = O.rms_norm(v, g, eps)
    expect = torch.zeros(H, dtype=F64)
    expect[j] = a * math.sqrt(H) * g[j] / math.sqrt(a * a + H * eps)
    np.testing.assert_allclose(out, expect, rtol=1e-15, atol=0)
    # scale invariance (exact as eps -> 0; with eps, close for large norms)
    v = torch.randn(H, dtype=F64, generator=torch.Generator().manual_seed(0))
    np.testing.assert_allclose(O.rms_norm(v, g, 0.0), O.rms_norm(7.0 * v, g, 0.0), rtol=1e-14)
    # unit gain: output has unit root-mean-square
    out = O.rms_norm(v, torch.ones(H, dtype=F64), 0.0)
    assert abs(float((out * out).mean()) - 1.0) < 1e-14


# ------------------------------------------------------------- P3 GEMM, SiLU

def test_linear_brute_force():
    gen = torch.Generator().manual_seed(1)
    w = torch.randn(7, 13, generator=gen).to(torch.bfloat16)
    x = torch.randn(3, 13, generator=gen, dtype=F64)
    y = O.linear(x, w, rows_per_chunk=3)
    wl = w.to(F64).tolist()
    xl = x.tolist()
    for b in range(3):
        for n in range(7):
            s = 0.0
            for k in range(13):
                s += xl[b][k] * wl[n][k]
            assert abs(y[b, n].item() - s) < 1e-12


def test_silu_values():
    assert O.silu(torch.tensor([0.0], dtype=F64)).item() == 0.0
    assert abs(O.silu(torch.tensor([1.0], dtype=F64)).item() - 1.0 / (1.0 + math.exp(-1.0))) < 1e-16
    big = torch.tensor([40.0], dtype=F64)
    assert abs(O.silu(big).item() - 40.0) < 1e-12
    assert abs(O.silu(-big).item()) < 1e-15
    # SiLU(-z) = SiLU(z) - z
    z = torch.linspace(-5, 5, 11, dtype=F64)
    np.testing.assert_allclose(O.silu(-z), O.silu(z) - z, atol=1e-15)


# ------------------------------------------------------------- P6 RoPE/YaRN

def test_rope_closed_forms():
    theta = 10000.0
    inv = O.rope_inv_freq(4, theta)
    assert inv.tolist() == [1.0, 1.0 / 100.0]
    p = torch.tensor([3])
    # rotate-half pairs (0,2) and (1,3)
    x = torch.tensor([[[1.0, 0.0, 0.0, 0.0]]], dtype=F64)
    y = O.rope_rotate_half(x, p, inv)[0, 0]
    np.testing.assert_allclose(y, [math.cos(3), 0, math.sin(3), 0], atol=1e-15)
    x = torch.tensor([[[0.0, 1.0, 0.0, 0.0]]], dtype=F64)
    y = O.rope_rotate_half(x, p, inv)[0, 0]
    np.testing.assert_allclose(y, [0, math.cos(0.03), 0, math.sin(0.03)], atol=1e-15)
    # interleaved pairs (0,1) and (2,3)
    x = torch.tensor([[[1.0, 0.0, 0.0, 0.0]]], dtype=F64)
    y = O.rope_interleaved(x, p, inv)[0, 0]
    np.testing.assert_allclose(y, [math.cos(3), math.sin(3), 0, 0], atol=1e-15)
    x = torch.tensor([[[0.0, 0.0, 0.0, 1.0]]], dtype=F64)
    y = O.rope_interleaved(x, p, inv)[0, 0]
    np.testing.assert_allclose(y, [0, 0, -math.sin(0.03), math.cos(0.03)], atol=1e-15)


@pytest.mark.parametrize("fn", [O.rope_rotate_half, O.rope_interleaved])
def test_rope_invariants(fn):
    gen = torch.Generator().manual_seed(2)
    d = 64
    inv = O.yarn_inv_freq(d, 1e4, 40.0, 4096.0, 32.0, 1.0)
    q = torch.randn(1, 1, d, dtype=F64, generator=gen)
    k = torch.randn(1, 1, d, dtype=F64, generator=gen)
    # identity at position 0, norm preserving elsewhere
    np.testing.assert_allclose(fn(q, torch.tensor([0]), inv), q, atol=0)
    for p in (1, 77, 4099):
        np.testing.assert_allclose(fn(q, torch.tensor([p]), inv).norm(), q.norm(), rtol=1e-14)
    # scores depend only on the distance m - n
    def dot(m, n):
        return float((fn(q, torch.tensor([m]), inv) * fn(k, torch.tensor([n]), inv)).sum())
    assert abs(dot(10, 3) - dot(1007, 1000)) < 1e-9
    assert abs(dot(5, 5) - float((q * k).sum())) < 1e-12


def _ramp_weights(y, base, factor):
    """Interpolation weight w_i of each pair from t'_i = (1 - w_i) t_i + w_i t_i / factor."""
    return (base - y) / (base - base / factor)


def test_yarn_ramp():
    """NTK-by-parts at the DeepseekV3 shapes (rope dim 64, theta 1e4, original
    context 4096, beta_fast 32, beta_slow 1).  The boundaries come from the
    number of turns r_i = 4096 theta^(-2i/64) / (2 pi) each pair makes: pairs
    0..10 make more than 32 turns and keep their frequency, pairs 23..31 make
    less than one and are divided by the factor; in between the weight of the
    divided frequency is linear in the pair index (the DeepSeek YaRN rotary
    embedding the MLA head names), (i - 10) / 13."""
    d, theta = 64, 1e4
    base = O.rope_inv_freq(d, theta)
    # factor 1 reduces to plain RoPE
    np.testing.assert_allclose(O.yarn_inv_freq(d, theta, 1.0, 4096.0, 32.0, 1.0), base, rtol=1e-15)
    y = O.yarn_inv_freq(d, theta, 40.0, 4096.0, 32.0, 1.0)
    turns = 4096.0 * base / (2 * math.pi)
    assert (turns > 32.0).nonzero().flatten().tolist() == list(range(11))
    assert (turns < 1.0).nonzero().flatten().tolist() == list(range(23, 32))
    np.testing.assert_allclose(y[:11], base[:11], rtol=0)
    np.testing.assert_allclose(y[23:], base[23:] / 40.0, rtol=1e-15)
    w = _ramp_weights(y, base, 40.0)
    np.testing.assert_allclose(w[10:24], [(i - 10) / 13.0 for i in range(10, 24)], rtol=1e-12, atol=1e-13)
    assert abs(float(w[16]) - 6.0 / 13.0) < 1e-12
    assert abs(O.yarn_mscale(40.0) - 1.3688879454113936) < 1e-15      # 0.1 ln 40 + 1
    assert O.yarn_mscale(1.0) == 1.0


def test_yarn_equal_betas():
    """beta_fast = beta_slow (a draft may override the target's beta_fast 32
    with 1 [MAX-walkthrough section 5]).  At 4096 positions the pair making
    one turn lies between pairs 22 and 23, so the ramp spans one pair: 22
    keeps its frequency, 23 on are divided.  When the boundary is a whole
    pair index (orig_max_pos = 2 pi: pair 0 makes exactly one turn) the ramp
    is a step after it."""
    d, theta = 64, 1e4
    base = O.rope_inv_freq(d, theta)
    w = _ramp_weights(O.yarn_inv_freq(d, theta, 40.0, 4096.0, 1.0, 1.0), base, 40.0)
    expect = torch.tensor([0.0] * 23 + [1.0] * 9, dtype=F64)
    np.testing.assert_allclose(w, expect, atol=1e-13)
    w = _ramp_weights(O.yarn_inv_freq(d, theta, 40.0, 2 * math.pi, 1.0, 1.0), base, 40.0)
    expect = torch.tensor([0.0] + [1.0] * 31, dtype=F64)
    np.testing.assert_allclose(w, expect, atol=1e-13)


# ------------------------------------------------------------- attention score scales
# Two keys: a cached key whose score against the query is set by the test and
# a new key of zero score.  The first key's softmax weight is then
# e^D / (1 + e^D) with D = scale * (q . k), which the output reads back
# directly because the two values are orthogonal unit vectors (or zero).
# The scales are the published constants, evaluated by hand:
#   MHA: 1 / sqrt(head_dim) of scaled dot-product attention;
#   MLA: (0.1 ln s + 1)^2 / sqrt(qk_nope_dim + qk_rope_dim), YaRN's attention
#        temperature sqrt(1/t) = 0.1 ln s + 1 [YaRN section 3.4] on the
#        192-wide DeepseekV3 query-key dimension.

MHA_SCALE = {4: 0.5, 64: 0.125, 128: 0.08838834764831843}
MLA_TAU = {40.0: 0.1352337788608801, 4.0: 0.09356516759751217, 1.0: 0.07216878364870323}


def _sigmoid(z):
    return 1.0 / (1.0 + math.exp(-z))


@pytest.mark.parametrize("hd", [4, 64, 128])
def test_mha_two_key_score_scale(hd):
    H = 4
    cfg = W.Eagle3Config(name="two_key_mha", attn_kind=W.MHA, hidden=H, intermediate=8, draft_vocab=8,
                         target_vocab=8, n_heads=1, n_kv_heads=1, head_dim=hd, page_size=4, batch=1,
                         ctx=(1, 1), gamma=1)
    bf = torch.bfloat16
    q0 = torch.zeros(hd, dtype=F64)
    q0[:4] = torch.tensor([1.5, -0.5, 0.75, 1.0], dtype=F64)
    Wt = {"w_q": torch.zeros(hd, 2 * H, dtype=bf), "w_k": torch.zeros(hd, 2 * H, dtype=bf),
          "w_v": torch.zeros(hd, 2 * H, dtype=bf)}
    Wt["w_q"][:, 0] = q0.to(bf)
    Wt["w_v"][1, 0] = 1.0                                   # new value = e_1
    x = torch.zeros(1, 2 * H, dtype=F64)
    x[0, 0] = 1.0
    pos = torch.tensor([1])
    q_rot = O.rope_rotate_half(q0.view(1, 1, hd), pos, O.rope_inv_freq(hd, cfg.rope_theta)).view(hd)
    k0 = (q_rot * (3.0 * math.sqrt(hd) / 4.0 / float(q_rot @ q_rot))).to(torch.float32).to(bf)
    st = {"k_cache": torch.zeros(1, 4, 1, hd, dtype=bf), "v_cache": torch.zeros(1, 4, 1, hd, dtype=bf)}
    st["k_cache"][0, 0, 0] = k0
    st["v_cache"][0, 0, 0, 0] = 1.0                         # cached value = e_0
    out = OE._mha_attention(cfg, Wt, st, x, pos, torch.zeros(1, 1, dtype=torch.int32))[0]
    D = MHA_SCALE[hd] * float(q_rot @ k0.to(F64))
    assert abs(D - 0.75) < 0.01
    assert abs(float(out[0]) - _sigmoid(D)) < 1e-12
    assert abs(float(out[1]) - _sigmoid(-D)) < 1e-12
    assert float(out[2:].abs().max()) == 0.0


@pytest.mark.parametrize("factor", [40.0, 4.0, 1.0])
def test_mla_two_key_temperature(factor):
    H, r, dn, dr, dv = 2, 4, 128, 64, 2
    cfg = W.Eagle3Config(name="two_key_mla", attn_kind=W.MLA, hidden=H, intermediate=8, draft_vocab=8,
                         target_vocab=8, n_heads=1, q_lora_rank=2, kv_lora_rank=r, qk_nope_dim=dn,
                         qk_rope_dim=dr, v_head_dim=dv, yarn_factor=factor, yarn_orig_max_pos=4096.0,
                         page_size=4, batch=1, ctx=(1, 1), gamma=1)
    bf = torch.bfloat16
    gen = torch.Generator().manual_seed(11)
    n = (torch.rand(dn, generator=gen, dtype=torch.float32) * 0.5).to(bf)
    u = (torch.rand(dn, generator=gen, dtype=torch.float32) * 0.5).to(bf)
    Wt = {"w_qa": torch.zeros(2, 2 * H, dtype=bf), "norm_qa": torch.ones(2, dtype=bf),
          "w_qb": torch.zeros(dn + dr, 2, dtype=bf), "w_kva": torch.zeros(r + dr, 2 * H, dtype=bf),
          "norm_kv": torch.ones(r, dtype=bf), "w_kvb": torch.zeros(dn + dv, r, dtype=bf)}
    Wt["w_qa"][:, 0] = 1.0                                  # q_a = RMS((1, 1)) = 1 / sqrt(1 + eps)
    Wt["w_qb"][:dn, 0] = n                                  # q_nope = n q_a[0]; q_pe = 0
    Wt["w_kvb"][:dn, 0] = u                                 # W_UK c_0 = u
    Wt["w_kvb"][dn, 0] = 1.0                                # W_UV c_0 = e_0
    x = torch.zeros(1, 2 * H, dtype=F64)
    x[0, 0] = 1.0
    st = {"kv_cache": torch.zeros(1, 4, r + dr, dtype=bf)}
    st["kv_cache"][0, 0, 0] = 1.0                           # cached latent c_0 = e_0, k_pe_0 = 0
    out = OE._mla_attention(cfg, Wt, st, x, torch.tensor([1]), torch.zeros(1, 1, dtype=torch.int32))[0]
    qa = 1.0 / math.sqrt(1.0 + cfg.rms_eps)
    dot = float(n.to(F64) @ u.to(F64)) * qa
    D = MLA_TAU[factor] * dot
    assert 4.0 < dot < 20.0
    # the new entry is zero (W_kva = 0): score 0, value 0
    assert abs(float(out[0]) - _sigmoid(D)) < 1e-12
    assert float(out[1:].abs().max()) == 0.0


# ------------------------------------------------------------- P5 softmax

def test_softmax_invariants():
    gen = torch.Generator().manual_seed(3)
    V = torch.randn(9, 5, dtype=F64, generator=gen)
    s = torch.full((9,), 0.7, dtype=F64)
    np.testing.assert_allclose(O.softmax_attend(s, V), V.mean(0), rtol=1e-14)
    s = torch.randn(9, dtype=F64, generator=gen)
    np.testing.assert_allclose(O.softmax_attend(s + 123.0, V), O.softmax_attend(s, V), rtol=1e-12)
    perm = torch.randperm(9, generator=gen)
    np.testing.assert_allclose(O.softmax_attend(s[perm], V[perm]), O.softmax_attend(s, V), rtol=1e-13)
    # one dominant key returns its value
    s = torch.zeros(9, dtype=F64)
    s[4] = 1e4
    np.testing.assert_allclose(O.softmax_attend(s, V), V[4], rtol=1e-14)


def _repage(cfg, st, seed=7):
    """Same logical cache contents under a different random page assignment."""
    B = cfg.batch
    table = st["block_table"]
    g = torch.Generator().manual_seed(seed)
    key = "k_cache" if cfg.attn_kind == W.MHA else "kv_cache"
    npages = st[key].shape[0]
    perm = torch.randperm(npages, generator=g)
    new = {k: v.clone() for k, v in st.items()}
    new["block_table"] = perm[table.long()].to(torch.int32)
    for name in ("k_cache", "v_cache", "kv_cache"):
        if name in st:
            c = torch.empty_like(st[name])
            c[perm] = st[name]
            new[name] = c
    return new


@pytest.mark.parametrize("name", ["mha_small", "mla_small"])
def test_paging_invariance(name):
    cfg = W.get_config(name)
    Wt, st = W.make_weights(cfg), W.make_inputs(cfg)
    st2 = _repage(cfg, st)
    r1 = O.draft_chain(cfg, Wt, st, cfg.gamma)
    r2 = O.draft_chain(cfg, Wt, st2, cfg.gamma)
    assert torch.equal(r1["tokens"], r2["tokens"])
    for a, b in zip(r1["steps"], r2["steps"]):
        assert torch.equal(a["hidden_out"], b["hidden_out"])


# ------------------------------------------------------------- P4 one key

def test_single_token_attention_returns_v_mha():
    cfg = _cfg("mha_small", ctx=(0, 0))
    Wt, st = W.make_weights(cfg), W.make_inputs(cfg)
    B, H = cfg.batch, cfg.hidden
    gen = torch.Generator().manual_seed(4)
    x = torch.randn(B, 2 * H, dtype=F64, generator=gen)
    pos = st["ctx_len"].long()
    out = OE._mha_attention(cfg, Wt, st, x, pos, st["block_table"])
    v = (x @ Wt["w_v"].to(F64).T).view(B, cfg.n_kv_heads, cfg.head_dim)
    v = v.to(torch.float32).to(torch.bfloat16).to(F64)
    group = cfg.n_heads // cfg.n_kv_heads
    expect = v.repeat_interleave(group, dim=1).reshape(B, -1)
    np.testing.assert_allclose(out, expect, rtol=1e-14, atol=1e-14)


def test_single_token_attention_returns_v_mla():
    cfg = _cfg("mla_small", ctx=(0, 0))
    Wt, st = W.make_weights(cfg), W.make_inputs(cfg)
    B, H = cfg.batch, cfg.hidden
    gen = torch.Generator().manual_seed(5)
    x = torch.randn(B, 2 * H, dtype=F64, generator=gen)
    pos = st["ctx_len"].long()
    out = OE._mla_attention(cfg, Wt, st, x, pos, st["block_table"]).view(B, cfg.n_heads, -1)
    kv = x @ Wt["w_kva"].to(F64).T
    c = kv[:, : cfg.kv_lora_rank]
    c = c / torch.sqrt((c * c).mean(-1, keepdim=True) + cfg.rms_eps) * Wt["norm_kv"].to(F64)
    c = c.to(torch.float32).to(torch.bfloat16).to(F64)
    w_uv = Wt["w_kvb"].to(F64).view(cfg.n_heads, -1, cfg.kv_lora_rank)[:, cfg.qk_nope_dim:, :]
    for b in range(B):
        for h in range(cfg.n_heads):
            np.testing.assert_allclose(out[b, h], w_uv[h] @ c[b], rtol=1e-12, atol=1e-13)


# ------------------------------------------------------------- P7 GQA

def test_gqa_equals_mha_with_repeated_kv():
    cfg = _cfg("mha_small")                  # 6 q heads over 2 kv heads
    Wt, st = W.make_weights(cfg), W.make_inputs(cfg)
    g = cfg.n_heads // cfg.n_kv_heads
    hd = cfg.head_dim
    cfg2 = cfg.replace(n_kv_heads=cfg.n_heads)
    Wt2 = dict(Wt)
    for nm in ("w_k", "w_v"):
        Wt2[nm] = Wt[nm].view(cfg.n_kv_heads, hd, -1).repeat_interleave(g, 0).reshape(-1, 2 * cfg.hidden)
    st2 = dict(st)
    for nm in ("k_cache", "v_cache"):
        st2[nm] = st[nm].repeat_interleave(g, dim=2).contiguous()      # [pages, page, kv heads, hd]
    B = cfg.batch
    x = torch.randn(B, 2 * cfg.hidden, dtype=F64, generator=torch.Generator().manual_seed(6))
    pos = st["ctx_len"].long()
    a = OE._mha_attention(cfg, Wt, {k: v.clone() for k, v in st.items()}, x, pos, st["block_table"])
    b = OE._mha_attention(cfg2, Wt2, st2, x, pos, st["block_table"])
    np.testing.assert_allclose(a, b, rtol=1e-13, atol=1e-13)


# ------------------------------------------------------------- P8 absorbed MLA

def test_mla_absorbed_equals_decompressed():
    gen = torch.Generator().manual_seed(8)
    nh, dn, dr, dv, r, n = 3, 6, 4, 5, 8, 11
    q_nope = torch.randn(nh, dn, dtype=F64, generator=gen)
    q_pe = torch.randn(nh, dr, dtype=F64, generator=gen)
    c = torch.randn(n, r, dtype=F64, generator=gen)
    k_pe = torch.randn(n, dr, dtype=F64, generator=gen)
    w_uk = torch.randn(nh, dn, r, dtype=F64, generator=gen)
    w_uv = torch.randn(nh, dv, r, dtype=F64, generator=gen)
    tau = 0.37
    plain = O.mla_attend_plain(q_nope, q_pe, c, k_pe, w_uk, w_uv, tau)
    for h in range(nh):
        q_lat = w_uk[h].T @ q_nope[h]               # absorb W_UK into the query
        s = tau * (c @ q_lat + k_pe @ q_pe[h])
        p = torch.softmax(s, dim=0)
        o = w_uv[h] @ (p @ c)                       # attend in latent space, then W_UV
        np.testing.assert_allclose(plain[h], o, rtol=1e-12, atol=1e-13)


# ------------------------------------------------------------- P9 top-1, d2t

def test_argmax_lowest_index_on_ties_and_d2t():
    cfg = _cfg("tiny_mha_b1")
    Wt, st = W.make_weights(cfg), W.make_inputs(cfg)
    r = O.draft_step(cfg, Wt, {k: v.clone() for k, v in st.items()}, 0)
    d = int(r["draft_id"][0])
    assert torch.equal(r["token_out"], r["draft_id"])            # zero d2t: identity
    # duplicate the winning lm_head row at a lower index: exact tie, lower wins
    if d > 0:
        Wt2 = dict(Wt)
        lm = Wt["lm_head"].clone()
        lm[d - 1] = lm[d]
        Wt2["lm_head"] = lm
        r2 = O.draft_step(cfg, Wt2, {k: v.clone() for k, v in st.items()}, 0)
        assert int(r2["draft_id"][0]) == d - 1
        assert float(r2["margin"][0]) == 0.0


def test_sorted_d2t_map():
    cfg = W.get_config("llama3_8b_gqa_b32")
    d2t = W.make_d2t(cfg).long()
    tgt = torch.arange(cfg.draft_vocab) + d2t
    assert bool((tgt[1:] > tgt[:-1]).all())                     # strictly increasing => injective
    assert int(tgt[0]) >= 0 and int(tgt[-1]) < cfg.target_vocab


def test_d2t_offsets_applied():
    cfg = _cfg("mha_small")
    Wt, st = W.make_weights(cfg), W.make_inputs(cfg)
    r = O.draft_step(cfg, Wt, st, 0)
    d2t = Wt["d2t"].long()
    assert torch.equal(r["token_out"], r["draft_id"] + d2t[r["draft_id"]])
    assert bool((r["token_out"] < cfg.target_vocab).all())


# ------------------------------------------------------------- P10, P11 accept

def _accept_brute(draft, target):
    g = len(draft)
    best = 0
    for n in range(g + 1):
        if list(draft[:n]) == list(target[:n]):
            best = n
    return best, target[best]


@pytest.mark.parametrize("gamma", [1, 2, 3, 4])
def test_accept_exhaustive(gamma):
    cases = list(itertools.product(range(3), repeat=2 * gamma + 1))
    arr = torch.tensor(cases, dtype=torch.int32)
    draft, target = arr[:, :gamma], arr[:, gamma:]
    acc, bonus = O.greedy_accept(draft, target)
    for i, cse in enumerate(cases):
        a, bo = _accept_brute(cse[:gamma], cse[gamma:])
        assert int(acc[i]) == a and int(bonus[i]) == bo


def test_accept_synthesised_closed_form():
    cfg = W.get_config("dsv3_mla_b256_accept")
    draft = W.random_drafts(cfg)
    tgt, k = W.make_accept_targets(cfg, draft)
    acc, bonus = O.greedy_accept(draft, tgt)
    assert torch.equal(acc, k.long())
    assert torch.equal(bonus, tgt[torch.arange(cfg.batch), k.long()].long())
    # Geometric(0.3) - 1 capped at 7: rejection at the first draft is common
    assert int((k == 0).sum()) > 0 and int(k.max()) <= cfg.gamma


# ------------------------------------------------------------- P12-P14 chain

@pytest.mark.parametrize("name", ["mha_small", "mla_small"])
def test_chain_consistency(name):
    cfg = W.get_config(name)
    Wt = W.make_weights(cfg)
    st = W.make_inputs(cfg)
    one = O.draft_step(cfg, Wt, {k: v.clone() for k, v in st.items()}, 0)
    ch1 = O.draft_chain(cfg, Wt, {k: v.clone() for k, v in st.items()}, 1)
    assert torch.equal(ch1["steps"][0]["hidden_out"], one["hidden_out"])
    ch = O.draft_chain(cfg, Wt, {k: v.clone() for k, v in st.items()}, cfg.gamma)
    # steps after the first ignore the aux states (fc only fuses 3H inputs)
    st2 = {k: v.clone() for k, v in st.items()}
    s0 = O.draft_step(cfg, Wt, st2, 0)
    st2["aux"] = torch.zeros_like(st2["aux"])
    s1 = O.draft_step(cfg, Wt, st2, 1, hidden_in=s0["hidden_out"], token_in=s0["token_out"])
    assert torch.equal(s1["hidden_out"], ch["steps"][1]["hidden_out"])
    assert torch.equal(s1["token_out"], ch["tokens"][:, 1])


@pytest.mark.parametrize("name", ["mha_small", "mla_small"])
def test_batch_independence(name):
    cfg = W.get_config(name)
    Wt, st = W.make_weights(cfg), W.make_inputs(cfg)
    full = O.draft_chain(cfg, Wt, {k: v.clone() for k, v in st.items()}, cfg.gamma)
    perm = torch.tensor([3, 0, 4, 1, 2])
    st2 = {k: v.clone() for k, v in st.items()}
    for nm in ("aux", "token_in", "ctx_len", "block_table"):
        st2[nm] = st[nm][perm]
    r = O.draft_chain(cfg, Wt, st2, cfg.gamma)
    assert torch.equal(r["tokens"], full["tokens"][perm])
    np.testing.assert_allclose(r["steps"][-1]["hidden_out"], full["steps"][-1]["hidden_out"][perm],
                               rtol=1e-12, atol=1e-12)


# ------------------------------------------------------------- structured weights

def _structured_mha(H=8, hd=4, nq=2, I=8, V=8):
    """A head whose step can be followed by hand."""
    cfg = W.Eagle3Config(name="hand", attn_kind=W.MHA, hidden=H, intermediate=I, draft_vocab=V,
                         target_vocab=V, n_heads=nq, n_kv_heads=nq, head_dim=hd, batch=1,
                         ctx=(0, 0), gamma=1, paging="identity")
    gen = torch.Generator().manual_seed(9)
    bf = torch.bfloat16
    eye = torch.eye(H, dtype=bf)
    Wt = {
        "embed": torch.randn(V, H, generator=gen).to(bf),
        "fc": torch.cat([eye, torch.zeros(H, 2 * H, dtype=bf)], dim=1),      # g = early layer
        "norm_in": torch.ones(H, dtype=bf), "norm_hid": torch.ones(H, dtype=bf),
        "norm_post": torch.ones(H, dtype=bf), "norm_final": torch.ones(H, dtype=bf),
        "w_q": torch.randn(nq * hd, 2 * H, generator=gen).to(bf),
        "w_k": torch.randn(nq * hd, 2 * H, generator=gen).to(bf),
        "w_v": torch.cat([eye, torch.zeros(H, H, dtype=bf)], dim=1),        # v = norm(embedding)
        "w_o": eye.clone(),
        "w_gate": eye.clone(), "w_up": eye.clone(), "w_down": eye.clone(),
        "lm_head": eye.clone(),
        "d2t": torch.zeros(V, dtype=torch.int32),
    }
    st = W.make_inputs(cfg)
    st["aux"] = torch.randn(1, 3, H, generator=gen).to(bf)
    return cfg, Wt, st


def test_structured_step_by_hand():
    cfg, Wt, st = _structured_mha()
    r = O.draft_step(cfg, Wt, st, 0)
    eps = cfg.rms_eps
    a = st["aux"][0, 0].to(F64).numpy()                 # g = early aux (fc selects it, no bias)
    e = Wt["embed"][int(st["token_in"][0])].to(F64).numpy()
    en = e / np.sqrt((e ** 2).mean() + eps)
    v = en.astype(np.float32).astype(np.float64)
    v = torch.tensor(v).to(torch.bfloat16).to(F64).numpy()   # single key: attention returns bf16(v)
    h1 = a + v
    u = h1 / np.sqrt((h1 ** 2).mean() + eps)
    h_out = h1 + (u / (1 + np.exp(-u))) * u              # identity gate/up/down
    z = h_out / np.sqrt((h_out ** 2).mean() + eps)       # identity lm_head
    np.testing.assert_allclose(r["hidden_out"][0].numpy(), h_out, rtol=1e-13, atol=1e-13)
    np.testing.assert_allclose(r["logits"][0].numpy(), z, rtol=1e-13, atol=1e-13)
    assert int(r["draft_id"][0]) == int(np.argmax(z))


def test_structured_zero_branches_give_fc():
    cfg, Wt, st = _structured_mha()
    Wt = dict(Wt)
    Wt["w_o"] = torch.zeros_like(Wt["w_o"])
    Wt["w_down"] = torch.zeros_like(Wt["w_down"])
    H = cfg.hidden
    Wt["fc"] = torch.cat([torch.zeros(H, 2 * H), torch.eye(H)], dim=1).to(torch.bfloat16)  # late layer
    r = O.draft_step(cfg, Wt, st, 0)
    np.testing.assert_allclose(r["hidden_out"][0], st["aux"][0, 2].to(F64), rtol=0, atol=0)


# ------------------------------------------------ fc width and the target's lm_head
def test_two_way_fc_is_three_way_with_a_zero_block():
    """A head fusing two target layers (fc 2H -> H) equals a three-way head whose
    fc has a zero third block, whatever the third aux state holds: the fc
    input is the layers' concatenation [MAX-walkthrough section 11: fc is
    2-way or 3-way by its shape]."""
    c2 = W.get_config("mha_small_aux2_tgt_head")
    c3 = c2.replace(num_aux=3, aux_scales=(1.0, 0.5, 1.0))
    W2 = W.make_weights(c2)
    W3 = dict(W2)
    W3["fc"] = torch.cat([W2["fc"], torch.zeros(c2.hidden, c2.hidden, dtype=torch.bfloat16)], dim=1)
    s2 = W.make_inputs(c2)
    s3 = {k: v.clone() for k, v in s2.items()}
    s3["aux"] = torch.cat([s2["aux"], torch.randn(c2.batch, 1, c2.hidden).to(torch.bfloat16)], dim=1)
    r2 = O.draft_step(c2, W2, s2, 0)
    r3 = O.draft_step(c3, W3, s3, 0)
    assert W2["fc"].shape == (c2.hidden, 2 * c2.hidden)
    assert torch.allclose(r2["hidden_out"], r3["hidden_out"], rtol=1e-12, atol=1e-12)
    assert torch.equal(r2["draft_id"], r3["draft_id"])


def test_target_lm_head_ids_are_target_ids():
    """Without d2t the head scores through its target's lm_head over the target
    vocabulary, so its ids are target ids [MAX-API has_own_lm_head]; a zero
    d2t gives the same ids."""
    cfg = W.get_config("mha_small_aux2_tgt_head")
    Wt = W.make_weights(cfg)
    assert "d2t" not in Wt and cfg.draft_vocab == cfg.target_vocab
    st = W.make_inputs(cfg)
    r = O.draft_step(cfg, Wt, {k: v.clone() for k, v in st.items()}, 0)
    assert torch.equal(r["token_out"], r["draft_id"])
    Wz = dict(Wt, d2t=torch.zeros(cfg.draft_vocab, dtype=torch.int32))
    rz = O.draft_step(cfg, Wz, {k: v.clone() for k, v in st.items()}, 0)
    assert torch.equal(rz["token_out"], r["token_out"])
    assert torch.equal(rz["hidden_out"], r["hidden_out"])
