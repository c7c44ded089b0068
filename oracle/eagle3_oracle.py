"""CPU oracle of one EAGLE-3 draft-head step, a chain of steps, greedy chain
verification and its relaxed variant for thinking spans.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import, call or
link this module: only the tests, ``__graft_entry__.smoke()`` and the bench's
CPU-baseline leg use it.  It shares no code with the HIP library.

Arithmetic: float64 torch CPU ops throughout.  The only rounding to a
narrower type is where the interface fixes a storage type: the cache entry
a step appends is stored in bf16 (round to nearest even), and attention reads
every key, the new one included, back from that bf16 cache.

Sources, cited by page title and section:
  [MAX-walkthrough] "Eagle3 DeepseekV3 投机解码架构 — MAX 中 eagle3_deepseekV3
      模块的完整解析", section 4 (Eagle3MLADraft structure and forward),
      section 7 (one-layer paged draft cache), section 9 (decode-mode draft
      steps, and the prefill phase over accepted positions that
      draft_extend follows), section 10 (greedy acceptance, argmax
      proposals), section 11 (Llama-style MHA head).
  [MAX-API] "max.pipelines.architectures.eagle3_deepseekV3", the
      Eagle3DeepseekV3DraftConfig defaults (eps, rope theta, interleaved rope,
      MLA ranks, SiLU) and the MHA head's bf16 cache.
  [ModelOpt] "EAGLE头结构深潜：Model Optimizer投机解码草稿模型的内部设计",
      sections on the fc fusion, the doubled first-layer attention input with
      two RMSNorms, the draft lm_head with the d2t map, and multi-step drafting
      from the head's own hidden state.
  [YaRN] Peng et al., "YaRN: Efficient Context Window Extension of Large
      Language Models" (2023), section 3.2 (NTK-by-parts interpolation) and
      section 3.4 (attention temperature).  The pages name YaRN for the MLA
      head but do not write it out.

Readings where the pages are silent (the GPU path implements the same ones):
  * concat order is [norm(embedding) || norm(fused hidden)];
  * the residual stream is the fused hidden g (width H); only the attention
    input projections see 2H;
  * the hidden carried to the next step is h_out before the final norm;
  * MLA keeps DeepseekV3's q_a and kv-latent RMSNorms (gains, same eps);
  * MLP is gated SiLU: down(silu(gate(u)) * up(u));
  * GQA: query head h reads kv head h // (n_heads / n_kv_heads);
  * the new token sits at position ctx_len + step and attends to itself;
  * Llama RoPE pairs (i, i + d/2); MLA RoPE pairs (2i, 2i+1) (interleaved);
  * YaRN frequencies follow the DeepSeek YaRN rotary embedding the MLA head
    names (a ramp in the pair index), the temperature the YaRN paper
    (see yarn_*).
"""
from __future__ import annotations

import math
from typing import Dict, Optional

import torch

F64 = torch.float64

MHA = 0
MLA = 1


def f64(t: torch.Tensor) -> torch.Tensor:
    return t.to(F64)


def bf16_round(t: torch.Tensor) -> torch.Tensor:
    """Storage rounding of a cache entry: nearest-even bf16, back as float64."""
    return t.to(torch.float32).to(torch.bfloat16).to(F64)


# ---------------------------------------------------------------- primitives

def rms_norm(v: torch.Tensor, gain: torch.Tensor, eps: float) -> torch.Tensor:
    """RMSNorm over the last axis: v / sqrt(mean(v^2) + eps) * gain.

    eps = 1e-6 is the head's rms_norm_eps [MAX-API, draft config defaults].
    """
    v = f64(v)
    ms = (v * v).mean(dim=-1, keepdim=True)
    return v / torch.sqrt(ms + eps) * f64(gain)


# ---------------------------------------------------------------- weight formats
# A draft head may be post-training quantized to FP8 or NVFP4 [ModelOpt:
# export and PTQ section; MAX-walkthrough section 5: a quantized draft carries
# weight_scale tensors].  The pages name the formats only; the element
# encodings below are the published OCP 8-bit (E4M3, "FN": no infinities) and
# 4-bit (E2M1) floating-point definitions, and the scale layout is the reading
# stated for the kernels: FP8 codes times one fp32 scale per output row;
# NVFP4 codes times an E4M3 scale per 16 consecutive inputs of a row times
# one fp32 scale per output row (a per-tensor scale is that value repeated).

def decode_e4m3(codes: torch.Tensor) -> torch.Tensor:
    """OCP FP8 E4M3: sign, 4 exponent bits (bias 7), 3 mantissa bits;
    exponent 0 is subnormal (m/8 * 2^-6); S.1111.111 is NaN; no infinities."""
    c = codes.to(torch.int64)
    s = (c >> 7) & 1
    e = (c >> 3) & 15
    m = (c & 7).to(F64)
    mag = torch.where(e > 0, (1.0 + m / 8.0) * torch.pow(2.0, (e - 7).to(F64)), m / 8.0 * 2.0 ** -6)
    mag = torch.where((e == 15) & ((c & 7) == 7), torch.full_like(mag, math.nan), mag)
    return torch.where(s == 1, -mag, mag)


def decode_e2m1(nib: torch.Tensor) -> torch.Tensor:
    """OCP FP4 E2M1: sign, 2 exponent bits (bias 1), 1 mantissa bit; exponent 0
    is subnormal (m/2); magnitudes 0, 0.5, 1, 1.5, 2, 3, 4, 6."""
    c = nib.to(torch.int64)
    s = (c >> 3) & 1
    e = (c >> 1) & 3
    m = (c & 1).to(F64)
    mag = torch.where(e > 0, (1.0 + m / 2.0) * torch.pow(2.0, (e - 1).to(F64)), m / 2.0)
    return torch.where(s == 1, -mag, mag)


class QuantWeight:
    """A quantized [N, K] weight: rows are dequantized to float64 on demand."""

    def __init__(self, fmt: str, codes: torch.Tensor, row_scale: torch.Tensor,
                 block_scale: Optional[torch.Tensor] = None):
        self.fmt, self.codes, self.row_scale, self.block_scale = fmt, codes, row_scale, block_scale
        K = codes.shape[1] * (2 if fmt == "nvfp4" else 1)
        self.shape = (codes.shape[0], K)

    # every code's value, from the decoders above (a table lookup per element
    # is the same definition, evaluated faster on large matrices)
    _E4M3 = None
    _E2M1 = None

    @classmethod
    def _tables(cls):
        if cls._E4M3 is None:
            cls._E4M3 = decode_e4m3(torch.arange(256))
            cls._E2M1 = decode_e2m1(torch.arange(16))
        return cls._E4M3, cls._E2M1

    def rows(self, r0: int, r1: int) -> torch.Tensor:
        e4m3, e2m1 = self._tables()
        c = self.codes[r0:r1].to(torch.int64)
        if self.fmt == "fp8":
            w = e4m3[c]
        else:
            # element 2i in the low nibble of byte i, element 2i+1 in the high one
            w = e2m1[torch.stack([c & 15, c >> 4], dim=-1).reshape(c.shape[0], -1)]
            w = w * e4m3[self.block_scale[r0:r1].to(torch.int64)].repeat_interleave(16, dim=1)
        return w * f64(self.row_scale[r0:r1]).unsqueeze(1)

    def dense(self) -> torch.Tensor:
        return self.rows(0, self.shape[0])


GEMM_WEIGHTS = ("fc", "w_q", "w_k", "w_v", "w_qa", "w_qb", "w_kva", "w_kvb", "w_o", "w_gate", "w_up",
                "w_down", "lm_head")


def weight_view(cfg, W: Dict[str, torch.Tensor]) -> Dict[str, object]:
    """The head's weights with every GEMM matrix of a quantized head wrapped
    as a QuantWeight (codes in W[name], scales in W[name + ".row_scale"] and,
    for NVFP4, W[name + ".block_scale"])."""
    fmt = getattr(cfg, "weight_format", "bf16")
    if fmt == "bf16":
        return W
    V = dict(W)
    for n in GEMM_WEIGHTS:
        if n in W:
            V[n] = QuantWeight(fmt, W[n], W[n + ".row_scale"], W.get(n + ".block_scale"))
    return V


def dense(w) -> torch.Tensor:
    return w.dense() if isinstance(w, QuantWeight) else f64(w)


def linear(x: torch.Tensor, w, rows_per_chunk: int = 8192) -> torch.Tensor:
    """y = x @ w.T with w stored [out, in] (bf16, or a QuantWeight); no bias.

    The weight is widened to float64 a block of output rows at a time so that
    vocabulary-sized matrices fit in host memory; every output element is one
    whole dot product over the input axis.
    """
    x = f64(x)
    out = torch.empty(*x.shape[:-1], w.shape[0], dtype=F64)
    for r0 in range(0, w.shape[0], rows_per_chunk):
        r1 = min(w.shape[0], r0 + rows_per_chunk)
        out[..., r0:r1] = x @ (w.rows(r0, r1) if isinstance(w, QuantWeight) else f64(w[r0:r1])).T
    return out


def silu(z: torch.Tensor) -> torch.Tensor:
    """SiLU(z) = z / (1 + exp(-z)) (hidden_act 'silu' [MAX-API])."""
    return z / (1.0 + torch.exp(-z))


def rope_inv_freq(dim: int, theta: float) -> torch.Tensor:
    """theta^(-2i/dim) for i = 0 .. dim/2 - 1."""
    i = torch.arange(dim // 2, dtype=F64)
    return theta ** (-2.0 * i / dim)


def yarn_correction_pair(turns: float, dim: int, theta: float, orig_max_pos: float) -> float:
    """The (fractional) pair index i whose base frequency theta^(-2i/dim) makes
    `turns` full turns over orig_max_pos positions: solves
    orig_max_pos * theta^(-2i/dim) / (2 pi) = turns for i."""
    return dim * math.log(orig_max_pos / (2.0 * math.pi * turns)) / (2.0 * math.log(theta))


def yarn_inv_freq(dim: int, theta: float, factor: float, orig_max_pos: float,
                  beta_fast: float, beta_slow: float) -> torch.Tensor:
    """YaRN 'NTK-by-parts' frequencies [YaRN section 3.2] in the form of the
    DeepSeek YaRN rotary embedding that the MLA head uses [MAX-walkthrough
    section 4: its rope is DeepseekYarnRotaryEmbedding and needs
    rope_scaling].

    Pair i keeps its base frequency t_i = theta^(-2i/dim) when it turns fast
    over the original context and is interpolated to t_i / factor when it
    turns slowly.  The boundaries are whole pair indices: lo is the floor of
    the pair that makes beta_fast turns, hi the ceil of the pair that makes
    beta_slow turns, both clamped to [0, dim - 1].  Between them the
    interpolation weight ramps linearly in the pair index,
        w_i = clamp((i - lo) / (hi - lo), 0, 1),
    and it is a step (w_i = 1 exactly for i > lo) when hi <= lo, e.g. for
    beta_fast = beta_slow at an integer boundary.  Then
        t'_i = (1 - w_i) * t_i + w_i * t_i / factor.
    Needs theta > 1 and beta_fast >= beta_slow > 0.
    """
    assert theta > 1.0 and beta_fast >= beta_slow > 0.0
    t = rope_inv_freq(dim, theta)
    lo = min(max(math.floor(yarn_correction_pair(beta_fast, dim, theta, orig_max_pos)), 0), dim - 1)
    hi = min(max(math.ceil(yarn_correction_pair(beta_slow, dim, theta, orig_max_pos)), 0), dim - 1)
    i = torch.arange(dim // 2, dtype=F64)
    if hi > lo:
        w = ((i - lo) / (hi - lo)).clamp(0.0, 1.0)
    else:
        w = (i > lo).to(F64)
    return (1.0 - w) * t + w * t / factor


def yarn_mscale(factor: float) -> float:
    """sqrt(1/t) = 0.1 ln(s) + 1 for s > 1 [YaRN section 3.4]; 1 otherwise."""
    return 0.1 * math.log(factor) + 1.0 if factor > 1.0 else 1.0


def rope_rotate_half(x: torch.Tensor, pos: torch.Tensor, inv_freq: torch.Tensor) -> torch.Tensor:
    """Llama RoPE: pairs (i, i + d/2) turned by pos * inv_freq[i].

    x: [B, heads, d]; pos: [B] integer positions.
    """
    d = x.shape[-1]
    ang = f64(pos).view(-1, 1, 1) * inv_freq.view(1, 1, -1)      # [B,1,d/2]
    c, s = torch.cos(ang), torch.sin(ang)
    a, b = x[..., : d // 2], x[..., d // 2:]
    return torch.cat([a * c - b * s, a * s + b * c], dim=-1)


def rope_interleaved(x: torch.Tensor, pos: torch.Tensor, inv_freq: torch.Tensor) -> torch.Tensor:
    """Interleaved RoPE (rope_interleave=True [MAX-API]): pairs (2i, 2i+1).

    x: [B, heads, d]; pos: [B].
    """
    ang = f64(pos).view(-1, 1, 1) * inv_freq.view(1, 1, -1)
    c, s = torch.cos(ang), torch.sin(ang)
    a, b = x[..., 0::2], x[..., 1::2]
    out = torch.empty_like(x)
    out[..., 0::2] = a * c - b * s
    out[..., 1::2] = a * s + b * c
    return out


def softmax_attend(scores: torch.Tensor, values: torch.Tensor) -> torch.Tensor:
    """sum_j softmax(scores)_j * values_j over the key axis (-1 of scores)."""
    m = scores.max(dim=-1, keepdim=True).values
    p = torch.exp(scores - m)
    p = p / p.sum(dim=-1, keepdim=True)
    return p @ values


# ---------------------------------------------------------------- cache view

def cache_positions(block_table_row: torch.Tensor, n: int, page_size: int):
    """(page, slot) of positions 0..n-1 of one sequence in the paged cache."""
    j = torch.arange(n)
    return block_table_row[j // page_size].long(), j % page_size


# ---------------------------------------------------------------- one step

def draft_step(cfg, W: Dict[str, torch.Tensor], state: Dict[str, torch.Tensor],
               step_index: int, hidden_in: Optional[torch.Tensor] = None,
               token_in: Optional[torch.Tensor] = None) -> Dict[str, torch.Tensor]:
    """One draft-head step for every row of the batch.

    state holds aux [B, 3, H] bf16 (used when hidden_in is None), token_in [B],
    ctx_len [B], block_table [B, max_pages] and the cache tensors, which this
    call updates in place with the new token's entry.

    Returns float64 hidden_out [B, H] and logits [B, Vd], int64 draft_id and
    token_out [B], and the top-1/top-2 logit margin [B].
    """
    W = weight_view(cfg, W)
    B, H = state["token_in"].shape[0], cfg.hidden
    tok = (state["token_in"] if token_in is None else token_in).long()
    ctx = state["ctx_len"].long()
    pos = ctx + step_index                        # the new token's position
    table = state["block_table"]

    # E1: fused hidden.  Step 1 fuses the three aux states with fc (3H -> H,
    # no bias) [MAX-walkthrough section 4; ModelOpt fc section]; later steps
    # take the previous step's own hidden, which is H wide and skips fc
    # [MAX-walkthrough section 4, "only a 3H-wide input goes through fc";
    # ModelOpt TTT section].
    if hidden_in is None:
        aux = state["aux"].reshape(B, cfg.num_aux * H)     # [early || middle || late]
        g = linear(aux, W["fc"])
    else:
        g = f64(hidden_in)
    assert g.shape == (B, H)

    # E2-E4: embedding of the (target-vocabulary) token, two separate
    # RMSNorms, concatenated to 2H [MAX-walkthrough section 4; ModelOpt
    # attention in-dim section].
    e = f64(W["embed"][tok])
    x = torch.cat([rms_norm(e, W["norm_in"], cfg.rms_eps),
                   rms_norm(g, W["norm_hid"], cfg.rms_eps)], dim=-1)
    assert x.shape == (B, 2 * H)

    if cfg.attn_kind == MHA:
        attn = _mha_attention(cfg, W, state, x, pos, table)
    else:
        attn = _mla_attention(cfg, W, state, x, pos, table)

    # E9: o_proj back to H, residual on the fused hidden [MAX-walkthrough
    # section 4: o_proj outputs H; residual -> post-attention norm -> MLP ->
    # residual].
    h1 = g + linear(attn, W["w_o"])
    # E10: dense gated-SiLU MLP with residual.
    u = rms_norm(h1, W["norm_post"], cfg.rms_eps)
    h_out = h1 + linear(silu(linear(u, W["w_gate"])) * linear(u, W["w_up"]), W["w_down"])
    # E11: final norm and the head's own lm_head over the draft vocabulary.
    logits = linear(rms_norm(h_out, W["norm_final"], cfg.rms_eps), W["lm_head"])
    assert logits.shape == (B, cfg.draft_vocab)
    # E12-E13: greedy top-1, lowest index among exact ties, mapped to the
    # target vocabulary by adding its d2t offset [ModelOpt lm_head section].
    draft_id = torch.argmax(logits, dim=-1)
    top2 = torch.topk(logits, k=min(2, logits.shape[-1]), dim=-1).values
    margin = top2[:, 0] - top2[:, -1] if top2.shape[-1] > 1 else torch.full((B,), math.inf)
    # A head without d2t scores through its target's lm_head over the target
    # vocabulary, so its ids already are target ids [MAX-API has_own_lm_head].
    d2t = W.get("d2t")
    token_out = draft_id + d2t.long()[draft_id] if d2t is not None else draft_id.clone()
    return {"hidden_out": h_out, "logits": logits, "draft_id": draft_id,
            "token_out": token_out, "margin": margin}


def _mha_attention(cfg, W, state, x, pos, table):
    """Llama-style attention of the new token over its one-layer cache
    [MAX-walkthrough section 11; MAX-API: the MHA head's cache is bf16].

    Cache: K and V in the plain paged layout [pages, page_size, n_kv_heads,
    head_dim]; position j of row b is slot j % page_size of page
    table[b, j // page_size].
    """
    B = x.shape[0]
    nq, nkv, hd = cfg.n_heads, cfg.n_kv_heads, cfg.head_dim
    q = linear(x, W["w_q"]).view(B, nq, hd)
    k = linear(x, W["w_k"]).view(B, nkv, hd)
    v = linear(x, W["w_v"]).view(B, nkv, hd)
    inv = rope_inv_freq(hd, cfg.rope_theta)
    q = rope_rotate_half(q, pos, inv)
    k = rope_rotate_half(k, pos, inv)
    kc, vc = state["k_cache"], state["v_cache"]
    P = cfg.page_size
    out = torch.empty(B, nq, hd, dtype=F64)
    group = nq // nkv
    for b in range(B):
        p = int(pos[b])
        page, slot = int(table[b, p // P]), p % P
        kc[page, slot] = k[b].to(torch.float32).to(torch.bfloat16)         # E7: append first
        vc[page, slot] = v[b].to(torch.float32).to(torch.bfloat16)
        pg, sl = cache_positions(table[b], p + 1, P)                        # keys 0..p
        K = f64(kc[pg, sl])                                                 # [p + 1, nkv, hd]
        V = f64(vc[pg, sl])
        for h in range(nq):
            kvh = h // group
            s = (K[:, kvh, :] @ q[b, h]) / math.sqrt(hd)
            out[b, h] = softmax_attend(s, V[:, kvh, :])
    return out.reshape(B, nq * hd)


def _mla_attention(cfg, W, state, x, pos, table):
    """DeepseekV3 multi-head latent attention of the new token, written in the
    plain (decompressed) form: every cached latent is expanded through kv_b
    into per-head keys and values [MAX-walkthrough section 4: one DeepseekV3
    decoder layer; MAX-API ranks q_lora 1536, kv_lora 512, rope 64, nope 128,
    v 128, interleaved rope].

    Cache: entries of kv_lora_rank + qk_rope_dim values (the normalised
    latent c, then the rotated k_pe) in the plain paged layout [pages,
    page_size, r + dr].
    """
    B = x.shape[0]
    nh, dn, dr, dv, r = cfg.n_heads, cfg.qk_nope_dim, cfg.qk_rope_dim, cfg.v_head_dim, cfg.kv_lora_rank
    q_a = rms_norm(linear(x, W["w_qa"]), W["norm_qa"], cfg.rms_eps)
    q = linear(q_a, W["w_qb"]).view(B, nh, dn + dr)
    q_nope, q_pe = q[..., :dn], q[..., dn:]
    kv = linear(x, W["w_kva"])
    c = rms_norm(kv[:, :r], W["norm_kv"], cfg.rms_eps)
    k_pe = kv[:, r:].reshape(B, 1, dr)
    inv = yarn_inv_freq(dr, cfg.rope_theta, cfg.yarn_factor, cfg.yarn_orig_max_pos,
                        cfg.yarn_beta_fast, cfg.yarn_beta_slow)
    q_pe = rope_interleaved(q_pe, pos, inv)
    k_pe = rope_interleaved(k_pe, pos, inv).reshape(B, dr)
    tau = yarn_mscale(cfg.yarn_factor) ** 2 / math.sqrt(dn + dr)
    wkvb = dense(W["w_kvb"]).view(nh, dn + dv, r)
    w_uk, w_uv = wkvb[:, :dn, :], wkvb[:, dn:, :]          # per head [nope | v] rows
    cache = state["kv_cache"]
    P = cfg.page_size
    out = torch.empty(B, nh, dv, dtype=F64)
    for b in range(B):
        p = int(pos[b])
        page, slot = int(table[b, p // P]), p % P
        cache[page, slot] = torch.cat([c[b], k_pe[b]]).to(torch.float32).to(torch.bfloat16)
        pg, sl = cache_positions(table[b], p + 1, P)
        ent = f64(cache[pg, sl])                                # [p + 1, r + dr]
        out[b] = mla_attend_plain(q_nope[b], q_pe[b], ent[:, :r], ent[:, r:], w_uk, w_uv, tau)
    return out.reshape(B, nh * dv)


def mla_attend_plain(q_nope, q_pe, c, k_pe, w_uk, w_uv, tau):
    """Attention of one query over n cached latents, decompressed per head.

    q_nope [nh, dn], q_pe [nh, dr], c [n, r], k_pe [n, dr], w_uk [nh, dn, r],
    w_uv [nh, dv, r].  Key of head h at j: [w_uk[h] c_j || k_pe_j]; value:
    w_uv[h] c_j; score: tau * (q_h . key).  Returns [nh, dv].
    """
    K_nope = torch.einsum("hdc,nc->hnd", w_uk, c)    # [nh, n, dn]
    V = torch.einsum("hvc,nc->hnv", w_uv, c)         # [nh, n, dv]
    out = torch.empty(w_uv.shape[0], w_uv.shape[1], dtype=F64)
    for h in range(w_uk.shape[0]):
        s = (K_nope[h] @ q_nope[h] + k_pe @ q_pe[h]) * tau
        out[h] = softmax_attend(s, V[h])
    return out


# ---------------------------------------------------------------- chain

def draft_chain(cfg, W, state, gamma: int):
    """gamma autoregressive steps; step k+1 takes step k's hidden_out and
    token_out [ModelOpt TTT section: each drafted step consumes the head's
    own previous hidden state; MAX-walkthrough section 9: steps run in decode
    mode, one token per row].  Appends gamma cache entries per row.
    """
    h, t = None, None
    steps = []
    for k in range(gamma):
        r = draft_step(cfg, W, state, k, hidden_in=h, token_in=t)
        steps.append(r)
        h, t = r["hidden_out"], r["token_out"]
    tokens = torch.stack([s["token_out"] for s in steps], dim=1)
    return {"tokens": tokens, "steps": steps}


def draft_extend(cfg, W, state, cu_seqlens: torch.Tensor, aux: torch.Tensor, token_in: torch.Tensor):
    """Multi-token extend over the positions the verifier accepted
    [MAX-walkthrough section 4: the draft forward in prefill mode over
    variable-length inputs; section 9: the proposer's prefill phase asks the
    draft for the hidden state and logits of every accepted position].

    New token i belongs to sequence b with cu_seqlens[b] <= i < cu_seqlens[b+1]
    and sits at position ctx_len[b] + j, j = i - cu_seqlens[b].  By definition
    it is the draft step at that position with g = fc(aux[i]) and token
    token_in[i]; the positions of a sequence are taken in order, each
    appending its entry before it attends, so position p sees positions 0..p
    of its own sequence (causal among the new tokens).  aux is [T, num_aux, H];
    state's cache is updated in place.  Returns per-position hidden_out [T, H],
    logits [T, Vd], draft_id, token_out and margin [T].
    """
    cu = [int(v) for v in cu_seqlens.tolist()]
    B = len(cu) - 1
    T = int(token_in.shape[0])
    assert cu[0] == 0 and cu[-1] == T and all(cu[b] <= cu[b + 1] for b in range(B))
    out = {"hidden_out": torch.zeros(T, cfg.hidden, dtype=F64),
           "logits": torch.zeros(T, cfg.draft_vocab, dtype=F64),
           "draft_id": torch.zeros(T, dtype=torch.long), "token_out": torch.zeros(T, dtype=torch.long),
           "margin": torch.zeros(T, dtype=F64)}
    q_max = max(cu[b + 1] - cu[b] for b in range(B))
    for j in range(q_max):
        rows = [b for b in range(B) if cu[b] + j < cu[b + 1]]
        idx = [cu[b] + j for b in rows]
        sub = {k: v for k, v in state.items() if k not in ("aux", "token_in", "ctx_len", "block_table")}
        sub["aux"] = aux[idx]
        sub["token_in"] = token_in[idx]
        sub["ctx_len"] = state["ctx_len"][rows]
        sub["block_table"] = state["block_table"][rows]
        r = draft_step(cfg, W, sub, j)
        for k in out:
            out[k][idx] = r[k]
    return out


# ---------------------------------------------------------------- verify

def greedy_accept(draft: torch.Tensor, target: torch.Tensor):
    """Greedy chain verification [MAX-walkthrough section 10: greedy argmax
    acceptance; ModelOpt validation section: draft, verify, accept].

    draft [B, gamma] target ids; target [B, gamma+1] the target's argmax ids.
    accept_len[b] = number of leading j with draft[b, j] == target[b, j];
    bonus[b] = target[b, accept_len[b]].
    """
    B, g = draft.shape
    assert target.shape == (B, g + 1)
    acc = torch.zeros(B, dtype=torch.int64)
    bonus = torch.zeros(B, dtype=torch.int64)
    for b in range(B):
        a = 0
        while a < g and int(draft[b, a]) == int(target[b, a]):
            a += 1
        acc[b] = a
        bonus[b] = int(target[b, a])
    return acc, bonus


def target_order(z: torch.Tensor) -> torch.Tensor:
    """Token ids of one target distribution from most to least likely, equal
    logits ordered by lowest id first (the same tie rule as the top-1)."""
    # ids are already ascending, so a stable sort on -z orders ties by id
    return torch.argsort(-f64(z), stable=True)


def relaxed_accept(draft: torch.Tensor, logits: torch.Tensor, relaxed: Optional[torch.Tensor],
                   topk: int, delta: float):
    """Chain verification with relaxed acceptance inside thinking spans
    [MAX-walkthrough section 10: use_relaxed_acceptance_for_thinking with
    relaxed_topk and relaxed_delta; the draft proposal is its argmax].

    draft [B, gamma] target ids; logits [B, gamma+1, V] the target's fp32
    logits at the verified positions; relaxed [B] bool (None: every row).

    A row outside a thinking span uses the greedy rule: draft[b, j] must be
    the target's top-1 at position j.  A row inside one accepts draft[b, j]
    when it is among the target's `topk` most likely tokens AND its
    log-probability is at least the top-1's minus `delta` (the reading of
    relaxed_delta: a log-probability margin below the best candidate).
    accept_len[b] counts the leading accepted positions; bonus[b] is the
    target's top-1 at position accept_len[b].

    The log-probability gap needs no normaliser: log_softmax(z)[t] -
    log_softmax(z)[u] = z[t] - z[u] exactly.  The gap of two fp32 logits is
    formed in fp64, where it is exact, and compared with -delta (delta as
    the fp32 value the caller passes), so the decision is not left to
    rounding.
    """
    B, g = draft.shape
    assert logits.shape[:2] == (B, g + 1)
    d32 = float(torch.tensor(delta, dtype=torch.float32))
    acc = torch.zeros(B, dtype=torch.int64)
    bonus = torch.zeros(B, dtype=torch.int64)
    for b in range(B):
        rel = True if relaxed is None else bool(relaxed[b])
        a = 0
        while a < g:
            z = logits[b, a]
            order = target_order(z)
            t = int(draft[b, a])
            if not rel:
                ok = t == int(order[0])
            else:
                cands = order[:topk].tolist()
                ok = t in cands and float(f64(z[t]) - f64(z[order[0]])) >= -d32
            if not ok:
                break
            a += 1
        acc[b] = a
        bonus[b] = int(target_order(logits[b, a])[0])
    return acc, bonus
