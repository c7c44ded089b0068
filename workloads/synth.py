"""Seeded synthetic tensors for the EAGLE-3 draft-head workloads.

This module draws numbers; it computes nothing of the draft head.  The
CPU oracle and the HIP path both take their inputs from here, as torch
CPU tensors (the caller moves them to the GPU).

Recipe (all seeds derive from a config's name and a tensor's name, so a
tensor does not change when another one is added):

* weight matrices: N(0, weight_std) drawn in fp32, rounded to bf16 (RNE);
  a quantized head's matrices are codes and scales drawn directly (see
  quant_codes);
* RMSNorm gains: 1 + N(0, gain_std) in bf16 (exactly 1 when gain_std = 0);
* aux hidden states [B, 3, H]: N(0, 1) times the per-layer scale, bf16;
* cache entries: N(0, 1) bf16 over every slot of every page in the pool,
  in the plain paged layout (MHA: K and V [pages, page, kv_heads, head_dim];
  MLA: [pages, page, latent + rope]); ``workloads.layout.to_tiled`` gives
  the library's tiled layout;
* token ids: uniform over the target vocabulary;
* context lengths: fixed or uniform integers in [lo, hi];
* page tables: per-row contiguous page ranges ("identity") or a random
  permutation of a pool holding exactly the pages the rows need
  ("shuffled"); unused table entries hold page 0;
* d2t: zeros when the draft vocabulary is the target vocabulary, else the
  offsets of a sorted random injective map draft id -> target id; a head that
  scores through its target's lm_head has none;
* greedy-verification targets: per row k ~ Geometric(p) - 1 capped at
  gamma; the first k target ids copy the drafts, the remaining drafted
  positions get a different id, the bonus position a uniform id.
* relaxed-verification logits [B, gamma+1, V] fp32: every token U(-4, 4)
  except 12 distinct "planted" ids per position with logits 8 - s * (r // 2)
  for r = 0..11 (pairs of equal logits, so ties decide ranks), the step s
  drawn per position from {0.05, 0.125, 0.2, 0.3}; each draft is a planted id
  with r = min(Geometric(0.3) - 1, 11) (probability 0.85) or a uniform id;
  relaxed flags Bernoulli(0.5).
"""
from __future__ import annotations

import hashlib
import os
from concurrent.futures import ThreadPoolExecutor
from typing import Dict, Optional

import numpy as np
import torch

from .configs import MHA, MLA, Eagle3Config

_CHUNK = 1 << 24  # elements per independently seeded chunk


def _seed(*parts) -> int:
    h = hashlib.sha256("/".join(str(p) for p in parts).encode()).digest()
    return int.from_bytes(h[:8], "little") & ((1 << 63) - 1)


def _workers() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def normal_bf16(shape, std: float, seed: int, mean: float = 0.0) -> torch.Tensor:
    """N(mean, std) rounded to bf16, drawn in independently seeded chunks."""
    n = int(np.prod(shape)) if len(shape) else 1
    out = torch.empty(n, dtype=torch.bfloat16)
    nchunks = max(1, (n + _CHUNK - 1) // _CHUNK)

    def fill(i):
        lo = i * _CHUNK
        hi = min(n, lo + _CHUNK)
        g = torch.Generator().manual_seed(_seed(seed, i))
        x = torch.randn(hi - lo, generator=g, dtype=torch.float32)
        if std != 1.0:
            x.mul_(std)
        if mean != 0.0:
            x.add_(mean)
        out[lo:hi] = x.to(torch.bfloat16)

    if nchunks == 1:
        fill(0)
    else:
        with ThreadPoolExecutor(_workers()) as ex:
            list(ex.map(fill, range(nchunks)))
    return out.view(*shape)


def quant_codes(fmt: str, rows: int, cols: int, std: float, seed: int) -> Dict[str, torch.Tensor]:
    """Codes and scales of a quantized [rows, cols] weight, drawn directly
    (nothing is rounded from a float weight):

    * fp8: sign uniform, exponent field 15 - G with G ~ Geometric(1/2) - 1
      (clipped at 0, so subnormals and zeros appear in large matrices),
      mantissa uniform (the NaN code is moved to the largest finite one);
    * nvfp4: uniform bytes (two E2M1 elements, low nibble first) and
      positive E4M3 block scales per 16 elements with exponent field
      uniform in 5..9 and mantissa uniform;
    * a row scale per output row, std / (typical code magnitude) times
      U(0.75, 1.25), in fp32.
    """
    out = {}
    if fmt == "fp8":
        codes = np.empty((rows, cols), dtype=np.uint8)
        typical = 250.0
    else:
        codes = np.empty((rows, cols // 2), dtype=np.uint8)
        blocks = np.empty((rows, cols // 16), dtype=np.uint8)
        typical = 2.93 * 3.2
    step = max(1, _CHUNK // max(1, cols))

    def fill(i):
        r0, r1 = i * step, min(rows, (i + 1) * step)
        rng = np.random.default_rng(_seed(seed, "q", i))
        n = r1 - r0
        if fmt == "fp8":
            u = rng.integers(0, 2 ** 32, size=(n, cols), dtype=np.uint32)
            sign = (u & 1).astype(np.uint8)
            man = ((u >> 1) & 7).astype(np.uint8)
            frac = ((u >> 8).astype(np.float64) + 0.5) / float(1 << 24)   # uniform (0, 1)
            g = np.minimum(np.floor(-np.log2(frac)), 15).astype(np.int64)
            exp = (15 - g).astype(np.uint8)
            man = np.where((exp == 15) & (man == 7), 6, man).astype(np.uint8)
            codes[r0:r1] = (sign << 7) | (exp << 3) | man
        else:
            codes[r0:r1] = rng.integers(0, 256, size=(n, cols // 2), dtype=np.uint8)
            e = rng.integers(5, 10, size=(n, cols // 16)).astype(np.uint8)
            m = rng.integers(0, 8, size=(n, cols // 16)).astype(np.uint8)
            blocks[r0:r1] = (e << 3) | m

    nchunks = (rows + step - 1) // step
    if nchunks == 1:
        fill(0)
    else:
        with ThreadPoolExecutor(_workers()) as ex:
            list(ex.map(fill, range(nchunks)))
    rng = np.random.default_rng(_seed(seed, "row_scale"))
    out["codes"] = torch.from_numpy(codes)
    out["row_scale"] = torch.from_numpy((std / typical * rng.uniform(0.75, 1.25, size=rows)).astype(np.float32))
    if fmt != "fp8":
        out["block_scale"] = torch.from_numpy(blocks)
    return out


def _family(cfg: Eagle3Config) -> str:
    return cfg.weight_family or cfg.name


def make_weights(cfg: Eagle3Config) -> Dict[str, torch.Tensor]:
    """Row-major ([out, in]) bf16 weights of one draft head, plus d2t (int32).
    A quantized head (weight_format fp8 / nvfp4) holds uint8 codes for every
    GEMM matrix with its scales under "<name>.row_scale" / "<name>.block_scale";
    the embedding stays bf16."""
    fam = _family(cfg)
    H, I = cfg.hidden, cfg.intermediate
    std = cfg.weight_std

    qfmt = cfg.weight_format
    W: Dict[str, torch.Tensor] = {}

    def mat(name, rows, cols):
        if qfmt == "bf16" or name == "embed":
            return normal_bf16((rows, cols), std, _seed(fam, name))
        q = quant_codes(qfmt, rows, cols, std, _seed(fam, name, qfmt))
        W[name + ".row_scale"] = q["row_scale"]
        if "block_scale" in q:
            W[name + ".block_scale"] = q["block_scale"]
        return q["codes"]

    def gain(name, n):
        if cfg.gain_std == 0.0:
            return torch.ones(n, dtype=torch.bfloat16)
        return normal_bf16((n,), cfg.gain_std, _seed(fam, name), mean=1.0)

    W["embed"] = mat("embed", cfg.target_vocab, H)
    W["fc"] = mat("fc", H, cfg.num_aux * H)
    W["norm_in"] = gain("norm_in", H)
    W["norm_hid"] = gain("norm_hid", H)
    W["norm_post"] = gain("norm_post", H)
    W["norm_final"] = gain("norm_final", H)
    if cfg.attn_kind == MHA:
        nq, nkv, hd = cfg.n_heads, cfg.n_kv_heads, cfg.head_dim
        W["w_q"] = mat("w_q", nq * hd, 2 * H)
        W["w_k"] = mat("w_k", nkv * hd, 2 * H)
        W["w_v"] = mat("w_v", nkv * hd, 2 * H)
        W["w_o"] = mat("w_o", H, nq * hd)
    else:
        nh = cfg.n_heads
        W["w_qa"] = mat("w_qa", cfg.q_lora_rank, 2 * H)
        W["norm_qa"] = gain("norm_qa", cfg.q_lora_rank)
        W["w_qb"] = mat("w_qb", nh * cfg.qk_head_dim, cfg.q_lora_rank)
        W["w_kva"] = mat("w_kva", cfg.kv_lora_rank + cfg.qk_rope_dim, 2 * H)
        W["norm_kv"] = gain("norm_kv", cfg.kv_lora_rank)
        W["w_kvb"] = mat("w_kvb", nh * (cfg.qk_nope_dim + cfg.v_head_dim), cfg.kv_lora_rank)
        W["w_o"] = mat("w_o", H, nh * cfg.v_head_dim)
    W["w_gate"] = mat("w_gate", I, H)
    W["w_up"] = mat("w_up", I, H)
    W["w_down"] = mat("w_down", H, I)
    W["lm_head"] = mat("lm_head", cfg.draft_vocab, H)
    if cfg.d2t_kind != "none":
        W["d2t"] = make_d2t(cfg)
    return W


def make_d2t(cfg: Eagle3Config) -> torch.Tensor:
    """d2t offsets; a head with d2t_kind "none" has no map (identity)."""
    if cfg.d2t_kind in ("zero", "none"):
        if cfg.draft_vocab > cfg.target_vocab:
            raise ValueError("draft vocabulary larger than target vocabulary")
        return torch.zeros(cfg.draft_vocab, dtype=torch.int32)
    rng = np.random.default_rng(_seed(_family(cfg), "d2t"))
    m = np.sort(rng.choice(cfg.target_vocab, size=cfg.draft_vocab, replace=False))
    return torch.from_numpy((m - np.arange(cfg.draft_vocab)).astype(np.int32))


def make_inputs(cfg: Eagle3Config, seed: int = 0) -> Dict[str, torch.Tensor]:
    """Per-batch inputs: aux states, tokens, context lengths, page table, cache."""
    tag = (cfg.name, "inputs", seed)
    B, H = cfg.batch, cfg.hidden
    rng = np.random.default_rng(_seed(*tag, "ints"))
    lo, hi = cfg.ctx
    if lo == hi:
        ctx = np.full(B, lo, dtype=np.int64)
    else:
        ctx = rng.integers(lo, hi + 1, size=B)
    pages = [cfg.pages_for(int(c)) for c in ctx]
    max_pages = cfg.pages_for(hi)
    table = np.zeros((B, max_pages), dtype=np.int32)
    if cfg.paging == "identity":
        for b in range(B):
            table[b, : pages[b]] = b * max_pages + np.arange(pages[b])
        num_pages = B * max_pages
    else:
        num_pages = int(sum(pages))
        perm = rng.permutation(num_pages).astype(np.int32)
        off = 0
        for b in range(B):
            table[b, : pages[b]] = perm[off: off + pages[b]]
            off += pages[b]
    tokens = rng.integers(0, cfg.target_vocab, size=B).astype(np.int32)

    aux = normal_bf16((B, cfg.num_aux, H), 1.0, _seed(*tag, "aux")).float()
    scales = torch.tensor(cfg.aux_scales[: cfg.num_aux], dtype=torch.float32).view(1, -1, 1)
    aux = (aux * scales).to(torch.bfloat16)  # power-of-two scales: exact in bf16

    out = {
        "aux": aux,
        "token_in": torch.from_numpy(tokens),
        "ctx_len": torch.from_numpy(ctx.astype(np.int32)),
        "block_table": torch.from_numpy(table),
    }
    if cfg.attn_kind == MHA:
        shape = (num_pages, cfg.page_size, cfg.n_kv_heads, cfg.head_dim)
        out["k_cache"] = normal_bf16(shape, 1.0, _seed(*tag, "k_cache"))
        out["v_cache"] = normal_bf16(shape, 1.0, _seed(*tag, "v_cache"))
    else:
        shape = (num_pages, cfg.page_size, cfg.kv_entry_dim)
        out["kv_cache"] = normal_bf16(shape, 1.0, _seed(*tag, "kv_cache"))
    return out


def make_accept_targets(cfg: Eagle3Config, draft: torch.Tensor, seed: int = 0):
    """Target argmax ids [B, gamma+1] whose matching prefix length is known.

    Returns (target_ids int32 [B, gamma+1], k int32 [B]) with k the number
    of leading drafts the targets copy.  k = Geometric(p) - 1 (failures
    before the first success), capped at gamma.
    """
    B, g = draft.shape
    V = cfg.target_vocab
    rng = np.random.default_rng(_seed(cfg.name, "accept", seed))
    k = np.minimum(rng.geometric(cfg.accept_p, size=B) - 1, g).astype(np.int64)
    d = draft.numpy().astype(np.int64)
    tgt = np.empty((B, g + 1), dtype=np.int64)
    shift = rng.integers(0, V - 1, size=(B, g))
    for b in range(B):
        kb = int(k[b])
        tgt[b, :kb] = d[b, :kb]
        tgt[b, kb:g] = (d[b, kb:g] + 1 + shift[b, kb:g]) % V
    tgt[:, g] = rng.integers(0, V, size=B)
    return torch.from_numpy(tgt.astype(np.int32)), torch.from_numpy(k.astype(np.int32))


def make_extend_inputs(cfg: Eagle3Config, q_lens, seed: int = 0) -> Dict[str, torch.Tensor]:
    """Inputs of a multi-token extend: q_lens[b] new positions per sequence
    (0 allowed).  cu_seqlens [B+1] int32, aux [T, num_aux, H] bf16 (N(0,1)
    times the per-layer scales), token_in [T] uniform target ids."""
    q = np.asarray(q_lens, dtype=np.int64)
    cu = np.concatenate([[0], np.cumsum(q)]).astype(np.int32)
    T = int(cu[-1])
    tag = (cfg.name, "extend", seed)
    rng = np.random.default_rng(_seed(*tag, "ints"))
    tokens = rng.integers(0, cfg.target_vocab, size=T).astype(np.int32)
    aux = normal_bf16((T, cfg.num_aux, cfg.hidden), 1.0, _seed(*tag, "aux")).float()
    scales = torch.tensor(cfg.aux_scales[: cfg.num_aux], dtype=torch.float32).view(1, -1, 1)
    return {"cu_seqlens": torch.from_numpy(cu), "aux": (aux * scales).to(torch.bfloat16),
            "token_in": torch.from_numpy(tokens)}


def random_drafts(cfg: Eagle3Config, seed: int = 0) -> torch.Tensor:
    """Uniform draft ids [B, gamma] over the target vocabulary."""
    rng = np.random.default_rng(_seed(cfg.name, "drafts", seed))
    return torch.from_numpy(
        rng.integers(0, cfg.target_vocab, size=(cfg.batch, cfg.gamma)).astype(np.int32))


def make_relaxed_inputs(cfg: Eagle3Config, seed: int = 0, batch: Optional[int] = None,
                        vocab: Optional[int] = None) -> Dict[str, torch.Tensor]:
    """Target logits with a planted head, drafts and thinking-span flags for
    relaxed verification: logits fp32 [B, gamma+1, V], draft int32 [B, gamma],
    relaxed uint8 [B], planted int64 [B, gamma+1, 12] (the planted ids by r)."""
    B = cfg.batch if batch is None else batch
    V = cfg.target_vocab if vocab is None else vocab
    g, n_hot = cfg.gamma, 12
    rng = np.random.default_rng(_seed(cfg.name, "relaxed", seed, B, V))
    z = rng.uniform(-4.0, 4.0, size=(B, g + 1, V)).astype(np.float32)
    steps = np.array([0.05, 0.125, 0.2, 0.3], dtype=np.float64)
    s = steps[rng.integers(0, len(steps), size=(B, g + 1))]
    planted = np.empty((B, g + 1, n_hot), dtype=np.int64)
    r = np.arange(n_hot)
    for b in range(B):
        for j in range(g + 1):
            ids = rng.choice(V, size=min(n_hot, V), replace=False)
            planted[b, j, :len(ids)] = ids
            z[b, j, ids] = (8.0 - s[b, j] * (r[:len(ids)] // 2)).astype(np.float32)
    pick = np.minimum(rng.geometric(0.3, size=(B, g)) - 1, n_hot - 1)
    use_planted = rng.random(size=(B, g)) < 0.85
    uniform = rng.integers(0, V, size=(B, g))
    draft = np.where(use_planted, np.take_along_axis(planted[:, :g], pick[..., None], 2)[..., 0], uniform)
    relaxed = (rng.random(size=B) < 0.5).astype(np.uint8)
    return {"logits": torch.from_numpy(z), "draft": torch.from_numpy(draft.astype(np.int32)),
            "relaxed": torch.from_numpy(relaxed), "planted": torch.from_numpy(planted)}
