"""Conversion between the plain paged cache and the library's tiled cache.

Pure index permutations: no value is computed, rounded or reordered within
an element.  The inputs (``workloads.synth``) and the CPU oracle use the
plain paged layout, position j of a sequence in slot j % page_size of page
block_table[j // page_size]:

* MHA: K and V [pages, page_size, n_kv_heads, head_dim];
* MLA: entries [pages, page_size, kv_lora_rank + qk_rope_dim] (the
  normalised latent, then the rotated rope key).

The HIP library reads and appends the tiled layouts its header declares:

* MHA K [pages, n_kv, head_dim / c, page_size, c] with c = min(32, head_dim):
  dimension d of slot s at [d // c, s, d % c];
* MHA V [pages, n_kv, head_dim / c, page_size / 16, c / 2, 16, 2]: dimension
  d of slot s at [d // c, s // 16, (d // 2) % (c / 2), s % 16, d % 2];
* MLA [pages, entry / 16, page_size, 16]: value e of slot s at
  [e // 16, s, e % 16].

A caller that keeps its cache in the plain layout converts it once with
``to_tiled`` and reads entries back with ``to_plain``.
"""
from __future__ import annotations

from typing import Dict

import torch

from .configs import MHA

_CACHE_KEYS = ("k_cache", "v_cache", "kv_cache")


def _mha_chunk(head_dim: int) -> int:
    return min(32, head_dim)


def k_to_tiled(k: torch.Tensor) -> torch.Tensor:
    pages, P, nkv, hd = k.shape
    c = _mha_chunk(hd)
    return k.reshape(pages, P, nkv, hd // c, c).permute(0, 2, 3, 1, 4).contiguous()


def k_to_plain(k: torch.Tensor) -> torch.Tensor:
    pages, nkv, hc, P, c = k.shape
    return k.permute(0, 3, 1, 2, 4).reshape(pages, P, nkv, hc * c).contiguous()


def v_to_tiled(v: torch.Tensor) -> torch.Tensor:
    pages, P, nkv, hd = v.shape
    c = _mha_chunk(hd)
    # slot s = 16 s1 + s0, dimension d = c d2 + 2 d1 + d0
    t = v.reshape(pages, P // 16, 16, nkv, hd // c, c // 2, 2)
    #   axes:    0      1 (s1) 2 (s0) 3 (n) 4 (d2) 5 (d1) 6 (d0)
    return t.permute(0, 3, 4, 1, 5, 2, 6).contiguous()


def v_to_plain(v: torch.Tensor) -> torch.Tensor:
    pages, nkv, hc, p16, c2, s16, two = v.shape
    #   axes: 0 page, 1 n, 2 d2, 3 s1, 4 d1, 5 s0, 6 d0
    return v.permute(0, 3, 5, 1, 2, 4, 6).reshape(pages, p16 * s16, nkv, hc * c2 * two).contiguous()


def latent_to_tiled(kv: torch.Tensor) -> torch.Tensor:
    pages, P, E = kv.shape
    return kv.reshape(pages, P, E // 16, 16).permute(0, 2, 1, 3).contiguous()


def latent_to_plain(kv: torch.Tensor) -> torch.Tensor:
    pages, e16, P, sixteen = kv.shape
    return kv.permute(0, 2, 1, 3).reshape(pages, P, e16 * sixteen).contiguous()


def to_tiled(cfg, state: Dict[str, torch.Tensor]) -> Dict[str, torch.Tensor]:
    """A copy of `state` whose cache tensors are in the library's layout
    (every other entry is passed through unchanged)."""
    out = dict(state)
    if cfg.attn_kind == MHA:
        out["k_cache"] = k_to_tiled(state["k_cache"])
        out["v_cache"] = v_to_tiled(state["v_cache"])
    else:
        out["kv_cache"] = latent_to_tiled(state["kv_cache"])
    return out


def to_plain(cfg, caches: Dict[str, torch.Tensor]) -> Dict[str, torch.Tensor]:
    """The cache tensors of `caches` (library layout, on any device) back in
    the plain layout, on the CPU; entries that are not caches are dropped."""
    if cfg.attn_kind == MHA:
        return {"k_cache": k_to_plain(caches["k_cache"].cpu()), "v_cache": v_to_plain(caches["v_cache"].cpu())}
    return {"kv_cache": latent_to_plain(caches["kv_cache"].cpu())}


def cache_keys(cfg):
    return ("k_cache", "v_cache") if cfg.attn_kind == MHA else ("kv_cache",)
