"""Helpers of the GPU parity tests: run the HIP path through the C ABI and
compare it with the CPU oracle under the stated tolerances."""
from __future__ import annotations

import numpy as np
import torch

from eagle_draft_head_step_amd import binding

ATOL = 3e-2      # max-abs on fp32 hidden states and logits
RTOL_L2 = 1e-2   # relative L2 error
MARGIN = 1e-2    # ids must match where the oracle's top-1/top-2 margin exceeds this

DEV = torch.device("cuda:0")


def to_dev(d):
    return {k: v.to(DEV) for k, v in d.items()}


def clone(d):
    return {k: v.clone() for k, v in d.items()}


def cache_keys(cfg):
    return ("k_cache", "v_cache") if cfg.attn_kind == 0 else ("kv_cache",)


def kc_vc(cfg, d):
    if cfg.attn_kind == 0:
        return d["k_cache"], d["v_cache"]
    return d["kv_cache"], None


def gpu_step(head, cfg, d, ws, k, *, hidden_in=None, token_in=None, use_aux=True, logits=True):
    """One eagle3_draft_step on device state d (the cache is updated in place)."""
    B = cfg.batch
    hout = torch.empty(B, cfg.hidden, dtype=torch.float32, device=DEV)
    tok = torch.empty(B, dtype=torch.int32, device=DEV)
    did = torch.empty(B, dtype=torch.int32, device=DEV)
    lg = torch.empty(B, cfg.draft_vocab, dtype=torch.float32, device=DEV) if logits else None
    kc, vc = kc_vc(cfg, d)
    head.draft_step(step_index=k, aux=d["aux"].reshape(B, -1) if use_aux else None,
                    hidden_in=hidden_in, token_in=d["token_in"] if token_in is None else token_in,
                    k_cache=kc, v_cache=vc, block_table=d["block_table"], ctx_len=d["ctx_len"],
                    max_ctx=int(d["ctx_len"].max().item()), hidden_out=hout, token_out=tok,
                    draft_id_out=did, logits_out=lg, workspace=ws)
    return hout, tok, did, lg


def gpu_chain(head, cfg, d, ws, gamma, *, logits=True, max_ctx=None):
    B = cfg.batch
    hid = torch.empty(gamma, B, cfg.hidden, dtype=torch.float32, device=DEV)
    tok = torch.empty(B, gamma, dtype=torch.int32, device=DEV)
    did = torch.empty(B, gamma, dtype=torch.int32, device=DEV)
    lg = torch.empty(gamma, B, cfg.draft_vocab, dtype=torch.float32, device=DEV) if logits else None
    kc, vc = kc_vc(cfg, d)
    head.draft_chain(gamma=gamma, aux=d["aux"].reshape(B, -1), hidden_in=None, token_in=d["token_in"],
                     k_cache=kc, v_cache=vc, block_table=d["block_table"], ctx_len=d["ctx_len"],
                     max_ctx=cfg.max_ctx if max_ctx is None else max_ctx, hidden_out=hid,
                     token_out=tok, draft_id_out=did, logits_out=lg, workspace=ws)
    return hid, tok, did, lg


def assert_close(what, gpu, ref, atol=ATOL, rtol_l2=RTOL_L2):
    g = gpu.detach().cpu().double()
    r = ref.detach().cpu().double()
    assert g.shape == r.shape, (what, g.shape, r.shape)
    err = (g - r).abs().max().item()
    rel = ((g - r).norm() / r.norm().clamp_min(1e-30)).item()
    assert err <= atol and rel <= rtol_l2, f"{what}: max-abs {err:.3e} (<= {atol}), rel-L2 {rel:.3e} (<= {rtol_l2})"
    return err, rel


def assert_ids(what, gpu_ids, ref_ids, margin):
    g = gpu_ids.detach().cpu().long()
    r = ref_ids.detach().cpu().long()
    ok = margin.cpu() > MARGIN
    bad = (g != r) & ok
    assert not bool(bad.any()), f"{what}: {int(bad.sum())} id mismatches at margin > {MARGIN}: rows {bad.nonzero().flatten().tolist()[:8]}"
    return int(ok.sum())


def cache_segments(cfg):
    """Lengths of the independently scaled parts of one cache entry: the
    RMS-normalised latent and the raw rotated rope key (MLA), or K and V (MHA)."""
    if cfg.attn_kind == 0:
        n = cfg.n_kv_heads * cfg.head_dim
        return [n, n]
    return [cfg.kv_lora_rank, cfg.qk_rope_dim]


def assert_cache_entry(what, gpu_e: torch.Tensor, ref_e: torch.Tensor, segments=None):
    """A cache entry the step wrote, against the oracle's (both bf16).

    The GPU feeds its projections bf16-rounded activations (relative error
    uniform in +-2^-9, std 2^-9/sqrt(3) = 1.1e-3), so a projected element
    moves by about 1.1e-3 of the RMS of the projection it belongs to before
    its own rounding.  Each segment (latent / rope, or K / V) has its own
    scale: the rope key is not normalised and runs about twice the latent's
    RMS.  Bound: |gpu - ref| <= ulp(ref) + 1e-2 * rms(segment)  (one storage
    step plus ~9 sigma).
    """
    g, r = gpu_e.cpu().float(), ref_e.cpu().float()
    segments = segments or [r.numel()]
    assert sum(segments) == r.numel()
    scale = torch.cat([seg.pow(2).mean().sqrt().expand(seg.numel()) for seg in torch.split(r, segments)])
    ulp = torch.where(r == 0, torch.zeros_like(r), 2.0 ** (torch.floor(torch.log2(r.abs().clamp_min(1e-30))) - 7))
    bad = (g - r).abs() > ulp + 1e-2 * scale
    assert not bool(bad.any()), (f"{what}: {int(bad.sum())} cache elements off, max |d| "
                                 f"{(g - r).abs().max().item():.3e} (segment rms {scale.unique().tolist()})")


def cache_entry(cfg, cache: dict, table: torch.Tensor, b: int, pos: int):
    P = cfg.page_size
    page, slot = int(table[b, pos // P]), pos % P
    if cfg.attn_kind == 0:
        return torch.cat([cache["k_cache"][page, :, :, slot, :].flatten(),
                          cache["v_cache"][page, :, :, slot // 16, :, slot % 16, :].flatten()])
    return cache["kv_cache"][page, :, slot, :].flatten()
