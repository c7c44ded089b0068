"""Helpers of the GPU parity tests: run the HIP path through the C ABI and
compare it with the CPU oracle under the stated tolerances."""
from __future__ import annotations

import numpy as np
import torch

import workloads as W
from eagle_draft_head_step_amd import binding

ATOL = 3e-2      # max-abs on fp32 hidden states and logits
RTOL_L2 = 1e-2   # relative L2 error
MARGIN = 1e-2    # ids must match where the oracle's top-1/top-2 margin exceeds this

DEV = torch.device("cuda:0")


def to_dev(d):
    return {k: v.to(DEV) for k, v in d.items()}


def dev_state(cfg, st):
    """Per-batch inputs on the device, caches in the library's tiled layout."""
    return to_dev(W.to_tiled(cfg, st))


def gpu_caches(cfg, d):
    """The device caches of state d, back in the plain layout on the CPU."""
    return W.to_plain(cfg, {k: d[k] for k in W.cache_keys(cfg)})


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


CACHE_REL_L2 = 4e-3   # per segment, over every entry a step wrote


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


def assert_cache_entries(what, gpu_es, ref_es, segments=None):
    """Every entry a step wrote (lists of per-row entries): each within the
    per-element bound above, and, per segment over all of them, a relative
    L2 error <= CACHE_REL_L2.  The bf16 rounding of the activations alone
    gives about 2.0e-3 there (a N(0, 1.1e-3 rms) perturbation before the
    entry's own rounding); a systematic error of 0.5% of the segment's RMS,
    as a scale or an offset, gives 5.6e-3 or more and fails."""
    for i, (g, r) in enumerate(zip(gpu_es, ref_es)):
        assert_cache_entry(f"{what} entry {i}", g, r, segments)
    G = torch.stack([g.cpu().double() for g in gpu_es])
    R = torch.stack([r.cpu().double() for r in ref_es])
    segments = segments or [R.shape[1]]
    o = 0
    for n in segments:
        gs, rs = G[:, o:o + n], R[:, o:o + n]
        rel = ((gs - rs).norm() / rs.norm().clamp_min(1e-30)).item()
        assert rel <= CACHE_REL_L2, f"{what}: cache segment [{o}, {o + n}) rel-L2 {rel:.3e} > {CACHE_REL_L2}"
        o += n


def cache_entry(cfg, cache: dict, table: torch.Tensor, b: int, pos: int):
    """The entry of row b at position pos in plain-layout caches."""
    P = cfg.page_size
    page, slot = int(table[b, pos // P]), pos % P
    if cfg.attn_kind == 0:
        return torch.cat([cache["k_cache"][page, slot].flatten(), cache["v_cache"][page, slot].flatten()])
    return cache["kv_cache"][page, slot].flatten()
