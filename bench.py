#!/usr/bin/env python3
"""Throughput of the EAGLE-3 draft-head hot path on one MI355X.

One timed step = one pass of the whole hot path over one batch: a chain of
gamma draft steps (fc fusion, embedding and norms, the decoder layer with its
paged-cache attention, the MLP, lm_head top-1 and d2t) followed by greedy
verification of the drafted chain.  The default workload is the largest
one: the DeepseekV3-shaped MLA head at batch 256, context 2048, gamma 7, with
greedy acceptance; the other workloads are timed after it and reported in the
same line under per_config.  --config picks another workload alone.  Inputs are seeded synthetic tensors, resident in HBM before
the timed region; the step sequence is captured once into a HIP graph and
replayed.

Prints one JSON line on stdout (progress goes to stderr).
"""
from __future__ import annotations

import argparse
import ctypes
import gc
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK = 8.0e12          # bytes/s, MI355X HBM3E
MFMA_BF16_PEAK = 2.5e15    # dense bf16 flop/s


def log(*a):
    print(*a, file=sys.stderr, flush=True)


# ------------------------------------------------------------------ byte/flop model
# weight bytes per element of each storage format (NVFP4: a 4-bit code plus an
# E4M3 scale per 16); quantized matrices add one fp32 scale per row
WEIGHT_BYTES = {"bf16": 2.0, "fp8": 1.0, "nvfp4": 0.5 + 1.0 / 16}


def role_format(cfg, role):
    """Storage of a GEMM role's weights: the head's format, except the MLA
    absorb halves of kv_b, which are widened to bf16 at packing."""
    return "bf16" if role in ("gemm.uk_absorb", "gemm.uv") else cfg.weight_format


def gemm_roles(cfg, B):
    """(role, N, K, batch, out_bytes_per_elem) of every GEMM of one step."""
    H, I = cfg.hidden, cfg.intermediate
    r = []
    if cfg.attn_kind == 0:
        r.append(("gemm.qkv", (cfg.n_heads + 2 * cfg.n_kv_heads) * cfg.head_dim, 2 * H, 1, 4))
    else:
        r.append(("gemm.qa_kva", cfg.q_lora_rank + cfg.kv_lora_rank + cfg.qk_rope_dim, 2 * H, 1, 4))
        r.append(("gemm.qb", cfg.n_heads * (cfg.qk_nope_dim + cfg.qk_rope_dim), cfg.q_lora_rank, 1, 4))
        r.append(("gemm.uk_absorb", cfg.kv_lora_rank, cfg.qk_nope_dim, cfg.n_heads, 2))
        r.append(("gemm.uv", cfg.v_head_dim, cfg.kv_lora_rank, cfg.n_heads, 2))
    r.append(("gemm.o", H, cfg.attn_out_dim, 1, 4))
    r.append(("gemm.gate_up", 2 * I, H, 1, 4))
    r.append(("gemm.down", H, I, 1, 4))
    r.append(("gemm.lm_head", cfg.draft_vocab, H, 1, 0))
    return r


def gemm_bytes_flops(B, N, K, batch, ob, fmt="bf16"):
    """Algorithmic bytes: weights once (in their storage format), activations
    in, results out."""
    wbytes = N * K * WEIGHT_BYTES[fmt] + (N * 4 if fmt != "bf16" else 0)
    byts = batch * (wbytes + B * K * 2 + B * N * ob) + (B * 8 if ob == 0 else 0)
    return byts, 2.0 * batch * B * N * K


def chain_model(cfg, ctx_lens, gamma):
    """Algorithmic HBM bytes and flops of one chain + verification."""
    B, H = len(ctx_lens), cfg.hidden
    fc_b, fc_f = gemm_bytes_flops(B, H, cfg.num_aux * H, 1, 4, cfg.weight_format)
    per_tok = (2 * cfg.n_kv_heads * cfg.head_dim * 2) if cfg.attn_kind == 0 else cfg.kv_entry_dim * 2
    total_b, total_f = fc_b, fc_f
    gemm_b, gemm_f = fc_b, fc_f
    for k in range(gamma):
        for role, N, K, bt, ob in gemm_roles(cfg, B):
            b_, f_ = gemm_bytes_flops(B, N, K, bt, ob, role_format(cfg, role))
            total_b += b_; total_f += f_; gemm_b += b_; gemm_f += f_
        keys = sum(int(c) + k + 1 for c in ctx_lens)
        total_b += keys * per_tok + B * per_tok              # cache read + the appended entry
        if cfg.attn_kind == 0:
            total_f += 4.0 * cfg.n_heads * cfg.head_dim * keys
        else:
            total_f += 2.0 * cfg.n_heads * (cfg.kv_entry_dim + cfg.kv_lora_rank) * keys
        total_b += B * H * 2 + B * H * 4                     # embedding rows, hidden out
    total_b += B * cfg.num_aux * H * 2 + B * (2 * gamma + 1) * 4 * 2   # aux in, accept ids
    return {"bytes": total_b, "flops": total_f, "gemm_bytes": gemm_b, "gemm_flops": gemm_f}


# ------------------------------------------------------------------ per-kernel timing
def kernel_times(run_once, steps, ms_per_run):
    """{launch name: [total ms, launches]} over `steps` eager runs, from HIP
    events the library's launch hook records on the launch stream around each
    launch (a GPU spin is queued first so the events bracket kernels, not
    host latency)."""
    import torch
    from eagle_draft_head_step_amd import binding
    kern, events = {}, []
    HOOK = ctypes.CFUNCTYPE(None, ctypes.c_char_p, ctypes.c_int32, ctypes.c_void_p, ctypes.c_void_p)

    def hook(name, phase, stream, user):
        e = torch.cuda.Event(enable_timing=True)
        e.record(torch.cuda.current_stream())
        events.append((name.decode(), phase, e))

    cb = HOOK(hook)
    binding.lib().eagle3_set_launch_hook.argtypes = [HOOK, ctypes.c_void_p]
    binding.lib().eagle3_set_launch_hook(cb, None)
    try:
        for _ in range(steps):
            torch.cuda._sleep(int(30e6))
            run_once()
        torch.cuda.synchronize()
    finally:
        binding.lib().eagle3_set_launch_hook(HOOK(), None)
    open_ = {}
    for name, phase, e in events:
        if phase == 0:
            open_[name] = e
        else:
            t = open_.pop(name).elapsed_time(e)
            k = kern.setdefault(name, [0.0, 0])
            k[0] += t
            k[1] += 1
    for name, (t, n) in sorted(kern.items(), key=lambda x: -x[1][0]):
        log(f"[kernels] {name:24s} launches {n:5d}  avg {1e3 * t / n:9.2f} us  share of runs "
            f"{100 * t / (ms_per_run * steps):5.1f}%")
    return kern


def copy_bandwidth(torch, dev):
    """Measured device-to-device copy bandwidth (reads + writes) in GB/s."""
    try:
        nbytes = 1 << 30
        src = torch.empty(nbytes // 4, dtype=torch.int32, device=dev)
        dst = torch.empty_like(src)
        dst.copy_(src)
        c0, c1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        c0.record()
        for _ in range(5):
            dst.copy_(src)
        c1.record()
        torch.cuda.synchronize()
        return 2 * 5 * nbytes / (c0.elapsed_time(c1) / 1e3) / 1e9
    except RuntimeError:
        return None


# ------------------------------------------------------------------ counters
def sources_hash(family="step"):
    from eagle_draft_head_step_amd.rocprof_summary import sources_hash as h
    return h(family)


def counter_traffic(workload, prefix, suffix, family="step"):
    """HBM bytes per dispatch of a kernel family (every instance whose name holds
    prefix and suffix), averaged over its dispatches like the algorithmic bytes,
    from the committed counter summary of this workload, scaled by the copy
    calibration recorded there; None when the summary is missing or the kernel
    sources changed since it was taken."""
    path = os.path.join(ROOT, "profiles", f"{workload}_hbm_counters.txt")
    if not os.path.exists(path):
        return None
    text = open(path).read()
    if f"sha256[:16] = {sources_hash(family)}" not in text:
        return None
    scale, sums, disp = {}, {}, {}
    cur_n = None
    for line in text.splitlines():
        if line.startswith("# scale "):              # "# scale FETCH_SIZE 2.0"
            _, _, cname, f = line.split()
            scale[cname] = float(f)
        elif line and not line.startswith((" ", "#", "kernel")):
            cur_n = int(line.split()[-4]) if prefix in line and suffix in line else None
        elif cur_n and ":" in line:                  # "    FETCH_SIZE: avg X ..."
            cname = line.split(":")[0].strip()
            sums[cname] = sums.get(cname, 0.0) + cur_n * float(line.split("avg")[1].split()[0])
            disp[cname] = disp.get(cname, 0) + cur_n
    if "FETCH_SIZE" not in sums or "WRITE_SIZE" not in sums or not scale:
        return None
    per = {c: sums[c] / disp[c] * scale.get(c, 1.0) for c in ("FETCH_SIZE", "WRITE_SIZE")}
    return round(1024 * (per["FETCH_SIZE"] + per["WRITE_SIZE"]))


def run_extend(args, cfg, Wt, st, head, d, dev):
    """One eagle3_draft_extend over the positions a verification accepted:
    q_len_b = min(k_b + 1, gamma), k_b ~ Geometric(p) - 1 (the accept recipe),
    timed like the chain (graph replays) and reported per new position."""
    import numpy as np
    import torch
    import workloads as W
    B, g = cfg.batch, cfg.gamma
    _, k = W.make_accept_targets(cfg, W.random_drafts(cfg))
    q = np.minimum(k.numpy() + 1, g).tolist()
    ex = W.make_extend_inputs(cfg, q)
    T, qmax = int(ex["token_in"].numel()), int(max(q))
    de = {kk: v.to(dev) for kk, v in ex.items()}
    aux = de["aux"].reshape(T, -1)
    ws = head.extend_workspace(T, B, cfg.max_ctx, qmax)
    hid = torch.empty(T, cfg.hidden, dtype=torch.float32, device=dev)
    tok = torch.empty(T, dtype=torch.int32, device=dev)
    kc = d["k_cache"] if cfg.attn_kind == 0 else d["kv_cache"]
    vc = d.get("v_cache")
    log(f"[bench] extend: {T} new positions over {B} rows (q_len 1..{qmax})")

    def once():
        head.draft_extend(cu_seqlens=de["cu_seqlens"], max_q_len=qmax, aux=aux, token_in=de["token_in"],
                          k_cache=kc, v_cache=vc, block_table=d["block_table"], ctx_len=d["ctx_len"],
                          max_ctx=cfg.max_ctx, hidden_out=hid, token_out=tok, workspace=ws)

    for _ in range(max(1, args.warmup)):
        once()
    torch.cuda.synchronize()
    graph = None
    if not args.no_graph:
        s_ = torch.cuda.Stream()
        s_.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(s_):
            once()
        torch.cuda.current_stream().wait_stream(s_)
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            once()
        graph.replay()
        torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record()
    for _ in range(args.steps):
        graph.replay() if graph is not None else once()
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / args.steps
    log(f"[bench] extend {ms:.3f} ms per call, {T / (ms / 1e3):.1f} positions/s")
    copy_gbps = copy_bandwidth(torch, dev)
    kern = {} if args.no_kernel_timing else kernel_times(once, args.steps, ms)

    # algorithmic bytes: every weight once, each sequence's cache once (its
    # prefix plus the new entries), aux / embedding rows in, hidden out
    per_tok = (2 * cfg.n_kv_heads * cfg.head_dim * 2) if cfg.attn_kind == 0 else cfg.kv_entry_dim * 2
    H = cfg.hidden
    byts, flops = gemm_bytes_flops(T, H, cfg.num_aux * H, 1, 4, cfg.weight_format)
    for role, N, K, bt, ob in gemm_roles(cfg, T):
        b_, f_ = gemm_bytes_flops(T, N, K, bt, ob, role_format(cfg, role))
        byts += b_
        flops += f_
    ctx = st["ctx_len"].tolist()
    byts += sum((int(c) + qq) * per_tok for c, qq in zip(ctx, q))
    keys = sum(sum(int(c) + j + 1 for j in range(qq)) for c, qq in zip(ctx, q))
    flops += (4.0 * cfg.n_heads * cfg.head_dim if cfg.attn_kind == 0
              else 2.0 * cfg.n_heads * (cfg.kv_entry_dim + cfg.kv_lora_rank)) * keys
    byts += T * (cfg.num_aux * H * 2 + H * 2 + H * 4)
    bw = byts / (ms / 1e3)
    roof = None
    dom = [r for r in ("gemm.fc", "gemm.qkv", "gemm.qa_kva", "gemm.qb", "gemm.uk_absorb", "gemm.uv", "gemm.o",
                       "gemm.lm_head") if r in kern]
    if dom:
        role_b = {role: gemm_bytes_flops(T, N, K, bt, ob, role_format(cfg, role))[0]
                  for role, N, K, bt, ob in gemm_roles(cfg, T)}
        role_b["gemm.fc"] = gemm_bytes_flops(T, H, cfg.num_aux * H, 1, 4, cfg.weight_format)[0]
        launches = sum(kern[r][1] for r in dom)
        tb = sum(role_b[r] * kern[r][1] for r in dom)
        dur = sum(kern[r][0] for r in dom) / 1e3
        kname = ("gemm_big_kernel" if cfg.weight_format == "bf16" and T > 64 else "gemm_kernel")
        roof = {"kernel": f"{kname}, bf16 activations ({', '.join(dom)})", "bound": "hbm",
                "achieved": round(tb / dur / 1e9, 1), "peak": HBM_PEAK / 1e9, "unit": "GB/s",
                "frac": round(tb / dur / HBM_PEAK, 4), "traffic": None,
                "algorithmic_bytes_per_launch": round(tb / launches), "avg_launch_us": round(1e6 * dur / launches, 2)}
    result = {
        "metric": "draft extend positions/s (accepted positions through the draft head, one call)",
        "value": round(T / (ms / 1e3), 1), "unit": "positions/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": cfg.name + "_extend", "global_batch": B, "new_positions": T, "max_q_len": qmax,
                   "ctx": list(cfg.ctx), "attention": "mha_gqa" if cfg.attn_kind == 0 else "mla",
                   "parallelism": "single GPU", "hip_graph": graph is not None},
        "whole_call": {"algorithmic_bytes": byts, "algorithmic_flops": flops, "hbm_GBps": round(bw / 1e9, 1),
                       "hbm_frac": round(bw / HBM_PEAK, 4), "mfma_frac": round(flops / (ms / 1e3) / MFMA_BF16_PEAK, 4)},
        "measured_copy_GBps": None if copy_gbps is None else round(copy_gbps, 1),
        "roofline": roof,
        "kernels_us_per_call": {n: round(1e3 * t / args.steps, 2) for n, (t, c) in kern.items()},
    }
    if not args.no_cpu_baseline:
        import oracle
        cu = ex["cu_seqlens"].tolist()
        n, b, dt = 0, 0, 0.0
        cache = {kk: v.clone() for kk, v in st.items() if kk not in ("aux", "token_in", "ctx_len", "block_table")}
        while dt < 10.0:
            sub = dict(cache)
            sub["ctx_len"] = st["ctx_len"][[b]]
            sub["block_table"] = st["block_table"][[b]]
            sl = slice(cu[b], cu[b + 1])
            t0 = time.time()
            oracle.draft_extend(cfg, Wt, sub, torch.tensor([0, cu[b + 1] - cu[b]], dtype=torch.int32),
                                ex["aux"][sl], ex["token_in"][sl])
            dt += time.time() - t0
            n += cu[b + 1] - cu[b]
            b = (b + 1) % B
        result["cpu_baseline"] = {
            "value": round(n / dt, 4), "unit": "positions/s", "cores": torch.get_num_threads(), "kind": "oracle",
            "sample": f"{n} positions: the extend of whole sequences in turn, float64 torch CPU, {dt:.1f} s",
            **cpu_info(torch)}
    return result


def run_relaxed(args, cfg, dev):
    """One eagle3_relaxed_accept call per step over the target's fp32 logits at
    the gamma + 1 verified positions of every row (relaxed_topk / relaxed_delta
    of the workload, half the rows in a thinking span), timed in a graph."""
    import torch
    import workloads as W
    from eagle_draft_head_step_amd import binding
    B, g, V = cfg.batch, cfg.gamma, cfg.target_vocab
    x = W.make_relaxed_inputs(cfg, 0)
    z, dr, rel = x["logits"].to(dev), x["draft"].to(dev), x["relaxed"].to(dev)
    acc = torch.empty(B, dtype=torch.int32, device=dev)
    bon = torch.empty(B, dtype=torch.int32, device=dev)
    ws = torch.empty(binding.relaxed_accept_workspace_size(B, g, V), dtype=torch.uint8, device=dev)
    log(f"[bench] relaxed verification: B={B} gamma={g} vocab={V} ({z.numel() * 4 / 1e6:.1f} MB of logits)")

    def once():
        binding.relaxed_accept(dr, z, rel, cfg.relaxed_topk, cfg.relaxed_delta, acc, bon, workspace=ws)

    for _ in range(max(1, args.warmup)):
        once()
    torch.cuda.synchronize()
    graph = None
    if not args.no_graph:
        s_ = torch.cuda.Stream()
        s_.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(s_):
            once()
        torch.cuda.current_stream().wait_stream(s_)
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            once()
        graph.replay()
        torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record()
    for _ in range(args.steps):
        graph.replay() if graph is not None else once()
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / args.steps
    log(f"[bench] relaxed verification {1e3 * ms:.2f} us per call")
    copy_gbps = copy_bandwidth(torch, dev)
    kern = {} if args.no_kernel_timing else kernel_times(once, args.steps, ms)
    # algorithmic bytes of the scan: every logit once, the drafts, one partial per chunk
    part_bytes = ws.numel()
    scan_bytes = B * (g + 1) * V * 4 + B * g * 4 + part_bytes
    roof = None
    if "relaxed_scan" in kern:
        us = 1e3 * kern["relaxed_scan"][0] / kern["relaxed_scan"][1]
        ach = scan_bytes / (us / 1e6)
        roof = {"kernel": "relaxed_scan_kernel", "bound": "hbm", "achieved": round(ach / 1e9, 1),
                "peak": HBM_PEAK / 1e9, "unit": "GB/s", "frac": round(ach / HBM_PEAK, 4),
                "traffic": counter_traffic(cfg.name + "_relaxed", "relaxed_scan_kernel", "", "relaxed"),
                "algorithmic_bytes_per_launch": scan_bytes, "avg_launch_us": round(us, 2)}
        if copy_gbps:
            roof["frac_of_measured_copy"] = round(roof["achieved"] / copy_gbps, 4)
    a = acc.float()
    result = {
        "metric": "relaxed-verified draft tokens/s (rows x gamma per call)",
        "value": round(B * g / (ms / 1e3), 1), "unit": "draft tokens/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "f32", "data": "synthetic",
        "config": {"workload": cfg.name + "_relaxed", "global_batch": B, "gamma": g, "vocab": V,
                   "relaxed_topk": cfg.relaxed_topk, "relaxed_delta": cfg.relaxed_delta,
                   "parallelism": "single GPU", "hip_graph": graph is not None},
        "measured_copy_GBps": None if copy_gbps is None else round(copy_gbps, 1),
        "roofline": roof,
        "kernels_us_per_call": {n: round(1e3 * t / args.steps, 2) for n, (t, c) in kern.items()},
        "accept": {"mean_accept_len": round(float(a.mean()), 4),
                   "mean_accept_len_relaxed_rows": round(float(a[rel.bool()].mean()), 4),
                   "mean_accept_len_greedy_rows": round(float(a[~rel.bool()].mean()), 4)},
    }
    if not args.no_cpu_baseline:
        import oracle
        n, b, t0 = 0, 0, time.time()
        while time.time() - t0 < 10.0:
            oracle.relaxed_accept(x["draft"][[b]], x["logits"][[b]], x["relaxed"][[b]], cfg.relaxed_topk,
                                  cfg.relaxed_delta)
            n += 1
            b = (b + 1) % B
        dt = time.time() - t0
        result["cpu_baseline"] = {
            "value": round(n * g / dt, 4), "unit": "draft tokens/s", "cores": torch.get_num_threads(),
            "kind": "oracle", "sample": f"{n} rows verified one at a time, cycling through the batch, {dt:.1f} s",
            **cpu_info(torch)}
    return result


# ------------------------------------------------------------------ chain
RIDGE = MFMA_BF16_PEAK / HBM_PEAK      # flop per byte where the MFMA peak meets the HBM peak


def gemm_family(cfg, B, kern):
    """The dominant kernel family of a step: the weight-streaming GEMM launches
    with bf16 activations in the head's weight format (fc, q/k/v or q_a/kv_a,
    q_b, o_proj, lm_head; the MLP's gate/up and down are another instance: f16
    tiles with f16 activations for a bf16 head, fp32 activations for a quantized
    one; above 64 rows the per-head absorb halves stay on the register-staged
    kernel).  Returns (roles, kernel name, counter-name match)."""
    roles = ["gemm.fc"] + [r for r, *_ in gemm_roles(cfg, B)
                           if r not in ("gemm.gate_up", "gemm.down") and role_format(cfg, r) == cfg.weight_format]
    big = cfg.weight_format == "bf16" and B > 64
    if big:
        roles = [r for r in roles if r not in ("gemm.uk_absorb", "gemm.uv")]
        # (waves, m-tiles, read schedule, f16): the bf16 instance of the block height
        name = "gemm_big_kernel<8, 16, 1, false>" if B > 128 else "gemm_big_kernel<8, 8, 2, false>"
        match = (name, "")
    else:
        wq = {"bf16": 0, "fp8": 1, "nvfp4": 2}[cfg.weight_format]
        name = "gemm_kernel"
        match = ("gemm_kernel<", f", false, {wq}>")
    return [r for r in roles if r in kern], name, match


def role_models(cfg, B):
    """Algorithmic (bytes, flops) per launch of every GEMM role and the attention."""
    m = {role: gemm_bytes_flops(B, N, K, bt, ob, role_format(cfg, role)) for role, N, K, bt, ob in gemm_roles(cfg, B)}
    m["gemm.fc"] = gemm_bytes_flops(B, cfg.hidden, cfg.num_aux * cfg.hidden, 1, 4, cfg.weight_format)
    return m


def roofline_of(cfg, B, kern, roles, name, match, family_traffic=True):
    """Roofline line of a kernel family: algorithmic bytes and flops per launch
    over the average launch time.  The bound follows the family's intensity
    against the ridge (312.5 flop/B); both fractions are reported."""
    if not roles:
        return None
    models = role_models(cfg, B)
    launches = sum(kern[r][1] for r in roles)
    tb = sum(models[r][0] * kern[r][1] for r in roles)
    tf = sum(models[r][1] * kern[r][1] for r in roles)
    dur = sum(kern[r][0] for r in roles) / 1e3
    intensity = tf / tb
    hbm, mf = tb / dur, tf / dur
    bound = "mfma" if intensity > RIDGE else "hbm"
    r = {"kernel": f"{name}, bf16 activations, {cfg.weight_format} weights ({', '.join(roles)})",
         "bound": bound}
    if bound == "hbm":
        r.update(achieved=round(hbm / 1e9, 1), peak=HBM_PEAK / 1e9, unit="GB/s", frac=round(hbm / HBM_PEAK, 4))
    else:
        r.update(achieved=round(mf / 1e12, 1), peak=MFMA_BF16_PEAK / 1e12, unit="TFLOP/s",
                 frac=round(mf / MFMA_BF16_PEAK, 4))
    r["traffic"] = counter_traffic(cfg.name, *match) if family_traffic else None
    r.update({"hbm_frac": round(hbm / HBM_PEAK, 4), "mfma_frac": round(mf / MFMA_BF16_PEAK, 4),
              "intensity_flop_per_byte": round(intensity, 1), "ridge_flop_per_byte": round(RIDGE, 1),
              "mfma_cap_at_hbm_peak": round(min(1.0, intensity / RIDGE), 4),
              "algorithmic_bytes_per_launch": round(tb / launches),
              "algorithmic_flops_per_launch": round(tf / launches),
              "avg_launch_us": round(1e6 * dur / launches, 2), "launches": launches})
    return r


def stage_table(cfg, B, g, ctx_l, kern):
    """Per-launch time, bandwidth and MFMA share of every GEMM role and the attention."""
    stages = {}
    per_tok = (2 * cfg.n_kv_heads * cfg.head_dim * 2) if cfg.attn_kind == 0 else cfg.kv_entry_dim * 2
    keys_avg = sum(sum(int(c) + k + 1 for c in ctx_l) for k in range(g)) / g
    model = role_models(cfg, B)
    attn_f = (4.0 * cfg.n_heads * cfg.head_dim if cfg.attn_kind == 0
              else 2.0 * cfg.n_heads * (cfg.kv_entry_dim + cfg.kv_lora_rank)) * keys_avg
    attn_b = keys_avg * per_tok
    if cfg.attn_kind != 0 and "gemm.uv" not in kern and "gemm.uv" in model:
        # up to 64 rows the attention launch also applies W_UV (merge + W_UV kernel)
        attn_b += model["gemm.uv"][0]
        attn_f += model["gemm.uv"][1]
    model["mha_attn" if cfg.attn_kind == 0 else "mla_attn"] = (attn_b, attn_f)
    if "gemm.uk_absorb" in model:
        # up to 64 rows the W_UK absorption runs in the q epilogue's launch
        model["mla_q_absorb"] = model["gemm.uk_absorb"]
    for role, (byts, flops) in model.items():
        if role not in kern:
            continue
        us = 1e3 * kern[role][0] / kern[role][1]
        stages[role] = {"us_per_launch": round(us, 2), "GBps": round(byts / us / 1e3, 1),
                        "hbm_frac": round(byts / (us / 1e6) / HBM_PEAK, 4),
                        "mfma_frac": round(flops / (us / 1e6) / MFMA_BF16_PEAK, 4),
                        # the MFMA share a kernel would reach if it streamed its bytes at 8 TB/s
                        "mfma_cap_at_hbm_peak": round(min(1.0, flops / byts * HBM_PEAK / MFMA_BF16_PEAK), 4)}
    return stages


def gemm_mfma_share(cfg, B, kern):
    """MFMA fraction of all of a step's GEMM launches together (time-weighted),
    with the cap the spec bandwidth puts on it."""
    model = role_models(cfg, B)
    roles = [r for r in model if r.startswith("gemm.") and r in kern]
    if not roles:
        return None
    tf = sum(model[r][1] * kern[r][1] for r in roles)
    tb = sum(model[r][0] * kern[r][1] for r in roles)
    dur = sum(kern[r][0] for r in roles) / 1e3
    return {"mfma_frac": round(tf / dur / MFMA_BF16_PEAK, 4), "hbm_frac": round(tb / dur / HBM_PEAK, 4),
            "mfma_cap_at_hbm_peak": round(min(1.0, tf / tb / RIDGE), 4)}


def run_chain(args, cfg, st, head, dev, steps, warmup, kernel_steps):
    """Times one step of the hot path -- eagle3_draft_chain (gamma steps) +
    eagle3_greedy_accept -- captured in a HIP graph and replayed `steps` times
    between two events; then a per-kernel event pass over `kernel_steps`
    eager runs.  Returns the measurements of one workload."""
    import torch
    import workloads as W
    from eagle_draft_head_step_amd import binding
    B, g = cfg.batch, cfg.gamma
    d = {k: v.to(dev) for k, v in W.to_tiled(cfg, st).items()}
    ws = head.workspace(B, cfg.max_ctx, g)
    tok = torch.empty(B, g, dtype=torch.int32, device=dev)
    tgt = torch.zeros(B, g + 1, dtype=torch.int32, device=dev)   # filled from the chain's drafts below
    acc = torch.empty(B, dtype=torch.int32, device=dev)
    bon = torch.empty(B, dtype=torch.int32, device=dev)
    aux = d["aux"].reshape(B, -1)
    kc = d["k_cache"] if cfg.attn_kind == 0 else d["kv_cache"]
    vc = d.get("v_cache")
    torch.cuda.synchronize()

    def one_step():
        head.draft_chain(gamma=g, aux=aux, hidden_in=None, token_in=d["token_in"], k_cache=kc, v_cache=vc,
                         block_table=d["block_table"], ctx_len=d["ctx_len"], max_ctx=cfg.max_ctx,
                         hidden_out=None, token_out=tok, draft_id_out=None, logits_out=None, workspace=ws)
        binding.greedy_accept(tok, tgt, acc, bon)

    for _ in range(max(1, warmup)):
        one_step()
    torch.cuda.synchronize()
    # verification targets synthesised against the drafts this chain produces (it is
    # deterministic): the first k ~ Geometric(p) - 1 drafts of a row match, the rest differ
    tgt_cpu, k_expect = W.make_accept_targets(cfg, tok.cpu())
    tgt.copy_(tgt_cpu)
    one_step()
    torch.cuda.synchronize()
    assert torch.equal(acc.cpu(), k_expect), "greedy accept disagrees with the synthesised targets"

    graph = None
    if not args.no_graph:
        s = torch.cuda.Stream()
        s.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(s):
            one_step()
        torch.cuda.current_stream().wait_stream(s)
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            one_step()
        graph.replay()
        torch.cuda.synchronize()

    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    marks = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
    torch.cuda.synchronize()
    start.record()
    for i in range(steps):
        if graph is not None:
            graph.replay()
        else:
            one_step()
        marks[i].record()
    end.record()
    torch.cuda.synchronize()
    ms = start.elapsed_time(end) / steps
    per = sorted([start.elapsed_time(marks[0])] +
                 [marks[i - 1].elapsed_time(marks[i]) for i in range(1, steps)])
    pct = lambda q: per[min(len(per) - 1, int(round(q * (len(per) - 1))))]
    log(f"[bench] {cfg.name}: {ms:.3f} ms per step, {B * g / (ms / 1e3):.1f} draft tokens/s")
    kern = {} if (args.no_kernel_timing or kernel_steps <= 0) else kernel_times(one_step, kernel_steps, ms)
    ctx_l = st["ctx_len"].tolist()
    model = chain_model(cfg, ctx_l, g)
    roles, name, match = gemm_family(cfg, B, kern)
    out = {"ms": ms, "pct": {"median": round(pct(0.5), 4), "p10": round(pct(0.1), 4), "p90": round(pct(0.9), 4)},
           "tokens_per_s": B * g / (ms / 1e3), "model": model, "kern": kern, "kernel_steps": kernel_steps,
           "stages": stage_table(cfg, B, g, ctx_l, kern),
           "roofline": roofline_of(cfg, B, kern, roles, name, match),
           "gemm_all": gemm_mfma_share(cfg, B, kern),
           "accept_len": acc.float(), "graph": graph is not None}
    del graph, d, ws
    torch.cuda.empty_cache()
    return out


def config_summary(cfg, r):
    """The per-workload object of the JSON line."""
    bw = r["model"]["bytes"] / (r["ms"] / 1e3)
    ks = max(1, r["kernel_steps"])
    return {"global_batch": cfg.batch, "gamma": cfg.gamma, "ctx": list(cfg.ctx),
            "tokens_per_s": round(r["tokens_per_s"], 1), "ms_per_step": round(r["ms"], 4),
            "us_per_draft_step": round(1e3 * r["ms"] / cfg.gamma, 2),
            "whole_step_hbm_frac": round(bw / HBM_PEAK, 4),
            "whole_step_mfma_frac": round(r["model"]["flops"] / (r["ms"] / 1e3) / MFMA_BF16_PEAK, 4),
            "launches_per_step": sum(c for t, c in r["kern"].values()) // ks if r["kern"] else None,
            "roofline": r["roofline"], "gemm_all": r["gemm_all"], "stages": r["stages"]}


def cpu_info(torch):
    model = None
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    import re
    m = re.search(r"BLAS_INFO=([\w.-]+)", torch.__config__.show())
    blas = m.group(1) if m else None
    return {"cpu_model": model, "affinity_cores": len(os.sched_getaffinity(0)),
            "torch_threads": torch.get_num_threads(), "blas": blas,
            "omp_num_threads": os.environ.get("OMP_NUM_THREADS")}


# ------------------------------------------------------------------ main
DEFAULT_CONFIG = "4"                    # the largest workload: MLA head, B 256, gamma 7, + greedy accept
PER_CONFIG = (0, 1, 2, 3)               # the other workloads, reported beside the headline


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--config", default=None,
                    help="workload index 0-4 or name (default 4: the MLA head at batch 256, gamma 7, "
                         "with greedy accept; 4 for --mode relaxed)")
    ap.add_argument("--no-graph", action="store_true", help="time eager launches instead of a HIP graph")
    ap.add_argument("--mode", choices=("chain", "extend", "relaxed"), default="chain",
                    help="chain: gamma draft steps + greedy accept (default); extend: one multi-token "
                         "extend over accepted positions (q_len = accepted + 1 per row); relaxed: "
                         "relaxed top-N verification over the target's logits")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-kernel-timing", action="store_true")
    ap.add_argument("--no-per-config", action="store_true",
                    help="skip the other workloads' per_config entries")
    args = ap.parse_args()

    if args.gpus != 1:
        print(f"bench.py: this build runs on one GPU only (asked for --gpus {args.gpus}); "
              "multi-GPU sharding of the draft head is not built", file=sys.stderr)
        sys.exit(2)

    import torch
    import workloads as W
    from eagle_draft_head_step_amd import binding

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    dev = torch.device("cuda:0")
    headline = args.config is None and args.mode == "chain"
    if args.config is None:
        args.config = "4" if args.mode == "relaxed" else DEFAULT_CONFIG
    key = int(args.config) if args.config.isdigit() else args.config
    cfg = W.get_config(key)
    B, g = cfg.batch, cfg.gamma
    log(f"[bench] workload {cfg.name}: B={B} gamma={g} ctx={cfg.ctx}")
    if args.mode == "relaxed":
        print(json.dumps(run_relaxed(args, cfg, dev)), flush=True)
        return

    t0 = time.time()
    Wt = W.make_weights(cfg)
    st = W.make_inputs(cfg)
    log(f"[bench] synthetic inputs in {time.time() - t0:.1f}s")
    head = binding.DraftHead(cfg, {k: v.to(dev) for k, v in Wt.items()})
    if args.mode == "extend":
        d = {k: v.to(dev) for k, v in W.to_tiled(cfg, st).items()}
        print(json.dumps(run_extend(args, cfg, Wt, st, head, d, dev)), flush=True)
        return

    r = run_chain(args, cfg, st, head, dev, args.steps, args.warmup, args.steps)
    ms = r["ms"]
    model = r["model"]
    copy_gbps = copy_bandwidth(torch, dev)
    chain_bw = model["bytes"] / (ms / 1e3)
    kern = r["kern"]
    roof = r["roofline"]
    result = {
        "metric": "draft tokens/s per EAGLE-3 head step",
        "value": round(r["tokens_per_s"], 1),
        "unit": "draft tokens/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(ms, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16", "data": "synthetic",
        "config": {"workload": cfg.name, "global_batch": B, "gamma": g, "ctx": list(cfg.ctx),
                   "hidden": cfg.hidden, "attention": "mha_gqa" if cfg.attn_kind == 0 else "mla",
                   "weights": cfg.weight_format,
                   "draft_vocab": cfg.draft_vocab, "target_vocab": cfg.target_vocab,
                   "verification": "greedy", "parallelism": "single GPU", "hip_graph": r["graph"]},
        "step_latency_us": round(1e3 * ms / g, 2),
        "ms_per_step_replays": r["pct"],
        "measured_copy_GBps": None if copy_gbps is None else round(copy_gbps, 1),
        "whole_step": {"algorithmic_bytes": model["bytes"], "algorithmic_flops": model["flops"],
                       "hbm_GBps": round(chain_bw / 1e9, 1), "hbm_frac": round(chain_bw / HBM_PEAK, 4),
                       "mfma_frac": round(model["flops"] / (ms / 1e3) / MFMA_BF16_PEAK, 4)},
        "roofline": roof,
        "gemm_all": r["gemm_all"],
        "kernels_us_per_step": {n: round(1e3 * t / args.steps, 2) for n, (t, c) in kern.items()},
        "stages": r["stages"],
        "accept": {"mean_accept_len": round(float(r["accept_len"].mean()), 4),
                   "mean_accepted_plus_bonus": round(float(r["accept_len"].mean()) + 1, 4),
                   "kernel_us": None if "greedy_accept" not in kern
                   else round(1e3 * kern["greedy_accept"][0] / kern["greedy_accept"][1], 2)},
    }
    if copy_gbps:
        result["whole_step"]["frac_of_measured_copy"] = round(chain_bw / 1e9 / copy_gbps, 4)
        if roof and roof["unit"] == "GB/s":
            roof["frac_of_measured_copy"] = round(roof["achieved"] / copy_gbps, 4)

    # ---- the CPU oracle on a bounded sample of the same workload: groups of rows
    # of the first draft step, cycling through the batch, until >= 10 s of CPU work
    if not args.no_cpu_baseline:
        import oracle
        group = min(B, 4 if cfg.attn_kind == 0 else 1)
        n, start, t0 = 0, 0, time.time()
        while True:
            rows = [(start + i) % B for i in range(group)]
            sub = {k: (v[rows].clone() if k in ("aux", "token_in", "ctx_len", "block_table") else v.clone())
                   for k, v in st.items()}
            oracle.draft_step(cfg, Wt, sub, 0)
            n += group
            start = (start + group) % B
            if time.time() - t0 >= 10.0:
                break
        dt = time.time() - t0
        info = cpu_info(torch)
        result["cpu_baseline"] = {
            "value": round(n / dt, 4), "unit": "draft tokens/s",
            "cores": info["torch_threads"], "kind": "oracle",
            "sample": f"{n} row-steps of the first draft step (fc, attention over the full cached "
                      f"context, MLP, lm_head, top-1) in groups of {group} rows cycling through the "
                      f"batch, float64 torch CPU, {dt:.1f} s", **info}
        log(f"[bench] cpu oracle: {n} tokens in {dt:.1f}s")

    # ---- the other workloads, each timed the same way (shorter), beside the headline
    if headline and not args.no_per_config:
        per = {}
        fam = cfg.weight_family or cfg.name
        others = [W.get_config(i) for i in PER_CONFIG if W.get_config(i).name != cfg.name]
        # workloads of the headline's weight family first, reusing its packed weights
        others.sort(key=lambda c: (c.weight_family or c.name) != fam)
        for c2 in others:
            if (c2.weight_family or c2.name) != fam:
                del head
                torch.cuda.empty_cache()
                Wt = W.make_weights(c2)
                head = binding.DraftHead(c2, {k: v.to(dev) for k, v in Wt.items()})
                fam = c2.weight_family or c2.name
            # fresh device allocations for each workload: blocks the caching
            # allocator kept from the previous one measured a few percent slower
            gc.collect()
            torch.cuda.empty_cache()
            st2 = W.make_inputs(c2)
            r2 = run_chain(args, c2, st2, head, dev, min(args.steps, 20), 2, min(args.steps, 5))
            per[c2.name] = config_summary(c2, r2)
        result["per_config"] = per
        b16 = per.get("dsv3_mla_b16")
        b128 = per.get("dsv3_mla_b128_ragged")
        result["targets"] = {
            "batch<=16 whole-step HBM fraction (dsv3_mla_b16), target 0.70":
                None if b16 is None else b16["whole_step_hbm_frac"],
            "batch-128 MLA GEMMs MFMA fraction (dsv3_mla_b128_ragged), target 0.50, cap at 8 TB/s":
                None if b128 is None or b128["gemm_all"] is None
                else [b128["gemm_all"]["mfma_frac"], b128["gemm_all"]["mfma_cap_at_hbm_peak"]],
        }

    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
