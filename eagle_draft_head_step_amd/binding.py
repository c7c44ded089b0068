"""ctypes binding of libeagle3.so.

Argument marshalling only: every step of the draft head runs in the HIP
kernels behind the C ABI declared in include/eagle3.h.  torch provides the
device memory and the stream; pointers and sizes cross the boundary.
If the library is not built, loading fails loudly -- there is no fallback.
"""
from __future__ import annotations

import ctypes
import os
import re
from typing import Dict, Optional

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libeagle3.so")
DEBUG_LIB_PATH = os.path.join(_PKG, "libeagle3_debug.so")   # host-side range checks (EAGLE3_DEBUG)
HEADER_PATH = os.path.join(os.path.dirname(_PKG), "include", "eagle3.h")

ATTN_MHA, ATTN_MLA = 0, 1
STATUS = {0: "ok", -1: "invalid argument", -2: "inconsistent shapes", -3: "unsupported configuration",
          -4: "buffer too small", -5: "HIP launch error"}


class Eagle3Error(RuntimeError):
    def __init__(self, fn: str, code: int):
        super().__init__(f"{fn}: {STATUS.get(code, 'unknown status')} ({code})")
        self.code = code


class Config(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in (
        "attn_kind", "hidden", "num_aux", "fc_in_features", "intermediate", "draft_vocab",
        "target_vocab", "n_heads", "n_kv_heads", "head_dim", "q_lora_rank", "kv_lora_rank",
        "qk_nope_dim", "qk_rope_dim", "v_head_dim", "page_size")] + [
        (n, ctypes.c_float) for n in (
            "rms_eps", "rope_theta", "yarn_factor", "yarn_orig_max_pos", "yarn_beta_fast",
            "yarn_beta_slow")] + [("weight_format", ctypes.c_int32), ("cache_dtype", ctypes.c_int32)]


WEIGHT_FORMATS = {"bf16": 0, "fp8": 1, "nvfp4": 2}
# GEMM matrices in the order of the header's EAGLE3_MAT_* (row_scale / block_scale index)
GEMM_MATS = ("fc", "w_q", "w_k", "w_v", "w_qa", "w_qb", "w_kva", "w_kvb", "w_o", "w_gate", "w_up", "w_down",
             "lm_head")


WEIGHT_NAMES = ("embed", "fc", "norm_in", "norm_hid", "norm_post", "norm_final", "w_q", "w_k", "w_v",
                "w_qa", "norm_qa", "w_qb", "w_kva", "norm_kv", "w_kvb", "w_o", "w_gate", "w_up",
                "w_down", "lm_head", "d2t")


class Weights(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in WEIGHT_NAMES] + [
        ("row_scale", ctypes.c_void_p * len(GEMM_MATS)), ("block_scale", ctypes.c_void_p * len(GEMM_MATS))]


class StepArgs(ctypes.Structure):
    _fields_ = [
        ("batch", ctypes.c_int32),
        ("aux", ctypes.c_void_p), ("hidden_in", ctypes.c_void_p), ("token_in", ctypes.c_void_p),
        ("k_cache", ctypes.c_void_p), ("v_cache", ctypes.c_void_p),
        ("block_table", ctypes.c_void_p), ("max_pages", ctypes.c_int32),
        ("ctx_len", ctypes.c_void_p), ("max_ctx", ctypes.c_int32),
        ("hidden_out", ctypes.c_void_p), ("token_out", ctypes.c_void_p),
        ("draft_id_out", ctypes.c_void_p), ("logits_out", ctypes.c_void_p),
        ("workspace", ctypes.c_void_p), ("workspace_bytes", ctypes.c_size_t),
        ("num_pages", ctypes.c_int32),
    ]


class ExtendArgs(ctypes.Structure):
    _fields_ = [
        ("num_tokens", ctypes.c_int32), ("batch", ctypes.c_int32),
        ("cu_seqlens", ctypes.c_void_p), ("max_q_len", ctypes.c_int32),
        ("aux", ctypes.c_void_p), ("token_in", ctypes.c_void_p),
        ("k_cache", ctypes.c_void_p), ("v_cache", ctypes.c_void_p),
        ("block_table", ctypes.c_void_p), ("max_pages", ctypes.c_int32),
        ("ctx_len", ctypes.c_void_p), ("max_ctx", ctypes.c_int32),
        ("hidden_out", ctypes.c_void_p), ("token_out", ctypes.c_void_p),
        ("draft_id_out", ctypes.c_void_p), ("logits_out", ctypes.c_void_p),
        ("workspace", ctypes.c_void_p), ("workspace_bytes", ctypes.c_size_t),
        ("num_pages", ctypes.c_int32),
    ]


_libs = {}


def lib(debug: bool = False) -> ctypes.CDLL:
    """The loaded libeagle3.so, or with debug=True libeagle3_debug.so (the same
    kernels; each call first checks its device-resident indices on the host).
    Raises if the library has not been built."""
    path = DEBUG_LIB_PATH if debug else LIB_PATH
    if path not in _libs:
        if not os.path.exists(path):
            raise ImportError(f"{path} is missing: build it with "
                              "`python -m eagle_draft_head_step_amd.build`")
        L = ctypes.CDLL(path)
        P, I32, SZ, F32 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_size_t, ctypes.c_float
        sigs = {
            "eagle3_workspace_size": [P, I32, I32, I32, P],
            "eagle3_packed_weights_size": [P, P],
            "eagle3_pack_weights": [P, P, P, SZ, P],
            "eagle3_draft_step": [P, P, P, P, I32, P],
            "eagle3_draft_chain": [P, P, P, P, I32, P],
            "eagle3_extend_workspace_size": [P, I32, I32, I32, I32, P],
            "eagle3_draft_extend": [P, P, P, P, P],
            "eagle3_greedy_accept": [P, P, I32, I32, P, P, P],
            "eagle3_relaxed_accept_workspace_size": [I32, I32, I32, P],
            "eagle3_relaxed_accept": [P, P, P, I32, I32, I32, I32, F32, P, P, P, SZ, P],
            "eagle3_relaxed_accept_noalloc": [P, P, P, I32, I32, I32, I32, F32, P, P, P],
        }
        for name, argt in sigs.items():
            fn = getattr(L, name)
            fn.argtypes = argt
            fn.restype = ctypes.c_int
        L.eagle3_status_string.argtypes = [ctypes.c_int]
        L.eagle3_status_string.restype = ctypes.c_char_p
        _libs[path] = L
    return _libs[path]


def header_symbols():
    """Function names the public header declares."""
    with open(HEADER_PATH) as f:
        text = f.read()
    return sorted(set(re.findall(r"\b(eagle3_[a-z_]+)\s*\(", text)))


def _check(fn: str, code: int):
    if code != 0:
        raise Eagle3Error(fn, code)


def make_config(c) -> Config:
    """C config from any object with the draft-head shape attributes."""
    g = (lambda k, d=0: getattr(c, k, d)) if not isinstance(c, dict) else (lambda k, d=0: c.get(k, d))
    return Config(
        attn_kind=int(g("attn_kind")), hidden=int(g("hidden")), num_aux=int(g("num_aux", 3)),
        fc_in_features=int(g("fc_in_features", g("num_aux", 3) * g("hidden"))),
        intermediate=int(g("intermediate")), draft_vocab=int(g("draft_vocab")),
        target_vocab=int(g("target_vocab")), n_heads=int(g("n_heads")),
        n_kv_heads=int(g("n_kv_heads")), head_dim=int(g("head_dim")),
        q_lora_rank=int(g("q_lora_rank")), kv_lora_rank=int(g("kv_lora_rank")),
        qk_nope_dim=int(g("qk_nope_dim")), qk_rope_dim=int(g("qk_rope_dim")),
        v_head_dim=int(g("v_head_dim")), page_size=int(g("page_size", 64)),
        rms_eps=float(g("rms_eps", 1e-6)), rope_theta=float(g("rope_theta", 1e4)),
        yarn_factor=float(g("yarn_factor", 0.0)), yarn_orig_max_pos=float(g("yarn_orig_max_pos", 0.0)),
        yarn_beta_fast=float(g("yarn_beta_fast", 32.0)), yarn_beta_slow=float(g("yarn_beta_slow", 1.0)),
        weight_format=_weight_format(g("weight_format", "bf16")), cache_dtype=int(g("cache_dtype", 0)))


def _weight_format(f) -> int:
    return WEIGHT_FORMATS[f] if isinstance(f, str) else int(f)


def _ptr(t: Optional[torch.Tensor], dtype=None, name="") -> int:
    if t is None:
        return 0
    if not t.is_cuda:
        raise ValueError(f"{name}: expected a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name}: expected a contiguous tensor")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name}: expected {dtype}, got {t.dtype}")
    return t.data_ptr()


def _stream(stream) -> int:
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


def workspace_size(cfg, max_batch: int, max_ctx: int, max_gamma: int) -> int:
    n = ctypes.c_size_t(0)
    _check("eagle3_workspace_size",
           lib().eagle3_workspace_size(ctypes.byref(make_config(cfg)), max_batch, max_ctx, max_gamma,
                                       ctypes.byref(n)))
    return n.value


def packed_weights_size(cfg) -> int:
    n = ctypes.c_size_t(0)
    _check("eagle3_packed_weights_size",
           lib().eagle3_packed_weights_size(ctypes.byref(make_config(cfg)), ctypes.byref(n)))
    return n.value


def extend_workspace_size(cfg, max_tokens: int, max_batch: int, max_ctx: int, max_q_len: int) -> int:
    n = ctypes.c_size_t(0)
    _check("eagle3_extend_workspace_size",
           lib().eagle3_extend_workspace_size(ctypes.byref(make_config(cfg)), max_tokens, max_batch, max_ctx,
                                              max_q_len, ctypes.byref(n)))
    return n.value


class DraftHead:
    """One draft head's weights on the device, packed once for the GEMMs.

    weights: dict of device tensors named like the fields of eagle3_weights
    (bf16 matrices [out, in], bf16 gains, int32 d2t).  A quantized head
    (cfg.weight_format "fp8" / "nvfp4") holds uint8 codes for the GEMM
    matrices and their scales as "<name>.row_scale" (fp32) and
    "<name>.block_scale" (uint8 E4M3).
    """

    def __init__(self, cfg, weights: Dict[str, torch.Tensor], stream=None, debug: bool = False):
        self.cfg = cfg
        self.c = make_config(cfg)
        self.L = lib(debug)
        quant = self.c.weight_format != 0
        self.tensors = {k: v for k, v in weights.items()
                        if k in WEIGHT_NAMES or k.endswith((".row_scale", ".block_scale"))}
        self.w = Weights()
        for name in WEIGHT_NAMES:
            t = self.tensors.get(name)
            dt = torch.int32 if name == "d2t" else (torch.uint8 if quant and name in GEMM_MATS else torch.bfloat16)
            setattr(self.w, name, _ptr(t, dt, name) or None)
        for i, name in enumerate(GEMM_MATS):
            self.w.row_scale[i] = _ptr(self.tensors.get(name + ".row_scale"), torch.float32, name) or None
            self.w.block_scale[i] = _ptr(self.tensors.get(name + ".block_scale"), torch.uint8, name) or None
        nbytes = packed_weights_size(self.c)
        dev = next(iter(self.tensors.values())).device
        self.packed = torch.empty(nbytes, dtype=torch.uint8, device=dev)
        _check("eagle3_pack_weights",
               self.L.eagle3_pack_weights(ctypes.byref(self.c), ctypes.byref(self.w),
                                         self.packed.data_ptr(), nbytes, _stream(stream)))

    def workspace(self, max_batch: int, max_ctx: int, max_gamma: int) -> torch.Tensor:
        n = workspace_size(self.c, max_batch, max_ctx, max_gamma)
        return torch.empty(max(n, 256), dtype=torch.uint8, device=self.packed.device)

    def _args(self, *, aux, hidden_in, token_in, k_cache, v_cache, block_table, ctx_len, max_ctx,
              hidden_out, token_out, draft_id_out, logits_out, workspace) -> StepArgs:
        a = StepArgs()
        a.batch = int(token_in.shape[0])
        a.aux = _ptr(aux, torch.bfloat16, "aux") or None
        a.hidden_in = _ptr(hidden_in, torch.float32, "hidden_in") or None
        a.token_in = _ptr(token_in, torch.int32, "token_in")
        a.k_cache = _ptr(k_cache, torch.bfloat16, "k_cache")
        a.v_cache = _ptr(v_cache, torch.bfloat16, "v_cache") or None
        a.block_table = _ptr(block_table, torch.int32, "block_table")
        a.max_pages = int(block_table.shape[1])
        a.ctx_len = _ptr(ctx_len, torch.int32, "ctx_len")
        a.max_ctx = int(max_ctx)
        a.hidden_out = _ptr(hidden_out, torch.float32, "hidden_out") or None
        a.token_out = _ptr(token_out, torch.int32, "token_out")
        a.draft_id_out = _ptr(draft_id_out, torch.int32, "draft_id_out") or None
        a.logits_out = _ptr(logits_out, torch.float32, "logits_out") or None
        a.workspace = _ptr(workspace, None, "workspace")
        a.workspace_bytes = workspace.numel() * workspace.element_size()
        a.num_pages = int(k_cache.shape[0])
        return a

    def draft_step(self, *, step_index: int, stream=None, **kw) -> None:
        """eagle3_draft_step: outputs go to the given hidden_out / token_out tensors."""
        a = self._args(**kw)
        _check("eagle3_draft_step",
               self.L.eagle3_draft_step(ctypes.byref(self.c), ctypes.byref(self.w), self.packed.data_ptr(),
                                       ctypes.byref(a), int(step_index), _stream(stream)))

    def draft_chain(self, *, gamma: int, stream=None, **kw) -> None:
        """eagle3_draft_chain: token_out [B, gamma]; hidden_out None or [gamma, B, H]."""
        a = self._args(**kw)
        _check("eagle3_draft_chain",
               self.L.eagle3_draft_chain(ctypes.byref(self.c), ctypes.byref(self.w), self.packed.data_ptr(),
                                        ctypes.byref(a), int(gamma), _stream(stream)))


    def extend_workspace(self, max_tokens: int, max_batch: int, max_ctx: int, max_q_len: int) -> torch.Tensor:
        n = extend_workspace_size(self.c, max_tokens, max_batch, max_ctx, max_q_len)
        return torch.empty(max(n, 256), dtype=torch.uint8, device=self.packed.device)

    def draft_extend(self, *, cu_seqlens, max_q_len, aux, token_in, k_cache, v_cache, block_table, ctx_len,
                     max_ctx, hidden_out, token_out, draft_id_out=None, logits_out=None, workspace,
                     stream=None) -> None:
        """eagle3_draft_extend over T = token_in.numel() new positions of cu_seqlens.numel() - 1 rows."""
        a = ExtendArgs()
        a.num_tokens = int(token_in.shape[0])
        a.batch = int(cu_seqlens.shape[0]) - 1
        a.cu_seqlens = _ptr(cu_seqlens, torch.int32, "cu_seqlens")
        a.max_q_len = int(max_q_len)
        a.aux = _ptr(aux, torch.bfloat16, "aux")
        a.token_in = _ptr(token_in, torch.int32, "token_in")
        a.k_cache = _ptr(k_cache, torch.bfloat16, "k_cache")
        a.v_cache = _ptr(v_cache, torch.bfloat16, "v_cache") or None
        a.block_table = _ptr(block_table, torch.int32, "block_table")
        a.max_pages = int(block_table.shape[1])
        a.ctx_len = _ptr(ctx_len, torch.int32, "ctx_len")
        a.max_ctx = int(max_ctx)
        a.hidden_out = _ptr(hidden_out, torch.float32, "hidden_out")
        a.token_out = _ptr(token_out, torch.int32, "token_out")
        a.draft_id_out = _ptr(draft_id_out, torch.int32, "draft_id_out") or None
        a.logits_out = _ptr(logits_out, torch.float32, "logits_out") or None
        a.workspace = _ptr(workspace, None, "workspace")
        a.workspace_bytes = workspace.numel() * workspace.element_size()
        a.num_pages = int(k_cache.shape[0])
        _check("eagle3_draft_extend",
               self.L.eagle3_draft_extend(ctypes.byref(self.c), ctypes.byref(self.w), self.packed.data_ptr(),
                                         ctypes.byref(a), _stream(stream)))


def greedy_accept(draft: torch.Tensor, target: torch.Tensor, accept_len: torch.Tensor,
                  bonus: torch.Tensor, stream=None) -> None:
    """eagle3_greedy_accept on int32 device tensors draft [B, g], target [B, g+1]."""
    B, g = draft.shape
    if tuple(target.shape) != (B, g + 1):
        raise ValueError("target must be [B, gamma + 1]")
    _check("eagle3_greedy_accept",
           lib().eagle3_greedy_accept(_ptr(draft, torch.int32, "draft"), _ptr(target, torch.int32, "target"),
                                      B, g, _ptr(accept_len, torch.int32, "accept_len"),
                                      _ptr(bonus, torch.int32, "bonus"), _stream(stream)))


def relaxed_accept_workspace_size(batch: int, gamma: int, vocab: int) -> int:
    n = ctypes.c_size_t(0)
    _check("eagle3_relaxed_accept_workspace_size",
           lib().eagle3_relaxed_accept_workspace_size(batch, gamma, vocab, ctypes.byref(n)))
    return n.value


def relaxed_accept(draft: torch.Tensor, logits: torch.Tensor, relaxed, topk: int, delta: float,
                   accept_len: torch.Tensor, bonus: torch.Tensor, workspace: torch.Tensor = None,
                   stream=None) -> None:
    """eagle3_relaxed_accept: draft int32 [B, g], logits fp32 [B, g+1, V],
    relaxed uint8 [B] or None (every row relaxed); outputs int32 [B].  Without
    a workspace tensor one is allocated here, outside the library."""
    B, g = draft.shape
    if logits.dim() != 3 or tuple(logits.shape[:2]) != (B, g + 1):
        raise ValueError("logits must be [B, gamma + 1, vocab]")
    V = int(logits.shape[2])
    if workspace is None:
        workspace = torch.empty(max(relaxed_accept_workspace_size(B, g, V), 16), dtype=torch.uint8,
                                device=logits.device)
    _check("eagle3_relaxed_accept",
           lib().eagle3_relaxed_accept(_ptr(draft, torch.int32, "draft"), _ptr(logits, torch.float32, "logits"),
                                       _ptr(relaxed, torch.uint8, "relaxed") or None, B, g, V, int(topk),
                                       float(delta), _ptr(accept_len, torch.int32, "accept_len"),
                                       _ptr(bonus, torch.int32, "bonus"), _ptr(workspace, None, "workspace"),
                                       workspace.numel() * workspace.element_size(), _stream(stream)))


def relaxed_accept_noalloc(draft: torch.Tensor, logits: torch.Tensor, relaxed, topk: int, delta: float,
                           accept_len: torch.Tensor, bonus: torch.Tensor, stream=None) -> None:
    """eagle3_relaxed_accept_noalloc: as relaxed_accept, with the partials in
    the library's fixed per-GPU scratch array (nothing is allocated)."""
    B, g = draft.shape
    if logits.dim() != 3 or tuple(logits.shape[:2]) != (B, g + 1):
        raise ValueError("logits must be [B, gamma + 1, vocab]")
    V = int(logits.shape[2])
    _check("eagle3_relaxed_accept_noalloc",
           lib().eagle3_relaxed_accept_noalloc(_ptr(draft, torch.int32, "draft"),
                                               _ptr(logits, torch.float32, "logits"),
                                               _ptr(relaxed, torch.uint8, "relaxed") or None, B, g, V, int(topk),
                                               float(delta), _ptr(accept_len, torch.int32, "accept_len"),
                                               _ptr(bonus, torch.int32, "bonus"), _stream(stream)))


# C-ABI names
eagle3_greedy_accept = greedy_accept
eagle3_relaxed_accept = relaxed_accept
eagle3_relaxed_accept_noalloc = relaxed_accept_noalloc
