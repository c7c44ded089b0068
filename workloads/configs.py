"""Shapes of the EAGLE-3 draft-head workloads.

Plain data only: no arithmetic of the draft head lives here.  Both the
CPU oracle and the HIP path read these records; the seeded tensors that
go with them come from ``workloads.synth``.

Sources for the constants (pages are cited by title and section):

* "Eagle3 DeepseekV3 投机解码架构 — MAX 中 eagle3_deepseekV3 模块的完整解析"
  (Modular MAX walkthrough), section 4 (the MLA draft: fc 3H->H without
  bias, a single DeepseekV3 decoder layer, dense SiLU MLP, own lm_head).
* "max.pipelines.architectures.eagle3_deepseekV3" (MAX Python API
  reference), ``Eagle3DeepseekV3DraftConfig`` defaults: hidden 7168,
  intermediate 18432, 128 heads, q_lora_rank 1536, kv_lora_rank 512,
  qk_rope_head_dim 64, qk_nope_head_dim 128, v_head_dim 128, vocab 129280,
  rms_norm_eps 1e-6, rope_theta 1e4, rope_interleave True,
  max_position_embeddings 4096.
* "EAGLE头结构深潜：Model Optimizer投机解码草稿模型的内部设计"
  (Model Optimizer EAGLE head deep dive), sections on fc fusion, the
  doubled first-layer attention input, and the draft vocabulary with its
  d2t offset map.
"""
from __future__ import annotations

import dataclasses
from dataclasses import dataclass, field
from typing import Optional, Tuple

MHA = 0
MLA = 1


@dataclass(frozen=True)
class Eagle3Config:
    name: str
    attn_kind: int                 # MHA (Llama-style, GQA allowed) or MLA (DeepseekV3)
    hidden: int
    intermediate: int
    draft_vocab: int
    target_vocab: int
    num_aux: int = 3               # early / middle / late target layers
    # MHA / GQA
    n_heads: int = 0
    n_kv_heads: int = 0
    head_dim: int = 0
    # MLA
    q_lora_rank: int = 0
    kv_lora_rank: int = 0
    qk_nope_dim: int = 0
    qk_rope_dim: int = 0
    v_head_dim: int = 0
    # shared
    page_size: int = 64
    rms_eps: float = 1e-6
    rope_theta: float = 10000.0
    yarn_factor: float = 0.0       # MLA only: YaRN scale s (required > 0 for MLA)
    yarn_orig_max_pos: float = 0.0
    yarn_beta_fast: float = 32.0
    yarn_beta_slow: float = 1.0
    # workload
    batch: int = 1
    ctx: Tuple[int, int] = (64, 64)  # cached context per row: fixed (a, a) or uniform [a, b]
    gamma: int = 1
    aux_scales: Tuple[float, float, float] = (1.0, 1.0, 1.0)
    d2t_kind: str = "zero"           # "zero" (draft vocab == target vocab), "sorted_map", or "none"
                                     # (no d2t: scores through the target's lm_head)
    paging: str = "identity"         # "identity" page tables or "shuffled" page pool
    weight_std: float = 0.02
    gain_std: float = 0.0            # RMSNorm gains are 1 + N(0, gain_std)
    weight_family: Optional[str] = None  # configs with one family share their weights
    weight_format: str = "bf16"      # GEMM weights: "bf16", "fp8" (E4M3 + row scale) or
                                     # "nvfp4" (E2M1 + E4M3 per 16 + row scale)
    accept: bool = False             # draft + greedy verification workload
    accept_p: float = 0.3            # Geometric success probability of the accept synthesis
    relaxed_topk: int = 10           # relaxed acceptance in thinking spans: candidates per position
    relaxed_delta: float = 0.6       # ... and their log-probability margin below the top-1

    # ---- derived sizes -------------------------------------------------
    @property
    def n_q_heads(self) -> int:
        return self.n_heads

    @property
    def qk_head_dim(self) -> int:
        return self.qk_nope_dim + self.qk_rope_dim

    @property
    def attn_out_dim(self) -> int:
        """Width of the attention output that feeds o_proj."""
        if self.attn_kind == MHA:
            return self.n_heads * self.head_dim
        return self.n_heads * self.v_head_dim

    @property
    def kv_entry_dim(self) -> int:
        """Elements one cached token holds per (page slot): MLA latent + rope."""
        return self.kv_lora_rank + self.qk_rope_dim

    @property
    def max_ctx(self) -> int:
        return self.ctx[1]

    def pages_for(self, ctx_len: int) -> int:
        need = ctx_len + self.gamma
        return (need + self.page_size - 1) // self.page_size

    def replace(self, **kw) -> "Eagle3Config":
        return dataclasses.replace(self, **kw)


_DSV3_MLA = dict(
    attn_kind=MLA, hidden=7168, intermediate=18432,
    draft_vocab=129280, target_vocab=129280,
    n_heads=128, q_lora_rank=1536, kv_lora_rank=512,
    qk_nope_dim=128, qk_rope_dim=64, v_head_dim=128,
    rope_theta=10000.0, yarn_factor=40.0, yarn_orig_max_pos=4096.0,
    yarn_beta_fast=32.0, yarn_beta_slow=1.0, weight_family="dsv3_mla_head",
)

# The five workloads.  Index 0 is the tiny head the oracle runs in seconds.
CONFIGS = [
    Eagle3Config(
        name="tiny_mha_b1", attn_kind=MHA, hidden=256, intermediate=688,
        draft_vocab=4096, target_vocab=4096, n_heads=4, n_kv_heads=4, head_dim=64,
        rope_theta=10000.0, batch=1, ctx=(64, 64), gamma=1, d2t_kind="zero"),
    Eagle3Config(
        name="llama3_8b_gqa_b32", attn_kind=MHA, hidden=4096, intermediate=14336,
        draft_vocab=32000, target_vocab=128256, n_heads=32, n_kv_heads=8, head_dim=128,
        rope_theta=500000.0, batch=32, ctx=(2048, 2048), gamma=3, d2t_kind="sorted_map"),
    Eagle3Config(name="dsv3_mla_b16", batch=16, ctx=(4096, 4096), gamma=3, **_DSV3_MLA),
    Eagle3Config(name="dsv3_mla_b128_ragged", batch=128, ctx=(1024, 8192), gamma=5,
                 aux_scales=(0.5, 1.0, 2.0), paging="shuffled", **_DSV3_MLA),
    Eagle3Config(name="dsv3_mla_b256_accept", batch=256, ctx=(2048, 2048), gamma=7,
                 accept=True, **_DSV3_MLA),
]

# Reduced heads with the same structure, sized so the oracle finishes in
# seconds while every GEMM still spans several tiles with a ragged tail
# (N not a multiple of 16, K not a multiple of 32, batch not a multiple of 16).
SMALL = {
    "mha_small": Eagle3Config(
        name="mha_small", attn_kind=MHA, hidden=160, intermediate=344,
        draft_vocab=1000, target_vocab=3000, n_heads=6, n_kv_heads=2, head_dim=32,
        rope_theta=10000.0, batch=5, ctx=(0, 150), gamma=3, d2t_kind="sorted_map",
        paging="shuffled", gain_std=0.1),
    "mha_small_b40": Eagle3Config(
        name="mha_small_b40", attn_kind=MHA, hidden=192, intermediate=400,
        draft_vocab=2000, target_vocab=2000, n_heads=4, n_kv_heads=1, head_dim=64,
        rope_theta=500000.0, batch=40, ctx=(1, 300), gamma=2, d2t_kind="zero",
        paging="shuffled", gain_std=0.1),
    "mla_small": Eagle3Config(
        name="mla_small", attn_kind=MLA, hidden=256, intermediate=400,
        draft_vocab=1500, target_vocab=2500, n_heads=16, q_lora_rank=96,
        kv_lora_rank=512, qk_nope_dim=128, qk_rope_dim=64, v_head_dim=128,
        rope_theta=10000.0, yarn_factor=40.0, yarn_orig_max_pos=64.0,
        batch=5, ctx=(0, 200), gamma=3, d2t_kind="sorted_map", paging="shuffled",
        gain_std=0.1),
    "mla_small_b48": Eagle3Config(
        name="mla_small_b48", attn_kind=MLA, hidden=128, intermediate=288,
        draft_vocab=1200, target_vocab=1200, n_heads=32, q_lora_rank=64,
        kv_lora_rank=512, qk_nope_dim=128, qk_rope_dim=64, v_head_dim=128,
        rope_theta=10000.0, yarn_factor=4.0, yarn_orig_max_pos=128.0,
        batch=48, ctx=(1, 260), gamma=2, d2t_kind="zero", paging="shuffled",
        gain_std=0.1),
    # large-batch tile shapes (batch > 64 and > 128 rows per GEMM)
    "mha_small_b100": Eagle3Config(
        name="mha_small_b100", attn_kind=MHA, hidden=160, intermediate=344,
        draft_vocab=1000, target_vocab=3000, n_heads=6, n_kv_heads=2, head_dim=32,
        rope_theta=10000.0, batch=100, ctx=(0, 90), gamma=2, d2t_kind="sorted_map",
        paging="shuffled", gain_std=0.1),
    "mla_small_b200": Eagle3Config(
        name="mla_small_b200", attn_kind=MLA, hidden=128, intermediate=288,
        draft_vocab=1200, target_vocab=1200, n_heads=16, q_lora_rank=64,
        kv_lora_rank=512, qk_nope_dim=128, qk_rope_dim=64, v_head_dim=128,
        rope_theta=10000.0, yarn_factor=4.0, yarn_orig_max_pos=128.0,
        batch=200, ctx=(1, 70), gamma=2, d2t_kind="zero", paging="shuffled",
        gain_std=0.1),
    # a head fusing two target layers (fc 2H -> H) that scores through its
    # target's lm_head (no d2t, draft vocabulary = target vocabulary)
    "mha_small_aux2_tgt_head": Eagle3Config(
        name="mha_small_aux2_tgt_head", attn_kind=MHA, hidden=160, num_aux=2, intermediate=344,
        draft_vocab=3000, target_vocab=3000, n_heads=6, n_kv_heads=2, head_dim=32,
        rope_theta=10000.0, batch=6, ctx=(0, 150), gamma=3, d2t_kind="none",
        paging="shuffled", gain_std=0.1, aux_scales=(1.0, 0.5)),
}

# YaRN with beta_fast = beta_slow = 1 (a draft may override the target's
# beta_fast of 32 with 1): the ramp spans one pair at the original context 4096
SMALL["mla_small_beta1"] = SMALL["mla_small"].replace(name="mla_small_beta1", yarn_beta_fast=1.0,
                                                      yarn_orig_max_pos=4096.0)
# more rows than one 256-row GEMM block: two row blocks and two candidate blocks
SMALL["mla_small_b300"] = SMALL["mla_small_b200"].replace(name="mla_small_b300", batch=300, ctx=(1, 40))
# a gate/up GEMM of 132 column blocks of 256 (fewer than the CUs) and 64
# k-tiles at 160 and 100 rows: the large-batch GEMM's stream-K schedule
# (33 units per workgroup, three partial slots)
SMALL["mla_small_b160_wide_mlp"] = SMALL["mla_small_b200"].replace(
    name="mla_small_b160_wide_mlp", hidden=2048, intermediate=16896, batch=160, ctx=(1, 40))
# 260 (row, kv head) pairs: one 8-wave attention block per pair, no key split
SMALL["mha_small_b130"] = SMALL["mha_small_b100"].replace(name="mha_small_b130", batch=130, ctx=(0, 200))
# the same path at head_dim 64 (256 pairs, GQA groups of 2)
SMALL["mha_small_hd64_b128"] = SMALL["mha_small_b40"].replace(name="mha_small_hd64_b128", n_kv_heads=2,
                                                               batch=128, ctx=(0, 300))
SMALL["mha_small_b100_wide_mlp"] = SMALL["mha_small_b100"].replace(
    name="mha_small_b100_wide_mlp", hidden=2048, intermediate=16896, ctx=(0, 40))

# Quantized heads (weight-only FP8 / NVFP4 GEMM weights).  NVFP4 needs every
# GEMM's input width to be a multiple of 16, hence the adjusted MLP widths.
SMALL.update({
    "mha_small_fp8": SMALL["mha_small"].replace(name="mha_small_fp8", weight_format="fp8"),
    "mla_small_fp8": SMALL["mla_small"].replace(name="mla_small_fp8", weight_format="fp8"),
    "mha_small_b40_nvfp4": SMALL["mha_small_b40"].replace(name="mha_small_b40_nvfp4", weight_format="nvfp4"),
    "mla_small_b48_nvfp4": SMALL["mla_small_b48"].replace(name="mla_small_b48_nvfp4", weight_format="nvfp4"),
    "mha_small_nvfp4": SMALL["mha_small"].replace(name="mha_small_nvfp4", intermediate=352,
                                                  weight_format="nvfp4"),
    "mha_small_b100_fp8": SMALL["mha_small_b100"].replace(name="mha_small_b100_fp8", weight_format="fp8"),
    "mla_small_b200_nvfp4": SMALL["mla_small_b200"].replace(name="mla_small_b200_nvfp4", weight_format="nvfp4"),
})

# The Llama-3 GQA and DeepseekV3 MLA batch-16 workloads with quantized heads.
QUANTIZED = {
    c.name + "_" + f: c.replace(name=c.name + "_" + f, weight_format=f)
    for c in (CONFIGS[1], CONFIGS[2]) for f in ("fp8", "nvfp4")
}


def get_config(key) -> Eagle3Config:
    """Config by 0-based index into CONFIGS, by name, or by SMALL key."""
    if isinstance(key, int):
        return CONFIGS[key]
    for c in CONFIGS:
        if c.name == key:
            return c
    if key in SMALL:
        return SMALL[key]
    if key in QUANTIZED:
        return QUANTIZED[key]
    raise KeyError(key)
