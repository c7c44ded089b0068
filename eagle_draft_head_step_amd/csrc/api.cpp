// Host side of the C ABI: argument validation, the per-call plan (GEMM split
// factors, attention split-KV, workspace carving) and the kernel sequence of
// one draft step.  No allocation, no synchronisation: every call only
// enqueues on the caller's stream.
#include <math.h>

#include <cmath>
#include <string.h>

#include <algorithm>
#include <vector>

#include "../../include/eagle3.h"
#include "internal.h"

using namespace e3;

namespace {

constexpr size_t ALIGN = 256;
inline size_t align_up(size_t x) { return (x + ALIGN - 1) / ALIGN * ALIGN; }
inline int cdiv(int a, int b) { return (a + b - 1) / b; }
inline int64_t cdiv64(int64_t a, int64_t b) { return (a + b - 1) / b; }

bool is_mla(const eagle3_config* c) { return c->attn_kind == EAGLE3_ATTN_MLA; }
int attn_out_dim(const eagle3_config* c) {
  return is_mla(c) ? c->n_heads * c->v_head_dim : c->n_heads * c->head_dim;
}

// ------------------------------------------------------------------ validation
eagle3_status check_config(const eagle3_config* c) {
  if (!c) return EAGLE3_ERR_INVALID_ARG;
  if (c->hidden <= 0 || c->num_aux <= 0 || c->intermediate <= 0 || c->draft_vocab <= 0 ||
      c->target_vocab <= 0 || c->n_heads <= 0 || c->page_size <= 0 || !(c->rms_eps >= 0.f) ||
      !(c->rope_theta > 0.f))
    return EAGLE3_ERR_INVALID_ARG;
  if (c->fc_in_features != c->num_aux * c->hidden) return EAGLE3_ERR_SHAPE;
  if (c->draft_vocab > c->target_vocab) return EAGLE3_ERR_INVALID_ARG;
  if (c->hidden % 8 || c->intermediate % 8 || c->hidden > 16384) return EAGLE3_ERR_UNSUPPORTED;
  if (c->attn_kind == EAGLE3_ATTN_MHA) {
    if (c->n_kv_heads <= 0 || c->head_dim <= 0) return EAGLE3_ERR_INVALID_ARG;
    if (c->n_heads % c->n_kv_heads) return EAGLE3_ERR_SHAPE;
    if (c->n_heads / c->n_kv_heads > 16) return EAGLE3_ERR_UNSUPPORTED;
    if (c->head_dim != 32 && c->head_dim != 64 && c->head_dim != 128) return EAGLE3_ERR_UNSUPPORTED;
    if (c->page_size % 16) return EAGLE3_ERR_UNSUPPORTED;   // 16-key attention tiles stay in a page
  } else if (c->attn_kind == EAGLE3_ATTN_MLA) {
    if (c->q_lora_rank <= 0 || c->kv_lora_rank <= 0 || c->qk_nope_dim <= 0 ||
        c->qk_rope_dim <= 0 || c->v_head_dim <= 0)
      return EAGLE3_ERR_INVALID_ARG;
    // the head's rope is YaRN-scaled: no scaling parameters, no MLA head
    if (!(c->yarn_factor > 0.f) || !(c->yarn_orig_max_pos > 0.f) || !(c->yarn_beta_slow > 0.f) ||
        !(c->yarn_beta_fast >= c->yarn_beta_slow) || !(c->rope_theta > 1.f))
      return EAGLE3_ERR_UNSUPPORTED;
    if (c->page_size % 32) return EAGLE3_ERR_UNSUPPORTED;   // 32-key attention tiles stay in a page
    if (c->kv_lora_rank != 512 || c->qk_rope_dim != 64 || c->n_heads % 16 ||
        c->q_lora_rank % 8 || c->q_lora_rank > 4096 || c->qk_nope_dim % 8 || c->v_head_dim % 8)
      return EAGLE3_ERR_UNSUPPORTED;
  } else {
    return EAGLE3_ERR_INVALID_ARG;
  }
  // the cache's dtype must match the bf16 q/k/v of the head's attention
  if (c->cache_dtype != EAGLE3_CACHE_BF16) return EAGLE3_ERR_UNSUPPORTED;
  if (c->weight_format < EAGLE3_WEIGHTS_BF16 || c->weight_format > EAGLE3_WEIGHTS_NVFP4)
    return EAGLE3_ERR_INVALID_ARG;
  if (c->weight_format == EAGLE3_WEIGHTS_NVFP4) {
    // every GEMM input width a whole number of 16-element scale blocks
    const int ks[] = {c->hidden, c->intermediate, attn_out_dim(c), is_mla(c) ? c->q_lora_rank : 16,
                      is_mla(c) ? c->kv_lora_rank : 16};
    for (int k : ks)
      if (k % 16) return EAGLE3_ERR_UNSUPPORTED;
  }
  return EAGLE3_OK;
}

// ------------------------------------------------------------------ packed weights
struct PackedMat {
  size_t off;     // bytes into the packed buffer
  int N, K, NT, KT, batch;
  int64_t bs;     // batch stride in uint4
  int wq;         // EAGLE3_WEIGHTS_* of the packed tiles
  size_t rs_off;  // quantized: fp32 row scales (NT*16)
  size_t bs_off;  // NVFP4: block-scale words (32 per tile)
};
struct PackedLayout {
  PackedMat fc, qkv, qa_kva, qb, uk, uv, o, gu, down, lm;
  size_t total;
};

PackedMat make_mat(size_t& off, int N, int K, int batch = 1, int wq = EAGLE3_WEIGHTS_BF16) {
  PackedMat m;
  memset(&m, 0, sizeof(m));
  const int kpw = wq_ktiles(wq);
  m.off = off;
  m.N = N; m.K = K; m.NT = cdiv(N, 16); m.KT = cdiv(cdiv(K, 32), kpw) * kpw; m.batch = batch;
  m.wq = wq;
  m.bs = (int64_t)m.NT * (m.KT / kpw) * 64;
  off = align_up(off + (size_t)m.bs * 16 * batch);
  if (wq_scaled(wq)) {
    m.rs_off = off;
    off = align_up(off + (size_t)m.NT * 16 * sizeof(float));
  }
  if (wq == EAGLE3_WEIGHTS_NVFP4) {
    m.bs_off = off;
    off = align_up(off + (size_t)m.NT * (m.KT / 4) * 32 * sizeof(uint32_t));
  }
  return m;
}

PackedLayout packed_layout(const eagle3_config* c) {
  PackedLayout L;
  memset(&L, 0, sizeof(L));
  size_t off = 0;
  const int H = c->hidden, wq = c->weight_format;
  L.fc = make_mat(off, H, c->num_aux * H, 1, wq);
  if (is_mla(c)) {
    L.qa_kva = make_mat(off, c->q_lora_rank + c->kv_lora_rank + c->qk_rope_dim, 2 * H, 1, wq);
    L.qb = make_mat(off, c->n_heads * (c->qk_nope_dim + c->qk_rope_dim), c->q_lora_rank, 1, wq);
    // the per-head absorbed halves of kv_b are widened to bf16 at packing
    L.uk = make_mat(off, c->kv_lora_rank, c->qk_nope_dim, c->n_heads);
    L.uv = make_mat(off, c->v_head_dim, c->kv_lora_rank, c->n_heads);
  } else {
    L.qkv = make_mat(off, (c->n_heads + 2 * c->n_kv_heads) * c->head_dim, 2 * H, 1, wq);
  }
  L.o = make_mat(off, H, attn_out_dim(c), 1, wq);
  // a bf16 head's MLP matrices are packed as f16 (its fp32 activations then
  // go to the matrix cores as one f16 operand)
  const int wmlp = wq == EAGLE3_WEIGHTS_BF16 ? WQ_F16 : wq;
  L.gu = make_mat(off, 2 * c->intermediate, H, 1, wmlp);
  L.down = make_mat(off, H, c->intermediate, 1, wmlp);
  L.lm = make_mat(off, c->draft_vocab, H, 1, wq);
  L.total = off;
  return L;
}

// ------------------------------------------------------------------ plan
struct GemmPlan {
  GemmShape shape;
  int splitk, kps, mblocks, mrows;   // rows per M block (<= 256; 128 for large-batch NVFP4)
  int blocks_x;
  bool big;                          // the LDS-staged large-batch kernel
  int streamk;                       // big: stream-K workgroups (splitk = partial slots), or 0
};

// Launch shape per batch size, from a sweep of the streaming GEMM on MI355X
// (fp32 activations cost a second MFMA and twice the activation bytes).
// 17..32 rows: n-tiles per wave and k-tiles per stage of the two instances.
// (Llama-3 GQA shape, batch 32: fp32-activation shapes 2x1x4, 2x1x8 and
// 2x2x8 measured 4-8% slower per step; bf16 2x1x4 equal, 2x2x8 2% slower.)
#ifndef E3_M32_AF32_NTW
#define E3_M32_AF32_NTW 2
#endif
#ifndef E3_M32_AF32_KC
#define E3_M32_AF32_KC 4
#endif
#ifndef E3_M32_BF16_NTW
#define E3_M32_BF16_NTW 1
#endif
#ifndef E3_M32_BF16_KC
#define E3_M32_BF16_KC 8
#endif

#ifndef E3_M16_BF16_NTW
#define E3_M16_BF16_NTW 1
#endif
#ifndef E3_M16_BF16_KC
#define E3_M16_BF16_KC 8
#endif
#ifndef E3_M16_AF32_NTW
#define E3_M16_AF32_NTW 1
#endif

GemmShape shape_for_m(int M, bool af32) {
  if (M <= 16)
    return af32 ? GemmShape{1, E3_M16_AF32_NTW, 4} : GemmShape{1, E3_M16_BF16_NTW, E3_M16_BF16_KC};
  if (M <= 32)
    return af32 ? GemmShape{2, E3_M32_AF32_NTW, E3_M32_AF32_KC} : GemmShape{2, E3_M32_BF16_NTW, E3_M32_BF16_KC};
  if (M <= 64) return GemmShape{4, 1, 4};
  // large batch: bf16 rows take 128 x 64 wave tiles (one wave per SIMD);
  // fp32 (hi + lo) rows and 256-row blocks take a 2 x 2 wave grid with two
  // waves per SIMD
  if (M <= 128) return af32 ? GemmShape{8, 4, 1, 2} : GemmShape{8, 4, 2, 1};
  return GemmShape{16, 4, 1, 2};
}

// Least (column block, k-tile) units per stream-K workgroup of the large-batch
// kernel.  (DeepseekV3 shapes at batch 128 and 256: gate/up, 126 units per
// workgroup, gains; q_b, 18 units in four partial slots instead of two, loses
// more to the partial traffic than the balance saves.)
#ifndef E3_STREAMK_MIN_UNITS
#define E3_STREAMK_MIN_UNITS 32
#endif
constexpr int kStreamKMinUnits = E3_STREAMK_MIN_UNITS;

// Small-batch split-K GEMM (17..64 rows): workgroups the splits aim at.
#ifndef E3_GEMM_SMALL_TARGET_BLOCKS
#define E3_GEMM_SMALL_TARGET_BLOCKS 512
#endif
constexpr int kGemmSmallTargetBlocks = E3_GEMM_SMALL_TARGET_BLOCKS;

// split_ok: whether the consumer reduces fp32 partials (else one split).
// m16_target: blocks the split aims at for a one-m-tile (<= 16 rows) plan.
GemmPlan plan_gemm(const PackedMat& w, int M, bool split_ok, bool af32, int m16_target = 1024) {
  GemmPlan g;
  // NVFP4 stages span 4 k-tiles, whose 256-row activation stage would not fit
  // in registers: large batches run as blocks of 128 rows
  const int mstep = (w.wq == EAGLE3_WEIGHTS_NVFP4 && M > 128) ? 128 : 256;
  g.mrows = std::min(M, mstep);
  g.mblocks = cdiv(M, mstep);
  g.shape = shape_for_m(g.mrows, af32);
  if (wq_scaled(w.wq)) {
    // a stage holds whole weight words of the format (2 or 4 k-tiles); the
    // large-batch tiles with such stages take one wave per SIMD (the 2 x 2
    // wave grid would spill)
    // (small batches: the fastest shapes of a sweep over the Llama-3 GQA and
    // DeepseekV3 projections on MI355X; NVFP4 prefers more n-tiles per wave)
    const int kpw = wq_ktiles(w.wq);
    const bool nv = w.wq == EAGLE3_WEIGHTS_NVFP4;
    if (g.mrows > 128)
      g.shape = GemmShape{16, 2, kpw, 1};
    else if (g.mrows > 64)
      g.shape = (!nv && af32) ? GemmShape{8, 4, 2, 2} : GemmShape{8, 4, kpw, 1};
    else if (g.mrows > 32)
      g.shape = GemmShape{4, 1, 4, 1};
    else if (g.mrows > 16)
      g.shape = nv ? (af32 ? GemmShape{2, 4, 8, 1} : GemmShape{2, 2, 8, 1})
                   : (af32 ? GemmShape{2, 2, 8, 1} : GemmShape{2, 1, 8, 1});
    else
      g.shape = nv ? (af32 ? GemmShape{1, 4, 4, 1} : GemmShape{1, 2, 8, 1})
                   : (af32 ? GemmShape{1, 1, 4, 1} : GemmShape{1, 1, 8, 1});
  }
  g.blocks_x = cdiv(w.NT, (4 / g.shape.wm) * g.shape.ntw);
  // 65..256 rows of bf16 weights with whole k-tiles: both operands through
  // LDS, in blocks of 128 or 256 rows (fp32 activations then come as bf16
  // hi + lo planes from their producer)
  // (a batch of matrices -- the MLA absorb halves -- writes bf16, unsplit)
  g.big = (w.wq == EAGLE3_WEIGHTS_BF16 || w.wq == WQ_F16) && (w.batch == 1 || !split_ok) && g.mrows > 64 &&
          w.K % 32 == 0;
  g.streamk = 0;
  if (g.big) {
    // (split-K: as many splits as keep every block in one round of 256 CUs,
    // at most 16 and at least 4 k-tiles per split; a second, partial round
    // measured slower on the DeepseekV3 projections at batch 256)
    g.blocks_x = cdiv(w.NT, 16);
    int sk = split_ok ? std::max(1, std::min(16, 256 / g.blocks_x)) : 1;
    sk = std::min(sk, std::max(1, w.KT / 4));
    g.kps = cdiv(w.KT, sk);
    g.splitk = cdiv(w.KT, g.kps);
    // Stream-K when the split-K grid leaves over a fifth of the CUs idle: 256
    // workgroups share all (column block, k-tile) units equally, given at
    // least kStreamKMinUnits each and no more partial slots than
    // max(4, the split count)
    const int64_t units = (int64_t)g.blocks_x * w.KT;
    if (split_ok && g.blocks_x * g.splitk < 205 && units >= 256 * kStreamKMinUnits) {
      const int slots = gemm_big_streamk_slots(w.NT, w.KT, 256);
      if (slots >= 1 && slots <= std::max(4, g.splitk)) {
        g.streamk = 256;
        g.splitk = slots;
        g.kps = w.KT;
      }
    }
    return g;
  }
  int splitk = 1;
  if (split_ok) {
    // enough blocks to keep every CU streaming: two per CU for the small-batch
    // shapes, one per CU for the one-wave-per-SIMD large tiles, four for the
    // two-wave grid; large batches cap the split, since each split writes
    // and reads back B x N fp32 partials
    const bool big = g.mrows > 64;
    // (batch <= 16: a block of the one-m-tile shapes keeps few bytes in
    // flight, so four blocks per CU; measured on the DeepseekV3 head at batch
    // 16: gate/up, down, o and fc gain, 1.4% per step, and quantized heads
    // likewise.  At larger batches the extra fp32 partials of the wide MLP
    // GEMMs cost more: the Llama-3 head at batch 32 loses 3%.)
    const bool m16 = g.mrows <= 16;
    const int target = !big ? (m16 ? m16_target : kGemmSmallTargetBlocks) : (g.shape.wm == 2 ? 1024 : 256);
    const int blocks = g.blocks_x * w.batch;
    splitk = big ? cdiv(target, std::max(1, blocks)) : std::max(1, (target + blocks / 2) / std::max(1, blocks));
    // at least two stages of KC k-tiles per split; four at batch <= 16, where
    // the split target is higher (the DeepseekV3 q_b, K = 1536, measured 1.2 us
    // slower in three splits of two stages than in one)
    splitk = std::min(splitk, std::max(1, w.KT / ((m16 && !big ? 4 : 2) * g.shape.kc)));
    splitk = std::min(splitk, big ? 8 : 16);
  }
  // batch <= 16, bf16: when the split grid outgrows one round of the 8-k-tile
  // stage's residency (3 blocks per CU), 4-k-tile stages (6 per CU) keep it to
  // one round (DeepseekV3 batch 16: o 45.9 -> 41.3 us, fc 56.2 -> 51.5 us;
  // unsplit and smaller grids measured slower with them)
  if (split_ok && g.mrows <= 16 && !af32 && (w.wq == EAGLE3_WEIGHTS_BF16 || w.wq == WQ_F16) && g.shape.kc == 8 &&
      g.blocks_x * w.batch * splitk > 3 * 256)
    g.shape.kc = 4;
  int kps = cdiv(w.KT, splitk);
  kps = cdiv(kps, g.shape.kc) * g.shape.kc;
  g.kps = kps;
  g.splitk = cdiv(w.KT, kps);
  return g;
}

struct AttnPlan { int nsplit, chunk, nblocks, nw; };

// MHA split-KV attention: workgroups the key splits aim at.  (Llama-3 GQA
// shape, batch 32: one split per (row, kv head) -- 256 workgroups, no combine
// -- and four splits both measured 2-3% slower per step than two.)
#ifndef E3_MHA_ATTN_TARGET_BLOCKS
#define E3_MHA_ATTN_TARGET_BLOCKS 512
#endif
constexpr int kMhaAttnTargetBlocks = E3_MHA_ATTN_TARGET_BLOCKS;
// (row, kv head) pairs from which one 8-wave block per pair takes a whole row.
#ifndef E3_MHA_ATTN_WHOLE_ROW_PAIRS
#define E3_MHA_ATTN_WHOLE_ROW_PAIRS 256
#endif
constexpr int kMhaAttnWholeRowPairs = E3_MHA_ATTN_WHOLE_ROW_PAIRS;

// MLA: one persistent workgroup per CU shares the batch's 32-key tiles.
constexpr int kMlaAttnBlocks = 256;

AttnPlan plan_attn(const eagle3_config* c, int B, int max_keys) {
  AttnPlan a;
  a.nblocks = 0;
  a.nw = 4;
  if (is_mla(c)) {
    a.nblocks = std::max(1, std::min(kMlaAttnBlocks, B * cdiv(max_keys, 32)));
    a.nsplit = 0;
    a.chunk = 0;
    return a;
  }
  const int per = B * c->n_kv_heads;
  if (per >= kMhaAttnWholeRowPairs) {
    // every CU gets a (row, kv head): one 8-wave block per pair takes the
    // whole row and writes the output, no split and no combine
    a.nw = 8;
    a.nsplit = 1;
    a.chunk = cdiv(std::max(1, max_keys), 128) * 128;
    return a;
  }
  // blocks of 4 waves x 16-key tiles: chunks of whole 64-key rounds; two
  // blocks fit a CU, so aim at one round of 2 x 256 resident blocks
  int ns = std::max(1, (kMhaAttnTargetBlocks + per / 2) / per);
  ns = std::min(ns, std::max(1, cdiv(max_keys, 64)));
  a.chunk = cdiv(cdiv(max_keys, ns), 64) * 64;
  a.nsplit = cdiv(max_keys, a.chunk);
  return a;
}

struct Plan {
  PackedLayout pk;
  GemmPlan fc, qkv, qa_kva, qb, uk, uv, o, gu, down, lm;
  AttnPlan attn;
  // workspace offsets (bytes)
  size_t part, cand, g, h1, hbuf, x, u, f, act, q, attn_out, apo, aml, sched, qa, qnope, qpe, qlat, olat;
  size_t u16, act16;                // f16 u / act for the MLP GEMMs of f16 tiles
  bool mlp_f16;                     // the MLP GEMMs take f16 activations (u16, act16)
  bool q_absorb;                    // MLA: q epilogue and W_UK absorption in one kernel
  bool uv_fused;                    // MLA: merge of split rows and W_UV in one kernel
  size_t total;
  int sched_stride;                 // ints per step schedule (MLA)
};

size_t part_bytes(const GemmPlan& g, const PackedMat& w, int M) {
  return (size_t)g.splitk * M * w.N * w.batch * sizeof(float);
}

// nsteps: draft steps whose attention schedules the workspace holds (MLA).
Plan make_plan(const eagle3_config* c, int B, int max_keys, int nsteps) {
  Plan p;
  memset(&p, 0, sizeof(p));
  p.pk = packed_layout(c);
  const PackedLayout& L = p.pk;
  const int H = c->hidden, I = c->intermediate;
  // bf16 fc, o and down up to 16 rows: splits aimed at 448 blocks (four per
  // 7168-column DeepseekV3 projection instead of nine): the residual-norm and
  // embedding kernels then read fewer fp32 partials per row, which outweighs
  // the GEMMs' shallower grids (DeepseekV3 batch 16 on MI355X: 1.742 -> 1.726
  // ms per chain; five or seven splits measured 1.748 / 1.762, three 1.776)
  const int narrow_target = 448;
  p.fc = plan_gemm(L.fc, B, true, false, L.fc.wq == EAGLE3_WEIGHTS_BF16 ? narrow_target : 1024);
  size_t part = part_bytes(p.fc, L.fc, B);
  if (is_mla(c)) {
    p.qa_kva = plan_gemm(L.qa_kva, B, true, false);
    p.qb = plan_gemm(L.qb, B, true, false);
    p.uk = plan_gemm(L.uk, B, false, false);
    // up to 64 rows the absorption runs inside the q epilogue's launch
    p.q_absorb = !p.uk.big && c->qk_nope_dim == 128 && c->kv_lora_rank == 512;
    p.uv = plan_gemm(L.uv, B, false, false);
    // up to 64 rows W_UV runs inside the attention's merge launch
    p.uv_fused = !p.uv.big && c->v_head_dim == 128 && c->kv_lora_rank == 512;
    part = std::max(part, part_bytes(p.qa_kva, L.qa_kva, B));
    part = std::max(part, part_bytes(p.qb, L.qb, B));
  } else {
    p.qkv = plan_gemm(L.qkv, B, true, false);
    part = std::max(part, part_bytes(p.qkv, L.qkv, B));
  }
  p.o = plan_gemm(L.o, B, true, false, L.o.wq == EAGLE3_WEIGHTS_BF16 ? narrow_target : 1024);
  // f16 MLP tiles (a bf16 head) take their activations as one f16 operand,
  // which the residual-norm and SiLU kernels write; quantized MLPs take fp32
  p.mlp_f16 = L.gu.wq == WQ_F16 && L.down.wq == WQ_F16;
  p.gu = plan_gemm(L.gu, B, true, !p.mlp_f16);
  p.down = plan_gemm(L.down, B, true, !p.mlp_f16, p.mlp_f16 ? narrow_target : 1024);
  p.lm = plan_gemm(L.lm, B, false, false);
  // bf16 lm_head up to 16 rows (unsplit: the top-1 epilogue) whose one-n-tile
  // grid would take more than one round at three blocks per CU: four n-tiles
  // per wave in 4-k-tile stages, so the grid (505 blocks for a 129280-row
  // vocabulary) is one round at two blocks per CU with more weight bytes in
  // flight per wave; one n-tile in 8-k-tile stages left 2.6 rounds (DeepseekV3
  // batch 16 on MI355X: 3 us less per step).  A small vocabulary keeps the
  // wider grid (a 4096-row one measured 2% slower per step in 16 blocks).
  if (L.lm.wq == EAGLE3_WEIGHTS_BF16 && !p.lm.big && p.lm.mblocks == 1 && p.lm.mrows <= 16 &&
      p.lm.blocks_x > 3 * 256) {
    p.lm.shape = GemmShape{1, 4, 4, 1};
    p.lm.blocks_x = cdiv(L.lm.NT, 16);
    p.lm.kps = cdiv(L.lm.KT, 4) * 4;
    p.lm.splitk = 1;
  }
  part = std::max(part, part_bytes(p.o, L.o, B));
  part = std::max(part, part_bytes(p.gu, L.gu, B));
  part = std::max(part, part_bytes(p.down, L.down, B));
  p.attn = plan_attn(c, B, max_keys);

  size_t off = 0;
  auto take = [&](size_t bytes) { size_t o = off; off = align_up(off + bytes); return o; };
  p.part = take(part);
  p.cand = take((size_t)p.lm.blocks_x * B * sizeof(uint64_t));
  p.g = take((size_t)B * H * 4);
  p.h1 = take((size_t)B * H * 4);
  p.hbuf = take((size_t)B * H * 4);
  p.x = take((size_t)B * 2 * H * 2);
  p.u = take(p.mlp_f16 ? 0 : (size_t)B * H * 4);        // fp32 MLP inputs (quantized heads)
  p.f = take((size_t)B * H * 2);
  p.act = take(p.mlp_f16 ? 0 : (size_t)B * I * 4);
  p.u16 = p.mlp_f16 ? take((size_t)B * H * 2) : 0;
  p.act16 = p.mlp_f16 ? take((size_t)B * I * 2) : 0;
  p.attn_out = take((size_t)B * attn_out_dim(c) * 2);
  if (is_mla(c)) {
    const int nh = c->n_heads, r = c->kv_lora_rank;
    p.qa = take((size_t)B * c->q_lora_rank * 2);
    p.qnope = take(p.q_absorb ? 0 : (size_t)B * nh * c->qk_nope_dim * 2);
    p.qpe = take((size_t)B * nh * c->qk_rope_dim * 2);
    p.qlat = take((size_t)B * nh * r * 2);
    p.olat = take((size_t)B * nh * r * 2);
    p.apo = take((size_t)2 * p.attn.nblocks * nh * r * 2);
    p.aml = take((size_t)2 * p.attn.nblocks * nh * 2 * 4);
    p.sched_stride = 3 * B + 2 * p.attn.nblocks + 2;
    p.sched = take((size_t)nsteps * p.sched_stride * 4);
  } else {
    p.q = take((size_t)B * c->n_heads * c->head_dim * 4);
    p.apo = take((size_t)B * c->n_heads * p.attn.nsplit * c->head_dim * 4);
    p.aml = take((size_t)B * c->n_heads * p.attn.nsplit * 2 * 4);
  }
  p.total = off;
  return p;
}

void fill_rope(const eagle3_config* c, RopeTable& t) {
  memset(&t, 0, sizeof(t));
  if (is_mla(c)) {
    // YaRN NTK-by-parts as the DeepSeek YaRN rotary embedding defines it:
    // the pair index at which a pair makes b turns over the original context
    // L0 is d ln(L0 / (2 pi b)) / (2 ln theta); pairs up to the floor of that
    // index for beta_fast keep theta_i, pairs from the ceil of it for
    // beta_slow take theta_i / s, and the weight of theta_i / s ramps
    // linearly in the pair index in between (a step when the two meet).
    const int d = c->qk_rope_dim;
    t.npairs = d / 2;
    const double s = c->yarn_factor, L0 = c->yarn_orig_max_pos, base = c->rope_theta;
    auto pair_at = [&](double turns) {
      return d * log(L0 / (2.0 * M_PI * turns)) / (2.0 * log(base));
    };
    auto clampi = [&](double v) { return std::min(std::max(v, 0.0), (double)(d - 1)); };
    const double lo = clampi(floor(pair_at(c->yarn_beta_fast)));
    const double hi = clampi(ceil(pair_at(c->yarn_beta_slow)));
    for (int i = 0; i < t.npairs; ++i) {
      const double th = pow(base, -2.0 * i / d);
      double w;
      if (hi > lo) {
        w = (i - lo) / (hi - lo);
        w = w < 0.0 ? 0.0 : (w > 1.0 ? 1.0 : w);
      } else {
        w = i > lo ? 1.0 : 0.0;
      }
      t.inv_freq[i] = (1.0 - w) * th + w * th / s;
    }
  } else {
    const int d = c->head_dim;
    t.npairs = d / 2;
    for (int i = 0; i < t.npairs; ++i) t.inv_freq[i] = pow((double)c->rope_theta, -2.0 * i / d);
  }
}

// ------------------------------------------------------------------ launches
eagle3_launch_hook g_hook = nullptr;
void* g_hook_user = nullptr;

// Brackets one launch (or fused pair) with the profiling hook, if set.
struct HookScope {
  const char* name;
  hipStream_t st;
  HookScope(const char* n, hipStream_t s) : name(n), st(s) {
    if (g_hook) g_hook(name, 0, reinterpret_cast<eagle3_stream_t>(st), g_hook_user);
  }
  ~HookScope() {
    if (g_hook) g_hook(name, 1, reinterpret_cast<eagle3_stream_t>(st), g_hook_user);
  }
};

#define E3_HIP(x)                                   \
  do {                                              \
    if ((x) != hipSuccess) return EAGLE3_ERR_HIP;   \
  } while (0)

template <typename T>
T* ws_at(void* ws, size_t off) { return reinterpret_cast<T*>(static_cast<char*>(ws) + off); }

// C (or candidates) of an A [M, K] x packed W GEMM, looping over blocks of g.mrows rows.
eagle3_status run_gemm(const GemmPlan& g, const PackedMat& w, const void* packed, const void* A,
                       bool a_f32, int64_t lda, int64_t a_bs, int M, int mode, void* C, int64_t ldc,
                       int64_t c_bs, uint64_t* cand, float* logits, hipStream_t st) {
  for (int mb = 0; mb < g.mblocks; ++mb) {
    const int m0 = mb * g.mrows;
    const int b0 = m0 / 256 * 256;                 // the 256-row block of the candidates
    GemmParams p;
    memset(&p, 0, sizeof(p));
    // A: fp32, or 16-bit (bf16, or f16 for f16 weights in the large-batch kernel)
    p.A = a_f32 ? static_cast<const void*>(static_cast<const float*>(A) + (int64_t)m0 * lda)
                : static_cast<const void*>(static_cast<const bf16_t*>(A) + (int64_t)m0 * lda);
    p.a_f32 = a_f32 ? 1 : 0;
    p.lda = lda; p.a_bs = a_bs;
    p.W = reinterpret_cast<const uint4*>(static_cast<const char*>(packed) + w.off);
    p.w_bs = w.bs;
    p.wq = w.wq;
    if (wq_scaled(w.wq))
      p.rscale = reinterpret_cast<const float*>(static_cast<const char*>(packed) + w.rs_off);
    if (w.wq == EAGLE3_WEIGHTS_NVFP4)
      p.bscale = reinterpret_cast<const uint32_t*>(static_cast<const char*>(packed) + w.bs_off);
    p.M = std::min(g.mrows, M - m0);
    p.N = w.N; p.K = w.K; p.NT = w.NT; p.KT = w.KT;
    p.kps = g.kps; p.splitk = g.splitk; p.streamk = g.streamk;
    p.mode = mode;
    if (mode == GEMM_F32_PARTIAL) {
      p.C = static_cast<float*>(C) + (int64_t)m0 * ldc;
      p.c_ss = (int64_t)M * ldc;     // splits stacked over the full M
    } else if (mode == GEMM_BF16) {
      p.C = static_cast<bf16_t*>(C) + (int64_t)m0 * ldc;
    } else {
      // candidates: [blocks_x, rows] per 256-row block of the batch
      p.cand = cand + (int64_t)g.blocks_x * b0 + (m0 - b0);
      p.cand_ld = std::min(256, M - b0);
      p.logits = logits ? logits + (int64_t)m0 * ldc : nullptr;
    }
    p.ldc = ldc; p.c_bs = c_bs;
    if (g.big) {
      if (!gemm_big_ok(p, w.batch)) return EAGLE3_ERR_HIP;
      E3_HIP(launch_gemm_big(p, w.batch, st));
    } else {
      E3_HIP(launch_gemm(p, g.shape, w.batch, st));
    }
  }
  return EAGLE3_OK;
}

eagle3_status check_args(const eagle3_config* cfg, const eagle3_step_args* a, int nsteps,
                         bool chain) {
  if (!a) return EAGLE3_ERR_INVALID_ARG;
  if (a->batch <= 0 || !a->token_in || !a->k_cache || !a->block_table || !a->ctx_len ||
      !a->token_out || a->max_pages <= 0 || a->max_ctx < 0 || !a->workspace)
    return EAGLE3_ERR_INVALID_ARG;
  if (!is_mla(cfg) && !a->v_cache) return EAGLE3_ERR_INVALID_ARG;
  if (!a->aux && !a->hidden_in) return EAGLE3_ERR_INVALID_ARG;
  if (a->num_pages < 0) return EAGLE3_ERR_INVALID_ARG;
  if (!chain && !a->hidden_out) return EAGLE3_ERR_INVALID_ARG;
  if ((int64_t)a->max_pages * cfg->page_size < (int64_t)a->max_ctx + nsteps)
    return EAGLE3_ERR_INVALID_ARG;
  if (((uintptr_t)a->aux | (uintptr_t)a->k_cache | (uintptr_t)a->v_cache |
       (uintptr_t)a->hidden_in | (uintptr_t)a->hidden_out | (uintptr_t)a->workspace) & 15)
    return EAGLE3_ERR_INVALID_ARG;
  return EAGLE3_OK;
}

// One step.  g source: aux (fc) when use_aux, else h_in.  Tokens read at
// tok_in[b * tok_in_stride]; written at tok_out[b * tok_stride].
// When fuse_prev is set, tok_in / draft_in are where the previous step's top-1
// goes: this step's embedding kernel reduces the candidates the previous
// lm_head left in the workspace, writes that token and embeds it.  When
// final_top1 is clear, this step's own candidates are left for the next step.
eagle3_status run_step(const eagle3_config* c, const eagle3_weights* w, const void* packed,
                       const eagle3_step_args* a, const Plan& p, int step, bool use_aux,
                       const float* h_in, const int32_t* tok_in, int tok_in_stride, bool fuse_prev,
                       int32_t* prev_tok, int32_t* prev_draft, float* h_out, int32_t* tok_out,
                       int32_t* draft_out, int tok_stride, float* logits, bool final_top1,
                       int sched_slot, const int32_t* tok_pos, const int32_t* tok_row,
                       hipStream_t st) {
  const int B = a->batch, H = c->hidden, I = c->intermediate;
  const PackedLayout& L = p.pk;
  void* ws = a->workspace;
  float* part = ws_at<float>(ws, p.part);
  float* g = ws_at<float>(ws, p.g);
  float* h1 = ws_at<float>(ws, p.h1);
  bf16_t* x = ws_at<bf16_t>(ws, p.x);
  float* u = ws_at<float>(ws, p.u);
  bf16_t* f = ws_at<bf16_t>(ws, p.f);
  float* act = ws_at<float>(ws, p.act);
  bf16_t* attn_out = ws_at<bf16_t>(ws, p.attn_out);
  const int aod = attn_out_dim(c);
  eagle3_status s;

  // fused hidden + embedding norms
  EmbedNormArgs en;
  memset(&en, 0, sizeof(en));
  en.tok = tok_in; en.tok_stride = tok_in_stride;
  if (fuse_prev) {
    en.cand = ws_at<uint64_t>(ws, p.cand); en.ncand = p.lm.blocks_x; en.d2t = w->d2t;
    en.top1_out = prev_tok; en.top1_draft = prev_draft; en.top1_stride = tok_in_stride;
  }
  en.embed = static_cast<const bf16_t*>(w->embed);
  if (use_aux) {
    {
      HookScope hs("gemm.fc", st);
      s = run_gemm(p.fc, L.fc, packed, a->aux, false, c->num_aux * H, 0, B,
                   GEMM_F32_PARTIAL, part, H, 0, nullptr, nullptr, st);
    }
    if (s != EAGLE3_OK) return s;
    en.g_part = part; en.g_splits = p.fc.splitk; en.g_ss = (int64_t)B * H;
  } else {
    en.g_in = h_in;
  }
  en.norm_in = static_cast<const bf16_t*>(w->norm_in);
  en.norm_hid = static_cast<const bf16_t*>(w->norm_hid);
  en.g_out = g; en.x = x; en.B = B; en.H = H; en.eps = c->rms_eps;
  {
    HookScope hs("embed_norm", st);
    E3_HIP(launch_embed_norm(en, st));
  }

  RopeTable rope;
  fill_rope(c, rope);

  if (!is_mla(c)) {
    const int nq = c->n_heads, nkv = c->n_kv_heads, hd = c->head_dim;
    const int nqkv = (nq + 2 * nkv) * hd;
    {
      HookScope hs("gemm.qkv", st);
      s = run_gemm(p.qkv, L.qkv, packed, x, false, 2 * H, 0, B, GEMM_F32_PARTIAL, part, nqkv, 0, nullptr,
                 nullptr, st);
    }
    if (s != EAGLE3_OK) return s;
    MhaQkvArgs qa;
    memset(&qa, 0, sizeof(qa));
    qa.part = part; qa.splits = p.qkv.splitk; qa.ss = (int64_t)B * nqkv; qa.ldp = nqkv;
    qa.q = ws_at<float>(ws, p.q);
    qa.k_cache = static_cast<bf16_t*>(a->k_cache); qa.v_cache = static_cast<bf16_t*>(a->v_cache);
    qa.table = a->block_table; qa.max_pages = a->max_pages; qa.ctx_len = a->ctx_len; qa.step = step;
    qa.tok_pos = tok_pos; qa.tok_row = tok_row;
    qa.B = B; qa.nq = nq; qa.nkv = nkv; qa.hd = hd; qa.page_size = c->page_size;
    qa.rope = rope;
    // whole-row attention blocks of a plain step (no per-token positions: each
    // row reads only its own new entry) take the q/k/v epilogue themselves
    const bool fuse_qkv = p.attn.nw == 8 && tok_pos == nullptr;
    if (!fuse_qkv) {
      HookScope hs("mha_qkv_rope_append", st);
      E3_HIP(launch_mha_qkv(qa, st));
    }
    MhaAttnArgs at;
    memset(&at, 0, sizeof(at));
    at.q = qa.q; at.k_cache = qa.k_cache; at.v_cache = qa.v_cache;
    at.table = a->block_table; at.max_pages = a->max_pages; at.ctx_len = a->ctx_len; at.step = step;
    at.tok_pos = tok_pos; at.tok_row = tok_row;
    at.B = B; at.nq = nq; at.nkv = nkv; at.hd = hd; at.page_size = c->page_size;
    at.nsplit = p.attn.nsplit; at.chunk = p.attn.chunk; at.nw = p.attn.nw;
    if (fuse_qkv) {
      at.part = qa.part; at.splits = qa.splits; at.ss = qa.ss; at.ldp = qa.ldp;
      at.k_app = qa.k_cache; at.v_app = qa.v_cache; at.rope = rope;
    }
    at.scale = (float)(1.0 / sqrt((double)hd));
    at.part_o = ws_at<float>(ws, p.apo); at.part_ml = ws_at<float>(ws, p.aml);
    at.out = attn_out;
    {
      HookScope hs("mha_attn", st);
      E3_HIP(launch_mha_attn(at, st));
    }
  } else {
    const int nh = c->n_heads, dn = c->qk_nope_dim, dr = c->qk_rope_dim, dv = c->v_head_dim;
    const int r = c->kv_lora_rank, ql = c->q_lora_rank;
    const int na = ql + r + dr;
    {
      HookScope hs("gemm.qa_kva", st);
      s = run_gemm(p.qa_kva, L.qa_kva, packed, x, false, 2 * H, 0, B, GEMM_F32_PARTIAL, part, na, 0, nullptr,
                 nullptr, st);
    }
    if (s != EAGLE3_OK) return s;
    MlaAArgs ma;
    memset(&ma, 0, sizeof(ma));
    ma.part = part; ma.splits = p.qa_kva.splitk; ma.ss = (int64_t)B * na; ma.ldp = na;
    ma.norm_qa = static_cast<const bf16_t*>(w->norm_qa);
    ma.norm_kv = static_cast<const bf16_t*>(w->norm_kv);
    ma.qa = ws_at<bf16_t>(ws, p.qa);
    ma.cache = static_cast<bf16_t*>(a->k_cache);
    ma.table = a->block_table; ma.max_pages = a->max_pages; ma.ctx_len = a->ctx_len; ma.step = step;
    ma.tok_pos = tok_pos; ma.tok_row = tok_row;
    ma.B = B; ma.q_lora = ql; ma.r = r; ma.dr = dr; ma.page_size = c->page_size; ma.eps = c->rms_eps;
    ma.rope = rope;
    {
      HookScope hs("mla_a_norm_rope_append", st);
      E3_HIP(launch_mla_a(ma, st));
    }
    const int nqb = nh * (dn + dr);
    {
      HookScope hs("gemm.qb", st);
      s = run_gemm(p.qb, L.qb, packed, ma.qa, false, ql, 0, B, GEMM_F32_PARTIAL, part, nqb, 0, nullptr,
                 nullptr, st);
    }
    if (s != EAGLE3_OK) return s;
    MlaQArgs mq;
    memset(&mq, 0, sizeof(mq));
    mq.part = part; mq.splits = p.qb.splitk; mq.ss = (int64_t)B * nqb; mq.ldp = nqb;
    mq.q_nope = ws_at<bf16_t>(ws, p.qnope); mq.q_pe = ws_at<bf16_t>(ws, p.qpe);
    mq.ctx_len = a->ctx_len; mq.step = step; mq.tok_pos = tok_pos;
    mq.B = B; mq.nh = nh; mq.dn = dn; mq.dr = dr; mq.rope = rope;
    bf16_t* qlat = ws_at<bf16_t>(ws, p.qlat);
    if (p.q_absorb) {
      // q epilogue and W_UK absorption in one launch
      HookScope hs("mla_q_absorb", st);
      E3_HIP(launch_mla_q_absorb(mq, reinterpret_cast<const uint4*>(static_cast<const char*>(packed) + L.uk.off),
                                 L.uk.bs, qlat, st));
    } else {
      {
        HookScope hs("mla_q_rope", st);
        E3_HIP(launch_mla_q(mq, st));
      }
      // absorb W_UK: q_lat[b, h] = W_UK[h]^T q_nope[b, h]  (per-head GEMMs)
      {
        HookScope hs("gemm.uk_absorb", st);
        s = run_gemm(p.uk, L.uk, packed, mq.q_nope, false, (int64_t)nh * dn, dn, B, GEMM_BF16, qlat,
                     (int64_t)nh * r, r, nullptr, nullptr, st);
      }
      if (s != EAGLE3_OK) return s;
    }
    MlaAttnArgs at;
    memset(&at, 0, sizeof(at));
    at.q_lat = qlat; at.q_pe = mq.q_pe; at.cache = ma.cache;
    at.table = a->block_table; at.max_pages = a->max_pages; at.ctx_len = a->ctx_len; at.step = step;
    at.tok_pos = tok_pos; at.tok_row = tok_row;
    at.B = B; at.nh = nh; at.r = r; at.dr = dr; at.page_size = c->page_size;
    at.nblocks = p.attn.nblocks;
    at.sched = ws_at<int32_t>(ws, p.sched) + (int64_t)sched_slot * p.sched_stride;
    const double ms = c->yarn_factor > 1.f ? 0.1 * log((double)c->yarn_factor) + 1.0 : 1.0;
    at.scale = (float)(ms * ms / sqrt((double)(dn + dr)));
    at.part_o = ws_at<uint16_t>(ws, p.apo); at.part_ml = ws_at<float>(ws, p.aml);
    at.out = ws_at<bf16_t>(ws, p.olat);
    if (p.uv_fused) {
      // attention, then the merge of split rows with W_UV in one launch
      HookScope hs("mla_attn", st);
      E3_HIP(launch_mla_attn(at, st, reinterpret_cast<const uint4*>(static_cast<const char*>(packed) + L.uv.off),
                             L.uv.bs, attn_out));
    } else {
      {
        HookScope hs("mla_attn", st);
        E3_HIP(launch_mla_attn(at, st));
      }
      // W_UV: o[b, h] = W_UV[h] o_lat[b, h]
      {
        HookScope hs("gemm.uv", st);
        s = run_gemm(p.uv, L.uv, packed, at.out, false, (int64_t)nh * r, r, B, GEMM_BF16, attn_out,
                     (int64_t)nh * dv, dv, nullptr, nullptr, st);
      }
      if (s != EAGLE3_OK) return s;
    }
  }

  // o_proj + residual + post-attention norm
  {
    HookScope hs("gemm.o", st);
    s = run_gemm(p.o, L.o, packed, attn_out, false, aod, 0, B, GEMM_F32_PARTIAL, part, H, 0, nullptr, nullptr, st);
  }
  if (s != EAGLE3_OK) return s;
  ResidNormArgs rn;
  memset(&rn, 0, sizeof(rn));
  rn.resid = g; rn.part = part; rn.splits = p.o.splitk; rn.ss = (int64_t)B * H; rn.ldp = H;
  rn.h_out = h1; rn.gain = static_cast<const bf16_t*>(w->norm_post);
  uint16_t* u16 = p.mlp_f16 ? ws_at<uint16_t>(ws, p.u16) : nullptr;
  uint16_t* act16 = p.mlp_f16 ? ws_at<uint16_t>(ws, p.act16) : nullptr;
  if (u16)
    rn.y_f16 = u16;
  else
    rn.y32 = u;
  rn.B = B; rn.N = H; rn.eps = c->rms_eps;
  {
    HookScope hs("resid_norm.post", st);
    E3_HIP(launch_resid_norm(rn, st));
  }
  // gated SiLU MLP
  {
    HookScope hs("gemm.gate_up", st);
    s = run_gemm(p.gu, L.gu, packed, u16 ? static_cast<const void*>(u16) : u, !u16, H, 0, B, GEMM_F32_PARTIAL,
                 part, 2 * I, 0, nullptr, nullptr, st);
  }
  if (s != EAGLE3_OK) return s;
  {
    HookScope hs("silu_mul", st);
    E3_HIP(launch_silu_mul(part, p.gu.splitk, (int64_t)B * 2 * I, 2 * I, act16 ? nullptr : act, act16, B, I, st));
  }
  {
    HookScope hs("gemm.down", st);
    s = run_gemm(p.down, L.down, packed, act16 ? static_cast<const void*>(act16) : act, !act16, I, 0, B,
                 GEMM_F32_PARTIAL, part, H, 0, nullptr, nullptr, st);
  }
  if (s != EAGLE3_OK) return s;
  rn.resid = h1; rn.splits = p.down.splitk; rn.h_out = h_out;
  rn.gain = static_cast<const bf16_t*>(w->norm_final); rn.y32 = nullptr; rn.y16 = f; rn.y_f16 = nullptr;
  {
    HookScope hs("resid_norm.final", st);
    E3_HIP(launch_resid_norm(rn, st));
  }
  // lm_head with fused top-1 candidates, then d2t
  uint64_t* cand = ws_at<uint64_t>(ws, p.cand);
  {
    HookScope hs("gemm.lm_head", st);
    s = run_gemm(p.lm, L.lm, packed, f, false, H, 0, B, GEMM_ARGMAX, nullptr, c->draft_vocab, 0, cand, logits, st);
  }
  if (s != EAGLE3_OK) return s;
  // candidates were written per 256-row block as [blocks_x, rows]; reduce each block
  if (!final_top1) return EAGLE3_OK;
  HookScope hs_top1("argmax_d2t", st);
  // (the candidate blocks are 256 rows whatever row blocks the GEMM ran in)
  for (int m0 = 0; m0 < B; m0 += 256) {
    const int rows = std::min(256, B - m0);
    E3_HIP(launch_argmax_final(cand + (int64_t)p.lm.blocks_x * m0, p.lm.blocks_x, rows, w->d2t,
                               tok_out + (int64_t)m0 * tok_stride, tok_stride,
                               draft_out ? draft_out + (int64_t)m0 * tok_stride : nullptr, st));
  }
  return EAGLE3_OK;
}

size_t workspace_need(const eagle3_config* c, int max_batch, int max_keys, int nsteps) {
  size_t need = 0;
  for (int b = 1; b <= max_batch; ++b) need = std::max(need, make_plan(c, b, max_keys, nsteps).total);
  return need;
}

// Extend: the step plan over T token rows, then the per-token (table row,
// position) arrays.
struct ExtendLayout { Plan p; size_t tok_row, tok_pos, total; };
ExtendLayout extend_layout(const eagle3_config* c, int T, int max_keys) {
  ExtendLayout e;
  e.p = make_plan(c, T, max_keys, 1);
  e.tok_row = align_up(e.p.total);
  e.tok_pos = align_up(e.tok_row + (size_t)T * 4);
  e.total = align_up(e.tok_pos + (size_t)T * 4);
  return e;
}

eagle3_status check_extend_args(const eagle3_config* cfg, const eagle3_extend_args* a) {
  if (!a) return EAGLE3_ERR_INVALID_ARG;
  if (a->num_tokens <= 0 || a->batch <= 0 || !a->cu_seqlens || a->max_q_len <= 0 || !a->aux ||
      !a->token_in || !a->k_cache || !a->block_table || a->max_pages <= 0 || !a->ctx_len ||
      a->max_ctx < 0 || !a->hidden_out || !a->token_out || !a->workspace)
    return EAGLE3_ERR_INVALID_ARG;
  if (!is_mla(cfg) && !a->v_cache) return EAGLE3_ERR_INVALID_ARG;
  if (a->num_pages < 0) return EAGLE3_ERR_INVALID_ARG;
  if ((int64_t)a->max_pages * cfg->page_size < (int64_t)a->max_ctx + a->max_q_len)
    return EAGLE3_ERR_INVALID_ARG;
  if (((uintptr_t)a->aux | (uintptr_t)a->k_cache | (uintptr_t)a->v_cache |
       (uintptr_t)a->hidden_out | (uintptr_t)a->workspace) & 15)
    return EAGLE3_ERR_INVALID_ARG;
  return EAGLE3_OK;
}

#ifdef EAGLE3_DEBUG
// Debug build: the device-resident indices a call will use are copied to the
// host (after the stream's earlier work, which may have written them) and
// checked against the range contract before anything is enqueued.
template <typename T>
bool to_host(std::vector<T>& v, const T* src, size_t n) {
  v.assign(n, T());
  return n == 0 || hipMemcpy(v.data(), src, n * sizeof(T), hipMemcpyDeviceToHost) == hipSuccess;
}

// d2t targets, token ids, context lengths, and the page ids of positions
// 0 .. ctx_len[r] + new_pos[r] - 1 of every row r.
eagle3_status debug_check(const eagle3_config* c, const eagle3_weights* w, const int32_t* token_in, int ntok,
                          const int32_t* ctx_len, const std::vector<int>& new_pos, const int32_t* table,
                          int max_pages, int max_ctx, int num_pages, hipStream_t st) {
  if (hipStreamSynchronize(st) != hipSuccess) return EAGLE3_ERR_HIP;
  std::vector<int32_t> d2t, tok, ctx, tab;
  const int rows = (int)new_pos.size();
  if ((w->d2t && !to_host(d2t, w->d2t, c->draft_vocab)) || !to_host(tok, token_in, ntok) ||
      !to_host(ctx, ctx_len, rows) || !to_host(tab, table, (size_t)rows * max_pages))
    return EAGLE3_ERR_HIP;
  for (int d = 0; d < (int)d2t.size(); ++d)
    if ((int64_t)d + d2t[d] < 0 || (int64_t)d + d2t[d] >= c->target_vocab) return EAGLE3_ERR_INVALID_ARG;
  for (int t : tok)
    if (t < 0 || t >= c->target_vocab) return EAGLE3_ERR_INVALID_ARG;
  for (int r = 0; r < rows; ++r) {
    if (ctx[r] < 0 || ctx[r] > max_ctx) return EAGLE3_ERR_INVALID_ARG;
    const int64_t last = (int64_t)ctx[r] + new_pos[r] - 1;   // last position the call touches
    for (int64_t pg = 0; last >= 0 && pg <= last / c->page_size; ++pg) {
      const int id = tab[(size_t)r * max_pages + pg];
      if (id < 0 || (num_pages > 0 && id >= num_pages)) return EAGLE3_ERR_INVALID_ARG;
    }
  }
  return EAGLE3_OK;
}
#endif

}  // namespace

extern "C" {

eagle3_status eagle3_workspace_size(const eagle3_config* cfg, int32_t max_batch, int32_t max_ctx,
                                    int32_t max_gamma, size_t* bytes) {
  eagle3_status s = check_config(cfg);
  if (s != EAGLE3_OK) return s;
  if (!bytes || max_batch <= 0 || max_ctx < 0 || max_gamma <= 0) return EAGLE3_ERR_INVALID_ARG;
  *bytes = workspace_need(cfg, max_batch, max_ctx + max_gamma, max_gamma);
  return EAGLE3_OK;
}

eagle3_status eagle3_packed_weights_size(const eagle3_config* cfg, size_t* bytes) {
  eagle3_status s = check_config(cfg);
  if (s != EAGLE3_OK) return s;
  if (!bytes) return EAGLE3_ERR_INVALID_ARG;
  *bytes = packed_layout(cfg).total;
  return EAGLE3_OK;
}

eagle3_status eagle3_pack_weights(const eagle3_config* c, const eagle3_weights* w, void* packed,
                                  size_t packed_bytes, eagle3_stream_t stream) {
  eagle3_status s = check_config(c);
  if (s != EAGLE3_OK) return s;
  if (!w || !packed || !w->fc || !w->w_o || !w->w_gate || !w->w_up || !w->w_down || !w->lm_head)
    return EAGLE3_ERR_INVALID_ARG;
  if (is_mla(c) ? (!w->w_qa || !w->w_qb || !w->w_kva || !w->w_kvb) : (!w->w_q || !w->w_k || !w->w_v))
    return EAGLE3_ERR_INVALID_ARG;
  const int wf = c->weight_format;
  if (wf != EAGLE3_WEIGHTS_BF16) {
    const int mha[] = {EAGLE3_MAT_FC, EAGLE3_MAT_Q, EAGLE3_MAT_K, EAGLE3_MAT_V, EAGLE3_MAT_O,
                       EAGLE3_MAT_GATE, EAGLE3_MAT_UP, EAGLE3_MAT_DOWN, EAGLE3_MAT_LM_HEAD};
    const int mla[] = {EAGLE3_MAT_FC, EAGLE3_MAT_QA, EAGLE3_MAT_QB, EAGLE3_MAT_KVA, EAGLE3_MAT_KVB,
                       EAGLE3_MAT_O, EAGLE3_MAT_GATE, EAGLE3_MAT_UP, EAGLE3_MAT_DOWN, EAGLE3_MAT_LM_HEAD};
    const int* used = is_mla(c) ? mla : mha;
    const int nused = is_mla(c) ? 10 : 9;
    for (int u = 0; u < nused; ++u) {
      if (!w->row_scale[used[u]]) return EAGLE3_ERR_INVALID_ARG;
      if (wf == EAGLE3_WEIGHTS_NVFP4 && !w->block_scale[used[u]]) return EAGLE3_ERR_INVALID_ARG;
    }
  }
  const PackedLayout L = packed_layout(c);
  if (packed_bytes < L.total) return EAGLE3_ERR_WORKSPACE;
  if ((uintptr_t)packed & 15) return EAGLE3_ERR_INVALID_ARG;
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  char* base = static_cast<char*>(packed);
  E3_HIP(launch_zero(packed, L.total, st));
  // rows [row0, row0 + nrows) of packed matrix m from checkpoint matrix `mat`
  // (K = m.K columns, row-major)
  auto pack = [&](const PackedMat& m, int row0, int nrows, const void* src, int mat) -> hipError_t {
    uint4* dst = reinterpret_cast<uint4*>(base + m.off);
    if (wf == EAGLE3_WEIGHTS_BF16)
      return launch_pack(dst, m.NT, m.KT, m.K, row0, nrows, src, m.wq == WQ_F16 ? 3 : 0, nullptr, nullptr, 0, 0,
                         m.K, 1, 1, 0, m.bs, st);
    hipError_t e = wf == EAGLE3_WEIGHTS_FP8
                       ? launch_pack_fp8(dst, m.NT, m.KT, m.K, row0, nrows, static_cast<const uint8_t*>(src),
                                         m.K, st)
                       : launch_pack_nvfp4(dst, reinterpret_cast<uint32_t*>(base + m.bs_off), m.NT, m.KT, m.K,
                                           row0, nrows, static_cast<const uint8_t*>(src), w->block_scale[mat],
                                           st);
    if (e != hipSuccess) return e;
    return hipMemcpyAsync(base + m.rs_off + (size_t)row0 * sizeof(float), w->row_scale[mat],
                          (size_t)nrows * sizeof(float), hipMemcpyDeviceToDevice, st);
  };
  const int H = c->hidden, I = c->intermediate;
  E3_HIP(pack(L.fc, 0, H, w->fc, EAGLE3_MAT_FC));
  if (is_mla(c)) {
    const int ql = c->q_lora_rank, r = c->kv_lora_rank, dr = c->qk_rope_dim;
    const int dn = c->qk_nope_dim, dv = c->v_head_dim, nh = c->n_heads;
    E3_HIP(pack(L.qa_kva, 0, ql, w->w_qa, EAGLE3_MAT_QA));
    E3_HIP(pack(L.qa_kva, ql, r + dr, w->w_kva, EAGLE3_MAT_KVA));
    E3_HIP(pack(L.qb, 0, nh * (dn + dr), w->w_qb, EAGLE3_MAT_QB));
    // kv_b [nh*(dn+dv), r], per head [W_UK | W_UV] rows; its absorbed halves
    // are packed as bf16 (a quantized kv_b is dequantized here)
    const float* rsc = w->row_scale[EAGLE3_MAT_KVB];
    const uint8_t* bsc = w->block_scale[EAGLE3_MAT_KVB];
    // W_UK^T of head h: element (n = latent c, k = nope d) = kv_b[h*(dn+dv) + d][c]
    E3_HIP(launch_pack(reinterpret_cast<uint4*>(base + L.uk.off), L.uk.NT, L.uk.KT, L.uk.K, 0, r, w->w_kvb, wf,
                       rsc, bsc, r, 0, 1, r, nh, (int64_t)(dn + dv) * r, L.uk.bs, st));
    // W_UV of head h: element (n = v, k = c) = kv_b[h*(dn+dv) + dn + v][c]
    E3_HIP(launch_pack(reinterpret_cast<uint4*>(base + L.uv.off), L.uv.NT, L.uv.KT, L.uv.K, 0, dv, w->w_kvb, wf,
                       rsc, bsc, r, (int64_t)dn * r, r, 1, nh, (int64_t)(dn + dv) * r, L.uv.bs, st));
  } else {
    const int hd = c->head_dim, nq = c->n_heads, nkv = c->n_kv_heads;
    E3_HIP(pack(L.qkv, 0, nq * hd, w->w_q, EAGLE3_MAT_Q));
    E3_HIP(pack(L.qkv, nq * hd, nkv * hd, w->w_k, EAGLE3_MAT_K));
    E3_HIP(pack(L.qkv, (nq + nkv) * hd, nkv * hd, w->w_v, EAGLE3_MAT_V));
  }
  E3_HIP(pack(L.o, 0, H, w->w_o, EAGLE3_MAT_O));
  E3_HIP(pack(L.gu, 0, I, w->w_gate, EAGLE3_MAT_GATE));
  E3_HIP(pack(L.gu, I, I, w->w_up, EAGLE3_MAT_UP));
  E3_HIP(pack(L.down, 0, H, w->w_down, EAGLE3_MAT_DOWN));
  E3_HIP(pack(L.lm, 0, c->draft_vocab, w->lm_head, EAGLE3_MAT_LM_HEAD));
  return EAGLE3_OK;
}

static eagle3_status check_weights(const eagle3_config* c, const eagle3_weights* w, const void* packed) {
  if (!w || !packed || !w->embed || !w->norm_in || !w->norm_hid || !w->norm_post || !w->norm_final)
    return EAGLE3_ERR_INVALID_ARG;
  // no d2t: the head scores over the target vocabulary (its target's lm_head)
  if (!w->d2t && c->draft_vocab != c->target_vocab) return EAGLE3_ERR_INVALID_ARG;
  if (is_mla(c) && (!w->norm_qa || !w->norm_kv)) return EAGLE3_ERR_INVALID_ARG;
  // embedding rows and gains are read 16 bytes at a time
  if (((uintptr_t)w->embed | (uintptr_t)w->norm_in | (uintptr_t)w->norm_hid |
       (uintptr_t)w->norm_post | (uintptr_t)w->norm_final) & 15)
    return EAGLE3_ERR_INVALID_ARG;
  return EAGLE3_OK;
}

eagle3_status eagle3_draft_step(const eagle3_config* cfg, const eagle3_weights* w, const void* packed,
                                const eagle3_step_args* a, int32_t step_index,
                                eagle3_stream_t stream) {
  eagle3_status s = check_config(cfg);
  if (s != EAGLE3_OK) return s;
  if ((s = check_weights(cfg, w, packed)) != EAGLE3_OK) return s;
  if (step_index < 0) return EAGLE3_ERR_INVALID_ARG;
  if ((s = check_args(cfg, a, step_index + 1, false)) != EAGLE3_OK) return s;
  const Plan p = make_plan(cfg, a->batch, a->max_ctx + step_index + 1, 1);
  if (a->workspace_bytes < p.total) return EAGLE3_ERR_WORKSPACE;
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
#ifdef EAGLE3_DEBUG
  if ((s = debug_check(cfg, w, a->token_in, a->batch, a->ctx_len, std::vector<int>(a->batch, step_index + 1),
                       a->block_table, a->max_pages, a->max_ctx, a->num_pages, st)) != EAGLE3_OK)
    return s;
#endif
  if (is_mla(cfg)) {
    HookScope hs("mla_attn_schedule", st);
    E3_HIP(launch_mla_attn_schedule(a->ctx_len, nullptr, step_index, 1, a->batch, p.attn.nblocks,
                                    ws_at<int32_t>(a->workspace, p.sched), p.sched_stride, st));
  }
  return run_step(cfg, w, packed, a, p, step_index, a->aux != nullptr, a->hidden_in, a->token_in, 1,
                  false, nullptr, nullptr, a->hidden_out, a->token_out, a->draft_id_out, 1,
                  a->logits_out, true, 0, nullptr, nullptr, st);
}

eagle3_status eagle3_draft_chain(const eagle3_config* cfg, const eagle3_weights* w, const void* packed,
                                 const eagle3_step_args* a, int32_t gamma, eagle3_stream_t stream) {
  eagle3_status s = check_config(cfg);
  if (s != EAGLE3_OK) return s;
  if ((s = check_weights(cfg, w, packed)) != EAGLE3_OK) return s;
  if (gamma < 1) return EAGLE3_ERR_INVALID_ARG;
  if ((s = check_args(cfg, a, gamma, true)) != EAGLE3_OK) return s;
  const Plan p = make_plan(cfg, a->batch, a->max_ctx + gamma, gamma);
  if (a->workspace_bytes < p.total) return EAGLE3_ERR_WORKSPACE;
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
#ifdef EAGLE3_DEBUG
  // (later steps embed draft tokens, in range when d2t is)
  if ((s = debug_check(cfg, w, a->token_in, a->batch, a->ctx_len, std::vector<int>(a->batch, gamma),
                       a->block_table, a->max_pages, a->max_ctx, a->num_pages, st)) != EAGLE3_OK)
    return s;
#endif
  const int B = a->batch, H = cfg->hidden;
  if (is_mla(cfg)) {   // the attention work split of every step of the chain, in one launch
    HookScope hs("mla_attn_schedule", st);
    E3_HIP(launch_mla_attn_schedule(a->ctx_len, nullptr, 0, gamma, B, p.attn.nblocks,
                                    ws_at<int32_t>(a->workspace, p.sched), p.sched_stride, st));
  }
  float* hbuf = ws_at<float>(a->workspace, p.hbuf);
  const float* h_prev = a->hidden_in;
  for (int k = 0; k < gamma; ++k) {
    float* h_out = a->hidden_out ? a->hidden_out + (int64_t)k * B * H : hbuf;
    // step k > 0 embeds the previous step's top-1, which its own embedding
    // kernel reduces from the candidates and writes to token_out[:, k-1]
    const int32_t* tin = k == 0 ? a->token_in : a->token_out + (k - 1);
    const int tin_stride = k == 0 ? 1 : gamma;
    float* logits = a->logits_out ? a->logits_out + (int64_t)k * B * cfg->draft_vocab : nullptr;
    s = run_step(cfg, w, packed, a, p, k, k == 0 && a->aux != nullptr, h_prev, tin, tin_stride, k > 0,
                 a->token_out + (k - 1), a->draft_id_out ? a->draft_id_out + (k - 1) : nullptr, h_out,
                 a->token_out + k, a->draft_id_out ? a->draft_id_out + k : nullptr, gamma, logits,
                 k == gamma - 1, k, nullptr, nullptr, st);
    if (s != EAGLE3_OK) return s;
    h_prev = h_out;
  }
  return EAGLE3_OK;
}

eagle3_status eagle3_extend_workspace_size(const eagle3_config* cfg, int32_t max_tokens, int32_t max_batch,
                                           int32_t max_ctx, int32_t max_q_len, size_t* bytes) {
  eagle3_status s = check_config(cfg);
  if (s != EAGLE3_OK) return s;
  if (!bytes || max_tokens <= 0 || max_batch <= 0 || max_ctx < 0 || max_q_len <= 0)
    return EAGLE3_ERR_INVALID_ARG;
  size_t need = 0;
  for (int t = 1; t <= max_tokens; ++t)
    need = std::max(need, extend_layout(cfg, t, max_ctx + max_q_len).total);
  *bytes = need;
  return EAGLE3_OK;
}

eagle3_status eagle3_draft_extend(const eagle3_config* cfg, const eagle3_weights* w, const void* packed,
                                  const eagle3_extend_args* a, eagle3_stream_t stream) {
  eagle3_status s = check_config(cfg);
  if (s != EAGLE3_OK) return s;
  if ((s = check_weights(cfg, w, packed)) != EAGLE3_OK) return s;
  if ((s = check_extend_args(cfg, a)) != EAGLE3_OK) return s;
  const int T = a->num_tokens;
  const ExtendLayout e = extend_layout(cfg, T, a->max_ctx + a->max_q_len);
  if (a->workspace_bytes < e.total) return EAGLE3_ERR_WORKSPACE;
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
#ifdef EAGLE3_DEBUG
  {
    // the sequence boundaries first: they give each sequence's new positions
    std::vector<int32_t> cu;
    if (hipStreamSynchronize(st) != hipSuccess || !to_host(cu, a->cu_seqlens, (size_t)a->batch + 1))
      return EAGLE3_ERR_HIP;
    if (cu[0] != 0 || cu[a->batch] != T) return EAGLE3_ERR_INVALID_ARG;
    std::vector<int> q(a->batch);
    for (int b = 0; b < a->batch; ++b) {
      q[b] = cu[b + 1] - cu[b];
      if (q[b] < 0 || q[b] > a->max_q_len) return EAGLE3_ERR_INVALID_ARG;
    }
    if ((s = debug_check(cfg, w, a->token_in, T, a->ctx_len, q, a->block_table, a->max_pages, a->max_ctx,
                         a->num_pages, st)) != EAGLE3_OK)
      return s;
  }
#endif
  int32_t* tok_row = ws_at<int32_t>(a->workspace, e.tok_row);
  int32_t* tok_pos = ws_at<int32_t>(a->workspace, e.tok_pos);
  {
    HookScope hs("extend_index", st);
    E3_HIP(launch_extend_index(a->cu_seqlens, a->ctx_len, a->batch, tok_row, tok_pos, st));
  }
  if (is_mla(cfg)) {
    HookScope hs("mla_attn_schedule", st);
    E3_HIP(launch_mla_attn_schedule(a->ctx_len, tok_pos, 0, 1, T, e.p.attn.nblocks,
                                    ws_at<int32_t>(a->workspace, e.p.sched), e.p.sched_stride, st));
  }
  // the step path over T token rows; every row reads its own page-table row
  // and position through tok_row / tok_pos
  eagle3_step_args sa;
  memset(&sa, 0, sizeof(sa));
  sa.batch = T; sa.aux = a->aux; sa.token_in = a->token_in;
  sa.k_cache = a->k_cache; sa.v_cache = a->v_cache; sa.block_table = a->block_table;
  sa.max_pages = a->max_pages; sa.ctx_len = a->ctx_len; sa.max_ctx = a->max_ctx;
  sa.hidden_out = a->hidden_out; sa.token_out = a->token_out; sa.draft_id_out = a->draft_id_out;
  sa.logits_out = a->logits_out; sa.workspace = a->workspace; sa.workspace_bytes = a->workspace_bytes;
  return run_step(cfg, w, packed, &sa, e.p, 0, true, nullptr, a->token_in, 1, false, nullptr, nullptr,
                  a->hidden_out, a->token_out, a->draft_id_out, 1, a->logits_out, true, 0, tok_pos, tok_row,
                  st);
}

eagle3_status eagle3_greedy_accept(const int32_t* draft, const int32_t* target, int32_t batch,
                                   int32_t gamma, int32_t* accept_len, int32_t* bonus,
                                   eagle3_stream_t stream) {
  if (!draft || !target || !accept_len || !bonus || batch <= 0 || gamma < 1)
    return EAGLE3_ERR_INVALID_ARG;
  HookScope hs("greedy_accept", reinterpret_cast<hipStream_t>(stream));
  if (launch_accept(draft, target, batch, gamma, accept_len, bonus,
                    reinterpret_cast<hipStream_t>(stream)) != hipSuccess)
    return EAGLE3_ERR_HIP;
  return EAGLE3_OK;
}

static eagle3_status relaxed_sizes(int32_t batch, int32_t gamma, int32_t vocab, size_t* bytes) {
  if (batch <= 0 || batch > 65535 || gamma < 1 || gamma > 1024 || vocab <= 0 || vocab > (1 << 30))
    return EAGLE3_ERR_INVALID_ARG;
  int nchunks, chunk;
  relaxed_layout(batch, gamma, vocab, &nchunks, &chunk);
  *bytes = (size_t)batch * (gamma + 1) * nchunks * sizeof(uint4);
  return EAGLE3_OK;
}

eagle3_status eagle3_relaxed_accept_workspace_size(int32_t batch, int32_t gamma, int32_t vocab,
                                                   size_t* bytes) {
  if (!bytes) return EAGLE3_ERR_INVALID_ARG;
  return relaxed_sizes(batch, gamma, vocab, bytes);
}

eagle3_status eagle3_relaxed_accept(const int32_t* draft, const float* logits, const uint8_t* relaxed,
                                    int32_t batch, int32_t gamma, int32_t vocab, int32_t topk, float delta,
                                    int32_t* accept_len, int32_t* bonus, void* workspace,
                                    size_t workspace_bytes, eagle3_stream_t stream) {
  if (!draft || !logits || !accept_len || !bonus || !workspace) return EAGLE3_ERR_INVALID_ARG;
  if (topk < 1 || !(delta >= 0.f) || !std::isfinite(delta)) return EAGLE3_ERR_INVALID_ARG;
  if (reinterpret_cast<uintptr_t>(logits) % 4 || reinterpret_cast<uintptr_t>(workspace) % 16)
    return EAGLE3_ERR_INVALID_ARG;
  size_t need = 0;
  const eagle3_status st = relaxed_sizes(batch, gamma, vocab, &need);
  if (st != EAGLE3_OK) return st;
  if (workspace_bytes < need) return EAGLE3_ERR_WORKSPACE;
  const hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  uint4* part = static_cast<uint4*>(workspace);
  {
    HookScope hs("relaxed_scan", s);
    if (launch_relaxed_scan(logits, draft, batch, gamma, vocab, part, s) != hipSuccess) return EAGLE3_ERR_HIP;
  }
  HookScope hs("relaxed_final", s);
  if (launch_relaxed_final(logits, draft, relaxed, batch, gamma, vocab, topk, delta, part, accept_len, bonus,
                           s) != hipSuccess)
    return EAGLE3_ERR_HIP;
  return EAGLE3_OK;
}

void eagle3_set_launch_hook(eagle3_launch_hook hook, void* user) {
  g_hook = hook;
  g_hook_user = user;
}

const char* eagle3_status_string(eagle3_status s) {
  switch (s) {
    case EAGLE3_OK: return "ok";
    case EAGLE3_ERR_INVALID_ARG: return "invalid argument";
    case EAGLE3_ERR_SHAPE: return "inconsistent shapes";
    case EAGLE3_ERR_UNSUPPORTED: return "unsupported configuration";
    case EAGLE3_ERR_WORKSPACE: return "buffer too small";
    case EAGLE3_ERR_HIP: return "HIP launch error";
  }
  return "unknown status";
}

}  // extern "C"
