// Internal launch interface between the host planner and the gfx950 kernels.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stddef.h>

namespace e3 {

typedef uint16_t bf16_t;

// ----------------------------------------------------------------- GEMM
// C[m, n] = sum_k A[m, k] * W[n, k] for a weight W packed into 16x32 tiles
// (see pack_weight), A row-major bf16 or fp32.  Optionally batched over grid.z with
// per-batch strides (per-head matrices of MLA).
enum GemmMode {
  GEMM_F32_PARTIAL = 0,  // fp32 partial sums: C + split * c_ss
  GEMM_BF16 = 1,         // bf16 result (single split)
  GEMM_ARGMAX = 2,       // per-block argmax candidates (+ optional fp32 logits)
};

struct GemmParams {
  const void* A;          // bf16 (f16 with f16 weights), or fp32 when
  int a_f32;              // a_f32 (split into bf16 hi + lo, or rounded to f16 for f16 weights)
  int64_t lda, a_bs;      // row stride, batch stride (elements)
  const uint4* W;         // packed tiles; 64 uint4 per tile
  int64_t w_bs;           // batch stride in uint4
  int wq;                 // weight storage: 0 bf16, 1 FP8 E4M3, 2 NVFP4 (EAGLE3_WEIGHTS_*), 3 f16 (WQ_F16)
  const float* rscale;    // quantized: fp32 scale per row, NT*16 entries
  const uint32_t* bscale; // NVFP4: E4M3 block scales, 32 words per tile
  int M, N, K, NT, KT;    // NT = ceil(N/16), KT = ceil(K/32) rounded up to whole tiles of the format
  int kps;                // k-tiles per split
  int splitk;             // splits (stream-K: partial slots per column block)
  int streamk;            // large-batch kernel: stream-K over this many workgroups, or 0
  int mode;
  void* C;
  int64_t ldc, c_bs, c_ss;
  uint64_t* cand;         // GEMM_ARGMAX: candidate of block x, row m at cand[x * cand_ld + m]
  int cand_ld;
  float* logits;          // GEMM_ARGMAX: optional [M, ldc] fp32 logits
};

// m-tiles (16 rows each) per block, n-tiles per wave, k-tiles per stage, waves along M (1 or 2)
struct GemmShape { int mt, ntw, kc, wm = 1; };

bool gemm_shape_supported(GemmShape s);
int gemm_blocks_x(const GemmParams& p, GemmShape s);
hipError_t launch_gemm(const GemmParams& p, GemmShape s, int batch, hipStream_t st);
// Large-batch kernel (up to 256 rows, planned for 65..256; bf16 weights with
// bf16 activations, or f16 weights with f16 activations; K a multiple of 32;
// a batch of matrices only with bf16 results): both operands through LDS by
// DMA, 256 columns per block.
bool gemm_big_ok(const GemmParams& p, int batch);
int gemm_big_blocks_x(const GemmParams& p);
// Stream-K over G workgroups: block w takes units (column block, k-tile)
// [w*U/G, (w+1)*U/G) of U = blocks_x * KT; returns the partial slots a
// column block needs (the most blocks sharing one), or 0 if G is not in 1..U.
int gemm_big_streamk_slots(int NT, int KT, int G);
hipError_t launch_gemm_big(const GemmParams& p, int batch, hipStream_t st);

// Packed f16 tiles: the MLP matrices of a bf16 head are widened to f16 at
// packing (exact in f16's normal range) so that the MLP GEMMs can take their
// fp32 activations as one f16 operand (relative rounding 2^-12) instead of
// bf16 hi + lo pairs, at the bf16 kernels' MFMA and byte cost.
constexpr int WQ_F16 = 3;
// k-tiles of 32 per packed tile (one 16-byte lane word): 1 bf16 or f16, 2 FP8, 4 NVFP4.
constexpr int wq_ktiles(int wq) { return wq == 1 ? 2 : (wq == 2 ? 4 : 1); }
// Whether the packed tiles carry fp32 row scales (the quantized formats).
constexpr bool wq_scaled(int wq) { return wq == 1 || wq == 2; }

// Writes bf16 tiles of W (N x K, element (n, k) at linear index
// src_off + (n - row0)*rs + k*cs of the source, rows [row0, row0+nrows) of a
// packed matrix of NT x KT tiles), batch copies at src_bs / dst_bs.  The
// source is bf16 (src_fmt 0), bf16 written as f16 tiles (src_fmt 3), or a
// quantized matrix with src_cols columns (src_fmt 1 FP8, 2 NVFP4) that is
// dequantized with its row and block scales and rounded to bf16.
hipError_t launch_pack(uint4* dst, int NT, int KT, int K, int row0, int nrows, const void* src, int src_fmt,
                       const float* src_rscale, const uint8_t* src_bscale, int64_t src_cols, int64_t src_off,
                       int64_t rs, int64_t cs, int batch, int64_t src_bs, int64_t dst_bs, hipStream_t st);
// FP8 [N, K] codes (row stride rs bytes) into 16 x 64 tiles; rows [row0, row0+nrows).
hipError_t launch_pack_fp8(uint4* dst, int NT, int KT, int K, int row0, int nrows, const uint8_t* src,
                           int64_t rs, hipStream_t st);
// NVFP4 [N, K/2] codes and [N, K/16] block scales into 16 x 128 tiles and
// 32 scale words per tile; rows [row0, row0+nrows).
hipError_t launch_pack_nvfp4(uint4* dst, uint32_t* bdst, int NT, int KT, int K, int row0, int nrows,
                             const uint8_t* codes, const uint8_t* blocks, hipStream_t st);
hipError_t launch_zero(void* dst, size_t bytes, hipStream_t st);

// ----------------------------------------------------------------- row kernels
struct EmbedNormArgs {
  const int32_t* tok; int tok_stride;
  // optional: the previous step's lm_head candidates; the block then takes its
  // row's top-1, maps it through d2t, writes it out and embeds it (tok unused)
  const uint64_t* cand; int ncand; const int32_t* d2t;
  int32_t* top1_out; int32_t* top1_draft; int top1_stride;
  const bf16_t* embed;
  const float* g_part; int g_splits; int64_t g_ss;   // fc partials, or
  const float* g_in;                                  // a previous hidden (g_part == null)
  const bf16_t* norm_in; const bf16_t* norm_hid;
  float* g_out;        // [B, H] residual stream
  bf16_t* x;           // [B, 2H]
  int B, H; float eps;
};
hipError_t launch_embed_norm(const EmbedNormArgs& a, hipStream_t st);

// h = resid + sum of partials; optional h store; y = RMS(h) * gain, stored
// as any of fp32 (y32), bf16 (y16) and f16 (y_f16).
struct ResidNormArgs {
  const float* resid; const float* part; int splits; int64_t ss; int64_t ldp;
  float* h_out; const bf16_t* gain; float* y32; bf16_t* y16;
  uint16_t* y_f16;                  // optional f16 copy of y
  int B, N; float eps;
};
hipError_t launch_resid_norm(const ResidNormArgs& a, hipStream_t st);

// act = silu(sum gate partials) * sum up partials -> fp32 [B, I] and / or
// f16 [B, I] (either may be null, not both)
hipError_t launch_silu_mul(const float* part, int splits, int64_t ss, int64_t ldp, float* act, uint16_t* act_f16,
                           int B, int I, hipStream_t st);

struct RopeTable { double inv_freq[64]; int npairs; };

struct MhaQkvArgs {
  const float* part; int splits; int64_t ss; int64_t ldp;
  float* q;                         // [B, nq, hd] rotated queries
  bf16_t* k_cache; bf16_t* v_cache; // K [pages, nkv, page, hd], V [pages, nkv, hd/2, page, 2]
  const int32_t* table; int max_pages; const int32_t* ctx_len; int step;
  const int32_t* tok_pos; const int32_t* tok_row;   // per-row position / table row (extend), or null
  int B, nq, nkv, hd, page_size;
  RopeTable rope;
};
hipError_t launch_mha_qkv(const MhaQkvArgs& a, hipStream_t st);

struct MhaAttnArgs {
  const float* q;                   // [B, nq, hd]
  const bf16_t* k_cache; const bf16_t* v_cache;
  const int32_t* table; int max_pages; const int32_t* ctx_len; int step;
  const int32_t* tok_pos; const int32_t* tok_row;   // per-row position / table row (extend), or null
  int B, nq, nkv, hd, page_size;
  int nsplit, chunk;                // key splits; keys per split (a multiple of 16 * nw)
  int nw;                           // waves per workgroup: 4 (split keys) or 8 (nsplit 1)
  // nw 8 and a plain step: the block reduces its kv head's q/k/v split-K
  // partials itself, rotates q and k, appends k and v (through k_app / v_app,
  // the same caches) and keeps q in LDS; q is then unused.  Null: q is read.
  const float* part; int splits; int64_t ss; int64_t ldp;
  bf16_t* k_app; bf16_t* v_app;
  RopeTable rope;
  float scale;
  float* part_o; float* part_ml;    // [B, nq, nsplit, hd], [B, nq, nsplit, 2]
  bf16_t* out;                      // [B, nq*hd]
};
hipError_t launch_mha_attn(const MhaAttnArgs& a, hipStream_t st);

struct MlaAArgs {
  const float* part; int splits; int64_t ss; int64_t ldp;   // [q_a | latent | rope]
  const bf16_t* norm_qa; const bf16_t* norm_kv;
  bf16_t* qa;                       // [B, q_lora]
  bf16_t* cache;                    // [pages, page, r + dr]
  const int32_t* table; int max_pages; const int32_t* ctx_len; int step;
  const int32_t* tok_pos; const int32_t* tok_row;   // per-row position / table row (extend), or null
  int B, q_lora, r, dr, page_size; float eps;
  RopeTable rope;
};
hipError_t launch_mla_a(const MlaAArgs& a, hipStream_t st);

struct MlaQArgs {
  const float* part; int splits; int64_t ss; int64_t ldp;   // q_b output [B, nh*(dn+dr)]
  bf16_t* q_nope;                   // [B, nh, dn]
  bf16_t* q_pe;                     // [B, nh, dr] rotated
  const int32_t* ctx_len; int step;
  const int32_t* tok_pos;           // per-row position (extend), or null
  int B, nh, dn, dr;
  RopeTable rope;
};
hipError_t launch_mla_q(const MlaQArgs& a, hipStream_t st);
// mla_q followed by W_UK absorption in one launch (qk_nope_dim 128, latent
// 512): wuk = the heads' packed bf16 W_UK tiles, w_bs uint4 per head;
// q_lat [B, nh, 512] bf16.  q_nope is not written.
hipError_t launch_mla_q_absorb(const MlaQArgs& a, const uint4* wuk, int64_t w_bs, bf16_t* q_lat, hipStream_t st);

struct MlaAttnArgs {
  const bf16_t* q_lat;              // [B, nh, r]
  const bf16_t* q_pe;               // [B, nh, dr]
  const bf16_t* cache;              // [pages, page, r + dr]
  const int32_t* table; int max_pages; const int32_t* ctx_len; int step;
  const int32_t* tok_pos; const int32_t* tok_row;   // per-row position / table row (extend), or null
  int B, nh, r, dr, page_size;      // page_size a multiple of 32
  int nblocks;                      // workgroups sharing the batch's tiles
  const int32_t* sched;             // [B + 1 + nblocks] tile prefix sums, first rows (this step)
  float scale;
  uint16_t* part_o;                 // [2*nblocks, nh, r] fp16 segment outputs / their sums
  float* part_ml;                   // [2*nblocks, nh, 2] segment (max, sum)
  bf16_t* out;                      // [B, nh, r] attended latent
};
// With wuv (the heads' packed bf16 W_UV tiles, w_bs uint4 per head; value
// head dim 128): the merge of split rows and the W_UV product run in one
// launch, writing attn_out [B, nh * 128] bf16 (out then holds only the rows
// written whole); else the merge writes out and W_UV is left to the caller.
hipError_t launch_mla_attn(const MlaAttnArgs& a, hipStream_t st, const uint4* wuv = nullptr, int64_t w_bs = 0,
                           bf16_t* attn_out = nullptr);
// Work schedules of steps step0 .. step0+nsteps-1, each [B + 1 + nblocks]
// ints at sched + s*stride; must run before those steps' attention.
hipError_t launch_mla_attn_schedule(const int32_t* ctx_len, const int32_t* tok_pos, int step0, int nsteps,
                                    int B, int nblocks, int32_t* sched, int stride, hipStream_t st);

// Multi-token extend: row i of the flattened token batch belongs to sequence
// b with cu[b] <= i < cu[b+1]; tok_row[i] = b, tok_pos[i] = ctx_len[b] + i - cu[b].
hipError_t launch_extend_index(const int32_t* cu, const int32_t* ctx_len, int B, int32_t* tok_row,
                               int32_t* tok_pos, hipStream_t st);

hipError_t launch_argmax_final(const uint64_t* cand, int ncand, int B, const int32_t* d2t,
                               int32_t* token_out, int tok_stride, int32_t* draft_out,
                               hipStream_t st);

hipError_t launch_accept(const int32_t* draft, const int32_t* target, int B, int gamma,
                         int32_t* accept_len, int32_t* bonus, hipStream_t st);

// Relaxed verification: `nchunks` vocabulary chunks of `chunk` logits per
// verified position; the partials take B * (gamma+1) * nchunks uint4.
void relaxed_layout(int B, int gamma, int V, int* nchunks, int* chunk);
hipError_t launch_relaxed_scan(const float* logits, const int32_t* draft, int B, int gamma, int V, uint4* part,
                               hipStream_t st);
hipError_t launch_relaxed_final(const float* logits, const int32_t* draft, const uint8_t* relaxed, int B,
                                int gamma, int V, int topk, float delta, const uint4* part, int32_t* accept_len,
                                int32_t* bonus, hipStream_t st);

}  // namespace e3
