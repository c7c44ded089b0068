/*
 * eagle3.h -- C ABI of an MI355X (gfx950) library that runs the hot path of
 * an EAGLE-3 speculative-decoding draft head:
 *
 *   eagle3_draft_step    one autoregressive draft step for a batch of rows,
 *   eagle3_draft_chain   gamma chained steps,
 *   eagle3_greedy_accept greedy verification of the drafted chain,
 *   eagle3_relaxed_accept its relaxed variant for thinking spans,
 *
 * plus the set-up calls they need (sizes, weight packing, status strings).
 *
 * Sources (pages cited by title and section):
 *  [MAX-walkthrough] "Eagle3 DeepseekV3 投机解码架构 — MAX 中 eagle3_deepseekV3
 *      模块的完整解析": section 4 gives the draft step (three target hidden
 *      states fused by fc from 3H to H without bias; token embedding; two
 *      RMSNorms concatenated to 2H; one DeepseekV3 MLA decoder layer whose
 *      o_proj returns to H; dense SiLU MLP; final norm and own lm_head);
 *      section 7 gives the one-layer paged draft cache; section 9 runs draft
 *      steps in decode mode, one token per row; section 10 gives greedy argmax
 *      acceptance with no allocation inside the graph; section 11 gives the
 *      Llama-style MHA head.
 *  [MAX-API] "max.pipelines.architectures.eagle3_deepseekV3": the draft
 *      config defaults (MLA ranks, eps 1e-6, rope theta, interleaved rope) and
 *      the MHA head's bf16 cache (q/k/v and cache dtypes must match).
 *  [ModelOpt] "EAGLE头结构深潜：Model Optimizer投机解码草稿模型的内部设计":
 *      fc fusion of three layers, doubled q/k/v input width, the smaller
 *      draft lm_head with its d2t offset map, multi-step drafting from the
 *      head's own hidden state.
 *  [YaRN] Peng et al. 2023, sections 3.2 and 3.4 (the MLA head's rope).
 *
 * Conventions shared by every call:
 *  - All tensor pointers are DEVICE pointers unless stated otherwise; the
 *    caller owns every buffer, the cache and the stream.  The library never
 *    allocates or frees device memory and (but for its debug build) never
 *    synchronises: each call only
 *    validates its arguments on the host and enqueues kernels on `stream`,
 *    so a call sequence can be captured into a HIP graph.
 *  - bf16 means IEEE bfloat16 bit patterns (uint16 storage).  Matrices are
 *    row-major; weights are [out_features, in_features] as checkpoints hold
 *    them.
 *  - Argument errors are reported before anything is enqueued.
 *  - Range contract: every token id in [0, target_vocab), every d2t target
 *    (d + d2t[d]) in [0, target_vocab), every ctx_len in [0, max_ctx], and
 *    every block-table id of a page a call reads or writes in [0, num_pages)
 *    (>= 0 when num_pages is 0).  The release library does not check these
 *    device-resident values; a violation is undefined behaviour.  The debug
 *    build (libeagle3_debug.so, compiled with EAGLE3_DEBUG) copies them to
 *    the host before enqueueing anything, returns EAGLE3_ERR_INVALID_ARG on a
 *    violation, and therefore synchronises and cannot be graph-captured.
 *  - Calls that share a workspace or a cache must be ordered on one stream.
 */
#ifndef EAGLE3_H_
#define EAGLE3_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct ihipStream_t* eagle3_stream_t;  /* a hipStream_t; NULL = default stream */

typedef enum {
  EAGLE3_OK = 0,
  EAGLE3_ERR_INVALID_ARG = -1, /* null pointer, non-positive size, gamma < 1, ... */
  EAGLE3_ERR_SHAPE = -2,       /* inconsistent sizes (e.g. fc width != num_aux * hidden) */
  EAGLE3_ERR_UNSUPPORTED = -3, /* a shape this build does not implement, MLA without valid YaRN */
  EAGLE3_ERR_WORKSPACE = -4,   /* workspace or packed-weight buffer too small */
  EAGLE3_ERR_HIP = -5          /* a HIP launch error */
} eagle3_status;

enum { EAGLE3_ATTN_MHA = 0, EAGLE3_ATTN_MLA = 1 };

/* Storage of the GEMM matrices (fc, attention projections, MLP, lm_head).  A
 * head may be post-training quantized to FP8 or NVFP4 [ModelOpt: export and
 * PTQ section; MAX-walkthrough section 5: a quantized draft carries
 * weight_scale tensors].  The pages name the formats only; the element
 * encodings are the OCP 8-bit E4M3 ("FN": no infinities, S.1111.111 is NaN)
 * and 4-bit E2M1 definitions, and the scales are laid out as follows:
 *   FP8:   w[n][k] = e4m3(code[n][k]) * row_scale[n]
 *   NVFP4: w[n][k] = e2m1(code[n][k]) * e4m3(block_scale[n][k / 16]) * row_scale[n]
 * (a per-tensor scale is passed as a row scale repeated over the rows).  The
 * kernels widen codes to bf16 exactly in registers (E4M3 values and E2M1 x
 * E4M3 products are bf16 values) and apply the fp32 row scale to the fp32
 * accumulator: activations keep their precision (weight-only quantization).
 * The MLA head's kv_b (absorbed per head into the attention) is widened to
 * bf16 once, at packing. */
enum { EAGLE3_WEIGHTS_BF16 = 0, EAGLE3_WEIGHTS_FP8 = 1, EAGLE3_WEIGHTS_NVFP4 = 2 };

/* eagle3_config.cache_dtype */
enum { EAGLE3_CACHE_BF16 = 0 };

/* GEMM matrices of eagle3_weights, indexing its row_scale / block_scale. */
enum {
  EAGLE3_MAT_FC = 0, EAGLE3_MAT_Q, EAGLE3_MAT_K, EAGLE3_MAT_V, EAGLE3_MAT_QA, EAGLE3_MAT_QB,
  EAGLE3_MAT_KVA, EAGLE3_MAT_KVB, EAGLE3_MAT_O, EAGLE3_MAT_GATE, EAGLE3_MAT_UP, EAGLE3_MAT_DOWN,
  EAGLE3_MAT_LM_HEAD, EAGLE3_NUM_MATS
};

/* Shape of one draft head.  All sizes in elements. */
typedef struct eagle3_config {
  int32_t attn_kind;      /* EAGLE3_ATTN_MHA (Llama-style, GQA allowed) or EAGLE3_ATTN_MLA */
  int32_t hidden;         /* H; multiple of 8 */
  int32_t num_aux;        /* target layers fused by fc (3 for EAGLE-3) */
  int32_t fc_in_features; /* width of fc's input; must equal num_aux * hidden */
  int32_t intermediate;   /* MLP width I; multiple of 8 */
  int32_t draft_vocab;    /* rows of lm_head */
  int32_t target_vocab;   /* rows of the embedding table; >= draft_vocab */
  /* MHA / GQA: n_heads query heads, n_kv_heads (divides n_heads, at most 16 query
     heads per kv head), head_dim in {32, 64, 128} */
  int32_t n_heads, n_kv_heads, head_dim;
  /* MLA (n_heads shared): q_lora_rank, kv_lora_rank (512), qk_nope_dim (128),
     qk_rope_dim (64), v_head_dim (128); n_heads a multiple of 16 */
  int32_t q_lora_rank, kv_lora_rank, qk_nope_dim, qk_rope_dim, v_head_dim;
  int32_t page_size;      /* tokens per cache page (>= 1; 64 in the workloads) */
  float rms_eps;          /* RMSNorm epsilon (1e-6) */
  float rope_theta;       /* RoPE base */
  /* YaRN (MLA: required, factor > 0, beta_fast >= beta_slow > 0, rope_theta > 1;
     MHA: ignored).  Frequencies follow the DeepSeek YaRN rotary embedding the
     MLA head names ([MAX-walkthrough] section 4; [YaRN] section 3.2): pair i
     keeps theta^(-2i/d) up to lo = floor of the pair making beta_fast turns
     over yarn_orig_max_pos positions, is divided by the factor from hi = ceil
     of the pair making beta_slow turns, with a linear ramp in i between them
     (a step after lo when hi <= lo); scores are scaled by
     (0.1 ln s + 1)^2 / sqrt(qk_nope_dim + qk_rope_dim) ([YaRN] section 3.4). */
  float yarn_factor, yarn_orig_max_pos, yarn_beta_fast, yarn_beta_slow;
  int32_t weight_format;  /* EAGLE3_WEIGHTS_*; NVFP4 needs every GEMM input width (K) to be a
                             multiple of 16 */
  int32_t cache_dtype;    /* EAGLE3_CACHE_BF16 (0): the cache dtype must match the bf16 q/k/v
                             of the head's attention ([MAX-walkthrough] section 7); any other
                             value is EAGLE3_ERR_UNSUPPORTED */
} eagle3_config;

/* Row-major weights as a checkpoint holds them, device pointers.
 * The step reads embed, the RMSNorm gains and d2t in place; the GEMM
 * matrices are read only by eagle3_pack_weights.  Unused members (the other
 * attention kind's) may be NULL.  The GEMM matrices are bf16 [N, K], or with
 * a quantized weight_format uint8 codes: FP8 [N, K]; NVFP4 [N, K/2] with
 * element 2i in the low nibble of byte i; their scales are in row_scale and
 * block_scale (the embedding and gains stay bf16). */
typedef struct eagle3_weights {
  const void* embed;       /* [target_vocab, H] shared token embedding */
  const void* fc;          /* [H, num_aux*H], no bias */
  const void* norm_in;     /* [H] gain of the embedding RMSNorm */
  const void* norm_hid;    /* [H] gain of the fused-hidden RMSNorm */
  const void* norm_post;   /* [H] post-attention RMSNorm */
  const void* norm_final;  /* [H] final RMSNorm before lm_head */
  /* MHA */
  const void* w_q;         /* [n_heads*head_dim, 2H] */
  const void* w_k;         /* [n_kv_heads*head_dim, 2H] */
  const void* w_v;         /* [n_kv_heads*head_dim, 2H] */
  /* MLA */
  const void* w_qa;        /* [q_lora_rank, 2H] */
  const void* norm_qa;     /* [q_lora_rank] */
  const void* w_qb;        /* [n_heads*(qk_nope_dim+qk_rope_dim), q_lora_rank], per head [nope | rope] */
  const void* w_kva;       /* [kv_lora_rank+qk_rope_dim, 2H], rows [latent | rope] */
  const void* norm_kv;     /* [kv_lora_rank] */
  const void* w_kvb;       /* [n_heads*(qk_nope_dim+v_head_dim), kv_lora_rank], per head [W_UK | W_UV] */
  /* both */
  const void* w_o;         /* [H, attention output width] */
  const void* w_gate;      /* [I, H] */
  const void* w_up;        /* [I, H] */
  const void* w_down;      /* [H, I] */
  const void* lm_head;     /* [draft_vocab, H] */
  const int32_t* d2t;      /* [draft_vocab]: target id = draft id + d2t[draft id].  NULL: the
                              head scores through its target's lm_head over the target
                              vocabulary (draft_vocab == target_vocab), ids are target ids
                              [MAX-API: has_own_lm_head] */
  /* quantized formats only, per GEMM matrix (index EAGLE3_MAT_*; entries of
     unused matrices may be NULL) */
  const float* row_scale[EAGLE3_NUM_MATS];     /* [N] fp32 */
  const uint8_t* block_scale[EAGLE3_NUM_MATS]; /* NVFP4: [N, K/16] E4M3 */
} eagle3_weights;

/* Per-call batch arguments of a step or a chain. */
typedef struct eagle3_step_args {
  int32_t batch;              /* B >= 1 */
  const void* aux;            /* [B, num_aux*H] bf16, layers [early | middle | late];
                                 fused through fc.  NULL: use hidden_in instead. */
  const float* hidden_in;     /* [B, H] fp32 hidden of a previous step (no fc); used when aux is NULL */
  const int32_t* token_in;    /* [B] target-vocabulary ids of the tokens being embedded */
  /* One-layer paged cache, bf16.
       MHA: k_cache [num_pages, n_kv_heads, head_dim/32, page_size, 32]
            (dimension d of slot s at [d/32, s, d%32]) and
            v_cache [num_pages, n_kv_heads, head_dim/32, page_size/16, 16, 16, 2]
            (dimension d of slot s at [d/32, s/16, (d/2)%16, s%16, d%2]): each
            16-byte-per-lane operand load of the attention is one contiguous
            KiB; page_size a multiple of 16.
       MLA: k_cache = latent cache [num_pages, (kv_lora_rank + qk_rope_dim)/16, page_size, 16]:
            each entry (the normalised latent, then the rotated k_pe) stored in
            chunks of 16 values, value e of slot s at [e/16, s, e%16], so each
            DMA instruction of the attention reads one contiguous KiB;
            v_cache = NULL; page_size a multiple of 32. */
  void* k_cache;
  void* v_cache;
  const int32_t* block_table; /* [B, max_pages] page ids of each row's positions */
  int32_t max_pages;
  const int32_t* ctx_len;     /* [B] tokens already cached per row (not modified) */
  int32_t max_ctx;            /* host-side bound: every ctx_len[b] <= max_ctx */
  /* Outputs. */
  float* hidden_out;          /* step: [B, H] fp32 (required).  chain: NULL or [gamma, B, H] */
  int32_t* token_out;         /* step: [B]; chain: [B, gamma] target-vocabulary ids (required) */
  int32_t* draft_id_out;      /* optional, same shape as token_out, draft-vocabulary ids */
  float* logits_out;          /* optional fp32 logits: step [B, Vd]; chain [gamma, B, Vd] */
  void* workspace;            /* scratch of at least eagle3_workspace_size() bytes, 256-B aligned */
  size_t workspace_bytes;
  int32_t num_pages;          /* pages the cache holds, or 0 if not given (see the range contract) */
} eagle3_step_args;

/* Bytes of scratch a step or chain needs for batch <= max_batch and
 * ctx_len <= max_ctx (gamma <= max_gamma).  Host only. */
eagle3_status eagle3_workspace_size(const eagle3_config* cfg, int32_t max_batch, int32_t max_ctx,
                                    int32_t max_gamma, size_t* bytes);

/* Bytes of the packed-weight buffer of one head.  Host only. */
eagle3_status eagle3_packed_weights_size(const eagle3_config* cfg, size_t* bytes);

/* Re-lays the GEMM weights (fc, q/k/v or q_a/kv_a/q_b/kv_b, o_proj,
 * gate/up, down, lm_head) into `packed`, a device buffer of at least
 * eagle3_packed_weights_size() bytes, in MFMA fragment order: tiles of 16
 * rows and 32 (bf16), 64 (FP8) or 128 (NVFP4) columns, 1 KiB each, stored in
 * lane order so that one wavefront load fetches one tile; NVFP4 block scales
 * and the fp32 row scales are packed beside them.  A bf16 head's gate/up and
 * down tiles hold the same weights widened to f16 (exact in f16's normal
 * range), and the MLP's inputs, formed in fp32, reach them rounded to f16.   Called once per set of
 * weights, before any step; enqueued on `stream`.  The row-major weights are
 * not modified.  A quantized format needs row_scale of every GEMM matrix the
 * head has (and block_scale for NVFP4): EAGLE3_ERR_INVALID_ARG otherwise. */
eagle3_status eagle3_pack_weights(const eagle3_config* cfg, const eagle3_weights* w, void* packed,
                                  size_t packed_bytes, eagle3_stream_t stream);

/* One draft step [MAX-walkthrough section 4; ModelOpt]: for every row b,
 *   g   = fc(aux[b])            if aux != NULL, else hidden_in[b]
 *   x   = [RMS(embed[token_in[b]]) * norm_in || RMS(g) * norm_hid]      (2H)
 *   attention of the new token at position p = ctx_len[b] + step_index
 *     (its K/V or latent entry is written into the cache at p first, so it
 *     attends to itself and to positions 0..p-1)
 *   h1  = g + o_proj(attn);  h_out = h1 + down(silu(gate(u)) * up(u)),
 *     u = RMS(h1) * norm_post
 *   d   = argmax lm_head(RMS(h_out) * norm_final)   (lowest index on ties)
 *   token_out[b] = d + d2t[d];  hidden_out[b] = h_out
 * `packed` holds the output of eagle3_pack_weights for `w`.
 * ctx_len[b] + step_index must stay below max_pages * page_size. */
eagle3_status eagle3_draft_step(const eagle3_config* cfg, const eagle3_weights* w,
                                const void* packed, const eagle3_step_args* args,
                                int32_t step_index, eagle3_stream_t stream);

/* gamma chained steps [ModelOpt: multi-step drafting; MAX-walkthrough
 * section 9]: step k (0-based) embeds token_out[:, k-1] (token_in for k = 0),
 * takes step k-1's h_out as its hidden (step 0 fuses aux, or takes
 * hidden_in), and writes its entry at position ctx_len[b] + k.  ctx_len is
 * not advanced: the caller does that after verification. */
eagle3_status eagle3_draft_chain(const eagle3_config* cfg, const eagle3_weights* w,
                                 const void* packed, const eagle3_step_args* args, int32_t gamma,
                                 eagle3_stream_t stream);

/* Per-call arguments of a multi-token extend (the draft's prefill over the
 * positions the verifier accepted). */
typedef struct eagle3_extend_args {
  int32_t num_tokens;         /* T >= 1: new positions over all sequences */
  int32_t batch;              /* B >= 1 sequences */
  const int32_t* cu_seqlens;  /* [B+1] device: sequence b's new tokens are rows cu[b] .. cu[b+1]-1
                                 of the token arrays; cu[0] = 0, non-decreasing, cu[B] = T
                                 (a sequence may have none) */
  int32_t max_q_len;          /* host-side bound: every cu[b+1] - cu[b] <= max_q_len */
  const void* aux;            /* [T, num_aux*H] bf16: the target's aux states at each new position */
  const int32_t* token_in;    /* [T] target-vocabulary ids embedded at each new position */
  void* k_cache;              /* cache, as in eagle3_step_args */
  void* v_cache;
  const int32_t* block_table; /* [B, max_pages] */
  int32_t max_pages;
  const int32_t* ctx_len;     /* [B] tokens cached before this call (not modified); new token j of
                                 sequence b sits at position ctx_len[b] + j */
  int32_t max_ctx;            /* host-side bound: every ctx_len[b] <= max_ctx */
  float* hidden_out;          /* [T, H] fp32 h_out of every new position (required) */
  int32_t* token_out;         /* [T] top-1 of every new position, target-vocabulary ids (required) */
  int32_t* draft_id_out;      /* optional [T] draft-vocabulary ids */
  float* logits_out;          /* optional [T, Vd] fp32 */
  void* workspace;            /* at least eagle3_extend_workspace_size() bytes, 256-B aligned */
  size_t workspace_bytes;
  int32_t num_pages;          /* pages the cache holds, or 0 if not given (see the range contract) */
} eagle3_extend_args;

/* Bytes of scratch an extend needs for num_tokens <= max_tokens, batch <=
 * max_batch, ctx_len <= max_ctx and q_len <= max_q_len.  Host only. */
eagle3_status eagle3_extend_workspace_size(const eagle3_config* cfg, int32_t max_tokens, int32_t max_batch,
                                           int32_t max_ctx, int32_t max_q_len, size_t* bytes);

/* Multi-token extend [MAX-walkthrough sections 4 and 9: the draft's prefill
 * phase runs over the accepted positions with variable-length inputs and
 * returns the hidden state and logits of every position].  Every new position
 * i (sequence b, j = i - cu[b]) runs the draft step with g = fc(aux[i]) and
 * token token_in[i] at position p = ctx_len[b] + j: all new entries are
 * written first, and position p attends to positions 0..p of its sequence
 * (causal among the new tokens).  Equivalent to q_len successive
 * eagle3_draft_step calls per sequence, each fed the given aux state and
 * token; the output for a position does not depend on later positions.
 * ctx_len[b] + max_q_len must stay within max_pages * page_size. */
eagle3_status eagle3_draft_extend(const eagle3_config* cfg, const eagle3_weights* w, const void* packed,
                                  const eagle3_extend_args* args, eagle3_stream_t stream);

/* Greedy chain verification [MAX-walkthrough section 10]:
 *   accept_len[b] = number of leading j < gamma with draft[b,j] == target[b,j]
 *   bonus[b]      = target[b, accept_len[b]]
 * draft [B, gamma] and target [B, gamma+1] (the target's argmax ids) are
 * int32 device arrays; outputs are int32 [B].  Allocates nothing. */
eagle3_status eagle3_greedy_accept(const int32_t* draft, const int32_t* target, int32_t batch,
                                   int32_t gamma, int32_t* accept_len, int32_t* bonus,
                                   eagle3_stream_t stream);

/* Chain verification with relaxed acceptance for rows inside a thinking span
 * [MAX-walkthrough section 10: use_relaxed_acceptance_for_thinking accepts a
 * draft proposal that is any of the target's top-N candidates; relaxed_topk
 * (default 10) and relaxed_delta (default 0.6) bound the candidates].
 *
 * Reading of relaxed_delta (the pages do not define it): a log-probability
 * margin, so a candidate must be at most delta below the target's top-1 in
 * log-probability, which is the same as in logit (the normaliser cancels).
 * With z the target's logits at verified position j and
 *   rank(t) = #{u : z[u] > z[t]} + #{u < t : z[u] == z[t]}
 * (ties ordered by lowest id, as for the top-1), draft[b,j] = d is accepted by
 *   a row with relaxed[b] == 0: rank(d) == 0 (the greedy rule);
 *   a row with relaxed[b] != 0: rank(d) < topk and
 *                               (double)z[d] - (double)max(z) >= -(double)delta.
 * accept_len[b] = number of leading accepted positions (0 .. gamma);
 * bonus[b]      = the target's top-1 id at position accept_len[b].
 *
 * draft    int32 [B, gamma] device, target ids; an id outside [0, vocab) is
 *          never accepted.
 * logits   fp32 [B, gamma+1, vocab] device, row-major, finite (no NaN), 4-byte
 *          aligned (16-byte aligned rows with vocab % 4 == 0 take the
 *          vectorised path).
 * relaxed  uint8 [B] device, or NULL: every row is in a thinking span.
 * topk >= 1, delta >= 0 and finite; B <= 65535, gamma <= 1024, vocab <= 2^30.
 * accept_len, bonus int32 [B] device outputs.
 * workspace: device memory, 16-byte aligned, of at least the size
 *   eagle3_relaxed_accept_workspace_size returns (per-chunk partials; nothing
 *   needs clearing).  Allocates nothing; enqueued on `stream`.
 * Errors: EAGLE3_ERR_INVALID_ARG for NULL or out-of-range arguments,
 * EAGLE3_ERR_WORKSPACE for a workspace that is too small. */
eagle3_status eagle3_relaxed_accept_workspace_size(int32_t batch, int32_t gamma, int32_t vocab,
                                                   size_t* bytes);
eagle3_status eagle3_relaxed_accept(const int32_t* draft, const float* logits, const uint8_t* relaxed,
                                    int32_t batch, int32_t gamma, int32_t vocab, int32_t topk, float delta,
                                    int32_t* accept_len, int32_t* bonus, void* workspace,
                                    size_t workspace_bytes, eagle3_stream_t stream);

/* Scratch of eagle3_relaxed_accept_noalloc on each GPU: 1 MiB, one 16-byte
 * partial per (row, verified position, vocabulary chunk), which covers
 * batch * (gamma + 1) <= 65536 at any vocabulary size. */
#define EAGLE3_NOALLOC_SCRATCH_BYTES (1u << 20)

/* eagle3_relaxed_accept for callers that cannot allocate (code under HIP
 * graph capture, tight serving loops, harnesses that forbid allocation): no
 * workspace argument.  The per-chunk partials live in a fixed device array
 * of the library, EAGLE3_NOALLOC_SCRATCH_BYTES on each GPU it runs on, held
 * until the process ends; its address on a GPU is looked up on the first
 * call made with that GPU current.  Same arguments, semantics and results as
 * eagle3_relaxed_accept.  Errors: as eagle3_relaxed_accept, plus
 * EAGLE3_ERR_WORKSPACE when the call needs more than the array
 * (eagle3_relaxed_accept_workspace_size above EAGLE3_NOALLOC_SCRATCH_BYTES)
 * and EAGLE3_ERR_HIP when the address lookup fails.  Calls no allocator.
 * Every call on one GPU shares that GPU's array: calls that overlap on one
 * GPU (streams without ordering between them) race; order them on one
 * stream. */
eagle3_status eagle3_relaxed_accept_noalloc(const int32_t* draft, const float* logits, const uint8_t* relaxed,
                                            int32_t batch, int32_t gamma, int32_t vocab, int32_t topk,
                                            float delta, int32_t* accept_len, int32_t* bonus,
                                            eagle3_stream_t stream);

/* Profiling aid: when set, every kernel launch (or fused launch pair) of a
 * step is bracketed by hook(name, 0, stream, user) before and
 * hook(name, 1, stream, user) after it is enqueued, so a caller can record
 * timing events on `stream` around it.  NULL clears the hook.  The hook is
 * process-wide and not thread-safe; leave it unset in production. */
typedef void (*eagle3_launch_hook)(const char* name, int32_t phase, eagle3_stream_t stream, void* user);
void eagle3_set_launch_hook(eagle3_launch_hook hook, void* user);

/* Static description of a status code. */
const char* eagle3_status_string(eagle3_status s);

#ifdef __cplusplus
}
#endif
#endif /* EAGLE3_H_ */
