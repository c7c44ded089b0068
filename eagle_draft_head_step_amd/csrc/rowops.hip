// Row-wise kernels of the draft step: split-K reductions fused with the
// RMSNorms, residual adds, SiLU gating, RoPE/YaRN rotations and cache
// appends; the final top-1 with the d2t map; and greedy acceptance.
// One workgroup handles one batch row (the rows are independent), so every
// reduction runs in a fixed order and results are bitwise reproducible.
#include "common.h"
#include "internal.h"

namespace e3 {

constexpr int RB = 256;  // threads per row block

__device__ __forceinline__ float sum_parts(const float* __restrict__ p, int splits, int64_t ss,
                                           int64_t idx) {
  float v = 0.f;
  for (int s = 0; s < splits; ++s) v += p[(int64_t)s * ss + idx];
  return v;
}

__device__ __forceinline__ float inv_rms(float sumsq, int n, float eps) {
  return 1.0f / sqrtf(sumsq / (float)n + eps);
}

// Fills cs/sn[0..npairs) with cos/sin of pos * inv_freq[i]; angles in double.
__device__ __forceinline__ void rope_angles(const RopeTable& t, int pos, float* cs, float* sn) {
  for (int i = threadIdx.x; i < t.npairs; i += blockDim.x) {
    double s, c;
    sincos((double)pos * t.inv_freq[i], &s, &c);
    cs[i] = (float)c;
    sn[i] = (float)s;
  }
}

// ------------------------------------------------------------ embed + norms
// x[b] = [RMS(embed[tok]) * norm_in || RMS(g) * norm_hid]; g kept in fp32.
__global__ __launch_bounds__(RB) void embed_norm_kernel(EmbedNormArgs a) {
  __shared__ float red[16];
  const int b = blockIdx.x, H = a.H;
  const int tok = a.tok[(int64_t)b * a.tok_stride];
  const bf16_t* __restrict__ e = a.embed + (int64_t)tok * H;
  float* __restrict__ g = a.g_out + (int64_t)b * H;
  float sg = 0.f, se = 0.f;
  for (int i = threadIdx.x; i < H; i += RB) {
    const float v = a.g_part ? sum_parts(a.g_part, a.g_splits, a.g_ss, (int64_t)b * H + i)
                             : a.g_in[(int64_t)b * H + i];
    g[i] = v;
    sg += v * v;
    const float ev = bf2f(e[i]);
    se += ev * ev;
  }
  const float rg = inv_rms(block_sum(sg, red), H, a.eps);
  const float re = inv_rms(block_sum(se, red), H, a.eps);
  bf16_t* __restrict__ x = a.x + (int64_t)b * 2 * H;
  for (int i = threadIdx.x; i < H; i += RB) {
    x[i] = f2bf(bf2f(e[i]) * re * bf2f(a.norm_in[i]));
    x[H + i] = f2bf(g[i] * rg * bf2f(a.norm_hid[i]));
  }
}

hipError_t launch_embed_norm(const EmbedNormArgs& a, hipStream_t st) {
  hipLaunchKernelGGL(embed_norm_kernel, dim3(a.B), dim3(RB), 0, st, a);
  return hipGetLastError();
}

// ------------------------------------------------------------ residual + norm
__global__ __launch_bounds__(RB) void resid_norm_kernel(ResidNormArgs a) {
  __shared__ float red[16];
  const int b = blockIdx.x, N = a.N;
  float s = 0.f;
  // first pass: h = resid + partials; keep it in h_out (or recompute below)
  for (int i = threadIdx.x; i < N; i += RB) {
    const float h = a.resid[(int64_t)b * N + i] + sum_parts(a.part, a.splits, a.ss, (int64_t)b * a.ldp + i);
    if (a.h_out) a.h_out[(int64_t)b * N + i] = h;
    s += h * h;
  }
  const float r = inv_rms(block_sum(s, red), N, a.eps);
  for (int i = threadIdx.x; i < N; i += RB) {
    const float h = a.h_out ? a.h_out[(int64_t)b * N + i]
                            : a.resid[(int64_t)b * N + i] +
                                  sum_parts(a.part, a.splits, a.ss, (int64_t)b * a.ldp + i);
    a.y[(int64_t)b * N + i] = f2bf(h * r * bf2f(a.gain[i]));
  }
}

hipError_t launch_resid_norm(const ResidNormArgs& a, hipStream_t st) {
  hipLaunchKernelGGL(resid_norm_kernel, dim3(a.B), dim3(RB), 0, st, a);
  return hipGetLastError();
}

// ------------------------------------------------------------ SiLU gate
__global__ __launch_bounds__(RB) void silu_mul_kernel(const float* __restrict__ part, int splits,
                                                      int64_t ss, int64_t ldp, bf16_t* __restrict__ act,
                                                      int I) {
  const int b = blockIdx.y;
  const int i = blockIdx.x * RB + threadIdx.x;
  if (i >= I) return;
  const float g = sum_parts(part, splits, ss, (int64_t)b * ldp + i);
  const float u = sum_parts(part, splits, ss, (int64_t)b * ldp + I + i);
  act[(int64_t)b * I + i] = f2bf(g / (1.0f + expf(-g)) * u);
}

hipError_t launch_silu_mul(const float* part, int splits, int64_t ss, int64_t ldp, bf16_t* act,
                           int B, int I, hipStream_t st) {
  hipLaunchKernelGGL(silu_mul_kernel, dim3((I + RB - 1) / RB, B), dim3(RB), 0, st, part, splits, ss,
                     ldp, act, I);
  return hipGetLastError();
}

// ------------------------------------------------------------ MHA q/k/v
// Reduces the fused q|k|v projection, rotates q and k (pairs i, i + hd/2),
// keeps q in fp32 and appends bf16 k, v at the row's new position.
__global__ __launch_bounds__(RB) void mha_qkv_kernel(MhaQkvArgs a) {
  __shared__ float cs[64], sn[64];
  const int b = blockIdx.x;
  const int pos = a.ctx_len[b] + a.step;
  rope_angles(a.rope, pos, cs, sn);
  __syncthreads();
  const int hd = a.hd, half = hd / 2;
  const int64_t row = (int64_t)b * a.ldp;
  const int page = a.table[(int64_t)b * a.max_pages + pos / a.page_size];
  const int slot = pos % a.page_size;
  const int nq_pairs = a.nq * half, nkv_pairs = a.nkv * half;
  for (int t = threadIdx.x; t < nq_pairs + nkv_pairs; t += RB) {
    const bool isq = t < nq_pairs;
    const int tt = isq ? t : t - nq_pairs;
    const int h = tt / half, i = tt % half;
    const int64_t base = isq ? (int64_t)h * hd : (int64_t)a.nq * hd + (int64_t)h * hd;
    const float x1 = sum_parts(a.part, a.splits, a.ss, row + base + i);
    const float x2 = sum_parts(a.part, a.splits, a.ss, row + base + i + half);
    const float y1 = x1 * cs[i] - x2 * sn[i];
    const float y2 = x1 * sn[i] + x2 * cs[i];
    if (isq) {
      float* q = a.q + ((int64_t)b * a.nq + h) * hd;
      q[i] = y1;
      q[i + half] = y2;
    } else {
      bf16_t* k = a.k_cache + (((int64_t)page * a.nkv + h) * a.page_size + slot) * hd;
      k[i] = f2bf(y1);
      k[i + half] = f2bf(y2);
    }
  }
  const int nv = a.nkv * hd;
  for (int t = threadIdx.x; t < nv; t += RB) {
    const int h = t / hd, d = t % hd;
    const float v = sum_parts(a.part, a.splits, a.ss, row + (int64_t)(a.nq + a.nkv) * hd + t);
    a.v_cache[(((int64_t)page * a.nkv + h) * a.page_size + slot) * hd + d] = f2bf(v);
  }
}

hipError_t launch_mha_qkv(const MhaQkvArgs& a, hipStream_t st) {
  hipLaunchKernelGGL(mha_qkv_kernel, dim3(a.B), dim3(RB), 0, st, a);
  return hipGetLastError();
}

// ------------------------------------------------------------ MLA down-projection epilogue
// From [q_a | latent | k_pe]: q_a -> RMS * norm_qa (bf16); latent -> RMS *
// norm_kv; k_pe rotated in interleaved pairs; [latent | k_pe] appended (bf16).
__global__ __launch_bounds__(RB) void mla_a_kernel(MlaAArgs a) {
  __shared__ float red[16];
  __shared__ float cs[64], sn[64];
  const int b = blockIdx.x;
  const int pos = a.ctx_len[b] + a.step;
  rope_angles(a.rope, pos, cs, sn);
  const int64_t row = (int64_t)b * a.ldp;
  float sq = 0.f, sc = 0.f;
  for (int i = threadIdx.x; i < a.q_lora; i += RB) {
    const float v = sum_parts(a.part, a.splits, a.ss, row + i);
    sq += v * v;
  }
  for (int i = threadIdx.x; i < a.r; i += RB) {
    const float v = sum_parts(a.part, a.splits, a.ss, row + a.q_lora + i);
    sc += v * v;
  }
  const float rq = inv_rms(block_sum(sq, red), a.q_lora, a.eps);
  const float rc = inv_rms(block_sum(sc, red), a.r, a.eps);
  for (int i = threadIdx.x; i < a.q_lora; i += RB) {
    const float v = sum_parts(a.part, a.splits, a.ss, row + i);
    a.qa[(int64_t)b * a.q_lora + i] = f2bf(v * rq * bf2f(a.norm_qa[i]));
  }
  const int page = a.table[(int64_t)b * a.max_pages + pos / a.page_size];
  const int slot = pos % a.page_size;
  bf16_t* ent = a.cache + ((int64_t)page * a.page_size + slot) * (a.r + a.dr);
  for (int i = threadIdx.x; i < a.r; i += RB) {
    const float v = sum_parts(a.part, a.splits, a.ss, row + a.q_lora + i);
    ent[i] = f2bf(v * rc * bf2f(a.norm_kv[i]));
  }
  for (int i = threadIdx.x; i < a.dr / 2; i += RB) {
    const float x1 = sum_parts(a.part, a.splits, a.ss, row + a.q_lora + a.r + 2 * i);
    const float x2 = sum_parts(a.part, a.splits, a.ss, row + a.q_lora + a.r + 2 * i + 1);
    ent[a.r + 2 * i] = f2bf(x1 * cs[i] - x2 * sn[i]);
    ent[a.r + 2 * i + 1] = f2bf(x1 * sn[i] + x2 * cs[i]);
  }
}

hipError_t launch_mla_a(const MlaAArgs& a, hipStream_t st) {
  hipLaunchKernelGGL(mla_a_kernel, dim3(a.B), dim3(RB), 0, st, a);
  return hipGetLastError();
}

// ------------------------------------------------------------ MLA query epilogue
// q_b output per head [nope | rope]: nope -> bf16 (input of the W_UK
// absorption); rope -> interleaved YaRN rotation -> bf16.
__global__ __launch_bounds__(RB) void mla_q_kernel(MlaQArgs a) {
  __shared__ float cs[64], sn[64];
  const int b = blockIdx.x;
  const int pos = a.ctx_len[b] + a.step;
  rope_angles(a.rope, pos, cs, sn);
  __syncthreads();
  const int dq = a.dn + a.dr;
  const int64_t row = (int64_t)b * a.ldp;
  for (int t = threadIdx.x; t < a.nh * a.dn; t += RB) {
    const int h = t / a.dn, d = t % a.dn;
    a.q_nope[(int64_t)b * a.nh * a.dn + t] = f2bf(sum_parts(a.part, a.splits, a.ss, row + (int64_t)h * dq + d));
  }
  const int hp = a.dr / 2;
  for (int t = threadIdx.x; t < a.nh * hp; t += RB) {
    const int h = t / hp, i = t % hp;
    const int64_t base = row + (int64_t)h * dq + a.dn;
    const float x1 = sum_parts(a.part, a.splits, a.ss, base + 2 * i);
    const float x2 = sum_parts(a.part, a.splits, a.ss, base + 2 * i + 1);
    bf16_t* o = a.q_pe + ((int64_t)b * a.nh + h) * a.dr;
    o[2 * i] = f2bf(x1 * cs[i] - x2 * sn[i]);
    o[2 * i + 1] = f2bf(x1 * sn[i] + x2 * cs[i]);
  }
}

hipError_t launch_mla_q(const MlaQArgs& a, hipStream_t st) {
  hipLaunchKernelGGL(mla_q_kernel, dim3(a.B), dim3(RB), 0, st, a);
  return hipGetLastError();
}

// ------------------------------------------------------------ top-1 + d2t
__global__ __launch_bounds__(RB) void argmax_final_kernel(const uint64_t* __restrict__ cand, int ncand,
                                                          int B, const int32_t* __restrict__ d2t,
                                                          int32_t* token_out, int tok_stride,
                                                          int32_t* draft_out) {
  __shared__ uint64_t red[RB / 64];
  const int b = blockIdx.x;
  uint64_t best = 0;
  for (int c = threadIdx.x; c < ncand; c += RB) {
    const uint64_t k = cand[(int64_t)c * B + b];
    best = k > best ? k : best;
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    const uint32_t lo = __shfl_xor((uint32_t)best, o, 64);
    const uint32_t hi = __shfl_xor((uint32_t)(best >> 32), o, 64);
    const uint64_t other = (uint64_t(hi) << 32) | lo;
    best = other > best ? other : best;
  }
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = best;
  __syncthreads();
  if (threadIdx.x == 0) {
    for (int w = 1; w < RB / 64; ++w) best = red[w] > best ? red[w] : best;
    best = red[0] > best ? red[0] : best;
    const int d = (int)argmax_key_index(best);
    token_out[(int64_t)b * tok_stride] = d + d2t[d];
    if (draft_out) draft_out[(int64_t)b * tok_stride] = d;
  }
}

hipError_t launch_argmax_final(const uint64_t* cand, int ncand, int B, const int32_t* d2t,
                               int32_t* token_out, int tok_stride, int32_t* draft_out,
                               hipStream_t st) {
  hipLaunchKernelGGL(argmax_final_kernel, dim3(B), dim3(RB), 0, st, cand, ncand, B, d2t, token_out,
                     tok_stride, draft_out);
  return hipGetLastError();
}

// ------------------------------------------------------------ greedy accept
// One lane per row: leading matches of draft against the target's argmax,
// then the target's id at the first mismatch (or after the last draft).
__global__ __launch_bounds__(RB) void accept_kernel(const int32_t* __restrict__ draft,
                                                    const int32_t* __restrict__ target, int B, int gamma,
                                                    int32_t* __restrict__ accept_len,
                                                    int32_t* __restrict__ bonus) {
  const int b = blockIdx.x * RB + threadIdx.x;
  if (b >= B) return;
  const int32_t* d = draft + (int64_t)b * gamma;
  const int32_t* t = target + (int64_t)b * (gamma + 1);
  int a = 0;
  while (a < gamma && d[a] == t[a]) ++a;
  accept_len[b] = a;
  bonus[b] = t[a];
}

hipError_t launch_accept(const int32_t* draft, const int32_t* target, int B, int gamma,
                         int32_t* accept_len, int32_t* bonus, hipStream_t st) {
  hipLaunchKernelGGL(accept_kernel, dim3((B + RB - 1) / RB), dim3(RB), 0, st, draft, target, B, gamma,
                     accept_len, bonus);
  return hipGetLastError();
}

}  // namespace e3
