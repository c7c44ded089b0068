// Row-wise kernels of the draft step: split-K reductions fused with the
// RMSNorms, residual adds, SiLU gating, RoPE/YaRN rotations and cache
// appends; the final top-1 with the d2t map; and greedy acceptance.
// Every reduction (split-K slabs, row sums) runs in a fixed order inside one
// workgroup, so results are bitwise reproducible.
#include "common.h"
#include "internal.h"

namespace e3 {

constexpr int RB = 256;  // threads per row block

// Split-K slabs whose loads are in flight together: the partials were just
// written by another kernel, so every round of loads costs a trip to memory.
constexpr int SLAB_GROUP = 4;

// Sum of the split-K slabs of one element, in split order; loads are issued
// SLAB_GROUP at a time so their latencies overlap.
__device__ __forceinline__ float sum_parts(const float* __restrict__ p, int splits, int64_t ss,
                                           int64_t idx) {
  float v = 0.f;
  for (int s = 0; s < splits; s += SLAB_GROUP) {
    float t[SLAB_GROUP];
#pragma unroll
    for (int u = 0; u < SLAB_GROUP; ++u) t[u] = s + u < splits ? p[(int64_t)(s + u) * ss + idx] : 0.f;
#pragma unroll
    for (int u = 0; u < SLAB_GROUP; ++u) v += t[u];
  }
  return v;
}

__device__ __forceinline__ float inv_rms(float sumsq, int n, float eps) {
  return 1.0f / sqrtf(sumsq / (float)n + eps);
}

// Wide row blocks: 1024 threads, 8 consecutive columns per thread and
// iteration (two float4 loads per split-K slab), so the split-K partials of a
// row stream in with many independent loads in flight.
constexpr int WB = 1024;
constexpr int GMAX = 2;            // 8-column groups per thread: rows up to 16384 wide

__device__ __forceinline__ void load8(const float* __restrict__ p, float* v) {
  const float4 x = *reinterpret_cast<const float4*>(p);
  const float4 y = *reinterpret_cast<const float4*>(p + 4);
  v[0] = x.x; v[1] = x.y; v[2] = x.z; v[3] = x.w; v[4] = y.x; v[5] = y.y; v[6] = y.z; v[7] = y.w;
}

__device__ __forceinline__ void store8(float* __restrict__ p, const float* v) {
  *reinterpret_cast<float4*>(p) = make_float4(v[0], v[1], v[2], v[3]);
  *reinterpret_cast<float4*>(p + 4) = make_float4(v[4], v[5], v[6], v[7]);
}

// v = sum over splits of p[s*ss + idx .. +7], in split order; SLAB_GROUP
// slabs' loads in flight at a time.
__device__ __forceinline__ void sum8_parts(const float* __restrict__ p, int splits, int64_t ss,
                                           int64_t idx, float* v) {
#pragma unroll
  for (int e = 0; e < 8; ++e) v[e] = 0.f;
  for (int s = 0; s < splits; s += SLAB_GROUP) {
    float t[SLAB_GROUP][8];
#pragma unroll
    for (int u = 0; u < SLAB_GROUP; ++u) {
      if (s + u < splits) load8(p + (int64_t)(s + u) * ss + idx, t[u]);
      else {
#pragma unroll
        for (int e = 0; e < 8; ++e) t[u][e] = 0.f;
      }
    }
#pragma unroll
    for (int u = 0; u < SLAB_GROUP; ++u)
#pragma unroll
      for (int e = 0; e < 8; ++e) v[e] += t[u][e];
  }
}

__device__ __forceinline__ uint4 pack8bf(const float* v) {
  return uint4{pack2bf(v[0], v[1]), pack2bf(v[2], v[3]), pack2bf(v[4], v[5]), pack2bf(v[6], v[7])};
}

// Eight fp32 values rounded to f16 (nearest even).
__device__ __forceinline__ uint4 pack8h(const float* v) {
  uint32_t o[4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
    o[i] = uint32_t(__builtin_bit_cast(uint16_t, (_Float16)v[2 * i])) |
           (uint32_t(__builtin_bit_cast(uint16_t, (_Float16)v[2 * i + 1])) << 16);
  return uint4{o[0], o[1], o[2], o[3]};
}

// ------------------------------------------------------------ embed + norms
// x[b] = [RMS(embed[tok]) * norm_in || RMS(g) * norm_hid]; g kept in fp32.
__device__ __forceinline__ uint64_t max_u64(uint64_t x, uint64_t y) { return x > y ? x : y; }

__device__ __forceinline__ uint64_t wave_max_u64(uint64_t v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    const uint32_t lo = __shfl_xor((uint32_t)v, o, 64);
    const uint32_t hi = __shfl_xor((uint32_t)(v >> 32), o, 64);
    v = max_u64(v, (uint64_t(hi) << 32) | lo);
  }
  return v;
}

// Top-1 of row b from the lm_head candidates ([ncand, rows] per block of 256
// rows), mapped to the target vocabulary; every thread gets the token.
__device__ int row_top1(const uint64_t* __restrict__ cand, int ncand, int B, int b,
                        const int32_t* __restrict__ d2t, int32_t* tok_out, int32_t* draft_out,
                        int stride) {
  __shared__ uint64_t red[32];
  __shared__ int tok;
  const int m0 = (b / 256) * 256, rows = min(256, B - m0);
  const uint64_t* c = cand + (int64_t)ncand * m0 + (b - m0);
  uint64_t best = 0;
  for (int i = threadIdx.x; i < ncand; i += blockDim.x) best = max_u64(best, c[(int64_t)i * rows]);
  best = wave_max_u64(best);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = best;
  __syncthreads();
  if (threadIdx.x == 0) {
    for (int w = 1; w < (int)(blockDim.x >> 6); ++w) best = max_u64(best, red[w]);
    const int d = (int)argmax_key_index(best);
    tok = d2t ? d + d2t[d] : d;
    tok_out[(int64_t)b * stride] = tok;
    if (draft_out) draft_out[(int64_t)b * stride] = d;
  }
  __syncthreads();
  return tok;
}

__global__ __launch_bounds__(WB) void embed_norm_kernel(EmbedNormArgs a) {
  __shared__ float red[16];
  const int b = blockIdx.x, H = a.H;
  // the fused-hidden half does not depend on the token: its loads go out
  // before the top-1 reduction that yields the token
  float gv[GMAX][8], ev[GMAX][8];
#pragma unroll
  for (int j = 0; j < GMAX; ++j) {
    const int c = (threadIdx.x + j * WB) * 8;
    if (c < H) {
      const int64_t idx = (int64_t)b * H + c;
      if (a.g_part) sum8_parts(a.g_part, a.g_splits, a.g_ss, idx, gv[j]);
      else load8(a.g_in + idx, gv[j]);
    }
  }
  const int tok = a.cand ? row_top1(a.cand, a.ncand, a.B, b, a.d2t, a.top1_out, a.top1_draft, a.top1_stride)
                         : a.tok[(int64_t)b * a.tok_stride];
  const bf16_t* __restrict__ e = a.embed + (int64_t)tok * H;
  float sg = 0.f, se = 0.f;
#pragma unroll
  for (int j = 0; j < GMAX; ++j) {
    const int c = (threadIdx.x + j * WB) * 8;
    if (c < H) {
      store8(a.g_out + (int64_t)b * H + c, gv[j]);
      unpack8(*reinterpret_cast<const uint4*>(e + c), ev[j]);
#pragma unroll
      for (int t = 0; t < 8; ++t) { sg += gv[j][t] * gv[j][t]; se += ev[j][t] * ev[j][t]; }
    }
  }
  const float rg = inv_rms(block_sum(sg, red), H, a.eps);
  const float re = inv_rms(block_sum(se, red), H, a.eps);
  bf16_t* __restrict__ x = a.x + (int64_t)b * 2 * H;
#pragma unroll
  for (int j = 0; j < GMAX; ++j) {
    const int c = (threadIdx.x + j * WB) * 8;
    if (c < H) {
      float gi[8], gh[8], yi[8], yh[8];
      unpack8(*reinterpret_cast<const uint4*>(a.norm_in + c), gi);
      unpack8(*reinterpret_cast<const uint4*>(a.norm_hid + c), gh);
#pragma unroll
      for (int t = 0; t < 8; ++t) { yi[t] = ev[j][t] * re * gi[t]; yh[t] = gv[j][t] * rg * gh[t]; }
      *reinterpret_cast<uint4*>(x + c) = pack8bf(yi);
      *reinterpret_cast<uint4*>(x + H + c) = pack8bf(yh);
    }
  }
}

hipError_t launch_embed_norm(const EmbedNormArgs& a, hipStream_t st) {
  if (a.H > GMAX * WB * 8 || a.H % 8) return hipErrorInvalidValue;
  hipLaunchKernelGGL(embed_norm_kernel, dim3(a.B), dim3(WB), 0, st, a);
  return hipGetLastError();
}

// ------------------------------------------------------------ residual + norm
__global__ __launch_bounds__(WB) void resid_norm_kernel(ResidNormArgs a) {
  __shared__ float red[16];
  const int b = blockIdx.x, N = a.N;
  float hv[GMAX][8];
  float s = 0.f;
#pragma unroll
  for (int j = 0; j < GMAX; ++j) {
    const int c = (threadIdx.x + j * WB) * 8;
    if (c < N) {
      float r[8];
      sum8_parts(a.part, a.splits, a.ss, (int64_t)b * a.ldp + c, hv[j]);
      load8(a.resid + (int64_t)b * N + c, r);
#pragma unroll
      for (int t = 0; t < 8; ++t) { hv[j][t] += r[t]; s += hv[j][t] * hv[j][t]; }
      if (a.h_out) store8(a.h_out + (int64_t)b * N + c, hv[j]);
    }
  }
  const float r = inv_rms(block_sum(s, red), N, a.eps);
#pragma unroll
  for (int j = 0; j < GMAX; ++j) {
    const int c = (threadIdx.x + j * WB) * 8;
    if (c < N) {
      float gn[8], y[8];
      unpack8(*reinterpret_cast<const uint4*>(a.gain + c), gn);
#pragma unroll
      for (int t = 0; t < 8; ++t) y[t] = hv[j][t] * r * gn[t];
      if (a.y32) store8(a.y32 + (int64_t)b * N + c, y);
      if (a.y16) *reinterpret_cast<uint4*>(a.y16 + (int64_t)b * N + c) = pack8bf(y);
      if (a.y_f16) *reinterpret_cast<uint4*>(a.y_f16 + (int64_t)b * N + c) = pack8h(y);
    }
  }
}

hipError_t launch_resid_norm(const ResidNormArgs& a, hipStream_t st) {
  if (a.N > GMAX * WB * 8 || a.N % 8) return hipErrorInvalidValue;
  hipLaunchKernelGGL(resid_norm_kernel, dim3(a.B), dim3(WB), 0, st, a);
  return hipGetLastError();
}

// ------------------------------------------------------------ SiLU gate
// act (fp32) and / or act rounded to f16, the form the large-batch GEMM reads.
__global__ __launch_bounds__(RB) void silu_mul_kernel(const float* __restrict__ part, int splits,
                                                      int64_t ss, int64_t ldp, float* __restrict__ act,
                                                      uint16_t* __restrict__ act_f16, int I) {
  const int b = blockIdx.y;
  const int i = blockIdx.x * RB + threadIdx.x;
  if (i >= I) return;
  const float g = sum_parts(part, splits, ss, (int64_t)b * ldp + i);
  const float u = sum_parts(part, splits, ss, (int64_t)b * ldp + I + i);
  const float v = g / (1.0f + expf(-g)) * u;
  if (act) act[(int64_t)b * I + i] = v;
  if (act_f16) act_f16[(int64_t)b * I + i] = __builtin_bit_cast(uint16_t, (_Float16)v);
}

__device__ __forceinline__ float4 ld4(const float* p) { return *reinterpret_cast<const float4*>(p); }
__device__ __forceinline__ float4 add4(float4 a, float4 b) { return make_float4(a.x + b.x, a.y + b.y, a.z + b.z, a.w + b.w); }

// Sum of the split-K slabs of 4 consecutive elements, in split order (each
// element's additions are those of sum_parts).
__device__ __forceinline__ float4 sum4_parts(const float* __restrict__ p, int splits, int64_t ss, int64_t idx) {
  float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
  for (int s = 0; s < splits; s += SLAB_GROUP) {
    float4 t[SLAB_GROUP];
#pragma unroll
    for (int u = 0; u < SLAB_GROUP; ++u)
      t[u] = s + u < splits ? ld4(p + (int64_t)(s + u) * ss + idx) : make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
    for (int u = 0; u < SLAB_GROUP; ++u) v = add4(v, t[u]);
  }
  return v;
}

__device__ __forceinline__ float silu_gate(float g, float u) { return g / (1.0f + expf(-g)) * u; }

// The same with 4 consecutive columns per thread (16-byte loads and stores),
// for rows whose width and strides are multiples of 4 (DeepseekV3 batch 256:
// 22.0 -> 19.4 us per launch).
__global__ __launch_bounds__(RB) void silu_mul4_kernel(const float* __restrict__ part, int splits, int64_t ss,
                                                       int64_t ldp, float* __restrict__ act,
                                                       uint16_t* __restrict__ act_f16, int I) {
  const int b = blockIdx.y;
  const int i = (blockIdx.x * RB + threadIdx.x) * 4;
  if (i >= I) return;
  const int64_t gi = (int64_t)b * ldp + i;
  const float4 g = sum4_parts(part, splits, ss, gi);
  const float4 u = sum4_parts(part, splits, ss, gi + I);
  const float4 v = make_float4(silu_gate(g.x, u.x), silu_gate(g.y, u.y), silu_gate(g.z, u.z), silu_gate(g.w, u.w));
  if (act) *reinterpret_cast<float4*>(act + (int64_t)b * I + i) = v;
  if (act_f16) {
    const float x[4] = {v.x, v.y, v.z, v.w};
    uint32_t o[2];
#pragma unroll
    for (int k = 0; k < 2; ++k)
      o[k] = uint32_t(__builtin_bit_cast(uint16_t, (_Float16)x[2 * k])) |
             (uint32_t(__builtin_bit_cast(uint16_t, (_Float16)x[2 * k + 1])) << 16);
    *reinterpret_cast<uint2*>(act_f16 + (int64_t)b * I + i) = uint2{o[0], o[1]};
  }
}

hipError_t launch_silu_mul(const float* part, int splits, int64_t ss, int64_t ldp, float* act, uint16_t* act_f16,
                           int B, int I, hipStream_t st) {
  if (!act && !act_f16) return hipErrorInvalidValue;
  if (I % 4 == 0 && ldp % 4 == 0 && ss % 4 == 0)
    hipLaunchKernelGGL(silu_mul4_kernel, dim3((I / 4 + RB - 1) / RB, B), dim3(RB), 0, st, part, splits, ss, ldp, act,
                       act_f16, I);
  else
    hipLaunchKernelGGL(silu_mul_kernel, dim3((I + RB - 1) / RB, B), dim3(RB), 0, st, part, splits, ss,
                       ldp, act, act_f16, I);
  return hipGetLastError();
}

// ------------------------------------------------------------ MHA q/k/v
// One block per (head of q|k|v, row), one thread per rotation pair
// (i, i + hd/2): reduces the fused projection's split-K partials, rotates q
// and k, keeps q in fp32 and appends bf16 k and v at the row's new position.
__global__ void mha_qkv_kernel(MhaQkvArgs a) {
  const int head = blockIdx.x, b = blockIdx.y, i = threadIdx.x;
  const int hd = a.hd, half = hd / 2;
  const int pos = new_token_pos(a.tok_pos, a.ctx_len, a.step, b);
  const int64_t base = (int64_t)b * a.ldp + (int64_t)head * hd;
  const float x1 = sum_parts(a.part, a.splits, a.ss, base + i);
  const float x2 = sum_parts(a.part, a.splits, a.ss, base + i + half);
  const int page = a.table[(int64_t)table_row(a.tok_row, b) * a.max_pages + pos / a.page_size];
  const int slot = pos % a.page_size;
  const int P = a.page_size;
  if (head >= a.nq + a.nkv) {
    // V pages: [kv_head][dim / 32][slot / 16][(dim / 2) % 16][slot % 16][dim % 2]
    bf16_t* v = a.v_cache + ((int64_t)page * a.nkv + (head - a.nq - a.nkv)) * hd * P;
    auto at = [&](int d) {
      return ((((int64_t)(d >> 5) * (P >> 4) + (slot >> 4)) * 16 + ((d >> 1) & 15)) * 16 + (slot & 15)) * 2 + (d & 1);
    };
    v[at(i)] = f2bf(x1);
    v[at(i + half)] = f2bf(x2);
    return;
  }
  double sd, cd;
  sincos((double)pos * a.rope.inv_freq[i], &sd, &cd);
  const float c = (float)cd, sn = (float)sd;
  const float y1 = x1 * c - x2 * sn, y2 = x1 * sn + x2 * c;
  if (head < a.nq) {
    float* q = a.q + ((int64_t)b * a.nq + head) * hd;
    q[i] = y1;
    q[i + half] = y2;
  } else {
    // K pages: [kv_head][dim / 32][slot][dim % 32]
    bf16_t* k = a.k_cache + ((int64_t)page * a.nkv + (head - a.nq)) * hd * P + (int64_t)slot * 32;
    k[(int64_t)(i >> 5) * P * 32 + (i & 31)] = f2bf(y1);
    k[(int64_t)((i + half) >> 5) * P * 32 + ((i + half) & 31)] = f2bf(y2);
  }
}

hipError_t launch_mha_qkv(const MhaQkvArgs& a, hipStream_t st) {
  hipLaunchKernelGGL(mha_qkv_kernel, dim3(a.nq + 2 * a.nkv, a.B), dim3(a.hd / 2), 0, st, a);
  return hipGetLastError();
}

// ------------------------------------------------------------ MLA down-projection epilogue
// From [q_a | latent | k_pe]: q_a -> RMS * norm_qa (bf16); latent -> RMS *
// norm_kv; k_pe rotated in interleaved pairs; [latent | k_pe] appended (bf16)
// into the page's 16-value chunks.
constexpr int QMAX = 4;   // q_lora elements per thread: q_lora_rank <= 4096
constexpr int AMAX = 6;   // row elements per thread: q_lora + r + dr <= 6144
__global__ __launch_bounds__(WB) void mla_a_kernel(MlaAArgs a) {
  __shared__ float red[16];
  __shared__ float rowv[AMAX * WB];
  const int b = blockIdx.x, tid = threadIdx.x;
  const int pos = new_token_pos(a.tok_pos, a.ctx_len, a.step, b);
  const int64_t row = (int64_t)b * a.ldp;
  const int na = a.q_lora + a.r + a.dr;
  // split-K reduction of the whole row, in split order, with the loads of
  // A_SLABS slabs x every element of the thread in flight together
  constexpr int A_SLABS = 8;
  {
    float v[AMAX];
#pragma unroll
    for (int j = 0; j < AMAX; ++j) v[j] = 0.f;
    for (int s = 0; s < a.splits; s += A_SLABS) {
      float t[A_SLABS][AMAX];
#pragma unroll
      for (int u = 0; u < A_SLABS; ++u)
#pragma unroll
        for (int j = 0; j < AMAX; ++j) {
          const int i = tid + j * WB;
          t[u][j] = (s + u < a.splits && i < na) ? a.part[(int64_t)(s + u) * a.ss + row + i] : 0.f;
        }
#pragma unroll
      for (int u = 0; u < A_SLABS; ++u)
#pragma unroll
        for (int j = 0; j < AMAX; ++j) v[j] += t[u][j];
    }
#pragma unroll
    for (int j = 0; j < AMAX; ++j)
      if (tid + j * WB < na) rowv[tid + j * WB] = v[j];
  }
  __syncthreads();
  float qv[QMAX];
  float sq = 0.f, sc = 0.f, cv = 0.f;
#pragma unroll
  for (int j = 0; j < QMAX; ++j) {
    const int i = tid + j * WB;
    qv[j] = i < a.q_lora ? rowv[i] : 0.f;
    sq += qv[j] * qv[j];
  }
  if (tid < a.r) {
    cv = rowv[a.q_lora + tid];
    sc = cv * cv;
  }
  float x1 = 0.f, x2 = 0.f;
  if (tid < a.dr / 2) {
    x1 = rowv[a.q_lora + a.r + 2 * tid];
    x2 = rowv[a.q_lora + a.r + 2 * tid + 1];
  }
  const float rq = inv_rms(block_sum(sq, red), a.q_lora, a.eps);
  const float rc = inv_rms(block_sum(sc, red), a.r, a.eps);
#pragma unroll
  for (int j = 0; j < QMAX; ++j) {
    const int i = tid + j * WB;
    if (i < a.q_lora) a.qa[(int64_t)b * a.q_lora + i] = f2bf(qv[j] * rq * bf2f(a.norm_qa[i]));
  }
  const int P = a.page_size;
  const int page = a.table[(int64_t)table_row(a.tok_row, b) * a.max_pages + pos / P];
  const int slot = pos % P;
  // cache page: entries [latent | rope] in chunks of 16 values, [chunk][slot][16]
  bf16_t* pg = a.cache + (int64_t)page * P * (a.r + a.dr) + (int64_t)slot * 16;
  auto ent = [&](int e) -> bf16_t& { return pg[(int64_t)(e >> 4) * P * 16 + (e & 15)]; };
  if (tid < a.r) ent(tid) = f2bf(cv * rc * bf2f(a.norm_kv[tid]));
  if (tid < a.dr / 2) {
    double sd, cd;
    sincos((double)pos * a.rope.inv_freq[tid], &sd, &cd);
    const float c = (float)cd, sn = (float)sd;
    ent(a.r + 2 * tid) = f2bf(x1 * c - x2 * sn);
    ent(a.r + 2 * tid + 1) = f2bf(x1 * sn + x2 * c);
  }
}

hipError_t launch_mla_a(const MlaAArgs& a, hipStream_t st) {
  if (a.q_lora > QMAX * WB || a.r > WB || a.dr / 2 > WB || a.q_lora + a.r + a.dr > AMAX * WB ||
      (a.r + a.dr) % 16)
    return hipErrorInvalidValue;
  hipLaunchKernelGGL(mla_a_kernel, dim3(a.B), dim3(WB), 0, st, a);
  return hipGetLastError();
}

// ------------------------------------------------------------ MLA query epilogue
// One block per (head, row): q_b output per head [nope | rope]; nope -> bf16
// (input of the W_UK absorption); rope -> interleaved YaRN rotation -> bf16.
__global__ __launch_bounds__(64) void mla_q_kernel(MlaQArgs a) {
  const int h = blockIdx.x, b = blockIdx.y, tid = threadIdx.x;
  const int pos = new_token_pos(a.tok_pos, a.ctx_len, a.step, b);
  const int dq = a.dn + a.dr;
  const int64_t base = (int64_t)b * a.ldp + (int64_t)h * dq;
  bf16_t* qn = a.q_nope + ((int64_t)b * a.nh + h) * a.dn;
  for (int d = tid; d < a.dn; d += 64) qn[d] = f2bf(sum_parts(a.part, a.splits, a.ss, base + d));
  for (int i = tid; i < a.dr / 2; i += 64) {
    const float x1 = sum_parts(a.part, a.splits, a.ss, base + a.dn + 2 * i);
    const float x2 = sum_parts(a.part, a.splits, a.ss, base + a.dn + 2 * i + 1);
    double sd, cd;
    sincos((double)pos * a.rope.inv_freq[i], &sd, &cd);
    const float c = (float)cd, sn = (float)sd;
    bf16_t* o = a.q_pe + ((int64_t)b * a.nh + h) * a.dr;
    o[2 * i] = f2bf(x1 * c - x2 * sn);
    o[2 * i + 1] = f2bf(x1 * sn + x2 * c);
  }
}

hipError_t launch_mla_q(const MlaQArgs& a, hipStream_t st) {
  hipLaunchKernelGGL(mla_q_kernel, dim3(a.nh, a.B), dim3(64), 0, st, a);
  return hipGetLastError();
}

// ------------------------------------------------------------ MLA query epilogue + W_UK absorption
// Small batches: one block per (head, quarter of the 512 latent columns,
// 16-row group).  Every wave builds the A fragments of the head's q_nope rows
// (bf16, reduced from the q_b split-K partials in split order) directly in
// MFMA lane order -- lane l holds row l % 16, dimensions 8 (l / 16) .. +7 of
// each 32-dimension k-tile -- and multiplies them with the head's packed W_UK
// tiles (16 latent columns x 32 dimensions, one 16-byte word per lane):
// q_lat[b, h] = W_UK[h]^T q_nope[b, h], rounded to bf16.  The blocks of the
// first quarter also rotate q_pe.  The roundings and the k order are those of
// the q epilogue above followed by the weight-streaming GEMM over the heads,
// and the q_nope round trip through memory and one launch are saved.
constexpr int QA_KT = 4;                      // k-tiles of qk_nope_dim = 128
constexpr int QA_NG = 4;                      // latent column groups per head
constexpr int QA_NTW = 512 / 16 / QA_NG / 4;  // latent n-tiles per wave

__global__ __launch_bounds__(256) void mla_q_absorb_kernel(MlaQArgs a, const uint4* __restrict__ wuk,
                                                           int64_t w_bs, bf16_t* __restrict__ q_lat) {
  const int h = blockIdx.x, ng = blockIdx.y, m0 = blockIdx.z * 16;
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  const int dq = a.dn + a.dr;
  const int nt0 = (ng * 4 + wid) * QA_NTW;
  const uint4* __restrict__ W = wuk + (int64_t)h * w_bs;
  uint4 w[QA_NTW][QA_KT];
#pragma unroll
  for (int j = 0; j < QA_NTW; ++j)
#pragma unroll
    for (int kt = 0; kt < QA_KT; ++kt) w[j][kt] = load_nt(&W[((int64_t)(nt0 + j) * QA_KT + kt) * 64 + lane]);
  const int m = m0 + (lane & 15);
  uint4 af[QA_KT];
#pragma unroll
  for (int kt = 0; kt < QA_KT; ++kt) {
    float v[8];
    if (m < a.B) sum8_parts(a.part, a.splits, a.ss, (int64_t)m * a.ldp + (int64_t)h * dq + 32 * kt + 8 * (lane >> 4), v);
    else {
#pragma unroll
      for (int e = 0; e < 8; ++e) v[e] = 0.f;
    }
    af[kt] = pack8bf(v);
  }
  f32x4 acc[QA_NTW];
#pragma unroll
  for (int j = 0; j < QA_NTW; ++j) acc[j] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int kt = 0; kt < QA_KT; ++kt)
#pragma unroll
    for (int j = 0; j < QA_NTW; ++j) acc[j] = mfma16x16x32(af[kt], w[j][kt], acc[j]);
  // D lane layout: column l % 16 of the n-tile, rows 4 (l / 16) .. +3
  const int64_t ldq = (int64_t)a.nh * 512;
#pragma unroll
  for (int j = 0; j < QA_NTW; ++j)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int mm = m0 + 4 * (lane >> 4) + r;
      if (mm < a.B) q_lat[(int64_t)mm * ldq + (int64_t)h * 512 + (nt0 + j) * 16 + (lane & 15)] = f2bf(acc[j][r]);
    }
  if (ng != 0) return;
  const int npair = a.dr / 2;
  for (int i = tid; i < 16 * npair; i += 256) {
    const int mm = m0 + i / npair, p = i % npair;
    if (mm >= a.B) break;
    const int pos = new_token_pos(a.tok_pos, a.ctx_len, a.step, mm);
    const int64_t base = (int64_t)mm * a.ldp + (int64_t)h * dq + a.dn;
    const float x1 = sum_parts(a.part, a.splits, a.ss, base + 2 * p);
    const float x2 = sum_parts(a.part, a.splits, a.ss, base + 2 * p + 1);
    double sd, cd;
    sincos((double)pos * a.rope.inv_freq[p], &sd, &cd);
    const float c = (float)cd, sn = (float)sd;
    bf16_t* o = a.q_pe + ((int64_t)mm * a.nh + h) * a.dr;
    o[2 * p] = f2bf(x1 * c - x2 * sn);
    o[2 * p + 1] = f2bf(x1 * sn + x2 * c);
  }
}

hipError_t launch_mla_q_absorb(const MlaQArgs& a, const uint4* wuk, int64_t w_bs, bf16_t* q_lat, hipStream_t st) {
  // float4 reads of the partials need 4-float alignment of every row, head and slab
  if (a.dn != QA_KT * 32 || a.B < 1 || a.dr % 2 || (a.dn + a.dr) % 4 || a.ldp % 4 || a.ss % 4 ||
      w_bs != (int64_t)(512 / 16) * QA_KT * 64)
    return hipErrorInvalidValue;
  hipLaunchKernelGGL(mla_q_absorb_kernel, dim3(a.nh, QA_NG, (a.B + 15) / 16), dim3(256), 0, st, a, wuk, w_bs, q_lat);
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
    token_out[(int64_t)b * tok_stride] = d2t ? d + d2t[d] : d;
    if (draft_out) draft_out[(int64_t)b * tok_stride] = d;
  }
}

hipError_t launch_argmax_final(const uint64_t* cand, int ncand, int B, const int32_t* d2t,
                               int32_t* token_out, int tok_stride, int32_t* draft_out,
                               hipStream_t st) {
  if (B <= 0 || ncand <= 0) return hipErrorInvalidValue;
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

// ------------------------------------------------------------ extend indexing
// One block per sequence: its new tokens [cu[b], cu[b+1]) get table row b and
// positions ctx_len[b] + j.
__global__ __launch_bounds__(256) void extend_index_kernel(const int32_t* __restrict__ cu,
                                                           const int32_t* __restrict__ ctx_len,
                                                           int32_t* __restrict__ tok_row,
                                                           int32_t* __restrict__ tok_pos) {
  const int b = blockIdx.x;
  const int i0 = cu[b], i1 = cu[b + 1], c = ctx_len[b];
  for (int i = i0 + threadIdx.x; i < i1; i += 256) {
    tok_row[i] = b;
    tok_pos[i] = c + (i - i0);
  }
}

hipError_t launch_extend_index(const int32_t* cu, const int32_t* ctx_len, int B, int32_t* tok_row,
                               int32_t* tok_pos, hipStream_t st) {
  hipLaunchKernelGGL(extend_index_kernel, dim3(B), dim3(256), 0, st, cu, ctx_len, tok_row, tok_pos);
  return hipGetLastError();
}

}  // namespace e3
