// Paged split-KV decode attention for the Llama-style (MHA/GQA) head, on the
// CDNA4 matrix cores.
//
// One workgroup per (key chunk, kv head, row); each wavefront takes tiles of
// 32 keys.  The query heads of the GQA group form the N dimension (padded to
// 16) of two MFMA products per tile:
//   S^T[keys x heads] = K[keys x hd] . Q^T        (2 x hd/32 MFMAs, Q split
//                                                    into bf16 hi + lo parts)
//   O^T[hd x heads]  += V^T[hd x keys] . P^T       (hd/16 MFMAs)
// The score tile comes out of the first MFMA already in the B-operand layout
// the second needs (each lane holds 8 keys of one head), so P never leaves
// the registers.  K pages are [slot][hd] (a lane reads 64 contiguous bytes of
// one key); V pages are stored dimension-major [hd][slot], so a lane reads
// 4 consecutive keys of one dimension twice (keys 4g..4g+3 and 16+4g..).
// Online softmax in fp32, base 2, one running max and sum per head.
#include <math.h>
#include "common.h"
#include "internal.h"

namespace e3 {

template <int HD>
__global__ __launch_bounds__(256) void mha_attn_split_kernel(MhaAttnArgs a) {
  constexpr int KS = HD / 32;      // k-steps of the score product
  constexpr int DT = HD / 16;      // 16-dim tiles of the output
  __shared__ float sm_m[4][16], sm_l[4][16];
  __shared__ float sm_o[4][HD][17];

  const int s = blockIdx.x, kvh = blockIdx.y, b = blockIdx.z;
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  const int col = lane & 15, g = lane >> 4;
  const int G = a.nq / a.nkv;
  const int P = a.page_size;
  const int n = a.ctx_len[b] + a.step + 1;                  // keys incl. the new one
  const int k_beg = s * a.chunk, k_end = min(n, k_beg + a.chunk);

  // Q^T as the B operand: column = head col (zero beyond the group), k-slots
  // of lane group g hold dims g*HD/4 + ks*8 .. +7 (the K tile uses the same order).
  uint4 qh[KS], ql[KS];
  {
    const float qs = a.scale * 1.4426950408889634f;        // base-2 softmax
    const float* qp = a.q + ((int64_t)b * a.nq + kvh * G + col) * HD;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const int d = g * (HD / 4) + ks * 8;
      float4 x0 = make_float4(0.f, 0.f, 0.f, 0.f), x1 = x0;
      if (col < G) {
        x0 = *reinterpret_cast<const float4*>(qp + d);
        x1 = *reinterpret_cast<const float4*>(qp + d + 4);
        x0.x *= qs; x0.y *= qs; x0.z *= qs; x0.w *= qs;
        x1.x *= qs; x1.y *= qs; x1.z *= qs; x1.w *= qs;
      }
      split_bf16x8(x0, x1, qh[ks], ql[ks]);
    }
  }
  f32x4 acc[DT];
#pragma unroll
  for (int i = 0; i < DT; ++i) acc[i] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m = -INFINITY, l = 0.f;

  const int32_t* table = a.table + (int64_t)b * a.max_pages;
  for (int t0 = k_beg + wid * 32; t0 < k_end; t0 += 4 * 32) {
    const int page = table[t0 / P], slot0 = t0 % P;          // 32 keys in one page
    const bf16_t* kp = a.k_cache + (((int64_t)page * a.nkv + kvh) * P + slot0) * HD + g * (HD / 4);
    const bf16_t* vp = a.v_cache + ((int64_t)page * a.nkv + kvh) * HD * P + slot0 + 4 * g;
    uint4 k0[KS], k1[KS];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      k0[ks] = *reinterpret_cast<const uint4*>(kp + (int64_t)col * HD + ks * 8);
      k1[ks] = *reinterpret_cast<const uint4*>(kp + (int64_t)(16 + col) * HD + ks * 8);
    }
    uint2 v0[DT], v1[DT];
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) {
      const bf16_t* vr = vp + (int64_t)(dt * 16 + col) * P;
      v0[dt] = *reinterpret_cast<const uint2*>(vr);
      v1[dt] = *reinterpret_cast<const uint2*>(vr + 16);
    }
    f32x4 s0 = f32x4{0.f, 0.f, 0.f, 0.f}, s1 = s0;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      s0 = mfma16x16x32(k0[ks], qh[ks], s0);
      s0 = mfma16x16x32(k0[ks], ql[ks], s0);
      s1 = mfma16x16x32(k1[ks], qh[ks], s1);
      s1 = mfma16x16x32(k1[ks], ql[ks], s1);
    }
    // lane holds keys t0 + 4g + r (s0) and t0 + 16 + 4g + r (s1) of head col
    const int nv0 = min(4, max(0, k_end - (t0 + 4 * g)));        // valid keys in each group of 4
    const int nv1 = min(4, max(0, k_end - (t0 + 16 + 4 * g)));
    float x[8];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      x[r] = r < nv0 ? s0[r] : -INFINITY;
      x[4 + r] = r < nv1 ? s1[r] : -INFINITY;
    }
    float mx = x[0];
#pragma unroll
    for (int e = 1; e < 8; ++e) mx = fmaxf(mx, x[e]);
    mx = fmaxf(mx, __shfl_xor(mx, 16, 64));
    mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
    const float mn = fmaxf(m, mx);                 // finite: key t0 is valid
    const float corr = exp2f(m - mn);
    m = mn;
    bf16_t pb[8];
    float ps = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      pb[e] = f2bf(exp2f(x[e] - mn));
      ps += bf2f(pb[e]);
    }
    l = l * corr + ps;
    const uint4 pf = uint4{pb[0] | (uint32_t(pb[1]) << 16), pb[2] | (uint32_t(pb[3]) << 16),
                           pb[4] | (uint32_t(pb[5]) << 16), pb[6] | (uint32_t(pb[7]) << 16)};
    // keys past the row's end have p = 0; their cache bytes may be anything
    const uint32_t m0 = nv0 >= 4 ? 0xFFFFFFFFu : (nv0 == 3 ? 0x0000FFFFu : 0u);
    const uint32_t m0l = nv0 >= 2 ? 0xFFFFFFFFu : (nv0 == 1 ? 0x0000FFFFu : 0u);
    const uint32_t m1 = nv1 >= 4 ? 0xFFFFFFFFu : (nv1 == 3 ? 0x0000FFFFu : 0u);
    const uint32_t m1l = nv1 >= 2 ? 0xFFFFFFFFu : (nv1 == 1 ? 0x0000FFFFu : 0u);
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) {
      const uint4 vf = uint4{v0[dt].x & m0l, v0[dt].y & m0, v1[dt].x & m1l, v1[dt].y & m1};
      acc[dt] *= corr;
      acc[dt] = mfma16x16x32(vf, pf, acc[dt]);
    }
  }
  l += __shfl_xor(l, 16, 64);
  l += __shfl_xor(l, 32, 64);
  // lane holds O^T[dim dt*16 + 4g + r][head col] of this wave's keys
  if (g == 0) { sm_m[wid][col] = m; sm_l[wid][col] = l; }
#pragma unroll
  for (int dt = 0; dt < DT; ++dt)
#pragma unroll
    for (int r = 0; r < 4; ++r) sm_o[wid][dt * 16 + 4 * g + r][col] = acc[dt][r];
  __syncthreads();
  for (int t = threadIdx.x; t < G * HD; t += 256) {
    const int h = t / HD, d = t % HD;
    float mm = -INFINITY, ll = 0.f, oo = 0.f;
    for (int w = 0; w < 4; ++w) {
      const float m2 = sm_m[w][h];
      const float mn = fmaxf(mm, m2);
      if (mn == -INFINITY) continue;
      const float x = exp2f(mm - mn), y = exp2f(m2 - mn);
      ll = ll * x + sm_l[w][h] * y;
      oo = oo * x + sm_o[w][d][h] * y;
      mm = mn;
    }
    const int64_t idx = ((int64_t)b * a.nq + kvh * G + h) * a.nsplit + s;
    a.part_o[idx * HD + d] = oo;
    if (d == 0) { a.part_ml[idx * 2] = mm; a.part_ml[idx * 2 + 1] = ll; }
  }
}

// out[b, h, :] = sum_s o_s 2^{m_s - M} / sum_s l_s 2^{m_s - M}  (bf16)
__global__ __launch_bounds__(128) void mha_attn_combine_kernel(MhaAttnArgs a) {
  const int h = blockIdx.x, b = blockIdx.y;
  const int64_t base = ((int64_t)b * a.nq + h) * a.nsplit;
  float M = -INFINITY;
  for (int s = 0; s < a.nsplit; ++s) M = fmaxf(M, a.part_ml[(base + s) * 2]);
  for (int d = threadIdx.x; d < a.hd; d += blockDim.x) {
    float L = 0.f, o = 0.f;
    for (int s = 0; s < a.nsplit; ++s) {
      const float ms = a.part_ml[(base + s) * 2];
      if (ms == -INFINITY) continue;
      const float w = exp2f(ms - M);
      L += a.part_ml[(base + s) * 2 + 1] * w;
      o += a.part_o[(base + s) * a.hd + d] * w;
    }
    a.out[((int64_t)b * a.nq + h) * a.hd + d] = f2bf(o / L);
  }
}

hipError_t launch_mha_attn(const MhaAttnArgs& a, hipStream_t st) {
  if (a.nq % a.nkv || a.nq / a.nkv > 16 || a.page_size % 32 || a.chunk % 32) return hipErrorInvalidValue;
  dim3 grid(a.nsplit, a.nkv, a.B);
  switch (a.hd) {
    case 32: hipLaunchKernelGGL(mha_attn_split_kernel<32>, grid, dim3(256), 0, st, a); break;
    case 64: hipLaunchKernelGGL(mha_attn_split_kernel<64>, grid, dim3(256), 0, st, a); break;
    case 128: hipLaunchKernelGGL(mha_attn_split_kernel<128>, grid, dim3(256), 0, st, a); break;
    default: return hipErrorInvalidValue;
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(mha_attn_combine_kernel, dim3(a.nq, a.B), dim3(128), 0, st, a);
  return hipGetLastError();
}

}  // namespace e3
