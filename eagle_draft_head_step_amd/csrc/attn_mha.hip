// Paged split-KV decode attention for the Llama-style (MHA/GQA) head.
//
// One workgroup per (key chunk, kv head, row).  A key's head_dim values are
// spread over hd/8 lanes (16 bytes each), so each wavefront load instruction
// reads whole cache rows of consecutive slots of one page -- contiguous,
// since a page stores [kv_head][slot][head_dim].  All query heads of the GQA
// group reuse each loaded key and value.  Every lane group runs its own
// online softmax (running max, running sum, rescaled accumulator in fp32);
// groups are merged with shuffles, waves through LDS, and chunks by the
// combine kernel.
#include <math.h>
#include "common.h"
#include "internal.h"

namespace e3 {

__device__ __forceinline__ void merge_state(float& m, float& l, float* o, float m2, float l2,
                                            const float* o2, int n) {
  const float mn = fmaxf(m, m2);
  if (mn == -INFINITY) return;
  const float a = expf(m - mn), b = expf(m2 - mn);
  l = l * a + l2 * b;
  for (int i = 0; i < n; ++i) o[i] = o[i] * a + o2[i] * b;
  m = mn;
}

template <int HD, int G>
__global__ __launch_bounds__(256) void mha_attn_split_kernel(MhaAttnArgs a) {
  constexpr int LPK = HD / 8;                        // lanes per key
  constexpr int KPW = 64 / LPK;                      // keys per wave per load instruction
  constexpr int U = KPW * 8 <= 64 ? 8 : 64 / KPW;    // keys per lane per step
  constexpr int STEP = KPW * U;                      // keys per wave per step
  __shared__ float sm_m[4][G], sm_l[4][G];
  __shared__ float sm_o[4][G][HD];

  const int s = blockIdx.x, kvh = blockIdx.y, b = blockIdx.z;
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  const int ks = lane / LPK, db = lane % LPK;
  const int n = a.ctx_len[b] + a.step + 1;                  // keys incl. the new one
  const int k_beg = s * a.chunk, k_end = min(n, k_beg + a.chunk);

  float q[G][8];
#pragma unroll
  for (int g = 0; g < G; ++g) {
    const float* qp = a.q + ((int64_t)b * a.nq + kvh * G + g) * HD + db * 8;
#pragma unroll
    for (int e = 0; e < 8; ++e) q[g][e] = qp[e] * a.scale;
  }
  float m[G], l[G], o[G][8];
#pragma unroll
  for (int g = 0; g < G; ++g) {
    m[g] = -INFINITY;
    l[g] = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) o[g][e] = 0.f;
  }

  const int32_t* table = a.table + (int64_t)b * a.max_pages;
  for (int base = k_beg + wid * STEP; base < k_end; base += 4 * STEP) {
    // issue every load of the step before using any of them
    uint4 kr[U], vr[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int j = base + u * KPW + ks;
      if (j < k_end) {
        const int page = table[j / a.page_size];
        const int64_t off =
            (((int64_t)page * a.nkv + kvh) * a.page_size + (j % a.page_size)) * HD + db * 8;
        kr[u] = *reinterpret_cast<const uint4*>(a.k_cache + off);
        vr[u] = *reinterpret_cast<const uint4*>(a.v_cache + off);
      } else {
        kr[u] = uint4{0u, 0u, 0u, 0u};
        vr[u] = kr[u];
      }
    }
    float sc[G][U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      float kf[8];
      unpack8(kr[u], kf);
      const bool valid = base + u * KPW + ks < k_end;
#pragma unroll
      for (int g = 0; g < G; ++g) {
        float t = 0.f;
#pragma unroll
        for (int e = 0; e < 8; ++e) t += q[g][e] * kf[e];
#pragma unroll
        for (int w = 1; w < LPK; w <<= 1) t += __shfl_xor(t, w, 64);
        sc[g][u] = valid ? t : -INFINITY;
      }
    }
#pragma unroll
    for (int g = 0; g < G; ++g) {
      float mx = sc[g][0];
#pragma unroll
      for (int u = 1; u < U; ++u) mx = fmaxf(mx, sc[g][u]);
      const float mn = fmaxf(m[g], mx);
      if (mn == -INFINITY) continue;                 // nothing valid yet for this lane group
      const float corr = expf(m[g] - mn);
      l[g] *= corr;
#pragma unroll
      for (int e = 0; e < 8; ++e) o[g][e] *= corr;
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const float p = expf(sc[g][u] - mn);
        float vf[8];
        unpack8(vr[u], vf);
        l[g] += p;
#pragma unroll
        for (int e = 0; e < 8; ++e) o[g][e] += p * vf[e];
      }
      m[g] = mn;
    }
  }
  // merge the KPW key slots of this wave (lanes differing in ks)
#pragma unroll
  for (int w = LPK; w < 64; w <<= 1) {
#pragma unroll
    for (int g = 0; g < G; ++g) {
      const float m2 = __shfl_xor(m[g], w, 64), l2 = __shfl_xor(l[g], w, 64);
      float o2[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) o2[e] = __shfl_xor(o[g][e], w, 64);
      merge_state(m[g], l[g], o[g], m2, l2, o2, 8);
    }
  }
  if (ks == 0) {
#pragma unroll
    for (int g = 0; g < G; ++g) {
      if (db == 0) { sm_m[wid][g] = m[g]; sm_l[wid][g] = l[g]; }
#pragma unroll
      for (int e = 0; e < 8; ++e) sm_o[wid][g][db * 8 + e] = o[g][e];
    }
  }
  __syncthreads();
  for (int t = threadIdx.x; t < G * HD; t += 256) {
    const int g = t / HD, d = t % HD;
    float mm = -INFINITY, ll = 0.f, oo = 0.f;
    for (int w = 0; w < 4; ++w) {
      const float m2 = sm_m[w][g];
      const float mn = fmaxf(mm, m2);
      if (mn == -INFINITY) continue;
      const float x = expf(mm - mn), y = expf(m2 - mn);
      ll = ll * x + sm_l[w][g] * y;
      oo = oo * x + sm_o[w][g][d] * y;
      mm = mn;
    }
    const int h = kvh * G + g;
    const int64_t idx = ((int64_t)b * a.nq + h) * a.nsplit + s;
    a.part_o[idx * HD + d] = oo;
    if (d == 0) { a.part_ml[idx * 2] = mm; a.part_ml[idx * 2 + 1] = ll; }
  }
}

// out[b, h, :] = sum_s o_s e^{m_s - M} / sum_s l_s e^{m_s - M}
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
      const float w = expf(ms - M);
      L += a.part_ml[(base + s) * 2 + 1] * w;
      o += a.part_o[(base + s) * a.hd + d] * w;
    }
    a.out[((int64_t)b * a.nq + h) * a.hd + d] = o / L;
  }
}

template <int HD, int G>
static hipError_t launch_split(const MhaAttnArgs& a, hipStream_t st) {
  hipLaunchKernelGGL((mha_attn_split_kernel<HD, G>), dim3(a.nsplit, a.nkv, a.B), dim3(256), 0, st, a);
  return hipGetLastError();
}

template <int HD>
static hipError_t launch_hd(const MhaAttnArgs& a, int G, hipStream_t st) {
  switch (G) {
    case 1: return launch_split<HD, 1>(a, st);
    case 2: return launch_split<HD, 2>(a, st);
    case 3: return launch_split<HD, 3>(a, st);
    case 4: return launch_split<HD, 4>(a, st);
    case 5: return launch_split<HD, 5>(a, st);
    case 6: return launch_split<HD, 6>(a, st);
    case 7: return launch_split<HD, 7>(a, st);
    case 8: return launch_split<HD, 8>(a, st);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_mha_attn(const MhaAttnArgs& a, hipStream_t st) {
  const int G = a.nq / a.nkv;
  hipError_t e;
  switch (a.hd) {
    case 32: e = launch_hd<32>(a, G, st); break;
    case 64: e = launch_hd<64>(a, G, st); break;
    case 128: e = launch_hd<128>(a, G, st); break;
    default: return hipErrorInvalidValue;
  }
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(mha_attn_combine_kernel, dim3(a.nq, a.B), dim3(128), 0, st, a);
  return hipGetLastError();
}

}  // namespace e3
