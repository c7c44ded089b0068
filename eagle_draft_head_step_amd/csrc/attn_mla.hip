// Paged split-KV decode attention of the MLA head in absorbed form, on the
// CDNA4 matrix cores.
//
// With W_UK absorbed into the query (q_lat = W_UK^T q_nope, per head) and
// W_UV applied after attention, every head attends over the same cached
// entries [latent c (512) | rotated k_pe (64)]:
//     s[h, j] = tau * (q_lat[h] . c_j + q_pe[h] . k_pe_j),
//     o_lat[h] = sum_j softmax_j(s[h, :]) c_j.
// The 16 heads of a wavefront form the M dimension of the MFMAs, so one
// 32-key tile of the cache is read once from HBM per block and used by all
// heads of the block:
//   * the tile is staged twice in LDS: key-major (the B operand of the
//     scores, 8 dims of one key per lane) and, through an in-register 8x8
//     transpose, dim-major (the B operand of P.V, 8 keys of one dim per lane);
//   * scores: 2 x 18 MFMAs (keys 0-15 and 16-31, k = 576 = 18 x 32);
//   * online softmax in fp32, base-2, with the running max per head row;
//   * P (bf16) goes through a small per-wave LDS tile into A-operand layout;
//   * P.V: 32 MFMAs into 16 x 512 fp32 accumulators per wave.
// Chunks of keys are split over blocks; the combine kernel merges them.
#include <math.h>
#include "common.h"
#include "internal.h"

namespace e3 {

namespace {
constexpr int TK = 32;       // keys per tile
constexpr int DQK = 576;     // latent + rope
constexpr int RL = 512;      // latent
constexpr int KSTR = 584;    // key-major row stride (elements)
constexpr int VSTR = 40;     // dim-major row stride (elements)
constexpr int PSTR = 40;     // per-wave P tile row stride (elements)
constexpr int ITEMS = (TK / 8) * (DQK / 8);  // 8x8 blocks per tile
}  // namespace

template <int NW>
__global__ __launch_bounds__(NW * 64) void mla_attn_split_kernel(MlaAttnArgs a) {
  __shared__ __attribute__((aligned(16))) bf16_t kt[TK * KSTR];
  __shared__ __attribute__((aligned(16))) bf16_t vt[RL * VSTR];
  __shared__ __attribute__((aligned(16))) bf16_t pw[NW][16 * PSTR];

  const int s = blockIdx.x, hg = blockIdx.y, b = blockIdx.z;
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  const int col = lane & 15, grp = lane >> 4;
  const int n = a.ctx_len[b] + a.step + 1;
  const int k_beg = s * a.chunk;
  const int k_end = min(n, k_beg + a.chunk);
  const int ntiles = k_end > k_beg ? (k_end - k_beg + TK - 1) / TK : 0;
  const int h0 = (hg * NW + wid) * 16;
  const float sl2 = a.scale * 1.4426950408889634f;   // tau * log2(e)

  // query fragments: row = head h0 + col, dims ks*32 + 8*grp .. +7
  uint4 qf[DQK / 32];
  {
    const int h = h0 + col;
    const bf16_t* ql = a.q_lat + ((int64_t)b * a.nh + h) * RL;
    const bf16_t* qp = a.q_pe + ((int64_t)b * a.nh + h) * 64;
#pragma unroll
    for (int ks = 0; ks < DQK / 32; ++ks) {
      const int d = ks * 32 + grp * 8;
      qf[ks] = d < RL ? *reinterpret_cast<const uint4*>(ql + d)
                      : *reinterpret_cast<const uint4*>(qp + (d - RL));
    }
  }

  f32x4 acc[RL / 16];
#pragma unroll
  for (int i = 0; i < RL / 16; ++i) acc[i] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m[4] = {-INFINITY, -INFINITY, -INFINITY, -INFINITY};
  float l[4] = {0.f, 0.f, 0.f, 0.f};

  const int32_t* table = a.table + (int64_t)b * a.max_pages;
  for (int t = 0; t < ntiles; ++t) {
    const int j0 = k_beg + t * TK;
    // ---- stage the tile: key-major and dim-major copies
    for (int it = tid; it < ITEMS; it += NW * 64) {
      const int db = it % (DQK / 8), kb = it / (DQK / 8);
      uint4 row[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int j = j0 + kb * 8 + i;
        if (j < k_end) {
          const int page = table[j / a.page_size], slot = j % a.page_size;
          row[i] = *reinterpret_cast<const uint4*>(
              a.cache + ((int64_t)page * a.page_size + slot) * DQK + db * 8);
        } else {
          row[i] = uint4{0u, 0u, 0u, 0u};
        }
        *reinterpret_cast<uint4*>(&kt[(kb * 8 + i) * KSTR + db * 8]) = row[i];
      }
      if (db < RL / 8) {
#pragma unroll
        for (int d = 0; d < 8; ++d) {
          uint32_t w[4];
#pragma unroll
          for (int k = 0; k < 4; ++k) {
            const uint32_t x = (&row[2 * k].x)[d >> 1], y = (&row[2 * k + 1].x)[d >> 1];
            w[k] = (d & 1) ? ((x >> 16) | (y & 0xFFFF0000u)) : ((x & 0xFFFFu) | (y << 16));
          }
          *reinterpret_cast<uint4*>(&vt[(db * 8 + d) * VSTR + kb * 8]) = uint4{w[0], w[1], w[2], w[3]};
        }
      }
    }
    __syncthreads();

    // ---- scores for keys j0 + [0, 16) and j0 + [16, 32)
    f32x4 s0 = f32x4{0.f, 0.f, 0.f, 0.f}, s1 = s0;
#pragma unroll
    for (int ks = 0; ks < DQK / 32; ++ks) {
      const int d = ks * 32 + grp * 8;
      const uint4 k0 = *reinterpret_cast<const uint4*>(&kt[col * KSTR + d]);
      const uint4 k1 = *reinterpret_cast<const uint4*>(&kt[(16 + col) * KSTR + d]);
      s0 = mfma16x16x32(qf[ks], k0, s0);
      s1 = mfma16x16x32(qf[ks], k1, s1);
    }
    const bool v0 = j0 + col < k_end, v1 = j0 + 16 + col < k_end;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const float x0 = v0 ? s0[r] * sl2 : -INFINITY;
      const float x1 = v1 ? s1[r] * sl2 : -INFINITY;
      float tm = fmaxf(x0, x1);
#pragma unroll
      for (int o = 1; o < 16; o <<= 1) tm = fmaxf(tm, __shfl_xor(tm, o, 64));
      const float mn = fmaxf(m[r], tm);            // finite: every tile has a valid key
      const float corr = exp2f(m[r] - mn);         // m = -inf -> 0
      const bf16_t p0 = f2bf(exp2f(x0 - mn)), p1 = f2bf(exp2f(x1 - mn));
      l[r] = l[r] * corr + bf2f(p0) + bf2f(p1);
      m[r] = mn;
#pragma unroll
      for (int i = 0; i < RL / 16; ++i) acc[i][r] *= corr;
      pw[wid][(grp * 4 + r) * PSTR + col] = p0;
      pw[wid][(grp * 4 + r) * PSTR + 16 + col] = p1;
    }
    __syncthreads();

    // ---- O += P . V
    const uint4 pf = *reinterpret_cast<const uint4*>(&pw[wid][col * PSTR + grp * 8]);
#pragma unroll
    for (int i = 0; i < RL / 16; ++i) {
      const uint4 vf = *reinterpret_cast<const uint4*>(&vt[(i * 16 + col) * VSTR + grp * 8]);
      acc[i] = mfma16x16x32(pf, vf, acc[i]);
    }
    __syncthreads();
  }

#pragma unroll
  for (int r = 0; r < 4; ++r) {
    float ls = l[r];
#pragma unroll
    for (int o = 1; o < 16; o <<= 1) ls += __shfl_xor(ls, o, 64);
    const int h = h0 + grp * 4 + r;
    const int64_t idx = ((int64_t)b * a.nh + h) * a.nsplit + s;
    float* po = a.part_o + idx * RL;
#pragma unroll
    for (int i = 0; i < RL / 16; ++i) po[i * 16 + col] = acc[i][r];
    if (col == 0) { a.part_ml[idx * 2] = m[r]; a.part_ml[idx * 2 + 1] = ls; }
  }
}

// o_lat[b, h, :] = sum_s o_s 2^{m_s - M} / sum_s l_s 2^{m_s - M}  (bf16)
__global__ __launch_bounds__(256) void mla_attn_combine_kernel(MlaAttnArgs a) {
  const int h = blockIdx.x, b = blockIdx.y;
  const int64_t base = ((int64_t)b * a.nh + h) * a.nsplit;
  float M = -INFINITY;
  for (int s = 0; s < a.nsplit; ++s) M = fmaxf(M, a.part_ml[(base + s) * 2]);
  for (int d = threadIdx.x; d < RL; d += blockDim.x) {
    float L = 0.f, o = 0.f;
    for (int s = 0; s < a.nsplit; ++s) {
      const float ms = a.part_ml[(base + s) * 2];
      if (ms == -INFINITY) continue;
      const float w = exp2f(ms - M);
      L += a.part_ml[(base + s) * 2 + 1] * w;
      o += a.part_o[(base + s) * RL + d] * w;
    }
    a.out[((int64_t)b * a.nh + h) * RL + d] = f2bf(o / L);
  }
}

hipError_t launch_mla_attn(const MlaAttnArgs& a, hipStream_t st) {
  if (a.r != RL || a.dr != 64 || a.nh % 16 != 0) return hipErrorInvalidValue;
  const int nw = a.nh >= 128 ? 8 : (a.nh >= 64 ? 4 : (a.nh >= 32 ? 2 : 1));
  const int nhg = a.nh / (16 * nw);
  if (nhg * 16 * nw != a.nh) return hipErrorInvalidValue;
  dim3 grid(a.nsplit, nhg, a.B);
  switch (nw) {
    case 8: hipLaunchKernelGGL(mla_attn_split_kernel<8>, grid, dim3(512), 0, st, a); break;
    case 4: hipLaunchKernelGGL(mla_attn_split_kernel<4>, grid, dim3(256), 0, st, a); break;
    case 2: hipLaunchKernelGGL(mla_attn_split_kernel<2>, grid, dim3(128), 0, st, a); break;
    default: hipLaunchKernelGGL(mla_attn_split_kernel<1>, grid, dim3(64), 0, st, a); break;
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(mla_attn_combine_kernel, dim3(a.nh, a.B), dim3(256), 0, st, a);
  return hipGetLastError();
}

}  // namespace e3
