// Paged split-KV decode attention of the MLA head in absorbed form, on the
// CDNA4 matrix cores.
//
// With W_UK absorbed into the query (q_lat = W_UK^T q_nope, per head) and
// W_UV applied after attention, every head attends over the same cached
// entries [latent c (512) | rotated k_pe (64)]:
//     s[h, j] = tau * (q_lat[h] . c_j + q_pe[h] . k_pe_j),
//     o_lat[h] = sum_j softmax_j(s[h, :]) c_j.
// One workgroup handles (row, key chunk, group of 16*NW heads); its waves
// take 16 heads each (the N dimension of the MFMAs).  Per tile of 16 keys:
//   S^T[keys x heads] = C[keys x 576] . Q^T        18 x v_mfma 16x16x32
//   O^T[512 x heads] += C^T[512 x keys] . P^T      32 x v_mfma 16x16x16
// The score tile leaves the first product in exactly the B-operand layout of
// the second (lane 16g+j holds keys 4g..4g+3 of head j), so P stays in
// registers.  The cache tile is staged in LDS twice: key-major (A operand of
// the scores, 8 dimensions of one key per lane) and, through an in-register
// 8x8 transpose, dimension-major (A operand of P.V, 4 keys of one dimension
// per lane).  Two LDS buffers and a ring of four register tiles: the global
// loads of the next three tiles are in flight while one tile is computed,
// with one barrier per tile.  Blocks are numbered
// so that the head groups of one (row, chunk) land on the same XCD and share
// its L2.  Chunks are merged by the combine kernel.
#include <math.h>
#include "common.h"
#include "internal.h"

namespace e3 {

namespace {
constexpr int TK = 16;       // keys per tile
constexpr int DQK = 576;     // latent + rope
constexpr int RL = 512;      // latent
constexpr int KSTR = 584;    // key-major row stride (elements): 8 lanes of 16 B hit 32 banks
constexpr int VSTR = 20;     // dim-major row stride (elements): 16 lanes of 8 B hit 32 banks
constexpr int ITEMS = (TK / 8) * (DQK / 8);  // 8x8 blocks per tile (144)
}  // namespace

template <int NW>
__global__ __launch_bounds__(NW * 64) void mla_attn_split_kernel(MlaAttnArgs a, int nhg, int units) {
  __shared__ __attribute__((aligned(16))) bf16_t kt[2][TK * KSTR];
  __shared__ __attribute__((aligned(16))) bf16_t vt[2][RL * VSTR];

  // XCD-aware numbering: the nhg head groups of a unit (row, chunk) are 8
  // block ids apart, and block ids go round-robin over the 8 XCDs.
  const int blk = blockIdx.x;
  const int hg = (blk % (8 * nhg)) / 8;
  const int unit = (blk / (8 * nhg)) * 8 + blk % 8;
  if (unit >= units) return;
  const int b = unit / a.nsplit, s = unit % a.nsplit;

  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  const int col = lane & 15, g = lane >> 4;
  const int n = a.ctx_len[b] + a.step + 1;
  const int k_beg = s * a.chunk;
  const int k_end = min(n, k_beg + a.chunk);
  const int ntiles = k_end > k_beg ? (k_end - k_beg + TK - 1) / TK : 0;
  const int h0 = (hg * NW + wid) * 16;
  const float sl2 = a.scale * 1.4426950408889634f;   // tau * log2(e)

  // Q^T fragments (B operand): column = head h0 + col, dims ks*32 + 8g .. +7
  uint4 qf[DQK / 32];
  {
    const int h = h0 + col;
    const bf16_t* ql = a.q_lat + ((int64_t)b * a.nh + h) * RL;
    const bf16_t* qp = a.q_pe + ((int64_t)b * a.nh + h) * 64;
#pragma unroll
    for (int ks = 0; ks < DQK / 32; ++ks) {
      const int d = ks * 32 + g * 8;
      qf[ks] = d < RL ? *reinterpret_cast<const uint4*>(ql + d)
                      : *reinterpret_cast<const uint4*>(qp + (d - RL));
    }
  }

  f32x4 acc[RL / 16];
#pragma unroll
  for (int i = 0; i < RL / 16; ++i) acc[i] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m = -INFINITY, l = 0.f;

  const int32_t* table = a.table + (int64_t)b * a.max_pages;
  // staging: 8x8 blocks (8 keys x 8 dims), item = tid + k*blockDim, held in
  // registers between their global load and their LDS store.  A ring of RING
  // tiles keeps RING-1 tiles of loads in flight; the page id of a tile (one
  // page per 16-key tile) is read one ring stage before its data.
  constexpr int IPT = (ITEMS + NW * 64 - 1) / (NW * 64);
  constexpr int RING = IPT == 1 ? 4 : 2;       // narrower blocks hold more items per thread
  uint4 row[RING][IPT][8];
  int pgid[RING];
  auto page_of = [&](int t) {
    const int j = k_beg + t * TK;
    return j < k_end ? table[j / a.page_size] : 0;
  };
  auto load_tile = [&](int t, int page, uint4 (&dst)[IPT][8]) {
#pragma unroll
    for (int it = 0; it < IPT; ++it) {
      const int item = tid + it * NW * 64;
      if (item >= ITEMS) break;
      const int kb = item / (DQK / 8), db = item % (DQK / 8);
      const int j0 = k_beg + t * TK + kb * 8;
      const bf16_t* src = a.cache + ((int64_t)page * a.page_size + j0 % a.page_size) * DQK + db * 8;
#pragma unroll
      for (int i = 0; i < 8; ++i)
        dst[it][i] = j0 + i < k_end ? *reinterpret_cast<const uint4*>(src + i * DQK)
                                    : uint4{0u, 0u, 0u, 0u};   // keys past the end contribute nothing
    }
  };
  auto store_tile = [&](int buf, uint4 (&src)[IPT][8]) {
#pragma unroll
    for (int it = 0; it < IPT; ++it) {
      const int item = tid + it * NW * 64;
      if (item >= ITEMS) break;
      const int kb = item / (DQK / 8), db = item % (DQK / 8);
#pragma unroll
      for (int i = 0; i < 8; ++i) *reinterpret_cast<uint4*>(&kt[buf][(kb * 8 + i) * KSTR + db * 8]) = src[it][i];
      if (db < RL / 8) {
#pragma unroll
        for (int d = 0; d < 8; ++d) {
          uint32_t w[4];
#pragma unroll
          for (int k = 0; k < 4; ++k) {
            const uint32_t x = (&src[it][2 * k].x)[d >> 1], y = (&src[it][2 * k + 1].x)[d >> 1];
            w[k] = (d & 1) ? ((x >> 16) | (y & 0xFFFF0000u)) : ((x & 0xFFFFu) | (y << 16));
          }
          bf16_t* dst = &vt[buf][(db * 8 + d) * VSTR + kb * 8];
          *reinterpret_cast<uint2*>(dst) = uint2{w[0], w[1]};
          *reinterpret_cast<uint2*>(dst + 4) = uint2{w[2], w[3]};
        }
      }
    }
  };
  auto compute_tile = [&](int t, int buf) {
    const int j0 = k_beg + t * TK;
    // scores: two accumulators break the dependency chain over k-steps
    f32x4 sa = f32x4{0.f, 0.f, 0.f, 0.f}, sb = sa;
#pragma unroll
    for (int ks = 0; ks < DQK / 32; ks += 2) {
      const uint4 c0 = *reinterpret_cast<const uint4*>(&kt[buf][col * KSTR + ks * 32 + g * 8]);
      const uint4 c1 = *reinterpret_cast<const uint4*>(&kt[buf][col * KSTR + (ks + 1) * 32 + g * 8]);
      sa = mfma16x16x32(c0, qf[ks], sa);
      sb = mfma16x16x32(c1, qf[ks + 1], sb);
    }
    // lane holds keys j0 + 4g + r of head h0 + col
    const int nv = min(4, max(0, k_end - (j0 + 4 * g)));
    float x[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) x[r] = r < nv ? (sa[r] + sb[r]) * sl2 : -INFINITY;
    float mx = fmaxf(fmaxf(x[0], x[1]), fmaxf(x[2], x[3]));
    mx = fmaxf(mx, __shfl_xor(mx, 16, 64));
    mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
    // Lazy rescaling: the reference max m only moves when a head's scores
    // exceed it by more than 2^8, so p stays <= 256 (exact enough in bf16
    // and fp32) and the 128 accumulators are rescaled on a handful of tiles
    // instead of every tile.  m = -inf on the first tile forces a move.
    if (__any(mx > m + 8.f)) {
      const float mn = mx > m + 8.f ? mx : m;       // finite: key j0 is valid
      const float corr = exp2f(m - mn);
      m = mn;
      l *= corr;
#pragma unroll
      for (int i = 0; i < RL / 16; ++i) acc[i] *= corr;
    }
    bf16_t pb[4];
    float ps = 0.f;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      pb[r] = f2bf(exp2f(x[r] - m));
      ps += bf2f(pb[r]);
    }
    l += ps;
    const uint2 pf = uint2{pb[0] | (uint32_t(pb[1]) << 16), pb[2] | (uint32_t(pb[3]) << 16)};
#pragma unroll
    for (int i = 0; i < RL / 16; ++i) {
      const uint2 vf = *reinterpret_cast<const uint2*>(&vt[buf][(i * 16 + col) * VSTR + g * 4]);
      acc[i] = mfma16x16x16(vf, pf, acc[i]);
    }
  };

  // stage t: page id of tile t+RING, loads of tile t+RING-1, compute tile t,
  // then tile t+1 (loaded RING-2 stages ago) goes to the other LDS buffer.
  auto stage = [&](int t, int r) {
    const int rl = (r + RING - 1) % RING, rn = (r + 1) % RING;
    if (t + RING - 1 < ntiles) load_tile(t + RING - 1, pgid[rl], row[rl]);
    if (t + RING < ntiles) pgid[r] = page_of(t + RING);
    compute_tile(t, t & 1);
    if (t + 1 < ntiles) store_tile((t + 1) & 1, row[rn]);
    __syncthreads();
  };
  if (ntiles > 0) {
#pragma unroll
    for (int r = 0; r < RING; ++r) pgid[r] = page_of(r);
#pragma unroll
    for (int r = 0; r < RING - 1; ++r)
      if (r < ntiles) load_tile(r, pgid[r], row[r]);
    store_tile(0, row[0]);
    __syncthreads();
    for (int t = 0; t < ntiles; t += RING) {
#pragma unroll
      for (int r = 0; r < RING; ++r)
        if (t + r < ntiles) stage(t + r, r);
    }
  }

  l += __shfl_xor(l, 16, 64);
  l += __shfl_xor(l, 32, 64);
  // lane holds O^T[dim 16i + 4g + r][head h0 + col]
  const int64_t idx = ((int64_t)b * a.nh + h0 + col) * a.nsplit + s;
  float* po = a.part_o + idx * RL;
#pragma unroll
  for (int i = 0; i < RL / 16; ++i)
    *reinterpret_cast<float4*>(po + i * 16 + 4 * g) = make_float4(acc[i][0], acc[i][1], acc[i][2], acc[i][3]);
  if (g == 0) { a.part_ml[idx * 2] = m; a.part_ml[idx * 2 + 1] = l; }
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

int mla_attn_waves(int nh) { return nh % 64 == 0 ? 4 : (nh % 32 == 0 ? 2 : 1); }

hipError_t launch_mla_attn(const MlaAttnArgs& a, hipStream_t st) {
  if (a.r != RL || a.dr != 64 || a.nh % 16 != 0) return hipErrorInvalidValue;
  const int nw = mla_attn_waves(a.nh);
  const int nhg = a.nh / (16 * nw);
  const int units = a.B * a.nsplit;
  const int blocks = (units + 7) / 8 * 8 * nhg;
  switch (nw) {
    case 4: hipLaunchKernelGGL(mla_attn_split_kernel<4>, dim3(blocks), dim3(256), 0, st, a, nhg, units); break;
    case 2: hipLaunchKernelGGL(mla_attn_split_kernel<2>, dim3(blocks), dim3(128), 0, st, a, nhg, units); break;
    default: hipLaunchKernelGGL(mla_attn_split_kernel<1>, dim3(blocks), dim3(64), 0, st, a, nhg, units); break;
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(mla_attn_combine_kernel, dim3(a.nh, a.B), dim3(256), 0, st, a);
  return hipGetLastError();
}

}  // namespace e3
