// Paged split-KV decode attention for the Llama-style (MHA/GQA) head, on the
// CDNA4 matrix cores.
//
// One workgroup of NW wavefronts per (key chunk, kv head, row); each wavefront
// takes tiles of 16 keys, with the next two tiles' loads in flight while it
// computes one.  When the batch alone gives every CU a (row, kv head), one
// 8-wave workgroup takes the whole row and writes the output directly;
// otherwise 4-wave workgroups split the keys and a combine kernel merges them.  The
// query heads of the GQA group form the N dimension (padded to 16) of two
// MFMA products per tile:
//   S^T[keys x heads] = K[keys x hd] . Q^T     (v_mfma 16x16x32, hd/32 steps,
//                                               Q split into bf16 hi + lo)
//   O^T[hd x heads]  += V^T[hd x keys] . P^T    (v_mfma 16x16x16, hd/16 tiles)
// The score tile comes out of the first product in exactly the B-operand
// layout of the second (lane 16g+j holds keys 4g..4g+3 of head j), so P never
// leaves the registers.  The cache pages are laid out so that every operand
// load of a wave reads one contiguous KiB (whole cache lines, each line read
// by one instruction): K pages are [hd/32][slot][32] (lane (key, g) reads
// dims 32ks + 8g .. +7 of its key); V pages are [hd/32][slot/16][16 dimension
// pairs][16 slots][2], so one 16-byte load gives a lane 4 consecutive keys of
// two dimensions (a 16-byte load per lane streams at full HBM rate, an 8-byte
// one does not); the pair is split in registers into the A operands of two
// MFMAs.
// Online softmax in fp32, base 2, one running max and sum per head.
#include <math.h>
#include "common.h"
#include "internal.h"

namespace e3 {

template <int HD, int NW>
__global__ __launch_bounds__(64 * NW) void mha_attn_split_kernel(MhaAttnArgs a) {
  constexpr int KS = HD / 32;      // k-steps of the score product
  constexpr int DT = HD / 16;      // 16-dim tiles of the output
  constexpr int R = 16 * NW;       // keys per round of the workgroup's waves
  __shared__ float sm_m[NW][16], sm_l[NW][16];
  __shared__ float sm_o[NW][HD][17];

  const int s = blockIdx.x, kvh = blockIdx.y, b = blockIdx.z;
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  const int col = lane & 15, g = lane >> 4;
  const int G = a.nq / a.nkv;
  const int P = a.page_size;
  const int n = new_token_pos(a.tok_pos, a.ctx_len, a.step, b) + 1;   // keys incl. the new one
  const int trow = table_row(a.tok_row, b);
  const int k_beg = s * a.chunk, k_end = min(n, k_beg + a.chunk);

  // Whole-row blocks of a plain step do the q/k/v epilogue themselves: this
  // block is the only reader of its kv head's cache for this row, so it can
  // append the new entry and then attend over it.  The entry's stores
  // complete before any tile load is issued, and no line of it was read
  // before, so the loads see it.
  constexpr int QR = NW == 8 ? 16 : 1;
  __shared__ float sm_q[QR][HD];
  const bool fused = NW == 8 && a.part != nullptr;
  if constexpr (NW == 8) {
    if (fused) {
      constexpr int half = HD / 2;
      const int pos = n - 1;
      const int page = a.table[(int64_t)trow * a.max_pages + pos / P], slot = pos % P;
      const int64_t pbase = ((int64_t)page * a.nkv + kvh) * HD * P;
      for (int t = threadIdx.x; t < (G + 2) * half; t += 64 * NW) {
        const int hh = t / half, i = t % half;     // hh < G: q head; G: k; G + 1: v
        const int head = hh < G ? kvh * G + hh : (hh == G ? a.nq + kvh : a.nq + a.nkv + kvh);
        const int64_t idx = (int64_t)b * a.ldp + (int64_t)head * HD + i;
        float x1 = 0.f, x2 = 0.f;                  // split-K sums, in split order
        for (int s0 = 0; s0 < a.splits; s0 += 4) {
          float t1[4], t2[4];
#pragma unroll
          for (int u = 0; u < 4; ++u) {
            const bool ok = s0 + u < a.splits;
            t1[u] = ok ? a.part[(int64_t)(s0 + u) * a.ss + idx] : 0.f;
            t2[u] = ok ? a.part[(int64_t)(s0 + u) * a.ss + idx + half] : 0.f;
          }
#pragma unroll
          for (int u = 0; u < 4; ++u) { x1 += t1[u]; x2 += t2[u]; }
        }
        if (hh == G + 1) {
          // V page: [dim / 32][slot / 16][(dim / 2) % 16][slot % 16][dim % 2]
          auto at = [&](int d) {
            return ((((int64_t)(d >> 5) * (P >> 4) + (slot >> 4)) * 16 + ((d >> 1) & 15)) * 16 + (slot & 15)) * 2 +
                   (d & 1);
          };
          a.v_app[pbase + at(i)] = f2bf(x1);
          a.v_app[pbase + at(i + half)] = f2bf(x2);
          continue;
        }
        double sd, cd;
        sincos((double)pos * a.rope.inv_freq[i], &sd, &cd);
        const float c = (float)cd, sn = (float)sd;
        const float y1 = x1 * c - x2 * sn, y2 = x1 * sn + x2 * c;
        if (hh < G) {
          sm_q[hh][i] = y1;
          sm_q[hh][i + half] = y2;
        } else {
          // K page: [dim / 32][slot][dim % 32]
          bf16_t* k = a.k_app + pbase + (int64_t)slot * 32;
          k[(int64_t)(i >> 5) * P * 32 + (i & 31)] = f2bf(y1);
          k[(int64_t)((i + half) >> 5) * P * 32 + ((i + half) & 31)] = f2bf(y2);
        }
      }
      __builtin_amdgcn_s_waitcnt(0);               // the entry's stores have completed
      __syncthreads();
    }
  }

  // Q^T as the B operand: column = head col (zero beyond the group), k-slots
  // of lane group g hold dims 32*ks + 8*g .. +7 (the K tile uses the same order).
  uint4 qh[KS], ql[KS];
  {
    const float qs = a.scale * 1.4426950408889634f;        // base-2 softmax
    const float* qp = fused ? &sm_q[col < QR ? col : 0][0] : a.q + ((int64_t)b * a.nq + kvh * G + col) * HD;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const int d = ks * 32 + g * 8;
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

  const int32_t* table = a.table + (int64_t)trow * a.max_pages;
  struct Tile { uint4 k[KS]; uint4 v[DT / 2]; };
  // issue every load of the 16-key tile starting at t0 (within one page)
  auto load_tile = [&](int t0, Tile& T) {
    const int page = table[t0 / P], slot0 = t0 % P;
    const int64_t pbase = ((int64_t)page * a.nkv + kvh) * HD * P;
    // K page: [dim chunk][slot][32]; lane reads dims 32ks + 8g .. +7 of key slot0 + col
    const bf16_t* kp = a.k_cache + pbase + (slot0 + col) * 32 + g * 8;
    // V page: [dim chunk][slot / 16][pair][slot % 16][2]; lane reads keys
    // 4g..4g+3 of dimension pair 16*d2 + col
    const bf16_t* vp = a.v_cache + pbase + ((slot0 >> 4) * 16 + col) * 32 + g * 8;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) T.k[ks] = *reinterpret_cast<const uint4*>(kp + (int64_t)ks * P * 32);
#pragma unroll
    for (int d2 = 0; d2 < DT / 2; ++d2)
      T.v[d2] = *reinterpret_cast<const uint4*>(vp + (int64_t)d2 * (P / 16) * 512);
  };
  auto process_tile = [&](int t0, const Tile& T) {
    f32x4 s0 = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      s0 = mfma16x16x32(T.k[ks], qh[ks], s0);
      s0 = mfma16x16x32(T.k[ks], ql[ks], s0);
    }
    // lane holds keys t0 + 4g + r of head col
    const int nv = min(4, max(0, k_end - (t0 + 4 * g)));
    float x[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) x[r] = r < nv ? s0[r] : -INFINITY;
    float mx = fmaxf(fmaxf(x[0], x[1]), fmaxf(x[2], x[3]));
    mx = fmaxf(mx, __shfl_xor(mx, 16, 64));
    mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
    const float mn = fmaxf(m, mx);                 // finite: key t0 is valid
    const float corr = exp2f(m - mn);
    m = mn;
    bf16_t pb[4];
    float ps = 0.f;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      pb[r] = f2bf(exp2f(x[r] - mn));
      ps += bf2f(pb[r]);
    }
    l = l * corr + ps;
    const uint2 pf = uint2{pb[0] | (uint32_t(pb[1]) << 16), pb[2] | (uint32_t(pb[3]) << 16)};
    // keys past the row's end have p = 0; their cache bytes may be anything
    const uint32_t mh = nv >= 4 ? 0xFFFFFFFFu : (nv == 3 ? 0x0000FFFFu : 0u);
    const uint32_t ml = nv >= 2 ? 0xFFFFFFFFu : (nv == 1 ? 0x0000FFFFu : 0u);
#pragma unroll
    for (int d2 = 0; d2 < DT / 2; ++d2) {
      const uint4 w = T.v[d2];       // (key, dim-pair) interleaved: lo half even dim, hi half odd
      const uint2 ve = uint2{((w.x & 0xFFFFu) | (w.y << 16)) & ml, ((w.z & 0xFFFFu) | (w.w << 16)) & mh};
      const uint2 vo = uint2{((w.x >> 16) | (w.y & 0xFFFF0000u)) & ml, ((w.z >> 16) | (w.w & 0xFFFF0000u)) & mh};
      acc[2 * d2] *= corr;
      acc[2 * d2] = mfma16x16x16(ve, pf, acc[2 * d2]);
      acc[2 * d2 + 1] *= corr;
      acc[2 * d2 + 1] = mfma16x16x16(vo, pf, acc[2 * d2 + 1]);
    }
  };
  // wave tiles t0 = k_beg + 16*wid + R*i; the loads of the next two tiles
  // are in flight while the current one is processed
  Tile tr[3];
  const int tb0 = k_beg + wid * 16;
  if (tb0 < k_end) load_tile(tb0, tr[0]);
  if (tb0 + R < k_end) load_tile(tb0 + R, tr[1]);
  for (int t0 = tb0; t0 < k_end; t0 += 3 * R) {
    if (t0 + 2 * R < k_end) load_tile(t0 + 2 * R, tr[2]);
    process_tile(t0, tr[0]);
    if (t0 + R >= k_end) break;
    if (t0 + 3 * R < k_end) load_tile(t0 + 3 * R, tr[0]);
    process_tile(t0 + R, tr[1]);
    if (t0 + 2 * R >= k_end) break;
    if (t0 + 4 * R < k_end) load_tile(t0 + 4 * R, tr[1]);
    process_tile(t0 + 2 * R, tr[2]);
  }
  l += __shfl_xor(l, 16, 64);
  l += __shfl_xor(l, 32, 64);
  // acc[2*d2 + par] row 4g + r holds O^T[dim 2*(16*d2 + 4g + r) + par][head col]
  if (g == 0) { sm_m[wid][col] = m; sm_l[wid][col] = l; }
#pragma unroll
  for (int dt = 0; dt < DT; ++dt)
#pragma unroll
    for (int r = 0; r < 4; ++r) sm_o[wid][2 * ((dt >> 1) * 16 + 4 * g + r) + (dt & 1)][col] = acc[dt][r];
  __syncthreads();
  const bool single = a.nsplit == 1;
  for (int t = threadIdx.x; t < G * HD; t += 64 * NW) {
    const int h = t / HD, d = t % HD;
    float mm = -INFINITY, ll = 0.f, oo = 0.f;
    for (int w = 0; w < NW; ++w) {
      const float m2 = sm_m[w][h];
      const float mn = fmaxf(mm, m2);
      if (mn == -INFINITY) continue;
      const float x = exp2f(mm - mn), y = exp2f(m2 - mn);
      ll = ll * x + sm_l[w][h] * y;
      oo = oo * x + sm_o[w][d][h] * y;
      mm = mn;
    }
    if (single) {                      // the whole row: the output itself
      a.out[((int64_t)b * a.nq + kvh * G + h) * HD + d] = f2bf(oo / ll);
      continue;
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
  if (a.nq % a.nkv || a.nq / a.nkv > 16 || a.page_size % 16 || (a.nw != 4 && a.nw != 8) ||
      a.chunk % (16 * a.nw) || a.nsplit < 1 || (a.nw == 8 && a.nsplit != 1) ||
      (a.part && (a.nw != 8 || a.tok_pos || !a.k_app || !a.v_app || a.splits < 1)))
    return hipErrorInvalidValue;
  dim3 grid(a.nsplit, a.nkv, a.B);
#define E3_MHA_LAUNCH(HDV, NWV) \
  hipLaunchKernelGGL((mha_attn_split_kernel<HDV, NWV>), grid, dim3(64 * NWV), 0, st, a)
  if (a.nw == 8) {
    switch (a.hd) {
      case 32: E3_MHA_LAUNCH(32, 8); break;
      case 64: E3_MHA_LAUNCH(64, 8); break;
      case 128: E3_MHA_LAUNCH(128, 8); break;
      default: return hipErrorInvalidValue;
    }
  } else {
    switch (a.hd) {
      case 32: E3_MHA_LAUNCH(32, 4); break;
      case 64: E3_MHA_LAUNCH(64, 4); break;
      case 128: E3_MHA_LAUNCH(128, 4); break;
      default: return hipErrorInvalidValue;
    }
  }
#undef E3_MHA_LAUNCH
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || a.nsplit == 1) return e;
  hipLaunchKernelGGL(mha_attn_combine_kernel, dim3(a.nq, a.B), dim3(128), 0, st, a);
  return hipGetLastError();
}

}  // namespace e3
