// Weight-streaming bf16 GEMM on CDNA4 matrix cores (v_mfma_f32_16x16x32_bf16).
//
// The draft head's projections are "skinny": M = batch rows (1..256) against
// weights of up to 129280 x 7168.  Every weight byte is read from HBM once,
// so the kernel is built around the weight stream:
//   * weights are pre-packed into 16 (n) x 32 (k) tiles of 1 KiB stored in
//     MFMA lane order, so one 16-byte load per lane fetches one tile fully
//     coalesced, straight into the B-operand registers;
//   * a workgroup of 4 wavefronts shares one K range; the activation rows for
//     a stage of KC k-tiles are staged once into LDS (in lane order, so every
//     ds_read_b128 is conflict free) and reused by all 4 waves;
//   * fp32 activations are split into bf16 high and low parts (x = hi + lo
//     to 2^-17 relative) and both go through the MFMA, so activations keep
//     fp32-level precision where bf16 rounding would cost accuracy;
//   * each wave owns NTW n-tiles and MT/WM m-tiles of accumulators: with
//     WM = 1 all four waves span the block's rows; with WM = 2 (large batch)
//     the waves form a 2 x 2 grid, so every activation fragment read from LDS
//     feeds NTW MFMAs with half the accumulators, and two waves per SIMD fit
//     (the pair that shares n-tiles loads the same weight tiles, the second
//     read served by the caches);
//   * the weights of the next two stages stream into a register ring while
//     the current stage's MFMAs run;
//   * split-K partials are stored in fp32 and reduced by the consumer kernel
//     in a fixed order (deterministic, no atomics); the lm_head variant
//     reduces to one (value, index) candidate per block and row instead;
//   * quantized weights (WQ = 1 FP8 E4M3, 2 NVFP4) keep the same 1 KiB lane
//     words, which then span 2 or 4 k-tiles: each word is widened to MFMA
//     operands in registers by the gfx950 converts, exactly (E4M3 values are
//     bf16 values; E2M1 x E4M3-block-scale products are f16 values, so the
//     NVFP4 instance runs f16 MFMAs on activations staged as f16 hi + lo) and
//     the fp32 row scale multiplies the accumulator in the epilogue, so the
//     activations keep their precision and only weight bytes shrink.
#include "common.h"
#include "internal.h"

#include <algorithm>

namespace e3 {

namespace {
typedef __bf16 bf16x2v __attribute__((ext_vector_type(2)));

__device__ __forceinline__ uint32_t bf2_bits(bf16x2v v) { return __builtin_bit_cast(uint32_t, v); }

// Eight E4M3 weights (k order, 4 per word) -> eight bf16 (an MFMA operand).
__device__ __forceinline__ uint4 fp8x8_to_bf16(uint32_t lo, uint32_t hi) {
  return uint4{bf2_bits(__builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(lo, 1.0f, false)),
               bf2_bits(__builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(lo, 1.0f, true)),
               bf2_bits(__builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(hi, 1.0f, false)),
               bf2_bits(__builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(hi, 1.0f, true))};
}

typedef _Float16 f16x2v __attribute__((ext_vector_type(2)));
typedef _Float16 f16x8v __attribute__((ext_vector_type(8)));

__device__ __forceinline__ uint32_t f16x2_bits(f16x2v v) { return __builtin_bit_cast(uint32_t, v); }

// Eight E2M1 weights (k order, low nibble first) times their E4M3 block
// scale s -> f16.  The scaled converts use only the exponent of their fp32
// scale operand (an E8M0-style power of two), so they apply 2^floor(log2 s)
// and one packed f16 multiply applies the rest of s (1 + m/8, 3 fraction
// bits).  Every step is exact: E2M1 x s has at most 6 significant bits and
// lies in [2^-10, 2880], inside f16's normal range.
__device__ __forceinline__ uint4 fp4x8_to_f16(uint32_t w, float s) {
  const float frac = __uint_as_float((__float_as_uint(s) & 0x807FFFFFu) | 0x3F800000u);
  const f16x2v f = {(_Float16)frac, (_Float16)frac};
  return uint4{f16x2_bits(__builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, s, 0) * f),
               f16x2_bits(__builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, s, 1) * f),
               f16x2_bits(__builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, s, 2) * f),
               f16x2_bits(__builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, s, 3) * f)};
}

// D(16x16, f32) += A(16x32) * B(32x16), f16 inputs (same lane layout as the bf16 form).
__device__ __forceinline__ f32x4 mfma16x16x32_f16(const uint4& a, const uint4& b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8v, a), __builtin_bit_cast(f16x8v, b), c,
                                                0, 0, 0);
}

// Eight activations -> f16 hi (and lo = f16(x - hi) for fp32 sources), for
// the NVFP4 instance, whose MFMAs take f16 operands.
__device__ __forceinline__ uint4 f32x8_to_f16(const float* x) {
  uint32_t o[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const f16x2v v = {(_Float16)x[2 * i], (_Float16)x[2 * i + 1]};
    o[i] = f16x2_bits(v);
  }
  return uint4{o[0], o[1], o[2], o[3]};
}
__device__ __forceinline__ void split_f16x8(const float* x, uint4& hi, uint4& lo) {
  float h[8], r[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    h[i] = (float)(_Float16)x[i];
    r[i] = x[i] - h[i];
  }
  hi = f32x8_to_f16(h);
  lo = f32x8_to_f16(r);
}

// A non-negative E4M3 code -> fp32, exactly: its 7 bits placed at the top of
// fp32's exponent/mantissa field read as 2^-120 times the value, subnormals
// included.
__device__ __forceinline__ float e4m3_pos_to_f32(uint32_t c) {
  return __uint_as_float((c & 0x7Fu) << 20) * 0x1p120f;
}
}  // namespace

template <int MT, int NTW, int KC, int WM, bool AF32, int WQ>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(WM)))
void gemm_kernel(GemmParams p) {
  static_assert(WM == 1 || WM == 2, "waves along M");
  static_assert(MT % WM == 0, "m-tiles split evenly over the waves along M");
  constexpr int KPW = wq_ktiles(WQ);             // k-tiles per 16-byte weight word
  static_assert(KC % KPW == 0, "a stage holds whole weight words");
  constexpr int KW = KC / KPW;                   // weight words per n-tile and stage
  constexpr int MTW = MT / WM;                   // m-tiles per wave
  constexpr int WN = 4 / WM;                     // waves along N
  constexpr int MP = MT * 16;
  constexpr int PIECES = MP * KC * 4;            // 8-element pieces of one A stage
  constexpr int APT = (PIECES + 255) / 256;      // pieces per thread
  // fp32 A: bf16 (or for NVFP4 f16) high and low parts; with f16 weights one f16 part
  constexpr int PLANES = (AF32 && WQ != WQ_F16) ? 2 : 1;
  __shared__ uint4 lds[1][PLANES][MT * KC * 64];
  __shared__ uint64_t red[WN][MP];

  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  const int wm = wid % WM, wn = wid / WM;
  const int mt0 = wm * MTW;
  const int bz = blockIdx.z, split = blockIdx.y;
  const int nt0 = (blockIdx.x * WN + wn) * NTW;
  const int kt_beg = split * p.kps;
  const int kt_end = min(p.KT, kt_beg + p.kps);
  const int nchunks = kt_end > kt_beg ? (kt_end - kt_beg + KC - 1) / KC : 0;
  const uint4* __restrict__ W = p.W + (int64_t)bz * p.w_bs;
  const int KG = p.KT / KPW;                     // weight words along K

  f32x4 acc[MTW][NTW];
#pragma unroll
  for (int i = 0; i < MTW; ++i)
#pragma unroll
    for (int j = 0; j < NTW; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  // Weights: a ring of three register stages, so two stages of weight loads
  // stay in flight while one is consumed.  Activations: raw (bf16 or fp32)
  // in registers until they are written to the LDS stage (fp32 is split into
  // bf16 hi/lo only then, so no load is waited on early: vmcnt is in order).
  uint4 wb[3][NTW][KW];
  uint32_t sb[3][NTW][WQ == 2 ? KW : 1];         // NVFP4 block scales of the lane's row
  constexpr int AW = AF32 ? 2 : 1;               // 16-byte words per piece held in registers
  uint4 ab[APT][AW];

  auto load_w = [&](int c, uint4 (&dst)[NTW][KW], uint32_t (&sdst)[NTW][WQ == 2 ? KW : 1]) {
#pragma unroll
    for (int j = 0; j < NTW; ++j) {
      const int nt = nt0 + j;
#pragma unroll
      for (int u = 0; u < KW; ++u) {
        const int kt = kt_beg + c * KC + u * KPW;
        const int64_t g = (int64_t)nt * KG + kt / KPW;
        if (nt < p.NT && kt < kt_end) {
          dst[j][u] = load_nt(&W[g * 64 + lane]);
          if constexpr (WQ == 2) sdst[j][u] = p.bscale[g * 32 + (lane & 15) * 2 + (lane >> 5)];
        } else {
          dst[j][u] = uint4{0u, 0u, 0u, 0u};
          if constexpr (WQ == 2) sdst[j][u] = 0u;
        }
      }
    }
  };
  auto load_a = [&](int c) {
#pragma unroll
    for (int i = 0; i < APT; ++i) {
      const int piece = tid + i * 256;
#pragma unroll
      for (int w = 0; w < AW; ++w) ab[i][w] = uint4{0u, 0u, 0u, 0u};
      if (piece < PIECES) {
        const int m = piece / (KC * 4), rem = piece % (KC * 4);
        const int kt = kt_beg + c * KC + rem / 4;
        const int k = kt * 32 + (rem & 3) * 8;
        if (m < p.M && kt < kt_end && k < p.K) {
          if constexpr (AF32) {
            const float* src = static_cast<const float*>(p.A) + (int64_t)bz * p.a_bs + (int64_t)m * p.lda + k;
            ab[i][0] = *reinterpret_cast<const uint4*>(src);
            ab[i][AW - 1] = *reinterpret_cast<const uint4*>(src + 4);
          } else {
            const bf16_t* src = static_cast<const bf16_t*>(p.A) + (int64_t)bz * p.a_bs + (int64_t)m * p.lda + k;
            ab[i][0] = *reinterpret_cast<const uint4*>(src);
          }
        }
      }
    }
  };
  auto store_a = [&](int buf) {
#pragma unroll
    for (int i = 0; i < APT; ++i) {
      const int piece = tid + i * 256;
      if (piece < PIECES) {
        const int m = piece / (KC * 4), rem = piece % (KC * 4);
        const int t = rem / 4, g = rem & 3;
        const int at = ((m >> 4) * KC + t) * 64 + (m & 15) + 16 * g;
        if constexpr (WQ == WQ_F16 && !AF32) {
          lds[buf][0][at] = ab[i][0];                 // f16 activations as written
        } else if constexpr (WQ == WQ_F16) {
          // f16 weights: fp32 activations rounded to one f16 operand
          float x[8];
          const float4 x0 = __builtin_bit_cast(float4, ab[i][0]), x1 = __builtin_bit_cast(float4, ab[i][AW - 1]);
          x[0] = x0.x; x[1] = x0.y; x[2] = x0.z; x[3] = x0.w; x[4] = x1.x; x[5] = x1.y; x[6] = x1.z; x[7] = x1.w;
          lds[buf][0][at] = f32x8_to_f16(x);
        } else if constexpr (WQ == 2) {
          // the NVFP4 instance multiplies in f16: activations to f16 (hi + lo for fp32)
          float x[8];
          if constexpr (AF32) {
            const float4 x0 = __builtin_bit_cast(float4, ab[i][0]), x1 = __builtin_bit_cast(float4, ab[i][AW - 1]);
            x[0] = x0.x; x[1] = x0.y; x[2] = x0.z; x[3] = x0.w; x[4] = x1.x; x[5] = x1.y; x[6] = x1.z; x[7] = x1.w;
            uint4 hi, lo;
            split_f16x8(x, hi, lo);
            lds[buf][0][at] = hi;
            lds[buf][PLANES - 1][at] = lo;
          } else {
            unpack8(ab[i][0], x);
            lds[buf][0][at] = f32x8_to_f16(x);
          }
        } else if constexpr (AF32) {
          uint4 hi, lo;
          split_bf16x8(__builtin_bit_cast(float4, ab[i][0]), __builtin_bit_cast(float4, ab[i][AW - 1]), hi, lo);
          lds[buf][0][at] = hi;
          lds[buf][PLANES - 1][at] = lo;
        } else {
          lds[buf][0][at] = ab[i][0];
        }
      }
    }
  };
  auto compute = [&](int buf, uint4 (&w)[NTW][KW], uint32_t (&sc)[NTW][WQ == 2 ? KW : 1]) {
#pragma unroll
    for (int t = 0; t < KC; ++t) {
      uint4 bw[NTW];
#pragma unroll
      for (int j = 0; j < NTW; ++j) {
        if constexpr (WQ == 0 || WQ == WQ_F16) {
          bw[j] = w[j][t];
        } else if constexpr (WQ == 1) {
          const uint4& q = w[j][t / 2];
          bw[j] = (t % 2 == 0) ? fp8x8_to_bf16(q.x, q.y) : fp8x8_to_bf16(q.z, q.w);
        } else {
          const uint4& q = w[j][t / 4];
          const uint32_t word = (t % 4 == 0) ? q.x : (t % 4 == 1) ? q.y : (t % 4 == 2) ? q.z : q.w;
          bw[j] = fp4x8_to_f16(word, e4m3_pos_to_f32(sc[j][t / 4] >> (8 * (t % 4))));
        }
      }
#pragma unroll
      for (int i = 0; i < MTW; ++i) {
#pragma unroll
        for (int pl = 0; pl < PLANES; ++pl) {
          const uint4 a = lds[buf][pl][((mt0 + i) * KC + t) * 64 + lane];
#pragma unroll
          for (int j = 0; j < NTW; ++j) {
            if constexpr (WQ == 2 || WQ == WQ_F16) acc[i][j] = mfma16x16x32_f16(a, bw[j], acc[i][j]);
            else acc[i][j] = mfma16x16x32(a, bw[j], acc[i][j]);
          }
        }
      }
    }
  };
  // stage c: activations of c go to LDS, activations of c+1 and weights of
  // c+2 are issued, then the weights of c (issued two stages ago) are used.
  // (A second LDS buffer, trading one of the two barriers for a later store,
  // measured slower at every batch size.)
  auto stage = [&](int c, int use, int fill) {
    __syncthreads();                 // every wave is done reading stage c-1
    store_a(0);
    if (c + 1 < nchunks) load_a(c + 1);
    if (c + 2 < nchunks) load_w(c + 2, wb[fill], sb[fill]);
    __syncthreads();                 // stage c visible
    compute(0, wb[use], sb[use]);
  };
  if (nchunks > 0) {
    load_a(0);
    load_w(0, wb[0], sb[0]);
    if (nchunks > 1) load_w(1, wb[1], sb[1]);
    for (int c = 0; c < nchunks; c += 3) {
      stage(c, 0, 2);
      if (c + 1 < nchunks) stage(c + 1, 1, 0);
      if (c + 2 < nchunks) stage(c + 2, 2, 1);
    }
  }

  const int col = lane & 15, rq = (lane >> 4) * 4;
  if constexpr (wq_scaled(WQ)) {
    // the row scale of a quantized weight, on the fp32 accumulator
#pragma unroll
    for (int j = 0; j < NTW; ++j) {
      const int nt = nt0 + j;
      const float sc = nt < p.NT ? p.rscale[nt * 16 + col] : 0.f;
#pragma unroll
      for (int i = 0; i < MTW; ++i) acc[i][j] *= sc;
    }
  }
  if (p.mode == GEMM_F32_PARTIAL || p.mode == GEMM_BF16) {
#pragma unroll
    for (int j = 0; j < NTW; ++j) {
      const int n = (nt0 + j) * 16 + col;
      if (n >= p.N) continue;
#pragma unroll
      for (int i = 0; i < MTW; ++i)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int m = (mt0 + i) * 16 + rq + r;
          if (m >= p.M) continue;
          if (p.mode == GEMM_F32_PARTIAL) {
            float* C = static_cast<float*>(p.C) + (int64_t)bz * p.c_bs + (int64_t)split * p.c_ss;
            C[(int64_t)m * p.ldc + n] = acc[i][j][r];
          } else {
            bf16_t* C = static_cast<bf16_t*>(p.C) + (int64_t)bz * p.c_bs;
            C[(int64_t)m * p.ldc + n] = f2bf(acc[i][j][r]);
          }
        }
    }
    return;
  }

  // GEMM_ARGMAX: best (value, lowest index) per row over this block's columns.
#pragma unroll
  for (int i = 0; i < MTW; ++i)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int m = (mt0 + i) * 16 + rq + r;
      uint64_t best = 0;
#pragma unroll
      for (int j = 0; j < NTW; ++j) {
        const int n = (nt0 + j) * 16 + col;
        if (n < p.N) {
          const float v = acc[i][j][r];
          if (p.logits && m < p.M) p.logits[(int64_t)m * p.ldc + n] = v;
          const uint64_t k = argmax_key(v, (uint32_t)n);
          best = k > best ? k : best;
        }
      }
#pragma unroll
      for (int o = 1; o < 16; o <<= 1) {
        const uint32_t lo = __shfl_xor((uint32_t)best, o, 64);
        const uint32_t hi = __shfl_xor((uint32_t)(best >> 32), o, 64);
        const uint64_t other = (uint64_t(hi) << 32) | lo;
        best = other > best ? other : best;
      }
      if (col == 0) red[wn][m] = best;
    }
  __syncthreads();
  for (int m = tid; m < MP; m += 256) {
    uint64_t b = red[0][m];
#pragma unroll
    for (int w = 1; w < WN; ++w) b = red[w][m] > b ? red[w][m] : b;
    if (m < p.M) p.cand[(int64_t)blockIdx.x * p.cand_ld + m] = b;
  }
}

// ----------------------------------------------------------------- large batch
// Batches of 65..256 rows (bf16 weights and activations, or f16 ones for the
// MLP; K a multiple of 32, one matrix): a block computes every row (128 or
// 256) x 256 columns.  Eight waves form a 2 x 4 grid of 64 x 64 or 128 x 64
// tiles (two waves per SIMD).  Both operands go HBM -> LDS by the LDS DMA,
// one k-tile per stage (16 activation fragments + 16 weight tiles, 32 KiB),
// into a ring of stages: each wave issues its share of a stage's DMAs, a
// ring's depth less one stages ahead, and waits for its own with vmcnt
// before the stage's barrier.  The MLP's fp32 activations come as f16,
// written so by the producing row kernels.
// No global load targets registers, so no wait is left to the compiler; the
// register-staged kernel above holds too few weight bytes in flight to feed
// the matrix cores at this batch.  Rows past M and columns past N read
// clamped (valid) addresses; their results are discarded.
namespace {
typedef __attribute__((address_space(3))) char lds_char_t;

// LDS DMA of 16 bytes per lane: lane i's 16 bytes at base + voff land at LDS
// byte address lds + 16*i.  Not tracked by the compiler: wait with vmcnt.
__device__ __forceinline__ void lds_dma16(const void* base, uint32_t voff, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1"
               :: "v"(voff), "s"(base), "s"(lds) : "memory", "m0");
}

__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0): this wave's LDS reads are done
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}
}  // namespace

#ifndef E3_BIG_NS_CAP
#define E3_BIG_NS_CAP 4
#endif

// s_waitcnt with only a vector-memory count (0..63).
#define E3_BIG_WAIT_VMCNT(n) __builtin_amdgcn_s_waitcnt(0x3F70 | ((n) & 15) | (((n) >> 4) << 14))

// NW waves: 8 (2 x 4 grid of 128 x 64 tiles, two waves per SIMD; a 4-wave
// grid of 128 x 128 tiles at one wave per SIMD measured slower).  MT m-tiles
// per block: 16 (256 rows, 128 x 64 wave tiles) or 8 (128 rows, 64 x 64 wave
// tiles).  F16: f16 weights and activations (the MLP of a bf16 head), else
// bf16.
// PIPE 2: the fragments of k-tile c + 1 are read from LDS into a second
// register set while the MFMAs of k-tile c run, so no MFMA waits on an LDS
// read (the register set doubles).  PIPE 1: all of a k-tile's fragment
// reads are issued before its first MFMA (the compiler would otherwise
// interleave small groups of reads with full waits), so only the first
// MFMA waits on LDS.  PIPE 0: the compiler's own order.
template <bool F16>
__device__ __forceinline__ f32x4 big_mfma(const uint4& a, const uint4& b, f32x4 c) {
  if constexpr (F16) return mfma16x16x32_f16(a, b, c);
  else return mfma16x16x32(a, b, c);
}

template <int NW, int MT, int PIPE, bool F16>
__global__ __launch_bounds__(64 * NW) void gemm_big_kernel(GemmParams p) {
  constexpr int NTW = 32 / NW;                    // n-tiles per wave
  constexpr int MTW = MT / 2;                     // m-tiles per wave
  constexpr int NFA = MT;                         // activation fragments per stage
  constexpr int NF = NFA + 16;                    // fragments per stage
  static_assert(NF % NW == 0, "whole DMAs per wave");
  constexpr int DPW = NF / NW;                    // DMAs per wave and stage
  constexpr int WC = NW / 2;                      // waves along N
  constexpr int BIG_STAGE = NF * 1024;
  // LDS stages (k-tiles), at most E3_BIG_NS_CAP and what 160 KiB hold (the
  // argmax epilogue reuses the ring for its per-row reduction).  Deeper
  // rings (5 or 6 stages) measured no faster: the loop is not bound by the
  // bytes in flight.
  constexpr int BIG_NS = (160 * 1024 / BIG_STAGE) < E3_BIG_NS_CAP ? (160 * 1024 / BIG_STAGE) : E3_BIG_NS_CAP;
  static_assert(BIG_NS >= 3 && WC * MT * 16 * 8 <= BIG_NS * BIG_STAGE, "ring and reduction fit in LDS");
  __shared__ __attribute__((aligned(1024))) char lds[BIG_NS * BIG_STAGE];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wid = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wid & 1, wn = wid >> 1;          // m-tiles MTW*wm.., n-tiles NTW*wn.. of the block
  const int bz = blockIdx.z;                      // matrix of a batch (the MLA per-head absorb halves)
  // The block's work is a range of units (column block cb, k-tile kt),
  // numbered cb*KT + kt.  Split-K: column block blockIdx.x, k-tiles of split
  // blockIdx.y.  Stream-K (p.streamk workgroups): an equal share of all
  // units, which may end one column block and start the next; each run of
  // units inside a column block is one partial sum.
  const int KT = p.KT;
  int64_t ubeg, uend;
  if (p.streamk) {
    const int64_t U = (int64_t)((p.NT + 15) / 16) * KT;
    ubeg = (int64_t)blockIdx.x * U / gridDim.x;
    uend = (int64_t)(blockIdx.x + 1) * U / gridDim.x;
  } else {
    ubeg = (int64_t)blockIdx.x * KT + (int64_t)blockIdx.y * p.kps;
    uend = (int64_t)blockIdx.x * KT + min(KT, (blockIdx.y + 1) * p.kps);
  }
  const uint32_t lds_addr = (uint32_t)(uintptr_t)(lds_char_t*)lds;

  // DMAs of wave w in a stage: fragments DPW*w .. +DPW-1 of the NF (first
  // the activation m-tiles, then the 16 weight n-tiles);
  // per-lane byte offsets are fixed but for the k-tile, which moves the base.
  uint32_t voff[DPW];
  const char* src[DPW];
#pragma unroll
  for (int i = 0; i < DPW; ++i) {
    const int f = DPW * wid + i;
    if (f < NFA) {
      const int row = min(16 * (f % MT) + (lane & 15), p.M - 1);
      voff[i] = (uint32_t)(((int64_t)row * p.lda + 8 * (lane >> 4)) * 2);
      src[i] = static_cast<const char*>(p.A) + (int64_t)bz * p.a_bs * 2;
    } else {
      voff[i] = (uint32_t)(lane * 16);
      src[i] = nullptr;                           // set per run
    }
  }

  f32x4 acc[MTW][NTW];
  const int col = lane & 15, rq = (lane >> 4) * 4;
  for (int64_t u0 = ubeg; u0 < uend;) {
    const int cb = (int)(u0 / KT);                // this run's column block
    const int kt_beg = (int)(u0 - (int64_t)cb * KT);
    const int64_t u1 = min(uend, (int64_t)(cb + 1) * KT);
    const int nk = (int)(u1 - u0);
    if (u0 != ubeg) __syncthreads();              // every wave is done with the last run's ring
#pragma unroll
    for (int i = 0; i < DPW; ++i) {
      const int f = DPW * wid + i;
      if (f >= NFA) {
        const int nt = min(cb * 16 + f - NFA, p.NT - 1);
        src[i] = reinterpret_cast<const char*>(p.W + (int64_t)bz * p.w_bs + (int64_t)nt * KT * 64);
      }
    }
    auto issue = [&](int s) {                     // k-tile kt_beg + s into ring slot s % BIG_NS
      const int kt = kt_beg + s;
      const uint32_t dst = lds_addr + (uint32_t)((s % BIG_NS) * BIG_STAGE + DPW * wid * 1024);
#pragma unroll
      for (int i = 0; i < DPW; ++i) {
        const int f = DPW * wid + i;
        const char* base = src[i] + (f < NFA ? (int64_t)kt * 64 : (int64_t)kt * 1024);
        lds_dma16(base, voff[i], dst + i * 1024);
      }
    };
#pragma unroll
    for (int i = 0; i < MTW; ++i)
#pragma unroll
      for (int j = 0; j < NTW; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

    if constexpr (PIPE == 2) {
      // Slot c % BIG_NS is free once every wave has read k-tile c into
      // registers, so stage c + BIG_NS is issued right after the barrier of
      // step c and the ring keeps BIG_NS - 1 stages in flight while the MFMAs
      // of k-tile c run from registers.
      uint4 fa0[MTW], fb0[NTW], fa1[MTW], fb1[NTW];
      auto read_stage = [&](int s, uint4 (&fa)[MTW], uint4 (&fb)[NTW]) {
        const uint4* st = reinterpret_cast<const uint4*>(lds + (s % BIG_NS) * BIG_STAGE);
#pragma unroll
        for (int j = 0; j < NTW; ++j) fb[j] = st[(NFA + NTW * wn + j) * 64 + lane];
#pragma unroll
        for (int i = 0; i < MTW; ++i) fa[i] = st[(MTW * wm + i) * 64 + lane];
      };
      auto mma = [&](const uint4 (&fa)[MTW], const uint4 (&fb)[NTW]) {
#pragma unroll
        for (int i = 0; i < MTW; ++i)
#pragma unroll
          for (int j = 0; j < NTW; ++j) acc[i][j] = big_mfma<F16>(fa[i], fb[j], acc[i][j]);
      };
      auto step = [&](int c, const uint4 (&ca)[MTW], const uint4 (&cb_)[NTW], uint4 (&na)[MTW],
                      uint4 (&nb)[NTW]) {
        if (c + 1 < nk) {
          // this wave's DMAs of k-tile c + 1 are done once at most those of
          // the later stages already issued (up to c + BIG_NS - 1) remain
          if (c + BIG_NS - 1 < nk) E3_BIG_WAIT_VMCNT(DPW * (BIG_NS - 2)); else E3_BIG_WAIT_VMCNT(0);
          lds_barrier();                          // k-tile c + 1 in LDS; k-tile c read by every wave
          if (c + BIG_NS < nk) issue(c + BIG_NS); // into the slot of k-tile c
          read_stage(c + 1, na, nb);
        }
        mma(ca, cb_);
      };
      const int pro = min(BIG_NS, nk);
      for (int s = 0; s < pro; ++s) issue(s);
      if (pro == BIG_NS) E3_BIG_WAIT_VMCNT(DPW * (BIG_NS - 1)); else E3_BIG_WAIT_VMCNT(0);
      lds_barrier();
      read_stage(0, fa0, fb0);
      for (int c = 0; c < nk; c += 2) {
        step(c, fa0, fb0, fa1, fb1);
        if (c + 1 < nk) step(c + 1, fa1, fb1, fa0, fb0);
      }
    } else {
      for (int s = 0; s < BIG_NS - 1 && s < nk; ++s) issue(s);
      for (int c = 0; c < nk; ++c) {
        // this wave's DMAs of stage c are done once at most those of the
        // BIG_NS - 2 later stages already issued are outstanding
        if (c + BIG_NS - 2 < nk) E3_BIG_WAIT_VMCNT(DPW * (BIG_NS - 2)); else E3_BIG_WAIT_VMCNT(0);
        lds_barrier();                            // stage c in LDS; stage c-1 read by every wave
        const bool refill = c + BIG_NS - 1 < nk;
        if (PIPE != 1 && refill) issue(c + BIG_NS - 1);
        const uint4* st = reinterpret_cast<const uint4*>(lds + (c % BIG_NS) * BIG_STAGE);
        uint4 b[NTW], a[MTW];
        if constexpr (PIPE == 1) {
          // reads in the order the MFMAs consume them (pinned: the compiler
          // would reorder them), every one issued before the first MFMA
#pragma unroll
          for (int j = 0; j < NTW; ++j) {
            b[j] = st[(NFA + NTW * wn + j) * 64 + lane];
            __builtin_amdgcn_sched_barrier(0);
          }
#pragma unroll
          for (int i = 0; i < MTW; ++i) {
            a[i] = st[(MTW * wm + i) * 64 + lane];
            __builtin_amdgcn_sched_barrier(0);
          }
#pragma unroll
          for (int i = 0; i < MTW; ++i) {
#pragma unroll
            for (int j = 0; j < NTW; ++j) acc[i][j] = big_mfma<F16>(a[i], b[j], acc[i][j]);
            __builtin_amdgcn_sched_barrier(0);    // m-tiles in the order their reads return
            // the refill DMAs go out after the first m-tile's MFMAs: issued
            // before them, they would make the compiler wait for every read
            // before the first MFMA
            if (i == 0 && refill) {
              issue(c + BIG_NS - 1);
              __builtin_amdgcn_sched_barrier(0);
            }
          }
        } else {
#pragma unroll
          for (int j = 0; j < NTW; ++j) b[j] = st[(NFA + NTW * wn + j) * 64 + lane];
#pragma unroll
          for (int i = 0; i < MTW; ++i) a[i] = st[(MTW * wm + i) * 64 + lane];
#pragma unroll
          for (int i = 0; i < MTW; ++i)
#pragma unroll
            for (int j = 0; j < NTW; ++j) acc[i][j] = big_mfma<F16>(a[i], b[j], acc[i][j]);
        }
      }
    }
    if (p.mode == GEMM_F32_PARTIAL) {
      // fp32 partial of the run.  Stream-K: its slot is the block's rank
      // among the blocks sharing the column block, and the first of them
      // also zeroes the slots the column block leaves unused, so a consumer
      // sums p.splitk slots everywhere.
      int slot = blockIdx.y, zero_from = p.splitk;
      if (p.streamk) {
        const int64_t U = (int64_t)((p.NT + 15) / 16) * KT, G = gridDim.x;
        auto owner = [&](int64_t v) { return (int)(((v + 1) * G + U - 1) / U - 1); };
        const int first = owner((int64_t)cb * KT);
        slot = blockIdx.x - first;
        if (slot == 0) zero_from = owner((int64_t)cb * KT + KT - 1) - first + 1;
      }
      // (opaque copies: no part of the store addressing may be hoisted out
      // of the run loop, where it would hold registers through the k-loop)
      float* C = static_cast<float*>(p.C);
      int64_t ldc = p.ldc, css = p.c_ss;
      int M = p.M, N = p.N;
      asm volatile("" : "+s"(C), "+s"(ldc), "+s"(css), "+s"(M), "+s"(N));
#pragma unroll
      for (int j = 0; j < NTW; ++j) {
        const int n = (cb * 16 + NTW * wn + j) * 16 + col;
        if (n >= N) continue;
#pragma unroll
        for (int i = 0; i < MTW; ++i)
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int m = (MTW * wm + i) * 16 + rq + r;
            if (m >= M) continue;
            C[(int64_t)slot * css + (int64_t)m * ldc + n] = acc[i][j][r];
          }
      }
      // (row-major over the run's M x 256 tile, 16 bytes per thread)
      for (int z = zero_from; z < p.splitk; ++z)
        for (int e = tid; e < M * 64; e += 64 * NW) {
          const int m = e >> 6, n = cb * 256 + (e & 63) * 4;
          float* row = C + (int64_t)z * css + (int64_t)m * ldc;
#pragma unroll
          for (int q = 0; q < 4; ++q)
            if (n + q < N) row[n + q] = 0.f;
        }
    }
    u0 = u1;
  }
  if (p.mode == GEMM_F32_PARTIAL || ubeg >= uend) return;
  // bf16 results and argmax candidates: split-K with one split
  const int ntb = blockIdx.x * 16;                // first n-tile of the block
  if (p.mode == GEMM_BF16) {
    // The block's bf16 tile goes through the (now idle) ring, row-major, and
    // leaves in 16-byte pieces of whole rows: the MFMA layout would give each
    // lane single 2-byte values 16 columns apart.  Column c of row m sits at
    // c ^ 16*((m / 4) % 4), so the four row groups of one LDS store fall on
    // different banks while every aligned 8-column piece stays contiguous.
    static_assert(MT * 16 * 256 * 2 <= BIG_NS * BIG_STAGE, "the tile fits in the ring");
    bf16_t* tile = reinterpret_cast<bf16_t*>(lds);
    auto at = [](int m, int c) { return m * 256 + (c ^ (((m >> 2) & 3) << 4)); };
    __syncthreads();                              // every wave is done reading the ring
#pragma unroll
    for (int j = 0; j < NTW; ++j)
#pragma unroll
      for (int i = 0; i < MTW; ++i)
#pragma unroll
        for (int r = 0; r < 4; ++r)
          tile[at((MTW * wm + i) * 16 + rq + r, (NTW * wn + j) * 16 + col)] = f2bf(acc[i][j][r]);
    __syncthreads();
    const int ncols = min(256, p.N - ntb * 16), rows = min(MT * 16, p.M);
    bf16_t* C = static_cast<bf16_t*>(p.C) + (int64_t)bz * p.c_bs + (int64_t)ntb * 16;
    for (int e = tid; e < rows * 32; e += 64 * NW) {
      const int m = e >> 5, c8 = (e & 31) * 8;
      if (c8 >= ncols) continue;
      const bf16_t* src = tile + at(m, c8);
      bf16_t* dst = C + (int64_t)m * p.ldc + c8;
      if (c8 + 8 <= ncols && (reinterpret_cast<uintptr_t>(dst) & 15) == 0) {
        *reinterpret_cast<uint4*>(dst) = *reinterpret_cast<const uint4*>(src);
      } else {
        for (int q = 0; q < 8 && c8 + q < ncols; ++q) dst[q] = src[q];
      }
    }
    return;
  }
  // GEMM_ARGMAX: best (value, lowest index) per row over the block's columns,
  // reduced across the waves along N in the (now idle) ring
  uint64_t (*red)[MT * 16] = reinterpret_cast<uint64_t (*)[MT * 16]>(lds);
  __syncthreads();                                // every wave is done reading the ring
#pragma unroll
  for (int i = 0; i < MTW; ++i)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int m = (MTW * wm + i) * 16 + rq + r;
      uint64_t best = 0;
#pragma unroll
      for (int j = 0; j < NTW; ++j) {
        const int n = (ntb + NTW * wn + j) * 16 + col;
        if (n < p.N) {
          const float v = acc[i][j][r];
          if (p.logits && m < p.M) p.logits[(int64_t)m * p.ldc + n] = v;
          const uint64_t k = argmax_key(v, (uint32_t)n);
          best = k > best ? k : best;
        }
      }
#pragma unroll
      for (int o = 1; o < 16; o <<= 1) {
        const uint32_t lo = __shfl_xor((uint32_t)best, o, 64);
        const uint32_t hi = __shfl_xor((uint32_t)(best >> 32), o, 64);
        const uint64_t other = (uint64_t(hi) << 32) | lo;
        best = other > best ? other : best;
      }
      if (col == 0) red[wn][m] = best;
    }
  __syncthreads();
  for (int m = tid; m < MT * 16; m += 64 * NW) {
    uint64_t b = red[0][m];
#pragma unroll
    for (int w = 1; w < WC; ++w) b = red[w][m] > b ? red[w][m] : b;
    if (m < p.M) p.cand[(int64_t)blockIdx.x * p.cand_ld + m] = b;
  }
}

int gemm_big_blocks_x(const GemmParams& p) { return (p.NT + 15) / 16; }

int gemm_big_streamk_slots(int NT, int KT, int G) {
  const int64_t U = (int64_t)((NT + 15) / 16) * KT;
  if (G <= 0 || G > U) return 0;
  // the block owning unit v (ranges [w*U/G, (w+1)*U/G)); a column block's
  // partials come from the blocks owning its first through last unit
  auto owner = [&](int64_t v) { return (int)(((v + 1) * G + U - 1) / U - 1); };
  int slots = 1;
  for (int64_t cb = 0; cb < U / KT; ++cb)
    slots = std::max(slots, owner(cb * KT + KT - 1) - owner(cb * KT) + 1);
  return slots;
}

bool gemm_big_ok(const GemmParams& p, int batch) {
  // stream-K: fp32 partials in p.splitk slots, every workgroup with work
  if (p.streamk && (p.mode != GEMM_F32_PARTIAL || p.streamk > (int64_t)gemm_big_blocks_x(p) * p.KT ||
                    p.splitk < gemm_big_streamk_slots(p.NT, p.KT, p.streamk)))
    return false;
  // split-K: every split has k-tiles; one split unless fp32 partials
  if (!p.streamk && (p.kps < 1 || (int64_t)(p.splitk - 1) * p.kps >= p.KT ||
                     (p.mode != GEMM_F32_PARTIAL && p.splitk != 1)))
    return false;
  // a batch of matrices: bf16 results only (blockIdx.z is the matrix)
  if (batch < 1 || (batch > 1 && (p.mode != GEMM_BF16 || p.a_bs % 8 != 0))) return false;
  return (p.wq == 0 || p.wq == WQ_F16) && !p.a_f32 && p.M >= 1 &&
         p.M <= 256 && p.K % 32 == 0 && p.KT * 32 == p.K && p.lda % 8 == 0 &&
         reinterpret_cast<uintptr_t>(p.A) % 16 == 0;
}

// Waves and read schedule (PIPE) of the large-batch kernel per block height,
// and the most LDS stages of its ring.
#ifndef E3_BIG_NW16
#define E3_BIG_NW16 8
#endif
#ifndef E3_BIG_PIPE16
#define E3_BIG_PIPE16 1
#endif
#ifndef E3_BIG_NW8
#define E3_BIG_NW8 8
#endif
#ifndef E3_BIG_PIPE8
#define E3_BIG_PIPE8 2
#endif

hipError_t launch_gemm_big(const GemmParams& p, int batch, hipStream_t st) {
  if (!gemm_big_ok(p, batch)) return hipErrorInvalidValue;
  const dim3 grid = p.streamk ? dim3(p.streamk, 1, 1) : dim3(gemm_big_blocks_x(p), p.splitk, batch);
  const bool f16 = p.wq == WQ_F16;
  // 128-row blocks when the rows fit (half the MFMAs and LDS traffic of 256)
  if (p.M <= 128) {
    constexpr int NW = E3_BIG_NW8;
    if (f16)
      hipLaunchKernelGGL((gemm_big_kernel<NW, 8, E3_BIG_PIPE8, true>), grid, dim3(64 * NW), 0, st, p);
    else
      hipLaunchKernelGGL((gemm_big_kernel<NW, 8, E3_BIG_PIPE8, false>), grid, dim3(64 * NW), 0, st, p);
  } else {
    constexpr int NW = E3_BIG_NW16;
    if (f16)
      hipLaunchKernelGGL((gemm_big_kernel<NW, 16, E3_BIG_PIPE16, true>), grid, dim3(64 * NW), 0, st, p);
    else
      hipLaunchKernelGGL((gemm_big_kernel<NW, 16, E3_BIG_PIPE16, false>), grid, dim3(64 * NW), 0, st, p);
  }
  return hipGetLastError();
}

// (m-tiles per block, n-tiles per wave, k-tiles per stage, waves along M); the
// last row holds the stages of 2 or 4 k-tiles that quantized weights need
#define E3_GEMM_SHAPES(X) \
  X(1, 1, 4, 1) X(1, 1, 8, 1) X(1, 2, 4, 1) X(1, 2, 8, 1) X(1, 4, 4, 1) \
  X(2, 1, 4, 1) X(2, 1, 8, 1) X(2, 2, 4, 1) X(2, 4, 4, 1)                \
  X(1, 2, 16, 1) X(2, 2, 8, 1) X(2, 4, 8, 1)                            \
  X(4, 1, 4, 1) X(4, 2, 4, 1) X(4, 4, 4, 1)                             \
  X(8, 2, 2, 1) X(8, 2, 4, 1) X(8, 4, 2, 1)                             \
  X(16, 2, 2, 1)                                                        \
  X(8, 4, 1, 2) X(16, 4, 1, 2)                                          \
  X(8, 4, 4, 1) X(8, 4, 2, 2)

bool gemm_shape_supported(GemmShape s) {
#define X(a, b, c, d) if (s.mt == a && s.ntw == b && s.kc == c && s.wm == d) return true;
  E3_GEMM_SHAPES(X)
#undef X
  return false;
}

int gemm_blocks_x(const GemmParams& p, GemmShape s) {
  const int per_block = (4 / s.wm) * s.ntw;
  return (p.NT + per_block - 1) / per_block;
}

template <int MT, int NTW, int KC, int WM, int WQ>
hipError_t launch_gemm_wq(const GemmParams& p, dim3 grid, hipStream_t st) {
  if constexpr (KC % wq_ktiles(WQ) != 0) {
    return hipErrorInvalidValue;                 // the format's words do not fit this stage
  } else {
    if (p.a_f32)
      hipLaunchKernelGGL((gemm_kernel<MT, NTW, KC, WM, true, WQ>), grid, dim3(256), 0, st, p);
    else
      hipLaunchKernelGGL((gemm_kernel<MT, NTW, KC, WM, false, WQ>), grid, dim3(256), 0, st, p);
    return hipGetLastError();
  }
}

hipError_t launch_gemm(const GemmParams& p, GemmShape s, int batch, hipStream_t st) {
  if (wq_scaled(p.wq) && (!p.rscale || (p.wq == 2 && !p.bscale) || batch != 1)) return hipErrorInvalidValue;
  if (p.KT % wq_ktiles(p.wq) || p.kps % wq_ktiles(p.wq)) return hipErrorInvalidValue;
  dim3 grid(gemm_blocks_x(p, s), p.splitk, batch);
#define X(a, b, c, d)                                                      \
  if (s.mt == a && s.ntw == b && s.kc == c && s.wm == d) {                 \
    switch (p.wq) {                                                        \
      case 0: return launch_gemm_wq<a, b, c, d, 0>(p, grid, st);           \
      case 1: return launch_gemm_wq<a, b, c, d, 1>(p, grid, st);           \
      case 2: return launch_gemm_wq<a, b, c, d, 2>(p, grid, st);           \
      case WQ_F16: return launch_gemm_wq<a, b, c, d, WQ_F16>(p, grid, st); \
      default: return hipErrorInvalidValue;                                \
    }                                                                      \
  }
  E3_GEMM_SHAPES(X)
#undef X
  return hipErrorInvalidValue;
}

// ----------------------------------------------------------------- packing
// Packed layout of an N x K bf16 weight: tile (nt, kt) at uint4 offset
// (nt*KT + kt)*64; lane l of a tile holds W[nt*16 + (l & 15)][kt*32 + 8*(l >> 4) .. +7].

// Element `idx` (linear index into a quantized source of `cols` columns),
// dequantized: E4M3 code times the row scale, or E2M1 (low nibble = even
// column) times its 16-column E4M3 block scale times the row scale.
template <int SRC>
__device__ __forceinline__ float dequant_at(const uint8_t* src, const float* rscale, const uint8_t* bscale,
                                            int64_t cols, int64_t idx) {
  const int64_t r = idx / cols, c = idx % cols;
  if constexpr (SRC == 1) {
    const uint32_t q = src[idx];
    const float m = e4m3_pos_to_f32(q);
    return ((q & 0x80u) ? -m : m) * rscale[r];
  } else {
    const uint32_t q = (src[r * (cols / 2) + c / 2] >> (4 * (c & 1))) & 15u;
    const int e = (q >> 1) & 3;
    const float m = e ? float(2 + (q & 1)) * float(1 << e) * 0.25f : 0.5f * float(q & 1);
    return ((q & 8u) ? -m : m) * e4m3_pos_to_f32(bscale[r * (cols / 16) + c / 16]) * rscale[r];
  }
}

template <int SRC>
__global__ void pack_kernel(uint4* __restrict__ dst, int NT, int KT, int K, int row0, int nrows,
                            const void* __restrict__ src_v, const float* __restrict__ rscale,
                            const uint8_t* __restrict__ bscale, int64_t cols, int64_t src_off, int64_t rs,
                            int64_t cs, int64_t src_bs, int64_t dst_bs) {
  const int64_t slot = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;   // (tile, lane)
  const int64_t nslots = (int64_t)NT * KT * 64;
  if (slot >= nslots) return;
  const int lane = int(slot & 63);
  const int64_t tile = slot >> 6;
  const int nt = int(tile / KT), kt = int(tile % KT);
  const int n = nt * 16 + (lane & 15);
  if (n < row0 || n >= row0 + nrows) return;
  const int64_t base = src_off + (int64_t)blockIdx.z * src_bs + (int64_t)(n - row0) * rs;
  const int k0 = kt * 32 + (lane >> 4) * 8;
  uint32_t h[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const int k = k0 + e;
    if (k >= K) {
      h[e] = 0u;
    } else if constexpr (SRC == 0) {
      h[e] = static_cast<const bf16_t*>(src_v)[base + (int64_t)k * cs];
    } else if constexpr (SRC == 3) {
      // bf16 -> f16, round to nearest even (exact in f16's normal range)
      const _Float16 v = (_Float16)bf2f(static_cast<const bf16_t*>(src_v)[base + (int64_t)k * cs]);
      h[e] = __builtin_bit_cast(uint16_t, v);
    } else {
      h[e] = f2bf(dequant_at<SRC>(static_cast<const uint8_t*>(src_v), rscale, bscale, cols,
                                  base + (int64_t)k * cs));
    }
  }
  dst[(int64_t)blockIdx.z * dst_bs + slot] =
      uint4{h[0] | (h[1] << 16), h[2] | (h[3] << 16), h[4] | (h[5] << 16), h[6] | (h[7] << 16)};
}

hipError_t launch_pack(uint4* dst, int NT, int KT, int K, int row0, int nrows, const void* src, int src_fmt,
                       const float* src_rscale, const uint8_t* src_bscale, int64_t src_cols, int64_t src_off,
                       int64_t rs, int64_t cs, int batch, int64_t src_bs, int64_t dst_bs, hipStream_t st) {
  const int64_t nslots = (int64_t)NT * KT * 64;
  dim3 grid((unsigned)((nslots + 255) / 256), 1, batch);
  if (src_fmt == 0)
    hipLaunchKernelGGL(pack_kernel<0>, grid, dim3(256), 0, st, dst, NT, KT, K, row0, nrows, src, src_rscale,
                       src_bscale, src_cols, src_off, rs, cs, src_bs, dst_bs);
  else if (src_fmt == 1)
    hipLaunchKernelGGL(pack_kernel<1>, grid, dim3(256), 0, st, dst, NT, KT, K, row0, nrows, src, src_rscale,
                       src_bscale, src_cols, src_off, rs, cs, src_bs, dst_bs);
  else if (src_fmt == 2)
    hipLaunchKernelGGL(pack_kernel<2>, grid, dim3(256), 0, st, dst, NT, KT, K, row0, nrows, src, src_rscale,
                       src_bscale, src_cols, src_off, rs, cs, src_bs, dst_bs);
  else if (src_fmt == 3)
    hipLaunchKernelGGL(pack_kernel<3>, grid, dim3(256), 0, st, dst, NT, KT, K, row0, nrows, src, src_rscale,
                       src_bscale, src_cols, src_off, rs, cs, src_bs, dst_bs);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

// FP8: word (nt, kg) at uint4 offset (nt*KG + kg)*64; lane l holds row
// nt*16 + (l & 15), bytes 0-7 columns kg*64 + 8*(l >> 4) .. +7 and bytes
// 8-15 the same 8 columns 32 further on (two 16 x 32 MFMA tiles).
__global__ void pack_fp8_kernel(uint4* __restrict__ dst, int NT, int KG, int K, int row0, int nrows,
                                const uint8_t* __restrict__ src, int64_t rs) {
  const int64_t slot = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (slot >= (int64_t)NT * KG * 64) return;
  const int lane = int(slot & 63);
  const int64_t g = slot >> 6;
  const int nt = int(g / KG), kg = int(g % KG);
  const int n = nt * 16 + (lane & 15);
  if (n < row0 || n >= row0 + nrows) return;
  const uint8_t* s = src + (int64_t)(n - row0) * rs;
  uint32_t w[4];
#pragma unroll
  for (int half = 0; half < 2; ++half)
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      uint32_t v = 0;
#pragma unroll
      for (int b = 0; b < 4; ++b) {
        const int k = kg * 64 + 32 * half + 8 * (lane >> 4) + 4 * q + b;
        v |= (k < K ? uint32_t(s[k]) : 0u) << (8 * b);
      }
      w[2 * half + q] = v;
    }
  dst[slot] = uint4{w[0], w[1], w[2], w[3]};
}

hipError_t launch_pack_fp8(uint4* dst, int NT, int KT, int K, int row0, int nrows, const uint8_t* src,
                           int64_t rs, hipStream_t st) {
  const int KG = KT / 2;
  const int64_t nslots = (int64_t)NT * KG * 64;
  hipLaunchKernelGGL(pack_fp8_kernel, dim3((unsigned)((nslots + 255) / 256)), dim3(256), 0, st, dst, NT, KG,
                     K, row0, nrows, src, rs);
  return hipGetLastError();
}

// NVFP4: word (nt, kg) at uint4 offset (nt*KG + kg)*64; lane l holds row
// nt*16 + (l & 15) and, in its 32-bit word u, the 8 columns
// kg*128 + 32u + 8*(l >> 4) .. +7 (4 bytes of codes).  Block scales: 32
// words per (nt, kg); word (l & 15)*2 + h holds, in byte u, the scale of
// columns kg*128 + 32u + 16h .. +15 of row nt*16 + (l & 15), which is the
// block of lanes with l >> 5 == h.
__global__ void pack_nvfp4_kernel(uint4* __restrict__ dst, uint32_t* __restrict__ bdst, int NT, int KG, int K,
                                  int row0, int nrows, const uint8_t* __restrict__ codes,
                                  const uint8_t* __restrict__ blocks) {
  const int64_t slot = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (slot >= (int64_t)NT * KG * 64) return;
  const int lane = int(slot & 63);
  const int64_t g = slot >> 6;
  const int nt = int(g / KG), kg = int(g % KG);
  const int n = nt * 16 + (lane & 15);
  if (n < row0 || n >= row0 + nrows) return;
  const uint8_t* c = codes + (int64_t)(n - row0) * (K / 2);
  const uint8_t* bs = blocks + (int64_t)(n - row0) * (K / 16);
  uint32_t w[4];
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const int k0 = kg * 128 + 32 * u + 8 * (lane >> 4);   // 8 columns = 4 bytes
    uint32_t v = 0;
#pragma unroll
    for (int b = 0; b < 4; ++b) {
      const int k = k0 + 2 * b;
      v |= (k < K ? uint32_t(c[k / 2]) : 0u) << (8 * b);
    }
    w[u] = v;
  }
  dst[slot] = uint4{w[0], w[1], w[2], w[3]};
  if (((lane >> 4) & 1) == 0) {            // one lane of each (row, half) writes the scales
    const int h = lane >> 5;
    uint32_t v = 0;
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int blk = kg * 8 + 2 * u + h;
      v |= (blk < K / 16 ? uint32_t(bs[blk]) : 0u) << (8 * u);
    }
    bdst[g * 32 + (lane & 15) * 2 + h] = v;
  }
}

hipError_t launch_pack_nvfp4(uint4* dst, uint32_t* bdst, int NT, int KT, int K, int row0, int nrows,
                             const uint8_t* codes, const uint8_t* blocks, hipStream_t st) {
  const int KG = KT / 4;
  const int64_t nslots = (int64_t)NT * KG * 64;
  hipLaunchKernelGGL(pack_nvfp4_kernel, dim3((unsigned)((nslots + 255) / 256)), dim3(256), 0, st, dst, bdst, NT,
                     KG, K, row0, nrows, codes, blocks);
  return hipGetLastError();
}

__global__ void zero_kernel(uint4* __restrict__ dst, int64_t n16) {
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n16;
       i += (int64_t)gridDim.x * blockDim.x)
    dst[i] = uint4{0u, 0u, 0u, 0u};
}

hipError_t launch_zero(void* dst, size_t bytes, hipStream_t st) {
  const int64_t n16 = (int64_t)(bytes / 16);
  if (n16 == 0) return hipSuccess;
  const int64_t blocks = (n16 + 255) / 256;
  hipLaunchKernelGGL(zero_kernel, dim3((unsigned)(blocks < 8192 ? blocks : 8192)), dim3(256), 0, st,
                     static_cast<uint4*>(dst), n16);
  return hipGetLastError();
}

}  // namespace e3
