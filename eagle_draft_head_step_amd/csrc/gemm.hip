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
//     reduces to one (value, index) candidate per block and row instead.
#include "common.h"
#include "internal.h"

namespace e3 {

template <int MT, int NTW, int KC, int WM, bool AF32>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(WM)))
void gemm_kernel(GemmParams p) {
  static_assert(WM == 1 || WM == 2, "waves along M");
  static_assert(MT % WM == 0, "m-tiles split evenly over the waves along M");
  constexpr int MTW = MT / WM;                   // m-tiles per wave
  constexpr int WN = 4 / WM;                     // waves along N
  constexpr int MP = MT * 16;
  constexpr int PIECES = MP * KC * 4;            // 8-element pieces of one A stage
  constexpr int APT = (PIECES + 255) / 256;      // pieces per thread
  constexpr int PLANES = AF32 ? 2 : 1;           // fp32 A: bf16 high and low parts
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

  f32x4 acc[MTW][NTW];
#pragma unroll
  for (int i = 0; i < MTW; ++i)
#pragma unroll
    for (int j = 0; j < NTW; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  // Weights: a ring of three register stages, so two stages of weight loads
  // stay in flight while one is consumed.  Activations: raw (bf16 or fp32)
  // in registers until they are written to the LDS stage (fp32 is split into
  // bf16 hi/lo only then, so no load is waited on early: vmcnt is in order).
  uint4 wb[3][NTW][KC];
  constexpr int AW = AF32 ? 2 : 1;               // 16-byte words per piece held in registers
  uint4 ab[APT][AW];

  auto load_w = [&](int c, uint4 (&dst)[NTW][KC]) {
#pragma unroll
    for (int j = 0; j < NTW; ++j) {
      const int nt = nt0 + j;
#pragma unroll
      for (int t = 0; t < KC; ++t) {
        const int kt = kt_beg + c * KC + t;
        if (nt < p.NT && kt < kt_end)
          dst[j][t] = load_nt(&W[((int64_t)nt * p.KT + kt) * 64 + lane]);
        else
          dst[j][t] = uint4{0u, 0u, 0u, 0u};
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
        if constexpr (AF32) {
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
  auto compute = [&](int buf, uint4 (&w)[NTW][KC]) {
#pragma unroll
    for (int t = 0; t < KC; ++t) {
#pragma unroll
      for (int i = 0; i < MTW; ++i) {
#pragma unroll
        for (int pl = 0; pl < PLANES; ++pl) {
          const uint4 a = lds[buf][pl][((mt0 + i) * KC + t) * 64 + lane];
#pragma unroll
          for (int j = 0; j < NTW; ++j) acc[i][j] = mfma16x16x32(a, w[j][t], acc[i][j]);
        }
      }
    }
  };
  // stage c: activations of c go to LDS, activations of c+1 and weights of
  // c+2 are issued, then the weights of c (issued two stages ago) are used.
  // (A second LDS buffer, trading one of the two barriers for a later store,
  // measured slower at every batch size.)
  auto stage = [&](int c, uint4 (&wuse)[NTW][KC], uint4 (&wfill)[NTW][KC]) {
    __syncthreads();                 // every wave is done reading stage c-1
    store_a(0);
    if (c + 1 < nchunks) load_a(c + 1);
    if (c + 2 < nchunks) load_w(c + 2, wfill);
    __syncthreads();                 // stage c visible
    compute(0, wuse);
  };
  if (nchunks > 0) {
    load_a(0);
    load_w(0, wb[0]);
    if (nchunks > 1) load_w(1, wb[1]);
    for (int c = 0; c < nchunks; c += 3) {
      stage(c, wb[0], wb[2]);
      if (c + 1 < nchunks) stage(c + 1, wb[1], wb[0]);
      if (c + 2 < nchunks) stage(c + 2, wb[2], wb[1]);
    }
  }

  const int col = lane & 15, rq = (lane >> 4) * 4;
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
    if (m < p.M) p.cand[(int64_t)blockIdx.x * p.M + m] = b;
  }
}

// (m-tiles per block, n-tiles per wave, k-tiles per stage, waves along M)
#define E3_GEMM_SHAPES(X) \
  X(1, 1, 4, 1) X(1, 1, 8, 1) X(1, 2, 4, 1) X(1, 2, 8, 1) X(1, 4, 4, 1) \
  X(2, 1, 4, 1) X(2, 1, 8, 1) X(2, 2, 4, 1) X(2, 4, 4, 1)                \
  X(4, 1, 4, 1) X(4, 2, 4, 1) X(4, 4, 4, 1)                             \
  X(8, 2, 2, 1) X(8, 2, 4, 1) X(8, 4, 2, 1)                             \
  X(16, 2, 2, 1)                                                        \
  X(8, 4, 1, 2) X(16, 4, 1, 2)

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

hipError_t launch_gemm(const GemmParams& p, GemmShape s, int batch, hipStream_t st) {
  dim3 grid(gemm_blocks_x(p, s), p.splitk, batch);
#define X(a, b, c, d)                                                                   \
  if (s.mt == a && s.ntw == b && s.kc == c && s.wm == d) {                              \
    if (p.a_f32)                                                                        \
      hipLaunchKernelGGL((gemm_kernel<a, b, c, d, true>), grid, dim3(256), 0, st, p);   \
    else                                                                                \
      hipLaunchKernelGGL((gemm_kernel<a, b, c, d, false>), grid, dim3(256), 0, st, p);  \
    return hipGetLastError();                                                           \
  }
  E3_GEMM_SHAPES(X)
#undef X
  return hipErrorInvalidValue;
}

// ----------------------------------------------------------------- packing
// Packed layout of an N x K weight: tile (nt, kt) at uint4 offset
// (nt*KT + kt)*64; lane l of a tile holds W[nt*16 + (l & 15)][kt*32 + 8*(l >> 4) .. +7].
__global__ void pack_kernel(uint4* __restrict__ dst, int NT, int KT, int K, int row0, int nrows,
                            const bf16_t* __restrict__ src, int64_t rs, int64_t cs, int64_t src_bs,
                            int64_t dst_bs) {
  const int64_t slot = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;   // (tile, lane)
  const int64_t nslots = (int64_t)NT * KT * 64;
  if (slot >= nslots) return;
  const int lane = int(slot & 63);
  const int64_t tile = slot >> 6;
  const int nt = int(tile / KT), kt = int(tile % KT);
  const int n = nt * 16 + (lane & 15);
  if (n < row0 || n >= row0 + nrows) return;
  const bf16_t* s = src + (int64_t)blockIdx.z * src_bs + (int64_t)(n - row0) * rs;
  const int k0 = kt * 32 + (lane >> 4) * 8;
  uint32_t h[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const int k = k0 + e;
    h[e] = k < K ? s[(int64_t)k * cs] : 0u;
  }
  dst[(int64_t)blockIdx.z * dst_bs + slot] =
      uint4{h[0] | (h[1] << 16), h[2] | (h[3] << 16), h[4] | (h[5] << 16), h[6] | (h[7] << 16)};
}

hipError_t launch_pack(uint4* dst, int NT, int KT, int K, int row0, int nrows, const bf16_t* src,
                       int64_t rs, int64_t cs, int batch, int64_t src_bs, int64_t dst_bs,
                       hipStream_t st) {
  const int64_t nslots = (int64_t)NT * KT * 64;
  dim3 grid((unsigned)((nslots + 255) / 256), 1, batch);
  hipLaunchKernelGGL(pack_kernel, grid, dim3(256), 0, st, dst, NT, KT, K, row0, nrows, src, rs, cs,
                     src_bs, dst_bs);
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
