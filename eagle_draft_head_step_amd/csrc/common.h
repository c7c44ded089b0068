// Device helpers shared by the gfx950 kernels of the draft head.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace e3 {

typedef uint16_t bf16_t;                                             // raw bf16 bits
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));           // MFMA operand
typedef float f32x4 __attribute__((ext_vector_type(4)));             // 16x16 MFMA accumulator

constexpr int WAVE = 64;

__device__ __forceinline__ float bf2f(bf16_t h) { return __uint_as_float(uint32_t(h) << 16); }

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

// float -> bf16, round to nearest even (gfx950 v_cvt_pk_bf16_f32).
__device__ __forceinline__ bf16_t f2bf(float f) { return __builtin_bit_cast(bf16_t, (__bf16)f); }

// x = hi + lo with hi = bf16(x) and lo = bf16(x - hi), for 8 floats.
__device__ __forceinline__ void split_bf16x8(const float4& a, const float4& b, uint4& hi, uint4& lo);

// Two floats -> two bf16 (round to nearest even) in one word, lo first.
__device__ __forceinline__ uint32_t pack2bf(float lo, float hi) {
  const bf16x2_t v = {(__bf16)lo, (__bf16)hi};
  return __builtin_bit_cast(uint32_t, v);
}

__device__ __forceinline__ void split_bf16x8(const float4& a, const float4& b, uint4& hi, uint4& lo) {
  const float x[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
  uint32_t h[8], r[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    h[i] = f2bf(x[i]);
    r[i] = f2bf(x[i] - bf2f((bf16_t)h[i]));
  }
  hi = uint4{h[0] | (h[1] << 16), h[2] | (h[3] << 16), h[4] | (h[5] << 16), h[6] | (h[7] << 16)};
  lo = uint4{r[0] | (r[1] << 16), r[2] | (r[3] << 16), r[4] | (r[5] << 16), r[6] | (r[7] << 16)};
}

// The 8 bf16 of a 16-byte word, widened.
__device__ __forceinline__ void unpack8(const uint4& v, float* f) {
  f[0] = __uint_as_float(v.x << 16); f[1] = __uint_as_float(v.x & 0xFFFF0000u);
  f[2] = __uint_as_float(v.y << 16); f[3] = __uint_as_float(v.y & 0xFFFF0000u);
  f[4] = __uint_as_float(v.z << 16); f[5] = __uint_as_float(v.z & 0xFFFF0000u);
  f[6] = __uint_as_float(v.w << 16); f[7] = __uint_as_float(v.w & 0xFFFF0000u);
}

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// Streaming 16-byte load (non-temporal: the data is used once).
__device__ __forceinline__ uint4 load_nt(const uint4* p) {
  const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
  return uint4{v.x, v.y, v.z, v.w};
}

__device__ __forceinline__ bf16x8 as_bf16x8(const uint4& v) { return __builtin_bit_cast(bf16x8, v); }

// D(16x16, f32) += A(16x32) * B(32x16), bf16 inputs.
// Lane l supplies A row (l & 15), k = 8*(l >> 4) .. +7 and B column (l & 15),
// the same k; it receives D rows 4*(l >> 4) .. +3 of column (l & 15).
__device__ __forceinline__ f32x4 mfma16x16x32(const uint4& a, const uint4& b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(a), as_bf16x8(b), c, 0, 0, 0);
}

typedef short s16x4 __attribute__((ext_vector_type(4)));

// D(16x16, f32) += A(16x16) * B(16x16), bf16 inputs: lane l supplies row/column
// (l & 15) with k = 4*(l >> 4) .. +3; D as for the 16x16x32 form.
__device__ __forceinline__ f32x4 mfma16x16x16(const uint2& a, const uint2& b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(s16x4, a),
                                                   __builtin_bit_cast(s16x4, b), c, 0, 0, 0);
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, WAVE);
  return v;
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, WAVE));
  return v;
}

// Sum over the whole block (blockDim.x a multiple of 64, <= 1024).  `red`
// holds >= 16 floats of shared memory.  All threads get the result.
__device__ __forceinline__ float block_sum(float v, float* red) {
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6, nw = blockDim.x >> 6;
  v = wave_sum(v);
  __syncthreads();
  if (lane == 0) red[wid] = v;
  __syncthreads();
  float t = 0.f;
  for (int i = 0; i < nw; ++i) t += red[i];
  return t;
}

// Order-preserving map of a float onto uint32 (larger float -> larger key).
__device__ __forceinline__ uint32_t ordered_key(float f) {
  uint32_t u = __float_as_uint(f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// 64-bit argmax candidate: value in the high word, and ~index in the low word
// so that among equal values the lowest index has the largest key.
__device__ __forceinline__ uint64_t argmax_key(float v, uint32_t idx) {
  return (uint64_t(ordered_key(v)) << 32) | uint64_t(0xFFFFFFFFu - idx);
}

// Position of row i's new token and the page-table row it reads: the
// per-token arrays when given (multi-token extend: row i is one new token),
// else ctx_len[i] + step with table row i (one draft step per sequence).
__device__ __forceinline__ int new_token_pos(const int32_t* tok_pos, const int32_t* ctx_len, int step, int i) {
  return tok_pos ? tok_pos[i] : ctx_len[i] + step;
}
__device__ __forceinline__ int table_row(const int32_t* tok_row, int i) { return tok_row ? tok_row[i] : i; }

__device__ __forceinline__ uint32_t argmax_key_index(uint64_t k) {
  return 0xFFFFFFFFu - uint32_t(k & 0xFFFFFFFFu);
}

}  // namespace e3
