// Relaxed chain verification for rows inside a thinking span (MAX-walkthrough
// section 10: relaxed acceptance with relaxed_topk and relaxed_delta).
//
// Draft token d at verified position j is accepted by a relaxed row when it
// is among the target's topk most likely tokens and its logit is at most
// delta below the target's best (the log-probability gap equals the logit
// gap: the softmax normaliser cancels).  Rows outside a thinking span keep
// the greedy rule (d is the target's top-1).  Both rules reduce to one
// number per position: rank(d) = the count of tokens ordered before d (a
// higher logit, or the same logit and a lower id), so the decision needs
// one pass over the logits and no sort.
//
// Pass 1 (grid chunks x positions x rows): each workgroup streams one chunk
// of one position's logits (HBM-bound, 16-byte non-temporal loads) and
// writes the chunk's (max key, count before d).  Pass 2 (one wave per row,
// one lane per position) combines each position's chunks, finds the first
// rejection with a ballot and reads the bonus token from that position's
// max key.
#include "common.h"
#include "internal.h"

namespace e3 {

namespace {
constexpr int RX_THREADS = 256;
constexpr int RX_VEC = 4 * RX_THREADS;        // floats per workgroup per iteration
constexpr int RX_TARGET_BLOCKS = 2048;        // >= 8 workgroups per CU over 256 CUs
constexpr int RX_MIN_CHUNK = 4 * RX_VEC;      // at least 4 loads per thread
constexpr int RX_UNROLL = 4;                  // loads in flight per thread

__device__ __forceinline__ float key_value(uint64_t k) {
  const uint32_t o = uint32_t(k >> 32);
  return __uint_as_float((o & 0x80000000u) ? (o & 0x7FFFFFFFu) : ~o);
}

__device__ __forceinline__ uint64_t umax64(uint64_t a, uint64_t b) { return a > b ? a : b; }

__device__ __forceinline__ uint64_t shfl_xor64(uint64_t v, int o) {
  const uint32_t lo = __shfl_xor(uint32_t(v), o, WAVE), hi = __shfl_xor(uint32_t(v >> 32), o, WAVE);
  return (uint64_t(hi) << 32) | lo;
}

// One logit into the chunk's state.  -0 is folded onto +0 so that the max key
// and the count treat the two zeros as the same value, as comparisons do.
__device__ __forceinline__ void rx_take(float e, uint32_t idx, float zd, int d, uint64_t& best,
                                        uint32_t& cnt) {
  const float v = e + 0.0f;
  best = umax64(best, argmax_key(v, idx));
  cnt += (v > zd) | ((v == zd) & (int(idx) < d));
}
}  // namespace

template <bool VEC>
__global__ __launch_bounds__(RX_THREADS) void relaxed_scan_kernel(const float* __restrict__ logits,
                                                                  const int32_t* __restrict__ draft,
                                                                  int gamma, int V, int chunk,
                                                                  uint4* __restrict__ part) {
  const int c = blockIdx.x, j = blockIdx.y, b = blockIdx.z, S = gridDim.x;
  const int64_t row = (int64_t)b * (gamma + 1) + j;
  const float* z = logits + row * V;
  int d = j < gamma ? draft[(int64_t)b * gamma + j] : -1;
  if (d >= V) d = -1;                                   // out of range: never accepted
  const float zd = d >= 0 ? z[d] + 0.0f : 0.f;
  const int lo = c * chunk, hi = min(V, lo + chunk);
  uint64_t best = 0;
  uint32_t cnt = 0;
  if (VEC) {
    // lo and hi - lo are multiples of 4 (chunk is, and V is) and the row
    // starts 16-byte aligned, so every float4 lies inside [lo, hi).  RX_UNROLL
    // loads are issued before any is used, to keep enough bytes in flight.
    for (int base = lo + 4 * threadIdx.x; base < hi; base += RX_UNROLL * RX_VEC) {
      uint4 w[RX_UNROLL];
#pragma unroll
      for (int u = 0; u < RX_UNROLL; ++u) {
        const int i = base + u * RX_VEC;
        if (i < hi) w[u] = load_nt(reinterpret_cast<const uint4*>(z + i));
      }
#pragma unroll
      for (int u = 0; u < RX_UNROLL; ++u) {
        const int i = base + u * RX_VEC;
        if (i < hi) {
          rx_take(__uint_as_float(w[u].x), i, zd, d, best, cnt);
          rx_take(__uint_as_float(w[u].y), i + 1, zd, d, best, cnt);
          rx_take(__uint_as_float(w[u].z), i + 2, zd, d, best, cnt);
          rx_take(__uint_as_float(w[u].w), i + 3, zd, d, best, cnt);
        }
      }
    }
  } else {
    for (int i = lo + threadIdx.x; i < hi; i += RX_THREADS) rx_take(z[i], i, zd, d, best, cnt);
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    best = umax64(best, shfl_xor64(best, o));
    cnt += __shfl_xor(cnt, o, WAVE);
  }
  __shared__ uint64_t rb[RX_THREADS / WAVE];
  __shared__ uint32_t rc[RX_THREADS / WAVE];
  const int lane = threadIdx.x & (WAVE - 1), wid = threadIdx.x / WAVE;
  if (lane == 0) {
    rb[wid] = best;
    rc[wid] = cnt;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
#pragma unroll
    for (int w = 1; w < RX_THREADS / WAVE; ++w) {
      best = umax64(best, rb[w]);
      cnt += rc[w];
    }
    part[row * S + c] = uint4{uint32_t(best), uint32_t(best >> 32), cnt, 0u};
  }
}

// One wave per row: lane l evaluates position base + l (all positions of a
// 64-wide window at once, each combining its chunks with independent loads),
// a ballot finds the first rejected position, and the bonus comes from that
// lane's max key.
__global__ __launch_bounds__(64) void relaxed_final_kernel(const float* __restrict__ logits,
                                                           const int32_t* __restrict__ draft,
                                                           const uint8_t* __restrict__ relaxed, int gamma,
                                                           int V, int S, int topk, float delta,
                                                           const uint4* __restrict__ part,
                                                           int32_t* __restrict__ accept_len,
                                                           int32_t* __restrict__ bonus) {
  const int b = blockIdx.x, lane = threadIdx.x;
  const bool rel = relaxed ? relaxed[b] != 0 : true;
  for (int base = 0; base <= gamma; base += WAVE) {
    const int j = base + lane;
    uint64_t best = 0;
    bool ok = false;
    if (j <= gamma) {
      const uint4* p = part + ((int64_t)b * (gamma + 1) + j) * S;
      uint32_t cnt = 0;
#pragma unroll 8
      for (int c = 0; c < S; ++c) {
        const uint4 q = p[c];
        best = umax64(best, (uint64_t(q.y) << 32) | q.x);
        cnt += q.z;
      }
      if (j < gamma) {
        const int d = draft[(int64_t)b * gamma + j];
        if (d >= 0 && d < V) {
          if (!rel) {
            ok = cnt == 0;
          } else {
            // the gap of two fp32 logits is exact in fp64
            const float zd = logits[((int64_t)b * (gamma + 1) + j) * V + d] + 0.0f;
            ok = cnt < uint32_t(topk) && (double)zd - (double)key_value(best) >= -(double)delta;
          }
        }
      }
    }
    // first position of the window that is not an accepted draft (position
    // gamma is never "ok", so the last window always stops)
    const uint64_t stop = __ballot(!ok);
    if (stop) {
      const int first = __builtin_ctzll(stop);
      const uint32_t lo = __shfl(uint32_t(best), first, WAVE), hi = __shfl(uint32_t(best >> 32), first, WAVE);
      if (lane == 0) {
        accept_len[b] = base + first;
        bonus[b] = (int32_t)argmax_key_index((uint64_t(hi) << 32) | lo);
      }
      return;
    }
  }
}

void relaxed_layout(int B, int gamma, int V, int* nchunks, int* chunk) {
  const int64_t rows = (int64_t)B * (gamma + 1);
  int64_t s = (RX_TARGET_BLOCKS + rows - 1) / rows;
  const int64_t smax = (V + RX_MIN_CHUNK - 1) / RX_MIN_CHUNK;
  if (s > smax) s = smax;
  if (s < 1) s = 1;
  // chunks of whole iterations; the last one may be short
  const int64_t c = ((V + s - 1) / s + RX_VEC - 1) / RX_VEC * RX_VEC;
  *chunk = (int)c;
  *nchunks = (int)((V + c - 1) / c);
}

hipError_t launch_relaxed_scan(const float* logits, const int32_t* draft, int B, int gamma, int V, uint4* part,
                               hipStream_t st) {
  int S, chunk;
  relaxed_layout(B, gamma, V, &S, &chunk);
  const dim3 grid(S, gamma + 1, B);
  const bool vec = (V % 4 == 0) && (reinterpret_cast<uintptr_t>(logits) % 16 == 0);
  if (vec)
    hipLaunchKernelGGL(relaxed_scan_kernel<true>, grid, dim3(RX_THREADS), 0, st, logits, draft, gamma, V,
                       chunk, part);
  else
    hipLaunchKernelGGL(relaxed_scan_kernel<false>, grid, dim3(RX_THREADS), 0, st, logits, draft, gamma, V,
                       chunk, part);
  return hipGetLastError();
}

hipError_t launch_relaxed_final(const float* logits, const int32_t* draft, const uint8_t* relaxed, int B,
                                int gamma, int V, int topk, float delta, const uint4* part, int32_t* accept_len,
                                int32_t* bonus, hipStream_t st) {
  int S, chunk;
  relaxed_layout(B, gamma, V, &S, &chunk);
  hipLaunchKernelGGL(relaxed_final_kernel, dim3(B), dim3(WAVE), 0, st, logits, draft, relaxed, gamma, V, S,
                     topk, delta, part, accept_len, bonus);
  return hipGetLastError();
}

}  // namespace e3
