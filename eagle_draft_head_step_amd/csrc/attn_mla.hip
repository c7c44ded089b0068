// Paged decode attention of the MLA head in absorbed form, on the CDNA4
// matrix cores.
//
// With W_UK absorbed into the query (q_lat = W_UK^T q_nope, per head) and
// W_UV applied after attention, every head attends over the same cached
// entries [latent c (512) | rotated k_pe (64)]:
//     s[h, j] = tau * (q_lat[h] . c_j + q_pe[h] . k_pe_j),
//     o_lat[h] = sum_j softmax_j(s[h, :]) c_j.
//
// Work split.  The (row, 32-key tile) pairs of the batch, numbered row by
// row, are cut into one equal contiguous range per workgroup of a grid sized
// to the chip (one workgroup per CU), so ragged context lengths leave no CU
// idle.  A range holds whole rows, written out directly, and at most two
// partial rows -- its first and its last -- whose (max, sum, output) partials
// the combine kernel merges.  A small schedule kernel (one launch per chain,
// a block per step) turns ctx_len into the row prefix sums, each workgroup's
// range and first row, and each row's first and last workgroup.  For the
// extend's token rows the ranges are cut at row starts instead, so that a
// sequence's new tokens read the same cache tiles side by side (L2 hits).
//
// Per tile, each wave takes 32 heads (the N dimension of
// v_mfma_f32_32x32x16_bf16):
//   S^T[32 keys x 32 heads] = C[keys x 576] . Q^T           36 MFMAs, K = 16 dims
//   O^T[512 x 32 heads]   += C^T[512 x 32 keys] . P^T       32 MFMAs, K = 16 keys
// The score accumulator is already the B operand of the second product: the
// order in which the 16 keys of each P.V contraction are summed is chosen to
// match the score layout, so P never leaves registers.
//
// Registers.  This file is compiled with the matrix-core results in VGPRs
// (the LLVM option amdgpu-mfma-vgpr-form): the 256 output accumulators then
// sit in VGPRs and the query fragments and long-lived offsets in AGPRs, which
// the MFMAs and v_accvgpr_read reach directly.  With the default placement
// the score accumulator takes AGPRs, 16 output accumulators and 21 other
// values fall out to scratch memory, and a kernel with scratch pays several
// microseconds more per dispatch.
//
// The cache tile (32 keys x 1152 bytes) is copied straight from HBM into LDS
// by the LDS DMA (global_load_lds_dwordx4: no registers, no VALU), into a
// ring of three tile buffers, two tiles in flight while one is computed.
// Cache pages store the entries in 16-value chunks ([chunk][slot][16]), so
// each DMA instruction (one chunk of 32 keys) reads one contiguous KiB.  In
// LDS each 16-dimension chunk of the tile is 1 KB of 16-byte pieces (key k,
// dimension half hs) at slot 32*hs + (k ^ 4*hs): the score MFMA reads one piece
// per lane (ds_read_b128) and the P.V MFMA reads four keys of one dimension
// per lane with the transposing ds_read_b64_tr_b16; the xor keeps the two
// dimension halves of a transposed read on different banks.
#include <math.h>
#include "common.h"
#include "internal.h"

namespace e3 {

typedef float f32x16 __attribute__((ext_vector_type(16)));

// D(32x32, f32) += A(32x16) * B(16x32), bf16 inputs.  Lane l supplies A row
// (l & 31) and B column (l & 31) with k = 8*(l >> 5) .. +7; it receives D
// column (l & 31), rows 8*(r/4) + 4*(l >> 5) + r%4 for r = 0..15.
__device__ __forceinline__ f32x16 mfma32x32x16(const uint4& a, const uint4& b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(a), as_bf16x8(b), c, 0, 0, 0);
}

namespace {
constexpr int TK = 32;                  // keys per tile
constexpr int DQK = 576;                // latent + rope
constexpr int RL = 512;                 // latent
constexpr int NCH = DQK / 16;           // 16-dimension chunks per tile, 1 KB each in LDS
constexpr int TILE_BYTES = NCH * 1024;
constexpr int NBUF = 3;                 // tile buffers in the LDS ring
constexpr int HPW = 32;                 // heads per wave
constexpr int NQR = 28;                 // query fragments held in registers; the rest in LDS
constexpr int PG_MAX = 2048;            // page ids of a row segment kept in LDS (the rest read from HBM)
constexpr int SCHED_THREADS = 1024;
constexpr float kRefSlack = 20.f;       // log2 headroom of the softmax reference
#ifndef E3_MLA_SR
#define E3_MLA_SR 3
#endif
#ifndef E3_MLA_PR
#define E3_MLA_PR 1
#endif

typedef __attribute__((address_space(3))) char lds_char;
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

__device__ __forceinline__ int slot_of(int key, int hs) { return 32 * hs + (key ^ (4 * hs)); }

typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
// two floats -> two fp16 (round to nearest even), low half first
__device__ __forceinline__ uint32_t pack2h(float x, float y) {
  const f16x2 v = {(_Float16)x, (_Float16)y};
  return __builtin_bit_cast(uint32_t, v);
}
__device__ __forceinline__ float4 unpack4h(uint2 u) {
  const f16x2 a = __builtin_bit_cast(f16x2, u.x), b = __builtin_bit_cast(f16x2, u.y);
  return make_float4((float)a.x, (float)a.y, (float)b.x, (float)b.y);
}

// LDS DMA of 16 bytes per lane: lane i's 16 bytes at base + voff (uniform
// base, per-lane 32-bit byte offset) land at LDS byte address lds + 16*i.
// The compiler does not track it; callers wait with vmcnt.
__device__ __forceinline__ void lds_dma16(const void* base, uint32_t voff, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1"
               :: "v"(voff), "s"(base), "s"(lds) : "memory", "m0");
}

// s_waitcnt with only a vector-memory count (0..63).
#define E3_WAIT_VMCNT(n) __builtin_amdgcn_s_waitcnt(0x3F70 | ((n) & 15) | (((n) >> 4) << 14))

__device__ __forceinline__ void block_barrier() {
  __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0): this wave's LDS reads are done
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

__device__ __forceinline__ uint2 lds_read_tr(lds_char* base, int off) {
  const s16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(base + off));
  return __builtin_bit_cast(uint2, v);
}

__device__ __forceinline__ int cdiv_i64(int64_t a, int64_t b) { return (int)((a + b - 1) / b); }
}  // namespace

// Work schedule of one step (block s computes step step0 + s into sched +
// s*stride), B rows and nb workgroups:
//   sched[0 .. B]                 running sum of 32-key tiles over rows (P);
//   sched[B+1+w]                  the row holding workgroup w's first tile;
//   sched[B+1+nb+w], w <= nb      first tile of workgroup w's range (its range
//                                 ends where workgroup w+1's starts);
//   sched[B+2+2nb+b], [+B]        the workgroups holding row b's first and last
//                                 tiles (equal when one workgroup has the row).
// Balanced: workgroup w owns tiles [w*T/nb, (w+1)*T/nb) of the T tiles, so
// ragged contexts cost no imbalance.  Row-aligned (the extend's token rows,
// when there are at most nb/2 of them): row b with t_b tiles gets
// n_b = 1 + floor(t_b (nb - B) / T) consecutive workgroups and cuts its tiles
// into that many equal chunks (the workgroups past the last row get empty
// ranges).  A sequence's consecutive new tokens have (nearly always) the same
// tile count, hence the same chunks, so they read the same keys at the same
// moment on neighbouring workgroups, which sit on one XCD, and the cache tile
// one token's workgroup reads is an L2 hit for the next's.
__device__ __forceinline__ int sched_first_row(const int32_t* sched, int B, int w) { return sched[B + 1 + w]; }
__device__ __forceinline__ int sched_start(const int32_t* sched, int B, int nb, int w) { return sched[B + 1 + nb + w]; }
__device__ __forceinline__ int sched_wlo(const int32_t* sched, int B, int nb, int b) { return sched[B + 2 + 2 * nb + b]; }
__device__ __forceinline__ int sched_whi(const int32_t* sched, int B, int nb, int b) { return sched[2 * B + 2 + 2 * nb + b]; }

__global__ __launch_bounds__(SCHED_THREADS) void mla_attn_schedule_kernel(const int32_t* __restrict__ ctx_len,
                                                                          const int32_t* __restrict__ tok_pos,
                                                                          int step0, int B, int nb,
                                                                          int32_t* __restrict__ sched_all,
                                                                          int stride) {
  __shared__ int wsum[SCHED_THREADS / 64], wsum_n[SCHED_THREADS / 64];
  __shared__ int used;
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  const int step = step0 + blockIdx.x;
  int32_t* sched = sched_all + (int64_t)blockIdx.x * stride;
  int32_t* first_row = sched + B + 1;
  int32_t* starts = sched + B + 1 + nb;
  int32_t* wlo = sched + B + 2 + 2 * nb;
  int32_t* whi = wlo + B;
  const bool aligned = tok_pos != nullptr && 2 * B <= nb;
  auto tiles = [&](int b) { return b < B ? (new_token_pos(tok_pos, ctx_len, step, b) + 1 + TK - 1) / TK : 0; };
  // pass 1: total
  int part = 0;
  for (int b = tid; b < B; b += SCHED_THREADS) part += tiles(b);
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) part += __shfl_xor(part, o, 64);
  if (lane == 0) wsum[wid] = part;
  __syncthreads();
  int total = 0;
  for (int i = 0; i < SCHED_THREADS / 64; ++i) total += wsum[i];
  __syncthreads();
  if (aligned) {
    // B <= nb / 2 <= MAX_ATTN_BLOCKS / 2 rows: one thread per row
    const int b = tid;
    const int v = tiles(b);
    const int n = b < B ? 1 + (int)((int64_t)v * (nb - B) / total) : 0;
    int iv = v, in = n;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int yv = __shfl_up(iv, o, 64), yn = __shfl_up(in, o, 64);
      if (lane >= o) { iv += yv; in += yn; }
    }
    if (lane == 63) { wsum[wid] = iv; wsum_n[wid] = in; }
    __syncthreads();
    int offv = 0, offn = 0;
    for (int i = 0; i < wid; ++i) { offv += wsum[i]; offn += wsum_n[i]; }
    const int pe = offv + iv, pb = pe - v, we = offn + in, w0 = we - n;
    if (b < B) {
      sched[b + 1] = pe;
      for (int c = 0; c < n; ++c) {
        starts[w0 + c] = pb + (int)((int64_t)c * v / n);
        first_row[w0 + c] = b;
      }
      wlo[b] = w0 + (n + v - 1) / v - 1;   // the first chunk that is not empty
      whi[b] = w0 + n - 1;
      if (b == B - 1) used = we;            // <= B + (nb - B) = nb
    }
    __syncthreads();
    for (int w = used + tid; w <= nb; w += SCHED_THREADS) {   // past the last row: empty
      starts[w] = total;
      if (w < nb) first_row[w] = B - 1;
    }
    if (tid == 0) sched[0] = 0;
    return;
  }
  for (int w = tid; w <= nb; w += SCHED_THREADS) starts[w] = (int)((int64_t)w * total / nb);
  // pass 2: prefix sums, first rows and row spans, one chunk of rows at a time
  int carry = 0;
  for (int base = 0; base < B; base += SCHED_THREADS) {
    const int b = base + tid;
    const int v = tiles(b);
    int inc = v;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int y = __shfl_up(inc, o, 64);
      if (lane >= o) inc += y;
    }
    if (lane == 63) wsum[wid] = inc;
    __syncthreads();
    int off = carry, tot = 0;
    for (int i = 0; i < SCHED_THREADS / 64; ++i) {
      if (i < wid) off += wsum[i];
      tot += wsum[i];
    }
    if (b < B) {
      const int pe = off + inc, pb = pe - v;
      sched[b + 1] = pe;
      const int wa = cdiv_i64((int64_t)pb * nb, total), wb = cdiv_i64((int64_t)pe * nb, total);
      for (int w = wa; w < wb; ++w) first_row[w] = b;
      wlo[b] = cdiv_i64((int64_t)(pb + 1) * nb, total) - 1;
      whi[b] = wb - 1;
    }
    carry += tot;
    __syncthreads();
  }
  if (tid == 0) sched[0] = 0;
}

template <int NW>
__global__ __launch_bounds__(NW * 64) void mla_attn_kernel(MlaAttnArgs a) {
  __shared__ __attribute__((aligned(1024))) char lds[NBUF * TILE_BYTES + NW * (NCH - NQR) * 1024];
  __shared__ int pg_lds[PG_MAX];        // page ids of the current row segment
  constexpr int DPW = NCH / NW;         // DMA chunks per wave per tile
  static_assert(NCH % NW == 0, "every wave issues the same number of DMA chunks");

  // Range index of this workgroup.  Workgroups are dealt round-robin to the
  // 8 XCDs (each with its own L2), so ranges w and w + 1 would sit on
  // different XCDs; numbering the ranges XCD by XCD keeps a row's neighbouring
  // ranges, which load the same queries, behind one L2.
  const int nb = gridDim.x, hg = blockIdx.y;
  const int w = (nb % 8 == 0) ? (int)(blockIdx.x % 8) * (nb / 8) + (int)(blockIdx.x / 8) : (int)blockIdx.x;
  const int start = sched_start(a.sched, a.B, nb, w);
  const int end = sched_start(a.sched, a.B, nb, w + 1);
  if (start >= end) return;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wid = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int hcol = lane & 31, hs = lane >> 5;
  const int head = (hg * NW + wid) * HPW + hcol;
  const bool head_ok = head < a.nh;
  const float sl2 = a.scale * 1.4426950408889634f;   // tau * log2(e)
  const uint32_t lds_addr = (uint32_t)(uintptr_t)(lds_char*)lds;

  // per-lane LDS byte offsets: score piece (key hcol, half hs), and the four
  // transposed reads (key group c, second half rho) of a 32-dimension block
  const int sc_off = 16 * slot_of(hcol, hs);
  int tr_off[2][2];
  {
    const int G = lane >> 4, j = lane & 15, e = j >> 2, q = j & 3;
#pragma unroll
    for (int c = 0; c < 2; ++c)
#pragma unroll
      for (int rho = 0; rho < 2; ++rho) {
        const int key = 16 * c + 8 * rho + 4 * (G >> 1) + e;
        tr_off[c][rho] = 1024 * (G & 1) + 16 * slot_of(key, q >> 1) + 8 * (q & 1);
      }
  }
  // DMA: lane s of a chunk fetches (key (s&31) ^ 4*(s>>5), dimension half s>>5)
  const int dma_key = (lane & 31) ^ (4 * (lane >> 5));
  const int dma_dim = 8 * (lane >> 5);

  int b = sched_first_row(a.sched, a.B, w);
  int cur = start;
  while (cur < end) {
    const int pb = a.sched[b], pe = a.sched[b + 1];
    const int t0 = cur - pb, t1 = min(end, pe) - pb;   // tiles [t0, t1) of row b
    const int n = new_token_pos(a.tok_pos, a.ctx_len, a.step, b) + 1;   // keys of row b
    const int nt = t1 - t0;

    const int32_t* table = a.table + (int64_t)table_row(a.tok_row, b) * a.max_pages;
    // The segment's page ids go to LDS, loaded together with the queries (one
    // wait for both).  A tile's DMA then takes its page id from LDS: a page id
    // read from HBM there would wait for every earlier vector-memory operation,
    // the previous tile's DMA included (they complete in order), and only one
    // tile would stream ahead.
    const int p_lo = (t0 * TK) / a.page_size;
    const int npg = min(((t1 - 1) * TK) / a.page_size - p_lo + 1, PG_MAX);
    const int pg0 = tid < npg ? table[p_lo + tid] : 0;
    // page id of tile t as held in LDS (per lane, all lanes equal; a tile
    // past the PG_MAX pages held there reads its id from HBM at the DMA)
    auto page_of = [&](int t) { return pg_lds[min((t * TK) / a.page_size - p_lo, PG_MAX - 1)]; };
    auto issue = [&](int t, int bi, int page_v) {
      const int j0 = t * TK;
      // page id and slot are uniform: scalar registers for the DMA base
      const int pidx = j0 / a.page_size;
      int page;
      if (pidx - p_lo < PG_MAX) page = __builtin_amdgcn_readfirstlane(page_v);
      else page = __builtin_amdgcn_readfirstlane(table[pidx]);
      const int jslot = __builtin_amdgcn_readfirstlane(j0 % a.page_size);
      // keys past the end re-read the row's last key (their scores are masked)
      // (the page's chunk offsets, at most 36 x page_size x 32 bytes, go in
      // the per-lane offset; the base stays uniform)
      const uint32_t chunk_bytes = (uint32_t)a.page_size * 32u;
      const uint32_t voff = (uint32_t)(min(dma_key, n - 1 - j0) * 16 + dma_dim) * 2u +
                            (uint32_t)(wid * DPW) * chunk_bytes;
      const char* base = reinterpret_cast<const char*>(
          a.cache + ((int64_t)page * DQK * a.page_size + (int64_t)jslot * 16));
      const uint32_t dst = lds_addr + bi * TILE_BYTES + wid * DPW * 1024;
#pragma unroll
      for (int i = 0; i < DPW; ++i) lds_dma16(base, voff + (uint32_t)i * chunk_bytes, dst + i * 1024);
    };
    // Q^T fragments (B operand of the scores): head, dims 16*ks + 8*hs .. +7.
    // The first NQR stay in registers; the others (rope included) go to this
    // wave's LDS area in lane order and are read with the cache fragments.
    uint4 qf[NQR];
    uint4* qlds = reinterpret_cast<uint4*>(lds + NBUF * TILE_BYTES + wid * (NCH - NQR) * 1024);
    {
      const bf16_t* ql = a.q_lat + ((int64_t)b * a.nh + head) * RL;
      const bf16_t* qp = a.q_pe + ((int64_t)b * a.nh + head) * 64;
#pragma unroll
      for (int ks = 0; ks < NCH; ++ks) {
        const int d = 16 * ks + 8 * hs;
        const uint4 v = !head_ok ? uint4{0u, 0u, 0u, 0u}
                        : d < RL ? *reinterpret_cast<const uint4*>(ql + d)
                                 : *reinterpret_cast<const uint4*>(qp + (d - RL));
        if (ks < NQR) qf[ks] = v;
        else qlds[(ks - NQR) * 64 + lane] = v;
      }
    }
    if (tid < npg) pg_lds[tid] = pg0;
    for (int k = tid + NW * 64; k < npg; k += NW * 64) pg_lds[k] = table[p_lo + k];
    block_barrier();                     // the segment's page ids are in LDS
    // the first two tiles go out after the query loads, so that waiting for
    // tile t0 (in-order vmcnt) also covers the queries
    issue(t0, 0, page_of(t0));
    if (nt > 1) issue(t0 + 1, 1, page_of(t0 + 1));
    // The page id of the tile two ahead is read from LDS one tile early, so
    // its LDS round trip is off the path from the barrier to the DMAs.
    int pg_next = nt > 2 ? page_of(t0 + 2) : 0;

    f32x16 acc[RL / 32];
#pragma unroll
    for (int i = 0; i < RL / 32; ++i)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][r] = 0.f;
    float m = -INFINITY, l = 0.f;
    int bi = 0, bi2 = 2;                 // ring slots of tiles t and t+2
    for (int i = 0; i < nt; ++i) {
      const int t = t0 + i;
      if (i + 1 < nt) E3_WAIT_VMCNT(DPW); else E3_WAIT_VMCNT(0);
      block_barrier();                   // tile t in LDS for every wave; tile t-1 done by every wave
      if (i + 2 < nt) issue(t + 2, bi2, pg_next);
      if (i + 3 < nt) pg_next = page_of(t + 3);

      const int tile_off = __builtin_amdgcn_readfirstlane(bi * TILE_BYTES);
      const char* tb = lds + tile_off;
      // scores: one accumulation chain (back-to-back accumulation into the
      // same registers is forwarded), LDS fragments read three steps ahead
      const char* sp = tb + sc_off;
      f32x16 sacc;
#pragma unroll
      for (int r = 0; r < 16; ++r) sacc[r] = 0.f;
      constexpr int SR = E3_MLA_SR;       // score fragments in flight
      uint4 cf[SR], qb[SR];
      auto fetch = [&](int ks) {
        cf[ks % SR] = *reinterpret_cast<const uint4*>(sp + ks * 1024);
        if (ks >= NQR) qb[ks % SR] = qlds[(ks - NQR) * 64 + lane];
      };
#pragma unroll
      for (int k = 0; k < SR; ++k) fetch(k);
#pragma unroll
      for (int ks = 0; ks < NCH; ++ks) {
        sacc = mfma32x32x16(cf[ks % SR], ks < NQR ? qf[ks < NQR ? ks : 0] : qb[ks % SR], sacc);
        if (ks + SR < NCH) fetch(ks + SR);
        __builtin_amdgcn_sched_barrier(0);
      }
      // P.V operands: transposed fragments of value block blk+PR are read
      // while blk is multiplied; block 0's go out before the softmax, whose
      // VALU work then covers their LDS latency
      lds_char* tbl = (lds_char*)lds + tile_off;   // LDS address space: offsets fold
      lds_char* tp0 = tbl + tr_off[0][0];
      lds_char* tp1 = tbl + tr_off[0][1];
      lds_char* tp2 = tbl + tr_off[1][0];
      lds_char* tp3 = tbl + tr_off[1][1];
      constexpr int PR = E3_MLA_PR;       // transposed value blocks in flight
      uint2 vf[PR + 1][4];
      auto read_blk = [&](int blk, uint2 (&d)[4]) {
        d[0] = lds_read_tr(tp0, blk * 2048);
        d[1] = lds_read_tr(tp1, blk * 2048);
        d[2] = lds_read_tr(tp2, blk * 2048);
        d[3] = lds_read_tr(tp3, blk * 2048);
      };
      read_blk(0, vf[0]);
      // lane holds keys t*32 + 8*(r/4) + 4*hs + r%4 of head `head`
      float x[16];
#pragma unroll
      for (int r = 0; r < 16; ++r) x[r] = sacc[r] * sl2;
      if ((t + 1) * TK > n) {
#pragma unroll
        for (int r = 0; r < 16; ++r)
          if (t * TK + 8 * (r >> 2) + 4 * hs + (r & 3) >= n) x[r] = -INFINITY;
      }
      // Lazy reference: m only moves when a score exceeds it by more than
      // 2^20 (p <= 2^20 is exact enough in bf16 and far from fp32 overflow),
      // so the accumulators are rescaled on very few tiles.  Whether any head
      // moves is decided from each lane's own scores (a wave vote, no
      // cross-lane exchange); the head maxima, which need the other half's
      // keys, are formed only on those tiles.  The rescale goes through AGPRs
      // (inline asm); with that form the main path's register allocation
      // measured slightly faster than with a plain multiply.
      const float thr = m + kRefSlack;
      bool up = false;
#pragma unroll
      for (int r = 0; r < 16; ++r) up |= x[r] > thr;
      if (__any(up)) {
        float mx = x[0];
#pragma unroll
        for (int r = 1; r < 16; ++r) mx = fmaxf(mx, x[r]);
        mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
        const float mn = mx > thr ? mx : m;
        if (i > 0) {                       // on the first tile acc and l are still zero
          const float corr = exp2f(m - mn);
#pragma unroll
          for (int blk = 0; blk < RL / 32; ++blk)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
              float tmp;
              asm volatile("v_accvgpr_read_b32 %1, %0\n\tv_mul_f32 %1, %1, %2\n\tv_accvgpr_write_b32 %0, %1"
                           : "+a"(acc[blk][r]), "=&v"(tmp) : "v"(corr));
            }
          l *= corr;
        }
        m = mn;
      }
      // p = 2^(x - m) in bf16 (x - m <= 20; far below, v_exp_f32 flushes to 0)
      uint32_t pw[8];
#pragma unroll
      for (int r = 0; r < 16; r += 2) {
        pw[r >> 1] = pack2bf(__builtin_amdgcn_exp2f(x[r] - m), __builtin_amdgcn_exp2f(x[r + 1] - m));
        l += __uint_as_float(pw[r >> 1] << 16) + __uint_as_float(pw[r >> 1] & 0xFFFF0000u);
      }
      const uint4 P0 = uint4{pw[0], pw[1], pw[2], pw[3]}, P1 = uint4{pw[4], pw[5], pw[6], pw[7]};
#pragma unroll
      for (int k = 1; k < PR; ++k) read_blk(k, vf[k]);
#pragma unroll
      for (int blk = 0; blk < RL / 32; ++blk) {
        if (blk + PR < RL / 32) read_blk(blk + PR, vf[(blk + PR) % (PR + 1)]);
        const uint2 (&v)[4] = vf[blk % (PR + 1)];
        acc[blk] = mfma32x32x16(uint4{v[0].x, v[0].y, v[1].x, v[1].y}, P0, acc[blk]);
        acc[blk] = mfma32x32x16(uint4{v[2].x, v[2].y, v[3].x, v[3].y}, P1, acc[blk]);
        __builtin_amdgcn_sched_barrier(0);
      }
      bi = bi == NBUF - 1 ? 0 : bi + 1;
      bi2 = bi2 == NBUF - 1 ? 0 : bi2 + 1;
    }
    l += __shfl_xor(l, 32, 64);
    auto out4 = [&](int blk, int g4) {
      return make_float4(acc[blk][4 * g4], acc[blk][4 * g4 + 1], acc[blk][4 * g4 + 2], acc[blk][4 * g4 + 3]);
    };
    // write the segment: a whole row directly (bf16, normalised), a partial row
    // to slot 2w (the range's first row) or 2w+1 (its last row)
    if (head_ok) {
      if (t0 == 0 && t1 == pe - pb) {
        const float inv = 1.f / l;
        bf16_t* o = a.out + ((int64_t)b * a.nh + head) * RL;
#pragma unroll
        for (int blk = 0; blk < RL / 32; ++blk)
#pragma unroll
          for (int g4 = 0; g4 < 4; ++g4) {
            const float4 v = out4(blk, g4);
            *reinterpret_cast<uint2*>(o + blk * 32 + 8 * g4 + 4 * hs) =
                uint2{pack2bf(v.x * inv, v.y * inv), pack2bf(v.z * inv, v.w * inv)};
          }
      } else {
        // the segment's output normalised by its own sum (a convex combination
        // of cached latents, so a few units in magnitude) in fp16, with its
        // (max, sum) in fp32: half the bytes of fp32 partials, and fp16's 11
        // significant bits add about a quarter of the final bf16 rounding
        const int slot = 2 * w + (cur == start ? 0 : 1);
        const float inv = 1.f / l;
        uint16_t* po = a.part_o + ((int64_t)slot * a.nh + head) * RL;
#pragma unroll
        for (int blk = 0; blk < RL / 32; ++blk)
#pragma unroll
          for (int g4 = 0; g4 < 4; ++g4) {
            const float4 v = out4(blk, g4);
            *reinterpret_cast<uint2*>(po + blk * 32 + 8 * g4 + 4 * hs) =
                uint2{pack2h(v.x * inv, v.y * inv), pack2h(v.z * inv, v.w * inv)};
          }
        if (hs == 0) {
          a.part_ml[((int64_t)slot * a.nh + head) * 2] = m;
          a.part_ml[((int64_t)slot * a.nh + head) * 2 + 1] = l;
        }
      }
    }
    cur = pb + t1;
    ++b;
    block_barrier();                     // every wave is done with the ring before the next row
  }
}

// Rows split over several workgroups: with o_s the segment's output normalised
// by its sum l_s, o = sum_s o_s l_s 2^{m_s - M} / sum_s l_s 2^{m_s - M}.
// One block per (head, row); the segments' (m, l) are fetched in parallel into
// LDS first, then each thread streams its 4 dimensions of every segment.
constexpr int MAX_ATTN_BLOCKS = 256;
__global__ __launch_bounds__(128) void mla_attn_combine_kernel(MlaAttnArgs a) {
  __shared__ float seg_w[MAX_ATTN_BLOCKS], seg_l[MAX_ATTN_BLOCKS];
  __shared__ int seg_slot[MAX_ATTN_BLOCKS];
  const int h = blockIdx.x, b = blockIdx.y, nb = a.nblocks, tid = threadIdx.x;
  const int pb = a.sched[b];
  const int w_lo = sched_wlo(a.sched, a.B, nb, b);                 // workgroup holding tile pb
  const int w_hi = sched_whi(a.sched, a.B, nb, b);                 // workgroup holding tile pe-1
  if (w_lo == w_hi) return;                                        // written directly
  const int nseg = w_hi - w_lo + 1;
  for (int i = tid; i < nseg; i += 128) {
    const int w = w_lo + i;
    const int s0 = sched_start(a.sched, a.B, nb, w), s1 = sched_start(a.sched, a.B, nb, w + 1);
    const int slot = 2 * w + (s0 >= pb ? 0 : 1);
    const bool empty = s0 >= s1;
    const int64_t idx = (int64_t)slot * a.nh + h;
    seg_slot[i] = slot;
    seg_w[i] = empty ? -INFINITY : a.part_ml[idx * 2];
    seg_l[i] = empty ? 0.f : a.part_ml[idx * 2 + 1];
  }
  __syncthreads();
  float M = -INFINITY;
  for (int i = 0; i < nseg; ++i) M = fmaxf(M, seg_w[i]);
  __syncthreads();
  for (int i = tid; i < nseg; i += 128) seg_w[i] = exp2f(seg_w[i] - M);   // 0 for empty ranges
  __syncthreads();
  // every thread weighs 4 dimensions of each segment
  const int d = tid * 4;
  float4 o = make_float4(0.f, 0.f, 0.f, 0.f);
  float L = 0.f;
  // eight segments' loads in flight at a time; a slot is always inside the
  // partial buffer, and one that holds no data (an empty range, weight 0) is
  // loaded but not added
  constexpr int SEG_GROUP = 8;
  for (int i0 = 0; i0 < nseg; i0 += SEG_GROUP) {
    uint2 v[SEG_GROUP];
#pragma unroll
    for (int u = 0; u < SEG_GROUP; ++u)
      v[u] = i0 + u < nseg
                 ? *reinterpret_cast<const uint2*>(a.part_o + ((int64_t)seg_slot[i0 + u] * a.nh + h) * RL + d)
                 : uint2{0u, 0u};
#pragma unroll
    for (int u = 0; u < SEG_GROUP; ++u) {
      if (i0 + u >= nseg) break;
      const float wt = seg_w[i0 + u], wl = seg_l[i0 + u] * wt;
      L += wl;
      if (wt != 0.f) {
        const float4 x = unpack4h(v[u]);
        o.x += x.x * wl; o.y += x.y * wl; o.z += x.z * wl; o.w += x.w * wl;
      }
    }
  }
  const float inv = 1.f / L;
  *reinterpret_cast<uint2*>(a.out + ((int64_t)b * a.nh + h) * RL + d) =
      uint2{pack2bf(o.x * inv, o.y * inv), pack2bf(o.z * inv, o.w * inv)};
}

// ------------------------------------------------------------ combine + W_UV
// Up to 64 rows: the merge above and the W_UV product of the merged latent in
// one launch, one block of 8 waves per (head, 8-row group); wave w owns row
// w of the group and, for the product, latent-output n-tile w.
//  1. every thread's 8 dimensions of its row's first CV_SEG segments are
//     requested at once; meanwhile the wave forms the row's segment weights
//     in LDS (the max over the segments is a wave reduction) and the head's
//     W_UV tiles of its n-tile are in flight;
//  2. each thread merges its 8 dimensions over the segments in order (a row
//     written whole by the attention is read as written), rounds them to bf16
//     and stores them in LDS as MFMA A fragments: lane l of k-tile kt holds
//     row l % 16, dimensions 32 kt + 8 (l / 16) .. +7 (rows 8..15 are zero);
//  3. wave w accumulates the 16 k-tiles in order against its W_UV tiles and
//     writes its 16 output columns as bf16.
// The roundings and orders are those of the combine kernel followed by the
// weight-streaming GEMM over the heads.
constexpr int CV_ROWS = 8;
constexpr int CV_SEG = 24;               // segments whose loads are in flight together
constexpr int CV_KT = RL / 32;           // k-tiles of the latent

__device__ __forceinline__ void unpack8h(const uint4& u, float* x) {
  const float4 a = unpack4h(uint2{u.x, u.y}), b = unpack4h(uint2{u.z, u.w});
  x[0] = a.x; x[1] = a.y; x[2] = a.z; x[3] = a.w; x[4] = b.x; x[5] = b.y; x[6] = b.z; x[7] = b.w;
}

__global__ __launch_bounds__(512) void mla_attn_combine_uv_kernel(MlaAttnArgs a, const uint4* __restrict__ wuv,
                                                                   int64_t w_bs, bf16_t* __restrict__ attn_out) {
  __shared__ float seg_w[CV_ROWS][MAX_ATTN_BLOCKS], seg_l[CV_ROWS][MAX_ATTN_BLOCKS];
  __shared__ uint4 afr[CV_KT][64];
  const int h = blockIdx.x, nb = a.nblocks, tid = threadIdx.x, lane = tid & 63;
  const int wid = __builtin_amdgcn_readfirstlane(tid >> 6);
  const uint4* __restrict__ W = wuv + (int64_t)h * w_bs;
  uint4 wt[CV_KT];
#pragma unroll
  // plain loads: the head's other row group reads the same tiles, on the same XCD
  for (int kt = 0; kt < CV_KT; ++kt) wt[kt] = W[((int64_t)wid * CV_KT + kt) * 64 + lane];

  const int b = blockIdx.y * CV_ROWS + wid;
  const bool row_ok = b < a.B;
  int pb = 0, w_lo = 0, w_hi = 0;
  if (row_ok) {
    pb = a.sched[b];
    w_lo = sched_wlo(a.sched, a.B, nb, b);                  // workgroup holding tile pb
    w_hi = sched_whi(a.sched, a.B, nb, b);                  // workgroup holding tile pe-1
  }
  const bool merged = row_ok && w_lo != w_hi;
  const int nseg = merged ? w_hi - w_lo + 1 : 0;
  // segment i: workgroup w_lo + i; its slot is 2w when the range starts at or
  // after the row's first tile (the row is the range's first), else 2w + 1
  // (the row is the range's last); only the first range can start before the row
  const int slot0 = 2 * w_lo + (sched_start(a.sched, a.B, nb, w_lo) >= pb ? 0 : 1);
  auto slot_of = [&](int i) { return i == 0 ? slot0 : 2 * (w_lo + i); };
  const int d = 8 * lane;
  // a slot is always inside the partial buffer; one that holds no data (an
  // empty range, weight 0) is loaded but not added
  auto part_at = [&](int i) {
    return *reinterpret_cast<const uint4*>(a.part_o + ((int64_t)slot_of(i) * a.nh + h) * RL + d);
  };
  uint4 v[CV_SEG];
#pragma unroll
  for (int u = 0; u < CV_SEG; ++u) v[u] = u < nseg ? part_at(u) : uint4{0u, 0u, 0u, 0u};
  const uint4 whole = (row_ok && !merged)
                          ? *reinterpret_cast<const uint4*>(a.out + ((int64_t)b * a.nh + h) * RL + d)
                          : uint4{0u, 0u, 0u, 0u};
  float M = -INFINITY;
  for (int i = lane; i < nseg; i += 64) {
    const int w = w_lo + i;
    const int s0 = sched_start(a.sched, a.B, nb, w), s1 = sched_start(a.sched, a.B, nb, w + 1);
    const int64_t idx = (int64_t)slot_of(i) * a.nh + h;
    const bool empty = s0 >= s1;
    const float m = empty ? -INFINITY : a.part_ml[idx * 2];
    seg_w[wid][i] = m;
    seg_l[wid][i] = empty ? 0.f : a.part_ml[idx * 2 + 1];
    M = fmaxf(M, m);
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) M = fmaxf(M, __shfl_xor(M, o, 64));
  for (int i = lane; i < nseg; i += 64) seg_w[wid][i] = exp2f(seg_w[wid][i] - M);   // 0 for empty ranges
  // rows 8..15 of every A fragment are zero
  afr[lane >> 2][CV_ROWS + wid + 16 * (lane & 3)] = uint4{0u, 0u, 0u, 0u};
  __syncthreads();                       // the row's weights are visible to the whole wave

  uint4 piece = whole;
  if (merged) {
    float o[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    float L = 0.f;
    for (int i0 = 0; i0 < nseg; i0 += CV_SEG) {
      if (i0 > 0) {
#pragma unroll
        for (int u = 0; u < CV_SEG; ++u) v[u] = i0 + u < nseg ? part_at(i0 + u) : uint4{0u, 0u, 0u, 0u};
      }
#pragma unroll
      for (int u = 0; u < CV_SEG; ++u) {
        if (i0 + u >= nseg) break;
        const float wt_s = seg_w[wid][i0 + u], wl = seg_l[wid][i0 + u] * wt_s;
        L += wl;
        if (wt_s != 0.f) {
          float x[8];
          unpack8h(v[u], x);
#pragma unroll
          for (int e = 0; e < 8; ++e) o[e] += x[e] * wl;
        }
      }
    }
    const float inv = 1.f / L;
    piece = uint4{pack2bf(o[0] * inv, o[1] * inv), pack2bf(o[2] * inv, o[3] * inv),
                  pack2bf(o[4] * inv, o[5] * inv), pack2bf(o[6] * inv, o[7] * inv)};
  }
  afr[lane >> 2][wid + 16 * (lane & 3)] = piece;
  __syncthreads();                       // A fragments complete

  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int kt = 0; kt < CV_KT; ++kt) acc = mfma16x16x32(afr[kt][lane], wt[kt], acc);
  // D lane layout: column l % 16 of the n-tile, rows 4 (l / 16) .. +3
  const int64_t ldo = (int64_t)a.nh * 128;
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int m = 4 * (lane >> 4) + r, row = blockIdx.y * CV_ROWS + m;
    if (m < CV_ROWS && row < a.B)
      attn_out[(int64_t)row * ldo + (int64_t)h * 128 + wid * 16 + (lane & 15)] = f2bf(acc[r]);
  }
}

namespace {
int mla_attn_waves(int nh) { return nh >= 4 * HPW ? 4 : nh > 2 * HPW ? 3 : nh > HPW ? 2 : 1; }
int mla_attn_head_groups(int nh) { return (nh + mla_attn_waves(nh) * HPW - 1) / (mla_attn_waves(nh) * HPW); }
}  // namespace

hipError_t launch_mla_attn_schedule(const int32_t* ctx_len, const int32_t* tok_pos, int step0, int nsteps,
                                    int B, int nblocks, int32_t* sched, int stride, hipStream_t st) {
  if (nsteps < 1 || B < 1 || nblocks < 1 || stride < 3 * B + 2 * nblocks + 2) return hipErrorInvalidValue;
  hipLaunchKernelGGL(mla_attn_schedule_kernel, dim3(nsteps), dim3(SCHED_THREADS), 0, st, ctx_len, tok_pos, step0,
                     B, nblocks, sched, stride);
  return hipGetLastError();
}

hipError_t launch_mla_attn(const MlaAttnArgs& a, hipStream_t st, const uint4* wuv, int64_t w_bs,
                           bf16_t* attn_out) {
  if (a.r != RL || a.dr != 64 || a.nh % 16 != 0 || a.page_size % TK != 0 || a.nblocks < 1 ||
      a.nblocks > MAX_ATTN_BLOCKS || a.B < 1)
    return hipErrorInvalidValue;
  // fused merge + W_UV: the packed tiles of a 128 x 512 W_UV per head
  if (wuv && w_bs != (int64_t)(128 / 16) * CV_KT * 64) return hipErrorInvalidValue;
  const dim3 grid(a.nblocks, mla_attn_head_groups(a.nh));
  switch (mla_attn_waves(a.nh)) {
    case 4: hipLaunchKernelGGL(mla_attn_kernel<4>, grid, dim3(256), 0, st, a); break;
    case 3: hipLaunchKernelGGL(mla_attn_kernel<3>, grid, dim3(192), 0, st, a); break;
    case 2: hipLaunchKernelGGL(mla_attn_kernel<2>, grid, dim3(128), 0, st, a); break;
    default: hipLaunchKernelGGL(mla_attn_kernel<1>, grid, dim3(64), 0, st, a); break;
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (wuv)
    hipLaunchKernelGGL(mla_attn_combine_uv_kernel, dim3(a.nh, (a.B + CV_ROWS - 1) / CV_ROWS), dim3(512), 0, st, a,
                       wuv, w_bs, attn_out);
  else
    hipLaunchKernelGGL(mla_attn_combine_kernel, dim3(a.nh, a.B), dim3(128), 0, st, a);
  return hipGetLastError();
}

}  // namespace e3
