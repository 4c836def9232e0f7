// dropout.hip -- the LoRA branch's dropout mask (gfx950).
//
// [QP] "第 04 篇：QLoRA 原理" §6.3: in training mode the LoRA branch takes
// D(x) instead of x, D an (inverted) dropout on the branch's input; the base
// branch takes x; inference turns it off.  The 1 / (1 - p) of D is folded
// into the LoRA scale by the caller, so here a dropped element becomes 0 and
// a kept one passes unchanged (exact in BF16).
//
// The mask comes from a counter-based generator, so the backward regenerates
// the forward's mask from (seed, offset) with no state in between:
// Philox4x32-10 (Salmon, Moraes, Dror, Shaw, "Parallel random numbers: as
// easy as 1, 2, 3", SC'11).  Element (m, k) of a row-major [M, d] input takes
// output word m % 4 of the generator at counter (k, m / 4, offset_lo,
// offset_hi) under key (seed_lo, seed_hi) and is kept when that word is at
// least thr = floor(p * 2^32).
//
// One thread owns two neighbouring columns and 16 rows: four generator calls
// per column give the 16 decisions, half of a keep word per column (bit
// m % 32 of word [k][m / 32], the layout the input-gradient GEMM reads), and
// the thread's 16 row pairs of X are copied with the dropped elements
// cleared.  A wavefront spans 64 column pairs, so every X access is a
// 256-byte row segment.
#include "qlora_device.h"
#include "qlora_kernels.h"

namespace qlora {

// One Philox round: (hi(M1 c2) ^ c1 ^ k0, lo(M1 c2), hi(M0 c0) ^ c3 ^ k1,
// lo(M0 c0)), M0 = 0xD2511F53, M1 = 0xCD9E8D57.  Each product is one 32 x 32
// -> 64-bit multiply (v_mad_u64_u32), not separate high and low multiplies.
__device__ __forceinline__ void philox_round(uint32_t& c0, uint32_t& c1, uint32_t& c2, uint32_t& c3,
                                             uint32_t k0, uint32_t k1) {
  const uint64_t p0 = (uint64_t)0xD2511F53u * c0;
  const uint64_t p1 = (uint64_t)0xCD9E8D57u * c2;
  const uint32_t n0 = (uint32_t)(p1 >> 32) ^ c1 ^ k0, n2 = (uint32_t)(p0 >> 32) ^ c3 ^ k1;
  c0 = n0;
  c1 = (uint32_t)p1;
  c2 = n2;
  c3 = (uint32_t)p0;
}

// Ten rounds, the key growing by (0x9E3779B9, 0xBB67AE85) between rounds.
__device__ __forceinline__ void philox4x32_10(uint32_t& c0, uint32_t& c1, uint32_t& c2,
                                              uint32_t& c3, uint32_t k0, uint32_t k1) {
#pragma unroll
  for (int i = 0; i < 10; ++i) {
    if (i > 0) {
      k0 += 0x9E3779B9u;
      k1 += 0xBB67AE85u;
    }
    philox_round(c0, c1, c2, c3, k0, k1);
  }
}

// Keep bits of column k for rows 32 w + 16 hh .. +16 (bit j = row 32 w +
// 16 hh + j): four generator calls.
__device__ __forceinline__ uint32_t keep_half(uint32_t k, uint32_t w, uint32_t hh,
                                              const DropoutArgs& a) {
  uint32_t bits = 0;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    uint32_t c0 = k, c1 = 8 * w + 4 * hh + j, c2 = a.off_lo, c3 = a.off_hi;
    philox4x32_10(c0, c1, c2, c3, a.key_lo, a.key_hi);
    bits |= (c0 >= a.thr ? 1u : 0u) << (4 * j);
    bits |= (c1 >= a.thr ? 1u : 0u) << (4 * j + 1);
    bits |= (c2 >= a.thr ? 1u : 0u) << (4 * j + 2);
    bits |= (c3 >= a.thr ? 1u : 0u) << (4 * j + 3);
  }
  return bits;
}

// One thread per (column pair, 16 rows): two threads fill one keep word,
// each its 16-bit half.
__global__ __launch_bounds__(256) void k_dropout(DropoutArgs a) {
  const int64_t pairs = a.d / 2;
  const int64_t tid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (tid >= pairs * 2 * a.ldw) return;
  const int64_t wh = tid / pairs;                       // 16-row unit: word w, half hh
  const uint32_t w = (uint32_t)(wh >> 1), hh = (uint32_t)(wh & 1);
  const uint32_t k = (uint32_t)(2 * (tid - wh * pairs));
  const int64_t m0 = 32 * (int64_t)w + 16 * hh;
  const int rows = a.M - m0 < 16 ? (a.M - m0 > 0 ? (int)(a.M - m0) : 0) : 16;
  // row pairs of X first, so the loads are in flight during the generator
  uint32_t x[16];
  if (a.Xm) {
#pragma unroll
    for (int j = 0; j < 16; ++j)
      x[j] = j < rows ? *reinterpret_cast<const uint32_t*>(a.X + (m0 + j) * a.d + k) : 0u;
  }
  // rows past M get keep bit 0
  const uint32_t live = (1u << rows) - 1u;
  const uint32_t b0 = keep_half(k, w, hh, a) & live;
  const uint32_t b1 = keep_half(k + 1, w, hh, a) & live;
  if (a.keep) {
    uint16_t* kh = reinterpret_cast<uint16_t*>(a.keep);
    kh[2 * ((int64_t)k * a.ldw + w) + hh] = (uint16_t)b0;
    kh[2 * ((int64_t)(k + 1) * a.ldw + w) + hh] = (uint16_t)b1;
  }
  if (a.Xm) {
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      if (j >= rows) break;
      const uint32_t lo = ((b0 >> j) & 1u) ? 0x0000FFFFu : 0u;
      const uint32_t hi = ((b1 >> j) & 1u) ? 0xFFFF0000u : 0u;
      *reinterpret_cast<uint32_t*>(a.Xm + (m0 + j) * a.d + k) = x[j] & (lo | hi);
    }
  }
}

// Keep bits only, for tiles of 32 rows x 32 columns: thread (quad q = t / 32,
// column c = t % 32) makes the one generator call of rows 4 q .. 4 q + 3 at
// column c.  A wavefront holds two quads x 32 columns, so a ballot of one row
// of a quad is that row's 32-column word; the column words (32 rows) are put
// together from the eight quads' nibbles in LDS.
__global__ __launch_bounds__(256) void k_dropout_bits(DropoutArgs a, uint32_t* __restrict__ rbits) {
  __shared__ uint8_t nib[8][32];
  const int64_t col_tiles = a.d / 32;
  const int64_t tile = blockIdx.x;
  const int64_t r0 = (tile / col_tiles) * 32, k0 = (tile % col_tiles) * 32;
  const int t = threadIdx.x, q = t >> 5, c = t & 31;
  uint32_t c0 = (uint32_t)(k0 + c), c1 = (uint32_t)(r0 / 4 + q), c2 = a.off_lo, c3 = a.off_hi;
  philox4x32_10(c0, c1, c2, c3, a.key_lo, a.key_hi);
  const int64_t m = r0 + 4 * q;
  const uint32_t live = a.M - m >= 4 ? 15u : (a.M > m ? (1u << (a.M - m)) - 1u : 0u);
  const uint32_t bits = ((c0 >= a.thr ? 1u : 0u) | (c1 >= a.thr ? 2u : 0u) |
                         (c2 >= a.thr ? 4u : 0u) | (c3 >= a.thr ? 8u : 0u)) & live;
  if (rbits) {
    const int64_t ldr = a.d / 32;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const uint64_t b = __ballot((bits >> r) & 1u);
      // lanes 0..31: quad 2 (t / 64); lanes 32..63: quad 2 (t / 64) + 1
      if ((t & 31) == 0) {
        const int64_t row = m + r;
        const uint32_t word = (t & 32) ? (uint32_t)(b >> 32) : (uint32_t)b;
        if (row < a.M) rbits[row * ldr + k0 / 32] = word;
      }
    }
  }
  if (a.keep) {
    nib[q][c] = (uint8_t)bits;
    __syncthreads();
    if (t < 32) {
      uint32_t word = 0;
#pragma unroll
      for (int qq = 0; qq < 8; ++qq) word |= (uint32_t)nib[qq][t] << (4 * qq);
      a.keep[(k0 + t) * a.ldw + r0 / 32] = word;
    }
  }
}

hipError_t launch_dropout_bits(const DropoutArgs& a, uint32_t* rbits, hipStream_t st) {
  const int64_t tiles = ((a.M + 31) / 32) * (a.d / 32);
  if (tiles == 0) return hipSuccess;
  hipLaunchKernelGGL(k_dropout_bits, dim3((unsigned)tiles), dim3(256), 0, st, a, rbits);
  return hipGetLastError();
}

hipError_t launch_dropout(const DropoutArgs& a, hipStream_t st) {
  const int64_t threads = (a.d / 2) * 2 * a.ldw;
  if (threads == 0) return hipSuccess;
  hipLaunchKernelGGL(k_dropout, dim3((unsigned)((threads + 255) / 256)), dim3(256), 0, st, a);
  return hipGetLastError();
}

}  // namespace qlora
