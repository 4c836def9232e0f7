// lora.hip -- the rank-r side of the LoRA linear layer (gfx950).
//
// [QP] "第 04 篇：QLoRA 原理" §2.2 (LoRA branch), §2.4 (gradients of A, B and
// the input), §6.3-6.4.  With s = alpha / r and token rows:
//   T = s X A^T,  U = s dY B,  dA = U^T X,  dB = dY^T T.
// Thin products run on the matrix cores with FP32 accumulation.  Reductions
// over K or over tokens are split across workgroups into FP32 partials that a
// finish kernel sums in split order, so every result is deterministic.  These
// kernels are bound by one pass over X (or dY); the rank-r operands are small
// and come from L2.
#include "qlora_device.h"
#include "qlora_kernels.h"

namespace qlora {

// ---------------------------------------------------------------------------
// Large M, one pass: v[m][n] = scale * sum_k P[m][k] Q[n][k], n < N <= 256.
// A workgroup owns 16 token rows and the whole K: its W wavefronts take
// consecutive K ranges (v_mfma_f32_16x16x32_bf16, 16 x 16*NB accumulators
// each) and the partial sums are added in wavefront order through LDS, so
// the result is deterministic and no partials reach HBM.  P is read once;
// Q (r x K, small) is shared through L2.  Loads go through buffer
// descriptors: rows of P past M and rows of Q past N read as zero.
// ---------------------------------------------------------------------------
// Buffer descriptor of a workgroup-uniform range, read through scalar
// registers so that every load using it is a single instruction.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t rank_rsrc(const void* base, int64_t bytes) {
  const int32_t n = bytes > 0x7FFFFFFF ? 0x7FFFFFFF : (bytes < 0 ? 0 : (int32_t)bytes);
  const uint64_t b = reinterpret_cast<uint64_t>(base);
  const uint64_t bu = ((uint64_t)(uint32_t)__builtin_amdgcn_readfirstlane((int)(b >> 32)) << 32) |
                      (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)b);
  return __builtin_amdgcn_make_buffer_rsrc(reinterpret_cast<void*>(bu), 0,
                                           __builtin_amdgcn_readfirstlane(n), 0x00020000);
}

// Eight BF16 values (natural order, two per dword) with the ones whose bit
// in b8 is 0 cleared (bit e for element e).
__device__ __forceinline__ u32x4 keep8_bf16(u32x4 v, uint32_t b8) {
  u32x4 m;
  m.x = ((b8 & 0x01u) ? 0x0000FFFFu : 0u) | ((b8 & 0x02u) ? 0xFFFF0000u : 0u);
  m.y = ((b8 & 0x04u) ? 0x0000FFFFu : 0u) | ((b8 & 0x08u) ? 0xFFFF0000u : 0u);
  m.z = ((b8 & 0x10u) ? 0x0000FFFFu : 0u) | ((b8 & 0x20u) ? 0xFFFF0000u : 0u);
  m.w = ((b8 & 0x40u) ? 0x0000FFFFu : 0u) | ((b8 & 0x80u) ? 0xFFFF0000u : 0u);
  return v & m;
}

// Row groups of 16 tokens per workgroup (RG) and wavefronts (W): every
// wavefront of a workgroup reads all of Q over its K range, so Q's L2
// traffic is (M / 16 RG) times its size; RG trades that against the number
// of workgroups.  Each wavefront keeps kRankDepth pairs of K slices (RG + NB
// 16-byte loads per slice) in flight.
#ifndef QLORA_RANK_RG4
#define QLORA_RANK_RG4 1
#endif
template <int NB>
constexpr int rank_rows_rg() { return NB == 4 ? QLORA_RANK_RG4 : 1; }
template <int NB>
constexpr int rank_rows_waves() { return NB <= 2 ? 16 : (NB == 4 ? 8 : (NB == 8 ? 4 : 2)); }
template <int NB, int RG>
constexpr int rank_depth() { return (RG + NB) * 2 * 4 * 3 + RG * NB * 4 <= 200 ? 3 : 2; }

// Two K slices (32 each, from k0) of the RG P rows and the NB Q rows of a
// lane.  The descriptors are passed by value so that they stay in scalar
// registers.
template <int NB, int RG>
__device__ __forceinline__ void rank_load_pair(__amdgpu_buffer_rsrc_t rp, __amdgpu_buffer_rsrc_t rq,
                                               const uint32_t (&vp)[RG], const uint32_t (&vq)[NB],
                                               int64_t k0, u32x4 (&x)[2][RG], u32x4 (&q)[2][NB]) {
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const uint32_t so = (uint32_t)((k0 + 32 * j) * 2);
#pragma unroll
    for (int rg = 0; rg < RG; ++rg)
      x[j][rg] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rp, vp[rg], so, 0));
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
      q[j][nb] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rq, vq[nb], so, 0));
  }
}

template <int NB, int RG>
__device__ __forceinline__ void rank_mma_pair(const u32x4 (&x)[2][RG], const u32x4 (&q)[2][NB],
                                              f32x4 (&acc)[RG][NB]) {
#pragma unroll
  for (int j = 0; j < 2; ++j)
#pragma unroll
    for (int rg = 0; rg < RG; ++rg)
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) acc[rg][nb] = mfma16(x[j][rg], q[j][nb], acc[rg][nb]);
}

template <int NB>
__global__ __launch_bounds__(64 * rank_rows_waves<NB>()) void k_rank_rows(RankRowsArgs a) {
  constexpr int W = rank_rows_waves<NB>();
  constexpr int RG = rank_rows_rg<NB>();
  constexpr int ROWS = 16 * RG;
  constexpr int NC = 16 * NB;                       // columns covered
  __shared__ float red[ROWS][NC];                   // wavefront partials, added in order
  // wavefront index read as a scalar, so that K offsets stay in scalar registers
  const int lane = threadIdx.x & 63, w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int r16 = lane & 15, g = lane >> 4;
  const int64_t m0 = (int64_t)blockIdx.x * ROWS;
  const int64_t K = a.K;
  const int64_t chunk = ((K + W - 1) / W + 31) / 32 * 32;
  const int64_t k_begin = (int64_t)w * chunk;
  const int64_t k_end = k_begin + chunk < K ? k_begin + chunk : K;

  const __amdgpu_buffer_rsrc_t rp = rank_rsrc(a.P + m0 * K, (a.M - m0) * K * 2);
  const __amdgpu_buffer_rsrc_t rq = rank_rsrc(a.Q, a.N * a.ldq * 2);
  uint32_t vp[RG], vq[NB];
#pragma unroll
  for (int rg = 0; rg < RG; ++rg) vp[rg] = (uint32_t)(((16 * rg + r16) * K + 8 * g) * 2);
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) vq[nb] = (uint32_t)(((16 * nb + r16) * a.ldq + 8 * g) * 2);
  const bool vec = (K % 8) == 0 && (a.ldq % 8) == 0;

  f32x4 acc[RG][NB];
#pragma unroll
  for (int rg = 0; rg < RG; ++rg)
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) acc[rg][nb] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
  // Full slices in pairs through a ring of D pair buffers: the loads of
  // pair i + D - 1 are issued before the MFMAs of pair i.  The prologue and
  // the steady loop load unconditionally (pairs past the range read zeros or
  // unused in-bounds data), which keeps the compiler's wait counts exact;
  // the last pairs run in a guarded tail.
  constexpr int D = rank_depth<NB, RG>();
  const int64_t k_full = k_begin + (vec ? (k_end - k_begin) / 64 * 64 : 0);
  const int np = (int)((k_full - k_begin) / 64);
  {
    u32x4 x[D][2][RG], q[D][2][NB];
#pragma unroll
    for (int i = 0; i < D - 1; ++i)
      rank_load_pair<NB, RG>(rp, rq, vp, vq, k_begin + 64 * i, x[i], q[i]);
    int i = 0;
    for (; i + 2 * D - 1 <= np; i += D) {
#pragma unroll
      for (int j = 0; j < D; ++j) {
        rank_load_pair<NB, RG>(rp, rq, vp, vq, k_begin + 64 * (i + j + D - 1), x[(j + D - 1) % D],
                               q[(j + D - 1) % D]);
        rank_mma_pair<NB, RG>(x[j], q[j], acc);
      }
    }
    for (; i < np; i += D) {
#pragma unroll
      for (int j = 0; j < D; ++j) {
        if (i + j < np) {
          if (i + j + D - 1 < np)
            rank_load_pair<NB, RG>(rp, rq, vp, vq, k_begin + 64 * (i + j + D - 1),
                                   x[(j + D - 1) % D], q[(j + D - 1) % D]);
          rank_mma_pair<NB, RG>(x[j], q[j], acc);
        }
      }
    }
  }
  for (int64_t k0 = k_full; k0 < k_end; k0 += 32) {
    // K tail or unaligned rows: element loads, zero at and past k_end
    const int64_t kk = k0 + 8 * g;
    uint32_t h[8];
    u32x4 x[RG];
#pragma unroll
    for (int rg = 0; rg < RG; ++rg) {
#pragma unroll
      for (int e = 0; e < 8; ++e)
        h[e] = kk + e < k_end ? (uint32_t)__builtin_amdgcn_raw_buffer_load_b16(
                                    rp, (uint32_t)(((16 * rg + r16) * K + kk + e) * 2), 0, 0)
                              : 0u;
      x[rg] = u32x4{h[0] | (h[1] << 16), h[2] | (h[3] << 16), h[4] | (h[5] << 16),
                    h[6] | (h[7] << 16)};
    }
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
#pragma unroll
      for (int e = 0; e < 8; ++e)
        h[e] = kk + e < k_end ? (uint32_t)__builtin_amdgcn_raw_buffer_load_b16(
                                    rq, (uint32_t)(((16 * nb + r16) * a.ldq + kk + e) * 2), 0, 0)
                              : 0u;
      const u32x4 q = {h[0] | (h[1] << 16), h[2] | (h[3] << 16), h[4] | (h[5] << 16),
                       h[6] | (h[7] << 16)};
#pragma unroll
      for (int rg = 0; rg < RG; ++rg) acc[rg][nb] = mfma16(x[rg], q, acc[rg][nb]);
    }
  }
  // wavefront partials added in wavefront order; accumulator lane l holds
  // rows 4 (l/16) + v, column l%16 of its 16 x 16 block
  for (int ww = 0; ww < W; ++ww) {
    if (w == ww) {
#pragma unroll
      for (int rg = 0; rg < RG; ++rg)
#pragma unroll
        for (int nb = 0; nb < NB; ++nb)
#pragma unroll
          for (int v = 0; v < 4; ++v) {
            float* e = &red[16 * rg + 4 * g + v][16 * nb + r16];
            *e = ww == 0 ? acc[rg][nb][v] : __fadd_rn(*e, acc[rg][nb][v]);
          }
    }
    __syncthreads();
  }

  const int64_t rows = a.ht ? a.ldt : a.M;   // transposed copies are padded with zeros
  for (int idx = threadIdx.x; idx < ROWS * NC; idx += W * 64) {
    const int row = idx / NC, n = idx % NC;
    const int64_t m = m0 + row;
    if (m >= rows) continue;
    const float v = __fmul_rn(a.scale, red[row][n]);   // zero for m >= M and n >= N
    float hi, lo;
    split_bf16(v, hi, lo);
    const uint16_t hb = (uint16_t)(__float_as_uint(hi) >> 16);
    const uint16_t lb = (uint16_t)(pack_bf16x2(lo, 0.0f) & 0xFFFFu);
    if (m < a.M) {
      if (a.out && n < a.N) a.out[m * a.N + n] = v;
      if (a.hl && n < a.rp) {
        a.hl[m * 2 * a.rp + n] = hb;
        a.hl[m * 2 * a.rp + a.rp + n] = lb;
      }
    }
    if (a.ht && n < (a.N + 31) / 32 * 32) {   // NC >= round_up(N, 32); zero past N
      a.ht[frag_index(n, m, a.ldt)] = hb;
      a.lt[frag_index(n, m, a.ldt)] = lb;
    }
  }
}

typedef short v4i16_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) v4i16_t lds_v4i16_t;

// ---------------------------------------------------------------------------
// Large M, split over K: part[s][m][n] = sum over k in split s of P[m][k]
// Q[n][k] (FP32), P [M][K], Q [N][ldq], N <= 16 NB.  Workgroup = 64 rows
// (16 per wavefront) x one K split.  K advances in chunks of KC columns: the
// Q chunk is staged in LDS once per workgroup (double-buffered, loaded into
// registers one chunk ahead) and read by all four wavefronts, so Q's L2
// traffic is (M / 64) times its size; each wavefront's P rows come straight
// from memory, one chunk ahead.  Rows past M or N and columns past the
// split read as zero.  k_rank_finish adds the splits in order.  K and ldq
// are multiples of 8 and P, Q 16-byte aligned (checked by the launcher).
// QT: Q is given as stored [K][ldq] (element (n, k) at Q[k * ldq + n], as
// the rank-r factor B [d_out][r] serves U = dY B); its chunk is staged in LDS
// row k by row k and the MFMA operand (eight consecutive k of one column per
// lane) comes from two transposing LDS reads.
#ifndef QLORA_RANK_KC4
#define QLORA_RANK_KC4 128
#endif
template <int NB>
constexpr int rank_kc() { return NB <= 4 ? QLORA_RANK_KC4 : (NB <= 8 ? 64 : 32); }

template <int NB, bool MASK, bool QT>
__global__ __launch_bounds__(256) void k_rank_part(RankRowsArgs a, float* __restrict__ part,
                                                   int64_t kper, int ks) {
  constexpr int KC = rank_kc<NB>();
  constexpr int NR = 16 * NB;                 // Q rows staged (zero past N)
  // LDS row, BF16 elements: [n][k] rows of KC (16 B pad: conflict-free
  // reads), or with QT [k][n] rows of NR
  constexpr int LQ = QT ? NR + 8 : KC + 8;
  constexpr int PIECES = NR * KC / 8 / 256;   // 16-byte Q pieces per thread per chunk
  constexpr int NS = KC / 32;                 // MFMA K slices per chunk
  __shared__ __attribute__((aligned(16))) uint16_t qs[2][QT ? KC * LQ : NR * LQ];
  const int lane = threadIdx.x & 63, w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int r16 = lane & 15, g = lane >> 4;
  const int rb = blockIdx.x / ks, sp = blockIdx.x % ks;
  const int64_t m0 = (int64_t)rb * 64;
  const int64_t K = a.K;
  const int64_t k_begin = (int64_t)sp * kper;
  const int64_t k_end = k_begin + kper < K ? k_begin + kper : K;
  const int nchunks = (int)((k_end - k_begin + KC - 1) / KC);

  const __amdgpu_buffer_rsrc_t rp = rank_rsrc(a.P + m0 * K, (a.M - m0) * K * 2);   // rows past M: zero
  const __amdgpu_buffer_rsrc_t rq = rank_rsrc(a.Q, (QT ? K : a.N) * a.ldq * 2);   // rows past N: zero
  const uint32_t prow = (uint32_t)((16 * w + r16) * K);                             // element offset
  // MASK: keep words of P's rows (K / 32 per row), rows past M read as zero
  const __amdgpu_buffer_rsrc_t rm =
      rank_rsrc(MASK ? a.pmask + m0 * (K / 32) : nullptr, MASK ? (a.M - m0) * (K / 32) * 4 : 0);
  const uint32_t mrow = (uint32_t)((16 * w + r16) * (K / 32));
  // Q pieces of this thread: LDS row qrow[u], 8 elements from qcol[u]
  // (row n and chunk columns k, or with QT chunk row k and columns n)
  uint32_t qrow[PIECES], qcol[PIECES];
#pragma unroll
  for (int u = 0; u < PIECES; ++u) {
    const int piece = threadIdx.x + 256 * u;
    constexpr int per_row = (QT ? NR : KC) / 8;
    qrow[u] = (uint32_t)(piece / per_row);
    qcol[u] = (uint32_t)(8 * (piece % per_row));
  }
  const uint32_t kend = (uint32_t)k_end;

  auto load_chunk = [&](int c, u32x4 (&qv)[PIECES], u32x4 (&xv)[NS], uint32_t (&mk)[NS]) {
    const uint32_t kc0 = (uint32_t)(k_begin + (int64_t)c * KC);
#pragma unroll
    for (int u = 0; u < PIECES; ++u) {
      uint32_t off;
      if (QT) {
        // row k of Q as stored; columns past N read zero
        const uint32_t k = kc0 + qrow[u];
        off = (k < kend && qcol[u] < (uint32_t)a.N) ? (k * (uint32_t)a.ldq + qcol[u]) * 2
                                                     : 0x80000000u;
      } else {
        const uint32_t col = kc0 + qcol[u];
        off = col < kend ? (qrow[u] * (uint32_t)a.ldq + col) * 2 : 0x80000000u;
      }
      qv[u] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rq, off, 0, 0));
    }
#pragma unroll
    for (int j = 0; j < NS; ++j) {
      const uint32_t col = kc0 + 32 * j + 8 * g;
      const uint32_t off = col < kend ? (prow + col) * 2 : 0x80000000u;
      xv[j] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rp, off, 0, 0));
      if (MASK)
        mk[j] = __builtin_amdgcn_raw_buffer_load_b32(
            rm, col < kend ? (mrow + ((kc0 >> 5) + j)) * 4 : 0x80000000u, 0, 0);
    }
  };
  auto store_q = [&](int buf, const u32x4 (&qv)[PIECES]) {
#pragma unroll
    for (int u = 0; u < PIECES; ++u)
      *reinterpret_cast<u32x4*>(&qs[buf][qrow[u] * LQ + qcol[u]]) = qv[u];
  };
  f32x4 acc[NB];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) acc[nb] = f32x4{0.f, 0.f, 0.f, 0.f};
  auto compute = [&](int buf, const u32x4 (&xv)[NS], const uint32_t (&mk)[NS]) {
#pragma unroll
    for (int j = 0; j < NS; ++j) {
      const u32x4 x = MASK ? keep8_bf16(xv[j], mk[j] >> (8 * g)) : xv[j];
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) {
        u32x4 qf;
        if (QT) {
          // lane group g reads rows k = 32 j + 8 g + (r16 / 4) (then + 4),
          // columns 16 nb + 4 (r16 % 4) .. +4; lane r16 receives column
          // 16 nb + r16 of the four rows
          const uint16_t* pb = &qs[buf][(32 * j + 8 * g + (r16 >> 2)) * LQ + 16 * nb + 4 * (r16 & 3)];
          const v4i16_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16_t*)(pb));
          const v4i16_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16_t*)(pb + 4 * LQ));
          const uint2 l2 = __builtin_bit_cast(uint2, lo), h2 = __builtin_bit_cast(uint2, hi);
          qf = u32x4{l2.x, l2.y, h2.x, h2.y};
        } else {
          qf = *reinterpret_cast<const u32x4*>(&qs[buf][(16 * nb + r16) * LQ + 32 * j + 8 * g]);
        }
        acc[nb] = mfma16(x, qf, acc[nb]);
      }
    }
  };

  u32x4 q0[PIECES], x0[NS], q1[PIECES], x1[NS];
  uint32_t m0k[NS], m1k[NS];
  if (nchunks > 0) {
    load_chunk(0, q0, x0, m0k);
    store_q(0, q0);
  }
  __syncthreads();
  for (int c = 0; c < nchunks; c += 2) {
    if (c + 1 < nchunks) load_chunk(c + 1, q1, x1, m1k);
    compute(0, x0, m0k);
    if (c + 1 >= nchunks) break;
    store_q(1, q1);
    __syncthreads();
    if (c + 2 < nchunks) load_chunk(c + 2, q0, x0, m0k);
    compute(1, x1, m1k);
    if (c + 2 < nchunks) store_q(0, q0);
    __syncthreads();
  }

  // accumulator lane (r16, g): rows 4 g + v of the wavefront's 16, column 16 nb + r16
  float* out = part + (int64_t)sp * a.M * a.N;
#pragma unroll
  for (int nb = 0; nb < NB; ++nb)
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int64_t m = m0 + 16 * w + 4 * g + v;
      const int64_t n = 16 * nb + r16;
      if (m < a.M && n < a.N) out[m * a.N + n] = acc[nb][v];
    }
}

// ---------------------------------------------------------------------------
// Small M (<= 16 tokens): partial sums part[s][m][n] of P Q^T over quarters
// of K, for a group of problems.  Workgroup = one 16-column block, problem
// and quarter; its four wavefronts take consecutive parts of the quarter
// (v_mfma_f32_16x16x32_bf16, rows past M read as zero; each part's loads
// issued in groups ahead of the MFMAs) and add their sums in wavefront
// order in LDS.  The problem's workgroups also write the permuted copy of P
// and clear the counters of the following weight-streaming launch.
// ---------------------------------------------------------------------------
constexpr int kSmallGroup = 4;   // K slices per load group

template <int G>
__device__ __forceinline__ void small_load(__amdgpu_buffer_rsrc_t rp, __amdgpu_buffer_rsrc_t rq,
                                           uint32_t vp, uint32_t vq, int64_t k0, u32x4 (&x)[G],
                                           u32x4 (&q)[G]) {
#pragma unroll
  for (int j = 0; j < G; ++j) {
    const uint32_t so = (uint32_t)((k0 + 32 * j) * 2);
    x[j] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rp, vp, so, 0));
    q[j] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rq, vq, so, 0));
  }
}

__global__ __launch_bounds__(256) void k_rank_small(RankSmallArgs a) {
  constexpr int S = kRankSmallSplits;
  __shared__ float red[16][16];
  const int wg = blockIdx.x;
  const int di = group_index(a.count, wg, [&](int i) { return a.d[i].wg_begin; });
  const RankSmallDesc& d = a.d[di];
  const int local = wg - d.wg_begin;
  const int nblk = (int)((d.N + 15) / 16);
  const int cb = local % nblk, sq = local / nblk;   // column block, K quarter
  const int lane = threadIdx.x & 63, w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int r16 = lane & 15, g = lane >> 4;
  const int64_t M = a.M, K = d.K;

  if (local == 0 && d.zero)
    for (int64_t i = threadIdx.x; i < d.zero_count; i += 256) d.zero[i] = 0u;

  // K part of the wavefront: part 4 sq + w of 16, whole load groups
  const int64_t chunk = ((K + 4 * S - 1) / (4 * S) + 32 * kSmallGroup - 1) / (32 * kSmallGroup) *
                        (32 * kSmallGroup);
  const int64_t part_id = (int64_t)sq * 4 + w;
  const int64_t k_begin = part_id * chunk < K ? part_id * chunk : K;
  const int64_t k_end = k_begin + chunk < K ? k_begin + chunk : K;
  const __amdgpu_buffer_rsrc_t rp = rank_rsrc(d.P, M * K * 2);             // rows past M: zero
  const __amdgpu_buffer_rsrc_t rq = rank_rsrc(d.Q + (int64_t)16 * cb * d.ldq,
                                             (d.N - 16 * cb) * d.ldq * 2);  // rows past N: zero
  const uint32_t vp = (uint32_t)((r16 * K + 8 * g) * 2);
  const uint32_t vq = (uint32_t)((r16 * d.ldq + 8 * g) * 2);
  const bool vec = (K % 8) == 0 && (d.ldq % 8) == 0;
  f32x4 acc = {0.0f, 0.0f, 0.0f, 0.0f};
  // full load groups (two in flight; loads unconditional in the prologue and
  // the steady loop, so the compiler's wait counts stay exact), then a tail
  constexpr int G = kSmallGroup;
  const int64_t k_full = k_begin + (vec ? (k_end - k_begin) / (32 * G) * (32 * G) : 0);
  const int ng = (int)((k_full - k_begin) / (32 * G));
  {
    u32x4 xa[G], qa[G], xb[G], qb[G];
    small_load<G>(rp, rq, vp, vq, k_begin, xa, qa);
    int i = 0;
    for (; i + 2 <= ng; i += 2) {
      small_load<G>(rp, rq, vp, vq, k_begin + 32 * G * (i + 1), xb, qb);
#pragma unroll
      for (int j = 0; j < G; ++j) acc = mfma16(xa[j], qa[j], acc);
      small_load<G>(rp, rq, vp, vq, k_begin + 32 * G * (i + 2), xa, qa);
#pragma unroll
      for (int j = 0; j < G; ++j) acc = mfma16(xb[j], qb[j], acc);
    }
    if (i < ng) {
#pragma unroll
      for (int j = 0; j < G; ++j) acc = mfma16(xa[j], qa[j], acc);
    }
  }
  for (int64_t k0 = k_full; k0 < k_end; k0 += 32) {
    const int64_t kk = k0 + 8 * g;
    uint32_t hx[8], hq[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const bool in = kk + e < k_end;
      hx[e] = in ? (uint32_t)__builtin_amdgcn_raw_buffer_load_b16(rp, (uint32_t)((r16 * K + kk + e) * 2), 0, 0) : 0u;
      hq[e] = in ? (uint32_t)__builtin_amdgcn_raw_buffer_load_b16(rq, (uint32_t)((r16 * d.ldq + kk + e) * 2), 0, 0) : 0u;
    }
    const u32x4 x = {hx[0] | (hx[1] << 16), hx[2] | (hx[3] << 16), hx[4] | (hx[5] << 16), hx[6] | (hx[7] << 16)};
    const u32x4 q = {hq[0] | (hq[1] << 16), hq[2] | (hq[3] << 16), hq[4] | (hq[5] << 16), hq[6] | (hq[7] << 16)};
    acc = mfma16(x, q, acc);
  }
  // wavefront sums added in order; accumulator lane l holds rows 4 (l/16) + v,
  // column l%16
  for (int ww = 0; ww < 4; ++ww) {
    if (w == ww) {
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        float* e = &red[4 * g + v][r16];
        *e = ww == 0 ? acc[v] : __fadd_rn(*e, acc[v]);
      }
    }
    __syncthreads();
  }
  {
    const int row = threadIdx.x >> 4, c = threadIdx.x & 15;
    const int64_t n = 16 * cb + c;
    if (row < M && n < d.N) d.part[((int64_t)sq * M + row) * d.N + n] = red[row][c];
  }
}

hipError_t launch_rank_small(const RankSmallArgs& a0, hipStream_t st) {
  RankSmallArgs a = a0;
  int wgs = 0;
  for (int i = 0; i < a.count; ++i) {
    a.d[i].wg_begin = wgs;
    wgs += (int)((a.d[i].N + 15) / 16) * kRankSmallSplits;
  }
  if (wgs == 0) return hipSuccess;
  hipLaunchKernelGGL(k_rank_small, dim3(wgs), dim3(256), 0, st, a);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Finish: v = scale * sum_s part[s] (s ascending).  Thread per element of the
// transposed [N][ldt] index space (the FP32 [M][N] output is written from
// the same thread when requested).
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void k_rank_finish(FinishArgs a) {
  const int wg = blockIdx.x;
  const int di = group_index(a.count, wg, [&](int i) { return a.d[i].wg_begin; });
  const FinishDesc& d = a.d[di];
  const int64_t idx = (int64_t)(wg - d.wg_begin) * 256 + threadIdx.x;
  const int64_t ldt = d.ldt > 0 ? d.ldt : d.M;
  // the transposed copies cover rows up to round_up(N, 32) (zeros past N)
  const int64_t nt = d.ht ? (d.N + 31) / 32 * 32 : d.N;
  if (idx >= nt * ldt) return;
  const int64_t n = idx / ldt, m = idx % ldt;
  float v = 0.0f;
  if (m < d.M && n < d.N) {
    const int64_t e = m * d.N + n, count = d.M * d.N;
    float acc = d.part[e];
    for (int s = 1; s < d.splits; ++s) acc = __fadd_rn(acc, d.part[(int64_t)s * count + e]);
    v = __fmul_rn(d.scale, acc);
    if (d.out) d.out[e] = v;
  }
  float hi, lo;
  split_bf16(v, hi, lo);
  const uint16_t hb = (uint16_t)(__float_as_uint(hi) >> 16);
  const uint16_t lb = (uint16_t)(pack_bf16x2(lo, 0.0f) & 0xFFFFu);
  if (d.ht) {
    d.ht[frag_index(n, m, ldt)] = hb;
    d.lt[frag_index(n, m, ldt)] = lb;
  }
  if (d.hl && m < d.M && n < d.N) {
    uint16_t* row = d.hl + m * 2 * d.rp;
    row[n] = hb;
    row[d.rp + n] = lb;
    if (n == d.N - 1) {
      for (int64_t j = d.N; j < d.rp; ++j) {
        row[j] = 0;
        row[d.rp + j] = 0;
      }
    }
  }
}

// Finish for many rows: one workgroup per 16 rows x 64 columns.  Same
// arithmetic and outputs as k_rank_finish (v = scale * sum of the splits in
// ascending order; out, hl with zeros for n in [N, rp), ht / lt with zeros
// for m in [M, ldt)), laid out for coalescing: partials and the row-major
// outputs are read and written along n, and the transposed copies go
// through an LDS tile so that they are written along m.  Each thread keeps
// four elements' partial loads in flight per split.
__global__ __launch_bounds__(256) void k_rank_finish_rows(FinishArgs fa) {
  constexpr int EU = 4;
  __shared__ uint16_t th[64][18], tl[64][18];   // [n][m], padded
  const FinishDesc& d = fa.d[blockIdx.z];
  const int64_t m0 = (int64_t)blockIdx.x * 16, nc = (int64_t)blockIdx.y * 64;
  {
    // this problem's tiles (the grid covers the largest problem of the list)
    const int64_t rows = d.ht && d.ldt > d.M ? d.ldt : d.M;
    const int64_t ncols = d.hl && d.rp > d.N ? d.rp : d.N;
    if (m0 >= rows || nc >= (ncols + 63) / 64 * 64) return;
  }
  const int t = threadIdx.x, col = t & 63, rq = t >> 6;
  const int64_t count = d.M * d.N;
  const int64_t ldt = d.ldt > 0 ? d.ldt : d.M;
  const int64_t n = nc + col;
  float acc[EU];
  int64_t e[EU];
  bool ok[EU];
#pragma unroll
  for (int u = 0; u < EU; ++u) {
    const int64_t m = m0 + rq + 4 * u;
    ok[u] = m < d.M && n < d.N;
    e[u] = m * d.N + n;
    acc[u] = 0.0f;
  }
  for (int s0 = 0; s0 < d.splits; s0 += 4) {
    float v[4][EU];
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int u = 0; u < EU; ++u)
        v[j][u] = (ok[u] && s0 + j < d.splits) ? d.part[(int64_t)(s0 + j) * count + e[u]] : 0.0f;
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int u = 0; u < EU; ++u)
        if (s0 + j < d.splits) acc[u] = (s0 + j == 0) ? v[j][u] : __fadd_rn(acc[u], v[j][u]);
  }
#pragma unroll
  for (int u = 0; u < EU; ++u) {
    const int r = rq + 4 * u;
    const int64_t m = m0 + r;
    const float val = ok[u] ? __fmul_rn(d.scale, acc[u]) : 0.0f;
    float hi, lo;
    split_bf16(val, hi, lo);
    const uint16_t hb = (uint16_t)(__float_as_uint(hi) >> 16);
    const uint16_t lb = (uint16_t)(pack_bf16x2(lo, 0.0f) & 0xFFFFu);
    if (ok[u] && d.out) d.out[e[u]] = val;
    if (d.hl && m < d.M && n < d.rp) {
      d.hl[m * 2 * d.rp + n] = hb;
      d.hl[m * 2 * d.rp + d.rp + n] = lb;
    }
    th[col][r] = hb;
    tl[col][r] = lb;
  }
  if (!d.ht) return;
  __syncthreads();
  // fragment order: the tile's 16 tokens are one 16-token slice, so each
  // (column, half) pair is one 16-byte piece
  if (t < 128) {
    const int cn = t >> 1, hh = t & 1;
    const int64_t nn = nc + cn, m = m0 + 8 * hh;
    if (nn < (d.N + 31) / 32 * 32 && m < ldt) {
      uint32_t ph[4], pl[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        ph[j] = (uint32_t)th[cn][8 * hh + 2 * j] | ((uint32_t)th[cn][8 * hh + 2 * j + 1] << 16);
        pl[j] = (uint32_t)tl[cn][8 * hh + 2 * j] | ((uint32_t)tl[cn][8 * hh + 2 * j + 1] << 16);
      }
      const int64_t f = frag_index(nn, m, ldt);
      *reinterpret_cast<u32x4*>(d.ht + f) = u32x4{ph[0], ph[1], ph[2], ph[3]};
      *reinterpret_cast<u32x4*>(d.lt + f) = u32x4{pl[0], pl[1], pl[2], pl[3]};
    }
  }
}

__global__ __launch_bounds__(256) void k_transpose_bf16(const uint16_t* __restrict__ in,
                                                        int64_t rows, int64_t cols,
                                                        uint16_t* __restrict__ out, int64_t ldo) {
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= cols * ldo) return;
  const int64_t c = idx / ldo, i = idx % ldo;
  out[idx] = (i < rows) ? in[i * cols + c] : (uint16_t)0;
}

// ---------------------------------------------------------------------------
// part[s][i][c] = sum_{m in split s} P[m][i] Q[m][c], i < R <= 256.  The
// contraction runs over tokens, the row index of both operands.  P arrives
// transposed and split (hi / lo BF16, zero past M and R) in fragment order,
// so the MFMA row operand of a 32-row block and 16 tokens is one contiguous
// 1 KB load per wavefront from L2.
// Q (X or dY) is streamed from HBM: each wavefront copies blocks of 64 token
// rows x 64 columns into an LDS region of its own and reads the column
// operands (eight consecutive tokens of one column) with transposing LDS
// reads (ds_read_b64_tr_b16); the global loads of the block two ahead are
// issued before the current block's MFMAs.  A workgroup covers all R rows x
// 256 columns x one token split, one 64-column tile per wavefront; the four
// wavefronts walk the same tokens and read the same P chunks at about the
// same time (mostly served by the compute unit's vector cache).
// ---------------------------------------------------------------------------
namespace {
constexpr int kGramRows = 64;                      // token rows per wavefront block
constexpr int kGramLd = 80;                        // LDS row: 64 columns + pad (40 dwords, = 8 mod 32)
constexpr int kGramWaveBytes = kGramRows * kGramLd * 2;
}  // namespace

// Q block (rows m .. m+63 of the wavefront, columns c0 .. c0+63): lane l
// loads row 8 i + l/8, columns 8 (l%8) .. +8, i = 0..7.
// The descriptor is based at the block's first token, so offsets stay below
// 64 rows of Q whatever M is; tokens past M read as zero.
// MASK: the keep words of Q's rows (qmask [M][N / 32], row-major bits; NULL:
// every element kept) are loaded beside the block into mk, word
// (row, col / 32), whose bits 8 (lane % 4) .. +8 are the lane's columns.
template <bool VEC, bool MASK>
__device__ __forceinline__ void gram_load(const uint16_t* Q, const uint32_t* qmask, int64_t M,
                                          int64_t m, int64_t c0, int64_t N, int lane, u32x4 (&x)[8],
                                          uint32_t (&mk)[8]) {
  const __amdgpu_buffer_rsrc_t rq = rank_rsrc(Q + (m < M ? m : M) * N, (M - m) * N * 2);
  if (MASK) {
    const int64_t nw = N / 32;
    const __amdgpu_buffer_rsrc_t rm =
        rank_rsrc(qmask ? qmask + (m < M ? m : M) * nw : nullptr, qmask ? (M - m) * nw * 4 : 0);
    const uint32_t all = qmask ? 0u : 0xFFFFFFFFu;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int64_t row = 8 * i + (lane >> 3), col = c0 + 8 * (lane & 7);
      mk[i] = all | __builtin_amdgcn_raw_buffer_load_b32(rm, (uint32_t)((row * nw + col / 32) * 4), 0, 0);
    }
  }
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int64_t row = 8 * i + (lane >> 3), col = c0 + 8 * (lane & 7);
    if (VEC) {
      x[i] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(
                                           rq, (uint32_t)((row * N + col) * 2), 0, 0));
    } else {
      uint32_t h[8];
#pragma unroll
      for (int e = 0; e < 8; ++e)
        h[e] = col + e < N ? (uint32_t)__builtin_amdgcn_raw_buffer_load_b16(
                                 rq, (uint32_t)((row * N + col + e) * 2), 0, 0)
                           : 0u;
      x[i] = u32x4{h[0] | (h[1] << 16), h[2] | (h[3] << 16), h[4] | (h[5] << 16),
                   h[6] | (h[7] << 16)};
    }
  }
}

// One 64-token block of a wavefront: stage Q block x (tokens m ..) in LDS,
// load the block's rank operands and the Q block two ahead into x, then 4
// token slices x RB x 2 x (hi, lo) MFMAs.
template <int RB, bool VEC, bool MASK>
__device__ __forceinline__ void gram_block(const uint16_t* Q, const uint32_t* qmask, int64_t M,
                                           __amdgpu_buffer_rsrc_t rh, __amdgpu_buffer_rsrc_t rl,
                                           int64_t ldp, int64_t c0, int64_t N, int64_t m, int lane,
                                           uint8_t* wl, uint32_t wr, uint32_t rd, u32x4 (&x)[8],
                                           uint32_t (&mk)[8], f32x16 (&acc)[RB][2]) {
#pragma unroll
  for (int i = 0; i < 8; ++i)
    *reinterpret_cast<u32x4*>(wl + wr + i * 8 * kGramLd * 2) =
        MASK ? keep8_bf16(x[i], mk[i] >> (8 * (lane & 3))) : x[i];
  u32x4 ph[4][RB], pl[4][RB];
#pragma unroll
  for (int t = 0; t < 4; ++t)
#pragma unroll
    for (int ib = 0; ib < RB; ++ib) {
      // fragment order: one contiguous 1 KB chunk per (row block, 16 tokens)
      const uint32_t po = (uint32_t)(((ib * (ldp >> 4) + (m >> 4) + t) * 64 + lane) * 16);
      ph[t][ib] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rh, po, 0, 0));
      pl[t][ib] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rl, po, 0, 0));
    }
  gram_load<VEC, MASK>(Q, qmask, M, m + 2 * kGramRows, c0, N, lane, x, mk);
  __builtin_amdgcn_sched_barrier(0);   // every load of the block ahead of its MFMAs
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    u32x4 b[2];
#pragma unroll
    for (int cb = 0; cb < 2; ++cb) {
      const uint8_t* pb = wl + rd + (16 * t * kGramLd + 32 * cb) * 2;
      const v4i16_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16_t*)(pb));
      const v4i16_t hi4 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16_t*)(pb + 4 * kGramLd * 2));
      const uint2 l2 = __builtin_bit_cast(uint2, lo), h2 = __builtin_bit_cast(uint2, hi4);
      b[cb] = u32x4{l2.x, l2.y, h2.x, h2.y};
    }
#pragma unroll
    for (int ib = 0; ib < RB; ++ib)
#pragma unroll
      for (int cb = 0; cb < 2; ++cb) {
        acc[ib][cb] = mfma32(ph[t][ib], b[cb], acc[ib][cb]);
        acc[ib][cb] = mfma32(pl[t][ib], b[cb], acc[ib][cb]);
      }
  }
}

struct GramDesc {
  const uint16_t* Pt_hi;
  const uint16_t* Pt_lo;
  const uint16_t* Q;
  const uint32_t* qmask;
  int64_t N, m_per_split;
  float* part;
  int cgroups;    // groups of four 64-column tiles
  int wg_begin;   // first workgroup of the problem
};
struct GramArgs {
  GramDesc d[2];
  int count;
  int64_t ldp, M, R;
};

// Workgroup = one token split and a group of four 64-column tiles; wavefront
// w takes column tile 4 g + w over the whole split.  The four wavefronts read
// the same rank fragments at about the same time, so the compute unit's
// vector cache serves most of them, and each wavefront's sums are complete
// for its columns: no reduction between wavefronts.
template <int RB, bool VEC, bool MASK>
__global__ __launch_bounds__(256) void k_gram(GramArgs ga) {
  extern __shared__ __attribute__((aligned(16))) uint8_t glds[];
  // problem of this workgroup, then its column group and token split
  const int di = (ga.count > 1 && (int)blockIdx.x >= ga.d[1].wg_begin) ? 1 : 0;
  const GramDesc& gd = ga.d[di];
  const uint16_t* __restrict__ Pt_hi = gd.Pt_hi;
  const uint16_t* __restrict__ Pt_lo = gd.Pt_lo;
  const uint16_t* __restrict__ Q = gd.Q;
  const uint32_t* qmask = gd.qmask;
  const int64_t ldp = ga.ldp, M = ga.M, R = ga.R, N = gd.N, m_per_split = gd.m_per_split;
  float* __restrict__ part = gd.part;
  const int local = (int)blockIdx.x - gd.wg_begin;
  const int lane = threadIdx.x & 63, w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int r32 = lane & 31, h = lane >> 5;
  const int g = lane >> 4, j = lane & 15;
  const int64_t c0 = ((int64_t)(local % gd.cgroups) * 4 + w) * 64;
  const int s = local / gd.cgroups;
  // m_per_split is a multiple of 128: whole pairs of 64-token blocks.  Tokens
  // at or past M read as zero in Q, so their (finite) products add nothing
  // and every block runs all four slices.  Columns at or past N (a ragged
  // last group) read in-bounds data or zeros and are never stored.
  const int64_t m_begin = (int64_t)s * m_per_split;
  int64_t m_end = m_begin + m_per_split;
  const int64_t m_lim = (M + 127) / 128 * 128;
  if (m_end > m_lim) m_end = m_lim;
  uint8_t* wl = glds + w * kGramWaveBytes;

  // fragment-ordered copies of round_up(R, 32) rows; row blocks past them read zero
  const __amdgpu_buffer_rsrc_t rh = rank_rsrc(Pt_hi, (R + 31) / 32 * 32 * ldp * 2);
  const __amdgpu_buffer_rsrc_t rl = rank_rsrc(Pt_lo, (R + 31) / 32 * 32 * ldp * 2);

  f32x16 acc[RB][2];
#pragma unroll
  for (int ib = 0; ib < RB; ++ib) acc[ib][0] = acc[ib][1] = f32x16{};

  // LDS block row of element (token k, column c): row k, byte (k * kGramLd + c) * 2.
  // Transposing read for MFMA column block cb, token slice t16: lane group g
  // covers columns 16 (g & 1) .. +16 and tokens 8 (g >> 1) .. +4 (+4 second read).
  const uint32_t wr = (uint32_t)(((8 * 0 + (lane >> 3)) * kGramLd + 8 * (lane & 7)) * 2);
  const uint32_t rd = (uint32_t)(((8 * (g >> 1) + (j >> 2)) * kGramLd + 16 * (g & 1) + 4 * (j & 3)) * 2);

  // Two Q blocks in flight: block j sits in register set j % 2 until it is
  // staged, and its registers then receive block j + 2.  Loads past the
  // range are in bounds or read zero and are never used; issuing them
  // unconditionally keeps the compiler's wait counts exact.
  u32x4 xa[8], xb[8];
  uint32_t ma[8], mb[8];
  gram_load<VEC, MASK>(Q, qmask, M, m_begin, c0, N, lane, xa, ma);
  __builtin_amdgcn_sched_barrier(0);   // issue order = use order
  gram_load<VEC, MASK>(Q, qmask, M, m_begin + kGramRows, c0, N, lane, xb, mb);
  __builtin_amdgcn_sched_barrier(0);
  for (int64_t m = m_begin; m < m_end; m += 2 * kGramRows) {
    gram_block<RB, VEC, MASK>(Q, qmask, M, rh, rl, ldp, c0, N, m, lane, wl, wr, rd, xa, ma, acc);
    gram_block<RB, VEC, MASK>(Q, qmask, M, rh, rl, ldp, c0, N, m + kGramRows, lane, wl, wr, rd,
                              xb, mb, acc);
  }

  // accumulator element v of lane l: row 32 ib + 8 (v/4) + 4 (l/32) + v%4,
  // column c0 + 32 cb + l%32; for each (ib, cb, v) the wavefront writes 32
  // consecutive columns of one row of the split's partial
  float* out = part + (int64_t)s * R * N;
#pragma unroll
  for (int ib = 0; ib < RB; ++ib)
#pragma unroll
    for (int cb = 0; cb < 2; ++cb)
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int64_t i = 32 * ib + 8 * (v >> 2) + 4 * h + (v & 3);
        const int64_t c = c0 + 32 * cb + r32;
        if (i < R && c < N) out[i * N + c] = acc[ib][cb][v];
      }
}

struct GramFinishArgs {
  const float* part[2];
  float* out[2];
  int64_t N[2];
  int splits[2];
  int transposed[2];
  int begin1;   // first workgroup of problem 1
  int count;
  int64_t R;
};

// Finish of the token-split partials: out = sum_s part[s] (s ascending).
// Workgroup = a tile of 32 rows (i < R) x 64 columns (c < N) of the [R][N]
// partials; the wavefronts read whole 256-byte row pieces of every split.
// out[i][c] is written the same way; the transposed out[c][i] (dB) goes
// through LDS so that each wavefront writes runs of 32 consecutive i.
constexpr int kGfTi = 32, kGfTc = 64;

__global__ __launch_bounds__(256) void k_gram_finish(GramFinishArgs a) {
  __shared__ float tile[kGfTi][kGfTc + 1];
  int wg = (int)blockIdx.x;
  const int di = (a.count > 1 && wg >= a.begin1) ? 1 : 0;
  if (di) wg -= a.begin1;
  const int64_t N = a.N[di], R = a.R, count = R * N;
  const int64_t ctiles = (N + kGfTc - 1) / kGfTc;
  const int64_t i0 = (wg / ctiles) * kGfTi, c0 = (wg % ctiles) * kGfTc;
  const float* __restrict__ part = a.part[di];
  float* __restrict__ out = a.out[di];
  const int S = a.splits[di];
  const int t = threadIdx.x;
  const int64_t c = c0 + (t & 63);
  constexpr int EU = kGfTi / 4;
  constexpr int SG = 8;   // splits whose loads are issued together
  float acc[EU];
  int64_t e[EU];
  bool ok[EU];
#pragma unroll
  for (int k = 0; k < EU; ++k) {
    const int64_t i = i0 + (t >> 6) + 4 * k;
    ok[k] = i < R && c < N;
    e[k] = ok[k] ? i * N + c : 0;
  }
  for (int s0 = 0; s0 < S; s0 += SG) {
    float v[SG][EU];
#pragma unroll
    for (int j = 0; j < SG; ++j)
#pragma unroll
      for (int k = 0; k < EU; ++k)
        v[j][k] = (ok[k] && s0 + j < S) ? part[(int64_t)(s0 + j) * count + e[k]] : 0.0f;
#pragma unroll
    for (int j = 0; j < SG; ++j)
#pragma unroll
      for (int k = 0; k < EU; ++k)
        if (s0 + j < S) acc[k] = (s0 + j == 0) ? v[j][k] : __fadd_rn(acc[k], v[j][k]);
  }
  if (!a.transposed[di]) {
#pragma unroll
    for (int k = 0; k < EU; ++k)
      if (ok[k]) out[e[k]] = acc[k];
    return;
  }
#pragma unroll
  for (int k = 0; k < EU; ++k) tile[(t >> 6) + 4 * k][t & 63] = acc[k];
  __syncthreads();
#pragma unroll
  for (int k = 0; k < kGfTc / 8; ++k) {
    const int ii = t & 31, cc = (t >> 5) + 8 * k;
    const int64_t i = i0 + ii, cn = c0 + cc;
    if (i < R && cn < N) out[cn * R + i] = tile[ii][cc];
  }
}

// ---------------------------------------------------------------------------
template <int NB>
static void launch_rank_rows_t(const RankRowsArgs& a, hipStream_t st) {
  const int64_t rows = a.ht ? a.ldt : a.M;
  constexpr int R = 16 * rank_rows_rg<NB>();
  const unsigned grid = (unsigned)((rows + R - 1) / R);
  if (grid == 0) return;
  hipLaunchKernelGGL(k_rank_rows<NB>, dim3(grid), dim3(64 * rank_rows_waves<NB>()), 0, st, a);
}

template <int NB>
static hipError_t launch_rank_part_t(const RankRowsArgs& a, float* part, int64_t kper, int ks,
                                     hipStream_t st) {
  const unsigned grid = (unsigned)(((a.M + 63) / 64) * ks);
  if (a.pmask)
    hipLaunchKernelGGL((k_rank_part<NB, true, false>), dim3(grid), dim3(256), 0, st, a, part, kper, ks);
  else if (a.q_kn)
    hipLaunchKernelGGL((k_rank_part<NB, false, true>), dim3(grid), dim3(256), 0, st, a, part, kper, ks);
  else
    hipLaunchKernelGGL((k_rank_part<NB, false, false>), dim3(grid), dim3(256), 0, st, a, part, kper, ks);
  return hipGetLastError();
}

hipError_t launch_rank_split(const RankRowsArgs& a, float* part, hipStream_t st,
                             const FinishDesc* extra) {
  // 16-byte row pieces need K and ldq multiples of 8 and aligned bases;
  // other layouts take the one-pass kernel, which loads elements
  if (a.pmask && (a.K % 32 != 0 || (reinterpret_cast<uintptr_t>(a.P) & 15)))
    return hipErrorInvalidValue;   // keep bits: whole words per row, 16-byte rows
  // Q as stored [K][ldq]: whole 16-byte pieces of its rows, only this kernel
  // takes that layout, and not with keep bits (U = dY B has none)
  if (a.q_kn && (a.pmask || a.N % 8 != 0 || a.ldq % 8 != 0 || a.K % 8 != 0 ||
                 (reinterpret_cast<uintptr_t>(a.P) & 15) || (reinterpret_cast<uintptr_t>(a.Q) & 15)))
    return hipErrorInvalidValue;
  if (a.K % 8 != 0 || a.ldq % 8 != 0 || (reinterpret_cast<uintptr_t>(a.P) & 15) ||
      (reinterpret_cast<uintptr_t>(a.Q) & 15)) {
    hipError_t e = launch_rank_rows(a, st);
    if (e == hipSuccess && extra) e = launch_rank_finish_rows(extra, 1, st);
    return e;
  }
  int64_t kper = 0;
  const int ks = rank_k_splits(a.M, a.K, &kper);
  hipError_t e;
  if (a.N <= 32) e = launch_rank_part_t<2>(a, part, kper, ks, st);
  else if (a.N <= 64) e = launch_rank_part_t<4>(a, part, kper, ks, st);
  else if (a.N <= 128) e = launch_rank_part_t<8>(a, part, kper, ks, st);
  else e = launch_rank_part_t<16>(a, part, kper, ks, st);
  if (e != hipSuccess) return e;
  FinishDesc d[2];
  d[0] = FinishDesc{part, a.out, a.ht, a.lt, a.M, a.N, a.ht ? a.ldt : a.M, a.scale, ks, 0, a.hl,
                    a.rp};
  if (extra) d[1] = *extra;
  return launch_rank_finish_rows(d, extra ? 2 : 1, st);
}

hipError_t launch_rank_finish_rows(const FinishDesc* d, int count, hipStream_t st) {
  FinishArgs a{};
  a.count = count;
  int64_t gx = 0, gy = 0;
  for (int i = 0; i < count; ++i) {
    a.d[i] = d[i];
    if (a.d[i].ldt <= 0) a.d[i].ldt = a.d[i].M;
    const int64_t rows = d[i].ht && a.d[i].ldt > d[i].M ? a.d[i].ldt : d[i].M;
    const int64_t ncols = d[i].hl && d[i].rp > d[i].N ? d[i].rp : d[i].N;
    gx = std::max(gx, (rows + 15) / 16);
    gy = std::max(gy, (ncols + 63) / 64);
  }
  if (gx == 0 || gy == 0) return hipSuccess;
  hipLaunchKernelGGL(k_rank_finish_rows, dim3((unsigned)gx, (unsigned)gy, (unsigned)count),
                     dim3(256), 0, st, a);
  return hipGetLastError();
}

hipError_t launch_rank_finish_rows(const float* part, int splits, int64_t M, int64_t N,
                                   float scale, float* out, uint16_t* ht, uint16_t* lt,
                                   int64_t ldt, uint16_t* hl, int64_t rp, hipStream_t st) {
  const FinishDesc d{part, out, ht, lt, M, N, ht ? ldt : M, scale, splits, 0, hl, rp};
  return launch_rank_finish_rows(&d, 1, st);
}

hipError_t launch_rank_rows(const RankRowsArgs& a, hipStream_t st) {
  if (a.N <= 32) launch_rank_rows_t<2>(a, st);
  else if (a.N <= 64) launch_rank_rows_t<4>(a, st);
  else if (a.N <= 128) launch_rank_rows_t<8>(a, st);
  else launch_rank_rows_t<16>(a, st);
  return hipGetLastError();
}

hipError_t launch_rank_finish(const FinishArgs& a0, hipStream_t st) {
  FinishArgs a = a0;
  int wgs = 0;
  for (int i = 0; i < a.count; ++i) {
    a.d[i].wg_begin = wgs;
    const int64_t ldt = a.d[i].ldt > 0 ? a.d[i].ldt : a.d[i].M;
    const int64_t nt = a.d[i].ht ? (a.d[i].N + 31) / 32 * 32 : a.d[i].N;
    wgs += (int)((nt * ldt + 255) / 256);
  }
  if (wgs == 0) return hipSuccess;
  hipLaunchKernelGGL(k_rank_finish, dim3(wgs), dim3(256), 0, st, a);
  return hipGetLastError();
}

hipError_t launch_rank_finish(const float* part, int splits, int64_t M, int64_t N, float scale,
                              float* out, uint16_t* ht, uint16_t* lt, int64_t ldt,
                              uint16_t* hl, int64_t rp, hipStream_t st) {
  FinishArgs a{};
  a.count = 1;
  a.d[0] = FinishDesc{part, out, ht, lt, M, N, ht ? ldt : M, scale, splits, 0, hl, rp};
  return launch_rank_finish(a, st);
}

hipError_t launch_transpose_bf16(const uint16_t* in, int64_t rows, int64_t cols, uint16_t* out,
                                 int64_t ldo, hipStream_t st) {
  const int64_t count = cols * ldo;
  hipLaunchKernelGGL(k_transpose_bf16, dim3((unsigned)((count + 255) / 256)), dim3(256), 0, st,
                     in, rows, cols, out, ldo);
  return hipGetLastError();
}

template <int RB, bool VEC, bool MASK>
static hipError_t launch_gram_t(const GramArgs& a, int wgs, hipStream_t st) {
  constexpr int lds = 4 * kGramWaveBytes;
  static hipError_t attr = hipFuncSetAttribute(reinterpret_cast<const void*>(&k_gram<RB, VEC, MASK>),
                                               hipFuncAttributeMaxDynamicSharedMemorySize, lds);
  if (attr != hipSuccess) return attr;
  hipLaunchKernelGGL((k_gram<RB, VEC, MASK>), dim3((unsigned)wgs), dim3(256), lds, st, a);
  return hipGetLastError();
}

// One contraction launch for problems sharing the 16-byte row loads or not.
static hipError_t launch_gram_group(const GramProblem* p, int count, int64_t ldp, int64_t M,
                                    int64_t R, bool vec, hipStream_t st) {
  GramArgs a{};
  a.count = count;
  a.ldp = ldp;
  a.M = M;
  a.R = R;
  int wgs = 0;
  bool mask = false;
  for (int i = 0; i < count; ++i) {
    a.d[i] = GramDesc{p[i].Pt_hi, p[i].Pt_lo, p[i].Q, p[i].qmask, p[i].N, p[i].m_per_split,
                      p[i].part, (int)((p[i].N + 255) / 256), wgs};
    wgs += a.d[i].cgroups * p[i].splits;
    if (p[i].qmask) {
      if (p[i].N % 32 != 0) return hipErrorInvalidValue;
      mask = true;
    }
  }
  if (wgs == 0) return hipSuccess;
  // keep bits: whole words per row and 16-byte row loads
  if (mask && !vec) return hipErrorInvalidValue;
#define QLORA_GRAM(RB) \
  return mask ? launch_gram_t<RB, true, true>(a, wgs, st) \
              : (vec ? launch_gram_t<RB, true, false>(a, wgs, st) : launch_gram_t<RB, false, false>(a, wgs, st))
  if (R <= 32) { QLORA_GRAM(1); }
  if (R <= 64) { QLORA_GRAM(2); }
  if (R <= 128) { QLORA_GRAM(4); }
  QLORA_GRAM(8);
#undef QLORA_GRAM
}

hipError_t launch_grams(const GramProblem* p, int count, int64_t ldp, int64_t M, int64_t R,
                        hipStream_t st) {
  if (count < 1 || count > 2) return hipErrorInvalidValue;
  const bool v0 = (p[0].N % 8) == 0;
  hipError_t e;
  if (count == 2 && ((p[1].N % 8) == 0) == v0) {
    e = launch_gram_group(p, 2, ldp, M, R, v0, st);
  } else {
    e = launch_gram_group(p, 1, ldp, M, R, v0, st);
    if (e == hipSuccess && count == 2)
      e = launch_gram_group(p + 1, 1, ldp, M, R, (p[1].N % 8) == 0, st);
  }
  if (e != hipSuccess) return e;
  GramFinishArgs f{};
  f.count = count;
  f.R = R;
  int64_t total = 0;
  for (int i = 0; i < count; ++i) {
    f.part[i] = p[i].part;
    f.out[i] = p[i].out;
    f.N[i] = p[i].N;
    f.splits[i] = p[i].splits;
    f.transposed[i] = p[i].transposed ? 1 : 0;
    if (i == 1) f.begin1 = (int)total;
    total += ((R + kGfTi - 1) / kGfTi) * ((p[i].N + kGfTc - 1) / kGfTc);
  }
  if (total == 0) return hipSuccess;
  hipLaunchKernelGGL(k_gram_finish, dim3((unsigned)total), dim3(256), 0, st, f);
  return hipGetLastError();
}

}  // namespace qlora
