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

// Eight BF16 values row[k0 .. k0+7], zero at and past `lim`.
__device__ __forceinline__ u32x4 load8_bf16(const uint16_t* row, int64_t k0, int64_t lim,
                                            bool vec) {
  if (vec && k0 + 8 <= lim) return *reinterpret_cast<const u32x4*>(row + k0);
  uint32_t h[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) h[e] = (k0 + e < lim) ? row[k0 + e] : 0u;
  u32x4 r;
  r.x = h[0] | (h[1] << 16);
  r.y = h[2] | (h[3] << 16);
  r.z = h[4] | (h[5] << 16);
  r.w = h[6] | (h[7] << 16);
  return r;
}

// ---------------------------------------------------------------------------
// Small M: part[s][m][n] = sum_{k in split s} P[m][k] Q[n][k].  One wavefront
// per 16 x 64 output tile and K split; a grid covers up to kMaxGroup
// problems.  The column-tile-0 wavefronts also write P permuted within each
// eight (the X operand of the weight-streaming kernel).
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(64) void k_rank_down(RankDownArgs a) {
  for (int z = 0; z < a.count; ++z) {
    if (!a.zero[z]) continue;
    for (int64_t i = (int64_t)blockIdx.x * 64 + threadIdx.x; i < a.zero_count[z];
         i += (int64_t)gridDim.x * 64)
      a.zero[z][i] = 0u;
  }
  const int wg = blockIdx.x;
  int di = 0;
  while (di + 1 < a.count && wg >= a.d[di + 1].wg_begin) ++di;
  const RankDownDesc& d = a.d[di];
  int local = wg - d.wg_begin;
  const int s = local % d.splits;
  local /= d.splits;
  const int tn = local % d.tiles_n;
  const int tm = local / d.tiles_n;

  const int lane = threadIdx.x;
  const int r16 = lane & 15, g = lane >> 4;
  const int64_t m = (int64_t)tm * 16 + r16;
  const int64_t k_begin = (int64_t)s * d.k_per_split;
  int64_t k_end = k_begin + d.k_per_split;
  if (k_end > d.K) k_end = d.K;
  const bool pvec = (d.K % 8) == 0;
  const bool qvec = (d.ldq % 8) == 0;

  f32x4 acc[4] = {};
  const uint16_t* prow = d.P + m * d.K;
  for (int64_t k0 = k_begin; k0 < k_end; k0 += 32) {
    const int64_t kk = k0 + 8 * g;
    u32x4 av = {0u, 0u, 0u, 0u};
    if (m < d.M && kk < k_end) av = load8_bf16(prow, kk, k_end, pvec);
    if (d.Xp && tn == 0 && m < d.M && kk < k_end)
      *reinterpret_cast<u32x4*>(d.Xp + m * d.K + kk) = perm8_bf16(av);
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const int64_t n = (int64_t)tn * 64 + 16 * t + r16;
      u32x4 bv = {0u, 0u, 0u, 0u};
      if (n < d.N && kk < k_end) bv = load8_bf16(d.Q + n * d.ldq, kk, k_end, qvec);
      acc[t] = mfma16(av, bv, acc[t]);
    }
  }
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    const int64_t n = (int64_t)tn * 64 + 16 * t + r16;
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int64_t mm = (int64_t)tm * 16 + 4 * g + v;
      if (mm < d.M && n < d.N) d.part[((int64_t)s * d.M + mm) * d.N + n] = acc[t][v];
    }
  }
}

// ---------------------------------------------------------------------------
// Large M: the same product with 256 x 64 workgroup tiles.  Wavefront w owns
// rows 64w .. 64w+63 of the tile: 2 x 2 tiles of v_mfma_f32_32x32x16_bf16.
// Operands come straight from global memory (P streamed once, Q shared
// through L1/L2); each iteration covers 64 of K.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void k_rank_down_big(const uint16_t* __restrict__ P,
                                                       const uint16_t* __restrict__ Q, int64_t M,
                                                       int64_t N, int64_t K, int64_t ldq,
                                                       int64_t k_per_split,
                                                       float* __restrict__ part) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int r32 = lane & 31, h = lane >> 5;
  const int64_t m0 = (int64_t)blockIdx.x * 256 + 64 * w;
  const int64_t n0 = (int64_t)blockIdx.y * 64;
  const int s = blockIdx.z;
  const int64_t k_begin = (int64_t)s * k_per_split;
  int64_t k_end = k_begin + k_per_split;
  if (k_end > K) k_end = K;
  const bool fast = (K % 8) == 0 && (ldq % 8) == 0 && m0 + 64 <= M && n0 + 64 <= N;

  f32x16 acc[2][2] = {};
  const uint16_t* pr[2];
  const uint16_t* qr[2];
  bool pok[2], qok[2];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int64_t m = m0 + 32 * i + r32, n = n0 + 32 * i + r32;
    pok[i] = m < M;
    qok[i] = n < N;
    pr[i] = P + (pok[i] ? m : 0) * K;
    qr[i] = Q + (qok[i] ? n : 0) * ldq;
  }
  for (int64_t k0 = k_begin; k0 < k_end; k0 += 64) {
    u32x4 a[4][2], b[4][2];
    if (fast && k0 + 64 <= k_end) {
#pragma unroll
      for (int ks = 0; ks < 4; ++ks)
#pragma unroll
        for (int i = 0; i < 2; ++i) {
          a[ks][i] = *reinterpret_cast<const u32x4*>(pr[i] + k0 + 16 * ks + 8 * h);
          b[ks][i] = *reinterpret_cast<const u32x4*>(qr[i] + k0 + 16 * ks + 8 * h);
        }
    } else {
      const u32x4 z = {0u, 0u, 0u, 0u};
#pragma unroll
      for (int ks = 0; ks < 4; ++ks)
#pragma unroll
        for (int i = 0; i < 2; ++i) {
          const int64_t kk = k0 + 16 * ks + 8 * h;
          a[ks][i] = pok[i] ? load8_bf16(pr[i], kk, k_end, (K % 8) == 0) : z;
          b[ks][i] = qok[i] ? load8_bf16(qr[i], kk, k_end, (ldq % 8) == 0) : z;
        }
    }
#pragma unroll
    for (int ks = 0; ks < 4; ++ks)
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) acc[i][j] = mfma32(a[ks][i], b[ks][j], acc[i][j]);
  }
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int64_t n = n0 + 32 * j + r32;
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int64_t m = m0 + 32 * i + 8 * (v >> 2) + 4 * h + (v & 3);
        if (m < M && n < N) part[((int64_t)s * M + m) * N + n] = acc[i][j][v];
      }
    }
}

// ---------------------------------------------------------------------------
// Finish: v = scale * sum_s part[s] (s ascending).  Thread per element of the
// transposed [N][ldt] index space (the FP32 [M][N] output is written from
// the same thread when requested).
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void k_rank_finish(FinishArgs a) {
  const int wg = blockIdx.x;
  int di = 0;
  while (di + 1 < a.count && wg >= a.d[di + 1].wg_begin) ++di;
  const FinishDesc& d = a.d[di];
  const int64_t idx = (int64_t)(wg - d.wg_begin) * 256 + threadIdx.x;
  const int64_t ldt = d.ldt > 0 ? d.ldt : d.M;
  if (idx >= d.N * ldt) return;
  const int64_t n = idx / ldt, m = idx % ldt;
  float v = 0.0f;
  if (m < d.M) {
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
    d.ht[idx] = hb;
    d.lt[idx] = lb;
  }
  if (d.hl && m < d.M) {
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

__global__ __launch_bounds__(256) void k_transpose_bf16(const uint16_t* __restrict__ in,
                                                        int64_t rows, int64_t cols,
                                                        uint16_t* __restrict__ out, int64_t ldo) {
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= cols * ldo) return;
  const int64_t c = idx / ldo, i = idx % ldo;
  out[idx] = (i < rows) ? in[i * cols + c] : (uint16_t)0;
}

// ---------------------------------------------------------------------------
// part[s][i][c] = sum_{m in split s} P[m][i] Q[m][c].  The contraction runs
// over tokens, the row index of both operands.  P arrives transposed
// (hi/lo BF16 [R][ldp]) so its MFMA operand is one 16-byte load; Q is
// transposed in registers: lane (c32, h) loads 4 columns of 8 token rows
// (8-byte loads, a wavefront reads 16 rows x 256 B) and one byte permute per
// output dword builds the 8-token column operands.  MFMA t of a lane then
// covers columns 4*c32 + t.  Wavefront tile: 64 (i) x 128 (c), 16 tokens per
// step; 4 wavefronts per workgroup side by side in c.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void k_gram(const uint16_t* __restrict__ Pt_hi,
                                              const uint16_t* __restrict__ Pt_lo, int64_t ldp,
                                              const uint16_t* __restrict__ Q, int64_t M,
                                              int64_t R, int64_t N, int64_t m_per_split,
                                              float* __restrict__ part) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int c32 = lane & 31, h = lane >> 5;
  const int64_t cb = (int64_t)blockIdx.x * 512 + 128 * w;
  const int64_t i0 = (int64_t)blockIdx.y * 64;
  const int s = blockIdx.z;
  const int64_t m_begin = (int64_t)s * m_per_split;
  int64_t m_end = m_begin + m_per_split;
  if (m_end > M) m_end = M;
  const int64_t col = cb + 4 * c32;
  const bool cvec = (N % 4) == 0 && col + 4 <= N;

  f32x16 acc[4][2] = {};
  for (int64_t m0 = m_begin; m0 < m_end; m0 += 16) {
    uint32_t q[8][2];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int64_t m = m0 + 8 * h + e;
      if (m < m_end && cvec) {
        const uint2 v = *reinterpret_cast<const uint2*>(Q + m * N + col);
        q[e][0] = v.x;
        q[e][1] = v.y;
      } else {
        uint32_t x[4];
#pragma unroll
        for (int t = 0; t < 4; ++t) x[t] = (m < m_end && col + t < N) ? Q[m * N + col + t] : 0u;
        q[e][0] = x[0] | (x[1] << 16);
        q[e][1] = x[2] | (x[3] << 16);
      }
    }
    u32x4 ah[2], al[2];
#pragma unroll
    for (int it = 0; it < 2; ++it) {
      const int64_t i = i0 + 32 * it + c32;
      const u32x4 z = {0u, 0u, 0u, 0u};
      ah[it] = i < R ? *reinterpret_cast<const u32x4*>(Pt_hi + i * ldp + m0 + 8 * h) : z;
      al[it] = i < R ? *reinterpret_cast<const u32x4*>(Pt_lo + i * ldp + m0 + 8 * h) : z;
    }
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const uint32_t sel = (t & 1) ? 0x07060302u : 0x05040100u;
      u32x4 b;
      b.x = __builtin_amdgcn_perm(q[1][t >> 1], q[0][t >> 1], sel);
      b.y = __builtin_amdgcn_perm(q[3][t >> 1], q[2][t >> 1], sel);
      b.z = __builtin_amdgcn_perm(q[5][t >> 1], q[4][t >> 1], sel);
      b.w = __builtin_amdgcn_perm(q[7][t >> 1], q[6][t >> 1], sel);
#pragma unroll
      for (int it = 0; it < 2; ++it) {
        acc[t][it] = mfma32(ah[it], b, acc[t][it]);
        acc[t][it] = mfma32(al[it], b, acc[t][it]);
      }
    }
  }
#pragma unroll
  for (int t = 0; t < 4; ++t)
#pragma unroll
    for (int it = 0; it < 2; ++it) {
      const int64_t c = col + t;
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int64_t i = i0 + 32 * it + 8 * (v >> 2) + 4 * h + (v & 3);
        if (i < R && c < N) part[((int64_t)s * R + i) * N + c] = acc[t][it][v];
      }
    }
}

__global__ __launch_bounds__(256) void k_gram_finish(const float* __restrict__ part, int splits,
                                                     int64_t R, int64_t N, int transposed,
                                                     float* __restrict__ out) {
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t count = R * N;
  if (idx >= count) return;
  float acc = part[idx];
  for (int s = 1; s < splits; ++s) acc = __fadd_rn(acc, part[(int64_t)s * count + idx]);
  const int64_t i = idx / N, c = idx % N;
  out[transposed ? c * R + i : idx] = acc;
}

// ---------------------------------------------------------------------------
hipError_t launch_rank_down(const RankDownArgs& a, int total_wgs, hipStream_t st) {
  hipLaunchKernelGGL(k_rank_down, dim3(total_wgs), dim3(64), 0, st, a);
  return hipGetLastError();
}

hipError_t launch_rank_down_big(const uint16_t* P, const uint16_t* Q, int64_t M, int64_t N,
                                int64_t K, int64_t ldq, int64_t k_per_split, int splits,
                                float* part, hipStream_t st) {
  dim3 grid((unsigned)((M + 255) / 256), (unsigned)((N + 63) / 64), (unsigned)splits);
  hipLaunchKernelGGL(k_rank_down_big, grid, dim3(256), 0, st, P, Q, M, N, K, ldq, k_per_split,
                     part);
  return hipGetLastError();
}

hipError_t launch_rank_finish(const FinishArgs& a0, hipStream_t st) {
  FinishArgs a = a0;
  int wgs = 0;
  for (int i = 0; i < a.count; ++i) {
    a.d[i].wg_begin = wgs;
    const int64_t ldt = a.d[i].ldt > 0 ? a.d[i].ldt : a.d[i].M;
    wgs += (int)((a.d[i].N * ldt + 255) / 256);
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

hipError_t launch_gram(const uint16_t* Pt_hi, const uint16_t* Pt_lo, int64_t ldp,
                       const uint16_t* Q, int64_t M, int64_t R, int64_t N, int64_t m_per_split,
                       int splits, float* part, hipStream_t st) {
  dim3 grid((unsigned)((N + 511) / 512), (unsigned)((R + 63) / 64), (unsigned)splits);
  hipLaunchKernelGGL(k_gram, grid, dim3(256), 0, st, Pt_hi, Pt_lo, ldp, Q, M, R, N, m_per_split,
                     part);
  return hipGetLastError();
}

hipError_t launch_gram_finish(const float* part, int splits, int64_t R, int64_t N,
                              bool transposed, float* out, hipStream_t st) {
  const int64_t count = R * N;
  hipLaunchKernelGGL(k_gram_finish, dim3((unsigned)((count + 255) / 256)), dim3(256), 0, st,
                     part, splits, R, N, transposed ? 1 : 0, out);
  return hipGetLastError();
}

}  // namespace qlora
