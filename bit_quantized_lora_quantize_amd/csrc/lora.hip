// lora.hip -- the rank-r side of the LoRA linear layer (gfx950).
//
// [QP] "第 04 篇：QLoRA 原理" §2.2 (LoRA branch), §2.4 (gradients of A, B and
// the input), §6.3-6.4.  With s = alpha / r and token rows:
//   T = s X A^T,  U = s dY B,  dA = U^T X,  dB = dY^T T.
// Thin products run on the matrix cores (v_mfma_f32_16x16x32_bf16) with FP32
// accumulation.  Reductions over K or over tokens are split across
// workgroups into FP32 partials that a finish kernel sums in split order, so
// every result is deterministic.
#include "qlora_device.h"
#include "qlora_kernels.h"

namespace qlora {

// Eight BF16 values P[k0 .. k0+7] of a row with K columns, zero past K.
__device__ __forceinline__ u32x4 load8_bf16(const uint16_t* row, int64_t k0, int64_t K,
                                            bool vec) {
  if (vec && k0 + 8 <= K) return *reinterpret_cast<const u32x4*>(row + k0);
  uint32_t h[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) h[e] = (k0 + e < K) ? row[k0 + e] : 0u;
  u32x4 r;
  r.x = h[0] | (h[1] << 16);
  r.y = h[2] | (h[3] << 16);
  r.z = h[4] | (h[5] << 16);
  r.w = h[6] | (h[7] << 16);
  return r;
}

// ---------------------------------------------------------------------------
// part[s][m][n] = sum_{k in split s} P[m][k] Q[n][k].  One wavefront per
// 16 x 64 output tile and K split; a grid covers up to kMaxGroup problems.
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

__global__ __launch_bounds__(256) void k_rank_finish(const float* __restrict__ part, int splits,
                                                     int64_t count, float scale,
                                                     float* __restrict__ out) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= count) return;
  float acc = part[i];
  for (int s = 1; s < splits; ++s) acc = __fadd_rn(acc, part[(int64_t)s * count + i]);
  out[i] = __fmul_rn(scale, acc);
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
// part[s][i][c] = sum_{m in split s} P[m][i] Q[m][c].  Workgroup tile 64 (i)
// x 128 (c); per 32-token step both operands are staged in LDS and read
// transposed (the contraction runs over tokens, the row index of both).
// P enters as hi + lo BF16 (two MFMAs per tile).
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void k_gram(const float* __restrict__ P,
                                              const uint16_t* __restrict__ Q, int64_t M,
                                              int64_t R, int64_t N, int64_t m_per_split,
                                              float* __restrict__ part) {
  __shared__ float Ps[32][64 + 1];
  __shared__ uint16_t Qs[32][128 + 2];
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int r16 = lane & 15, g = lane >> 4;
  const int64_t c0 = (int64_t)blockIdx.x * 128, i0 = (int64_t)blockIdx.y * 64;
  const int s = blockIdx.z;
  const int64_t m_begin = (int64_t)s * m_per_split;
  int64_t m_end = m_begin + m_per_split;
  if (m_end > M) m_end = M;

  f32x4 acc[4][2] = {};
  for (int64_t m0 = m_begin; m0 < m_end; m0 += 32) {
    {  // stage P[m0..m0+32][i0..i0+64] (FP32) and Q[m0..m0+32][c0..c0+128]
      const int row = tid >> 3, col = (tid & 7) * 8;
      const int64_t m = m0 + row;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int64_t i = i0 + col + e;
        Ps[row][col + e] = (m < m_end && i < R) ? P[m * R + i] : 0.0f;
      }
      const int qc = (tid & 7) * 16;
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int64_t c = c0 + qc + e;
        Qs[row][qc + e] = (m < m_end && c < N) ? Q[m * N + c] : (uint16_t)0;
      }
    }
    __syncthreads();
    u32x4 bq[2];
#pragma unroll
    for (int ct = 0; ct < 2; ++ct) {
      const int c = 32 * w + 16 * ct + r16;
      uint32_t h[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) h[e] = Qs[8 * g + e][c];
      bq[ct].x = h[0] | (h[1] << 16);
      bq[ct].y = h[2] | (h[3] << 16);
      bq[ct].z = h[4] | (h[5] << 16);
      bq[ct].w = h[6] | (h[7] << 16);
    }
#pragma unroll
    for (int it = 0; it < 4; ++it) {
      float hi[8], lo[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) split_bf16(Ps[8 * g + e][16 * it + r16], hi[e], lo[e]);
      u32x4 ah, al;
      ah.x = pack_bf16x2(hi[0], hi[1]);
      ah.y = pack_bf16x2(hi[2], hi[3]);
      ah.z = pack_bf16x2(hi[4], hi[5]);
      ah.w = pack_bf16x2(hi[6], hi[7]);
      al.x = pack_bf16x2(lo[0], lo[1]);
      al.y = pack_bf16x2(lo[2], lo[3]);
      al.z = pack_bf16x2(lo[4], lo[5]);
      al.w = pack_bf16x2(lo[6], lo[7]);
#pragma unroll
      for (int ct = 0; ct < 2; ++ct) {
        acc[it][ct] = mfma16(ah, bq[ct], acc[it][ct]);
        acc[it][ct] = mfma16(al, bq[ct], acc[it][ct]);
      }
    }
    __syncthreads();
  }
#pragma unroll
  for (int it = 0; it < 4; ++it)
#pragma unroll
    for (int ct = 0; ct < 2; ++ct) {
      const int64_t c = c0 + 32 * w + 16 * ct + r16;
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int64_t i = i0 + 16 * it + 4 * g + v;
        if (i < R && c < N) part[((int64_t)s * R + i) * N + c] = acc[it][ct][v];
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

hipError_t launch_rank_finish(const float* part, int splits, int64_t M, int64_t N, float scale,
                              float* out, hipStream_t st) {
  const int64_t count = M * N;
  if (count == 0) return hipSuccess;
  hipLaunchKernelGGL(k_rank_finish, dim3((unsigned)((count + 255) / 256)), dim3(256), 0, st,
                     part, splits, count, scale, out);
  return hipGetLastError();
}

hipError_t launch_transpose_bf16(const uint16_t* in, int64_t rows, int64_t cols, uint16_t* out,
                                 int64_t ldo, hipStream_t st) {
  const int64_t count = cols * ldo;
  hipLaunchKernelGGL(k_transpose_bf16, dim3((unsigned)((count + 255) / 256)), dim3(256), 0, st,
                     in, rows, cols, out, ldo);
  return hipGetLastError();
}

hipError_t launch_gram(const float* P, const uint16_t* Q, int64_t M, int64_t R, int64_t N,
                       int64_t m_per_split, int splits, float* part, hipStream_t st) {
  dim3 grid((unsigned)((N + 127) / 128), (unsigned)((R + 63) / 64), (unsigned)splits);
  hipLaunchKernelGGL(k_gram, grid, dim3(256), 0, st, P, Q, M, R, N, m_per_split, part);
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
