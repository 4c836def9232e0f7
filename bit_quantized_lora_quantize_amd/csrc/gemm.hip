// gemm.hip -- fused NF4-dequant GEMM with the LoRA term, forward (Y) and
// input-gradient (dX) directions, for larger token counts (gfx950).
//
// [QP] "第 04 篇：QLoRA 原理" §2.3 / §6.1: weights are restored tile by tile
// inside the kernel (codes + quantization state read, unpacked, scaled,
// converted to BF16) and fed to the matrix cores; no BF16 copy of W reaches
// HBM.  §2.4: the input gradient passes through the same restored weights
// (transposed); the base gets no gradient.
//
// Tiling.  256 threads (4 wavefronts, 2 x 2), output tile 128 x 256, K step
// 64 = one quantization block per weight row.  Each thread restores exactly
// one 64-weight block per K step: one scale, one 16-entry table, eight
// byte-permute lookups.  Both operands are staged in LDS as BF16; every
// wavefront computes a 64 x 128 sub-tile with v_mfma_f32_16x16x32_bf16
// (32 accumulator tiles).  The next K step's global data is loaded into
// registers while the current step runs on the matrix cores.
//
// Forward   Y[m][n]  = sum_k X[m][k] Wh[n][k]   (+ LoRA: T_hi/T_lo x B)
//   LDS  As[m][k] = X permuted within each eight, Bs[n][k] = table lookups
//        in the same permuted order (nf4_dequant8_perm).
// Backward  dX[m][c] = sum_n dY[m][n] Wh[n][c]  (+ LoRA: U_hi/U_lo x A)
//   LDS  As[m][k] = dY in natural order, Bs[c][n] = restored weights written
//        transposed, one 16-bit store per weight.
// LoRA term: extra K steps over [hi(0..RP) | lo(0..RP)], RP = r rounded up
// to 32, with the FP32 rank-r activations split into two BF16 terms.
#include "qlora_device.h"
#include "qlora_kernels.h"

namespace qlora {

constexpr int BM = 128, BN = 256, BK = 64;
constexpr int LDA = BK + 8;  // padded LDS row (BF16 elements)

template <bool BWD>
struct GemmStage {
  u32x4 a[4];      // 32 activation values of this thread's row half
  u32x4 c0, c1;    // the thread's 64-weight block
  uint32_t sc;
  float s2, mu;
};

template <bool BWD>
__device__ __forceinline__ void gemm_load(const GemmArgs& p, int64_t m0, int64_t n0, int64_t k0,
                                          int tid, GemmStage<BWD>& s) {
  const u32x4 z = {0u, 0u, 0u, 0u};
  // activations: row tid/2, 32 columns starting at 32*(tid%2)
  {
    const int row = tid >> 1, half = tid & 1;
    const int64_t m = m0 + row;
    const int64_t K = BWD ? p.d_out : p.d_in;
    const uint16_t* src = p.act + m * K + k0 + 32 * half;
    const bool vec = (K % 8) == 0;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int64_t kk = k0 + 32 * half + 8 * q;
      if (m >= p.M || kk >= K) {
        s.a[q] = z;
      } else if (vec && kk + 8 <= K) {
        s.a[q] = *reinterpret_cast<const u32x4*>(src + 8 * q);
      } else {
        uint32_t h[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) h[e] = (kk + e < K) ? src[8 * q + e] : 0u;
        s.a[q].x = h[0] | (h[1] << 16); s.a[q].y = h[2] | (h[3] << 16);
        s.a[q].z = h[4] | (h[5] << 16); s.a[q].w = h[6] | (h[7] << 16);
      }
    }
  }
  // weights: one block per thread
  {
    int64_t row, col;  // weight row n and first column of the block
    if (!BWD) {
      row = n0 + tid;
      col = k0;
    } else {
      row = k0 + (tid & 63);
      col = n0 + 64 * (tid >> 6);
    }
    s.c0 = z;
    s.c1 = z;
    s.sc = 0u;
    s.s2 = 0.0f;
    s.mu = 0.0f;
    if (row < p.d_out && col < p.d_in) {
      const u32x4* cp = reinterpret_cast<const u32x4*>(p.codes + row * (p.d_in / 2) + col / 2);
      s.c0 = cp[0];
      s.c1 = cp[1];
      const int64_t b = (row * p.d_in + col) / kBlock;
      s.sc = p.scodes[b];
      s.s2 = p.scale2[b >> 8];
      s.mu = p.mean[0];
    }
  }
}

template <bool BWD>
__device__ __forceinline__ void gemm_store(const GemmStage<BWD>& s, int tid, uint16_t* As,
                                           uint16_t* Bs) {
  {
    const int row = tid >> 1, half = tid & 1;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      u32x4 v = BWD ? s.a[q] : perm8_bf16(s.a[q]);
      *reinterpret_cast<u32x4*>(As + row * LDA + 32 * half + 8 * q) = v;
    }
  }
  const Nf4Table t = nf4_table(restored_scale(s.sc, s.s2, s.mu));
  const uint32_t cw[8] = {s.c0.x, s.c0.y, s.c0.z, s.c0.w, s.c1.x, s.c1.y, s.c1.z, s.c1.w};
  if (!BWD) {
#pragma unroll
    for (int j = 0; j < 8; ++j)
      *reinterpret_cast<u32x4*>(Bs + tid * LDA + 8 * j) = nf4_dequant8_perm(cw[j], t);
  } else {
    // Bs[c][n]: column c of the weight block, contraction index n = row
    const int nr = tid & 63, cb = tid >> 6;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const u32x4 v = nf4_dequant8(cw[j], t);  // natural order e = 8j .. 8j+7
      uint16_t* dst = Bs + (cb * 64 + 8 * j) * LDA + nr;
      dst[0 * LDA] = (uint16_t)(v.x & 0xFFFFu);
      dst[1 * LDA] = (uint16_t)(v.x >> 16);
      dst[2 * LDA] = (uint16_t)(v.y & 0xFFFFu);
      dst[3 * LDA] = (uint16_t)(v.y >> 16);
      dst[4 * LDA] = (uint16_t)(v.z & 0xFFFFu);
      dst[5 * LDA] = (uint16_t)(v.z >> 16);
      dst[6 * LDA] = (uint16_t)(v.w & 0xFFFFu);
      dst[7 * LDA] = (uint16_t)(v.w >> 16);
    }
  }
}

// 64 MFMAs of one wavefront on the staged K step.
__device__ __forceinline__ void gemm_mma(const uint16_t* As, const uint16_t* Bs, int wm, int wn,
                                         int r16, int g, f32x4 (&acc)[4][8]) {
#pragma unroll
  for (int ks = 0; ks < 2; ++ks) {
    u32x4 af[4], bf[8];
#pragma unroll
    for (int mt = 0; mt < 4; ++mt)
      af[mt] = *reinterpret_cast<const u32x4*>(As + (64 * wm + 16 * mt + r16) * LDA + 32 * ks + 8 * g);
#pragma unroll
    for (int nt = 0; nt < 8; ++nt)
      bf[nt] = *reinterpret_cast<const u32x4*>(Bs + (128 * wn + 16 * nt + r16) * LDA + 32 * ks + 8 * g);
#pragma unroll
    for (int mt = 0; mt < 4; ++mt)
#pragma unroll
      for (int nt = 0; nt < 8; ++nt) acc[mt][nt] = mfma16(af[mt], bf[nt], acc[mt][nt]);
  }
}

template <bool BWD>
__global__ __launch_bounds__(256) void k_gemm(GemmArgs p) {
  __shared__ __attribute__((aligned(16))) uint16_t As[BM * LDA];
  __shared__ __attribute__((aligned(16))) uint16_t Bs[BN * LDA];
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int wm = w & 1, wn = w >> 1;
  const int r16 = lane & 15, g = lane >> 4;
  const int64_t n0 = (int64_t)blockIdx.x * BN;  // output columns
  const int64_t m0 = (int64_t)blockIdx.y * BM;  // tokens
  const int64_t K = BWD ? p.d_out : p.d_in;     // contraction length
  const int64_t nsteps = (K + BK - 1) / BK;

  f32x4 acc[4][8];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 8; ++j) acc[i][j] = {0.f, 0.f, 0.f, 0.f};

  GemmStage<BWD> st;
  gemm_load<BWD>(p, m0, n0, 0, tid, st);
  for (int64_t s = 0; s < nsteps; ++s) {
    gemm_store<BWD>(st, tid, As, Bs);
    __syncthreads();
    if (s + 1 < nsteps) gemm_load<BWD>(p, m0, n0, (s + 1) * BK, tid, st);
    gemm_mma(As, Bs, wm, wn, r16, g, acc);
    __syncthreads();
  }

  // ---- LoRA term as extra K steps over [hi | lo] ----
  const int64_t RP = (p.r + 31) / 32 * 32;
  for (int64_t e0 = 0; e0 < 2 * RP; e0 += BK) {
    // As[m][j] = hi/lo part of lr[m][kappa]
    for (int idx = tid; idx < BM * BK; idx += 256) {
      const int row = idx / BK, j = idx % BK;
      const int64_t kv = e0 + j;
      const int64_t kap = kv < RP ? kv : kv - RP;
      const int64_t m = m0 + row;
      float v = 0.0f;
      if (kv < 2 * RP && kap < p.r && m < p.M) {
        float hi, lo;
        split_bf16(p.lr[m * p.r + kap], hi, lo);
        v = kv < RP ? hi : lo;
      }
      f32x2 pr = {v, 0.0f};
      As[row * LDA + j] =
          (uint16_t)(__builtin_bit_cast(uint32_t, __builtin_convertvector(pr, bf16x2)) & 0xFFFFu);
    }
    // Bs[col][j] = lw entry for output column col and rank kappa
    for (int idx = tid; idx < BN * BK; idx += 256) {
      const int col = idx / BK, j = idx % BK;
      const int64_t kv = e0 + j;
      const int64_t kap = kv < RP ? kv : kv - RP;
      const int64_t c = n0 + col;
      uint16_t v = 0;
      if (kv < 2 * RP && kap < p.r) {
        if (!BWD) {
          if (c < p.d_out) v = p.lw[c * p.r + kap];  // B[n][kappa]
        } else {
          if (c < p.d_in) v = p.lw[kap * p.d_in + c];  // A[kappa][c]
        }
      }
      Bs[col * LDA + j] = v;
    }
    __syncthreads();
    gemm_mma(As, Bs, wm, wn, r16, g, acc);
    __syncthreads();
  }

  // ---- epilogue: RNE to BF16 ----
  const int64_t NOUT = BWD ? p.d_in : p.d_out;
#pragma unroll
  for (int mt = 0; mt < 4; ++mt)
#pragma unroll
    for (int nt = 0; nt < 8; ++nt) {
      const int64_t n = n0 + 128 * wn + 16 * nt + r16;
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int64_t m = m0 + 64 * wm + 16 * mt + 4 * g + v;
        if (m < p.M && n < NOUT) {
          f32x2 pr = {acc[mt][nt][v], 0.0f};
          p.out[m * NOUT + n] = (uint16_t)(
              __builtin_bit_cast(uint32_t, __builtin_convertvector(pr, bf16x2)) & 0xFFFFu);
        }
      }
    }
}

hipError_t launch_gemm_fwd(const GemmArgs& a, hipStream_t st) {
  dim3 grid((unsigned)((a.d_out + BN - 1) / BN), (unsigned)((a.M + BM - 1) / BM));
  weight_kernel_begin(st);
  hipLaunchKernelGGL(k_gemm<false>, grid, dim3(256), 0, st, a);
  weight_kernel_end(st);
  return hipGetLastError();
}

hipError_t launch_gemm_bwd(const GemmArgs& a, hipStream_t st) {
  dim3 grid((unsigned)((a.d_in + BN - 1) / BN), (unsigned)((a.M + BM - 1) / BM));
  weight_kernel_begin(st);
  hipLaunchKernelGGL(k_gemm<true>, grid, dim3(256), 0, st, a);
  weight_kernel_end(st);
  return hipGetLastError();
}

}  // namespace qlora
