// gemm.hip -- fused NF4-dequant GEMM with the LoRA term, forward (Y) and
// input-gradient (dX) directions, for larger token counts (gfx950).
//
// [QP] "第 04 篇：QLoRA 原理" §2.3 / §6.1: weights are restored tile by tile
// inside the kernel (codes + quantization state read, unpacked, scaled,
// converted to BF16) and fed to the matrix cores; no BF16 copy of W reaches
// HBM.  §2.4: the input gradient passes through the same restored weights
// (transposed); the base gets no gradient.
//
// Tiling.  256 threads = 4 wavefronts in a 2 x 2 arrangement; output tile
// 256 x 256; K step 64 = one quantization block per weight row.  Each
// wavefront owns a 128 x 128 sub-tile: 4 x 4 tiles of v_mfma_f32_32x32x16_bf16
// with 256 FP32 accumulators per lane.  Both operands are staged in LDS as
// BF16, double-buffered (2 x 72 KB): while the matrix cores work on step s,
// the same wavefronts restore step s+1's weights into the other buffer from
// registers loaded one step earlier, and issue the global loads of step s+2.
// One barrier per K step.  Each thread restores exactly one 64-weight block
// per step: one scale, one 16-entry table, eight byte-permute lookups.
//
// Forward   Y[m][n]  = sum_k X[m][k] Wh[n][k]   (+ LoRA: T_hi/T_lo x B)
//   LDS  As[m][k] = X permuted within each eight, Bs[n][k] = table lookups in
//        the same permuted order (nf4_dequant8_perm).
// Backward  dX[m][c] = sum_n dY[m][n] Wh[n][c]  (+ LoRA: U_hi/U_lo x A)
//   LDS  As[m][k] = dY in natural order, Bs[c][n] = restored weights written
//        transposed, one 16-bit LDS store per weight.
// LoRA term: extra K steps over [hi(0..RP) | lo(0..RP)], RP = r rounded up
// to 32, with the FP32 rank-r activations split into two BF16 terms.
//
// Workgroup order: consecutive workgroup ids are spread over the 8 XCDs, so
// ids are remapped for each XCD to own a contiguous run of output tiles
// (same activation rows, neighbouring weight rows) in its own L2.
#include "qlora_device.h"
#include "qlora_kernels.h"

namespace qlora {

constexpr int BM = 256, BN = 256, BK = 64;
constexpr int LDA = BK + 8;                 // padded LDS row, BF16 elements
constexpr int kBufA = BM * LDA, kBufB = BN * LDA;
constexpr int kLdsBytes = 2 * (kBufA + kBufB) * 2;
constexpr int kXcds = 8;

struct GemmStage {
  u32x4 a[8];     // activations: 8 rows x 8 columns of this thread
  u32x4 c0, c1;   // the thread's 64-weight block
  uint32_t sc;
  float s2, mu;
};

// Activation rows of a K step: thread t loads rows t/8 + 32q (q = 0..7),
// columns 8*(t%8) .. +8 -- eight threads read one 128-byte row segment.
template <bool BWD>
__device__ __forceinline__ void load_stage(const GemmArgs& p, int64_t m0, int64_t n0, int64_t k0,
                                           int tid, GemmStage& s) {
  const u32x4 z = {0u, 0u, 0u, 0u};
  const int64_t K = BWD ? p.d_out : p.d_in;
  const bool vec = (K % 8) == 0;
  const int cc = (tid & 7) * 8;
  const int64_t kk = k0 + cc;
  // Interior tile (uniform over the workgroup): no per-lane bounds checks.
  const int64_t NW = BWD ? p.d_in : p.d_out;
  if (vec && m0 + BM <= p.M && k0 + BK <= K && n0 + BN <= NW) {
#pragma unroll
    for (int q = 0; q < 8; ++q)
      s.a[q] = *reinterpret_cast<const u32x4*>(p.act + (m0 + (tid >> 3) + 32 * q) * K + kk);
    const int64_t row = BWD ? k0 + (tid & 63) : n0 + tid;
    const int64_t col = BWD ? n0 + 64 * (tid >> 6) : k0;
    const u32x4* cp = reinterpret_cast<const u32x4*>(p.codes + row * (p.d_in / 2) + col / 2);
    s.c0 = cp[0];
    s.c1 = cp[1];
    const int64_t b = (row * p.d_in + col) / kBlock;
    s.sc = p.scodes[b];
    s.s2 = p.scale2[b >> 8];
    s.mu = p.mean[0];
    return;
  }
#pragma unroll
  for (int q = 0; q < 8; ++q) {
    const int64_t m = m0 + (tid >> 3) + 32 * q;
    const uint16_t* src = p.act + m * K + kk;
    if (m >= p.M || kk >= K) {
      s.a[q] = z;
    } else if (vec && kk + 8 <= K) {
      s.a[q] = *reinterpret_cast<const u32x4*>(src);
    } else {
      uint32_t h[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) h[e] = (kk + e < K) ? src[e] : 0u;
      s.a[q].x = h[0] | (h[1] << 16); s.a[q].y = h[2] | (h[3] << 16);
      s.a[q].z = h[4] | (h[5] << 16); s.a[q].w = h[6] | (h[7] << 16);
    }
  }
  int64_t row, col;  // weight row n and first column of the thread's block
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

template <bool BWD>
__device__ __forceinline__ void store_stage(const GemmStage& s, int tid, uint16_t* As,
                                            uint16_t* Bs) {
  const int cc = (tid & 7) * 8;
#pragma unroll
  for (int q = 0; q < 8; ++q) {
    const int row = (tid >> 3) + 32 * q;
    *reinterpret_cast<u32x4*>(As + row * LDA + cc) = BWD ? s.a[q] : perm8_bf16(s.a[q]);
  }
  const Nf4Table t = nf4_table(restored_scale(s.sc, s.s2, s.mu));
  const uint32_t cw[8] = {s.c0.x, s.c0.y, s.c0.z, s.c0.w, s.c1.x, s.c1.y, s.c1.z, s.c1.w};
  if (!BWD) {
#pragma unroll
    for (int j = 0; j < 8; ++j)
      *reinterpret_cast<u32x4*>(Bs + tid * LDA + 8 * j) = nf4_dequant8_perm(cw[j], t);
  } else {
    // Bs[c][n]: column c of the block's row n (the contraction index)
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

// 64 MFMAs (v_mfma_f32_32x32x16_bf16) of one wavefront on a staged K step:
// 4 x 4 tiles of 32 x 32, four K slices of 16.  Operand lane l holds row
// (A) / column (B) l%32 and contraction elements 8*(l/32) .. +8.
__device__ __forceinline__ void mma_stage(const uint16_t* As, const uint16_t* Bs, int wm, int wn,
                                          int r32, int h, f32x16 (&acc)[4][4]) {
#pragma unroll
  for (int ks = 0; ks < 4; ++ks) {
    u32x4 af[4], bf[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      af[i] = *reinterpret_cast<const u32x4*>(As + (128 * wm + 32 * i + r32) * LDA + 16 * ks + 8 * h);
      bf[i] = *reinterpret_cast<const u32x4*>(Bs + (128 * wn + 32 * i + r32) * LDA + 16 * ks + 8 * h);
    }
#pragma unroll
    for (int mt = 0; mt < 4; ++mt)
#pragma unroll
      for (int nt = 0; nt < 4; ++nt) acc[mt][nt] = mfma32(af[mt], bf[nt], acc[mt][nt]);
  }
}

// LoRA extension step e0: As[m][j] = hi/lo of lr[m][kappa], Bs[col][j] = the
// matching LoRA factor entry, for kappa-columns e0 .. e0+63 of [hi | lo].
template <bool BWD>
__device__ __forceinline__ void fill_lora_stage(const GemmArgs& p, int64_t m0, int64_t n0,
                                                int64_t e0, int64_t RP, int tid, uint16_t* As,
                                                uint16_t* Bs) {
  for (int idx = tid; idx < BM * BK; idx += 256) {
    const int row = idx >> 6, j = idx & 63;
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
  for (int idx = tid; idx < BN * BK; idx += 256) {
    const int col = idx >> 6, j = idx & 63;
    const int64_t kv = e0 + j;
    const int64_t kap = kv < RP ? kv : kv - RP;
    const int64_t c = n0 + col;
    uint16_t v = 0;
    if (kv < 2 * RP && kap < p.r) {
      if (!BWD) {
        if (c < p.d_out) v = p.lw[c * p.r + kap];      // B[n][kappa]
      } else {
        if (c < p.d_in) v = p.lw[kap * p.d_in + c];    // A[kappa][c]
      }
    }
    Bs[col * LDA + j] = v;
  }
}

template <bool BWD>
__global__ __launch_bounds__(256) void k_gemm(GemmArgs p) {
  extern __shared__ __attribute__((aligned(16))) uint16_t lds[];
  uint16_t* As0 = lds;
  uint16_t* Bs0 = lds + kBufA;
  uint16_t* As1 = lds + kBufA + kBufB;
  uint16_t* Bs1 = lds + 2 * kBufA + kBufB;

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int wm = w & 1, wn = w >> 1;
  const int r32 = lane & 31, h = lane >> 5;

  const int64_t NOUT = BWD ? p.d_in : p.d_out;
  const int tiles_n = (int)((NOUT + BN - 1) / BN);
  const int tiles_m = (int)((p.M + BM - 1) / BM);
  const int total = tiles_n * tiles_m;
  // XCD-aware remap: hardware places workgroup id i on XCD i % 8; give each
  // XCD a contiguous range of (m, n) tiles in n-fastest order.
  int id = blockIdx.x;
  {
    const int per = total / kXcds, extra = total % kXcds;
    const int x = id % kXcds, slot = id / kXcds;
    id = (x < extra ? x * (per + 1) : extra * (per + 1) + (x - extra) * per) + slot;
  }
  const int64_t n0 = (int64_t)(id % tiles_n) * BN;
  const int64_t m0 = (int64_t)(id / tiles_n) * BM;
  const int64_t K = BWD ? p.d_out : p.d_in;
  const int64_t nsteps = (K + BK - 1) / BK;

  f32x16 acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f32x16{};

  GemmStage st;
  load_stage<BWD>(p, m0, n0, 0, tid, st);
  store_stage<BWD>(st, tid, As0, Bs0);
  // step 1's data (a step at or past K loads zeros and is never consumed)
  load_stage<BWD>(p, m0, n0, BK, tid, st);
  __syncthreads();
  uint16_t* Ac = As0;
  uint16_t* Bc = Bs0;
  uint16_t* An = As1;
  uint16_t* Bn = Bs1;
  for (int64_t s = 0; s + 1 < nsteps; ++s) {
    mma_stage(Ac, Bc, wm, wn, r32, h, acc);
    store_stage<BWD>(st, tid, An, Bn);
    load_stage<BWD>(p, m0, n0, (s + 2) * BK, tid, st);
    __syncthreads();
    uint16_t* t0 = Ac; Ac = An; An = t0;
    uint16_t* t1 = Bc; Bc = Bn; Bn = t1;
  }
  mma_stage(Ac, Bc, wm, wn, r32, h, acc);
  __syncthreads();

  // ---- LoRA term as extra K steps over [hi | lo] ----
  const int64_t RP = (p.r + 31) / 32 * 32;
  for (int64_t e0 = 0; e0 < 2 * RP; e0 += BK) {
    fill_lora_stage<BWD>(p, m0, n0, e0, RP, tid, As0, Bs0);
    __syncthreads();
    mma_stage(As0, Bs0, wm, wn, r32, h, acc);
    __syncthreads();
  }

  // ---- epilogue: RNE to BF16.  Accumulator element v of lane l holds row
  // 8*(v/4) + 4*(l/32) + v%4 and column l%32 of its 32 x 32 tile. ----
#pragma unroll
  for (int mt = 0; mt < 4; ++mt)
#pragma unroll
    for (int nt = 0; nt < 4; ++nt) {
      const int64_t n = n0 + 128 * wn + 32 * nt + r32;
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int64_t m = m0 + 128 * wm + 32 * mt + 8 * (v >> 2) + 4 * h + (v & 3);
        if (m < p.M && n < NOUT) {
          f32x2 pr = {acc[mt][nt][v], 0.0f};
          p.out[m * NOUT + n] = (uint16_t)(
              __builtin_bit_cast(uint32_t, __builtin_convertvector(pr, bf16x2)) & 0xFFFFu);
        }
      }
    }
}

template <bool BWD>
static hipError_t launch_gemm(const GemmArgs& a, hipStream_t st) {
  static hipError_t attr = hipFuncSetAttribute(
      reinterpret_cast<const void*>(&k_gemm<BWD>), hipFuncAttributeMaxDynamicSharedMemorySize,
      kLdsBytes);
  if (attr != hipSuccess) return attr;
  const int64_t NOUT = BWD ? a.d_in : a.d_out;
  const int64_t tiles = ((NOUT + BN - 1) / BN) * ((a.M + BM - 1) / BM);
  weight_kernel_begin(st);
  hipLaunchKernelGGL(k_gemm<BWD>, dim3((unsigned)tiles), dim3(256), kLdsBytes, st, a);
  weight_kernel_end(st);
  return hipGetLastError();
}

hipError_t launch_gemm_fwd(const GemmArgs& a, hipStream_t st) { return launch_gemm<false>(a, st); }
hipError_t launch_gemm_bwd(const GemmArgs& a, hipStream_t st) { return launch_gemm<true>(a, st); }

}  // namespace qlora
