// quant.hip -- NF4 blockwise quantization with double quantization of the
// block scales, and double dequantization to BF16 (gfx950).
//
// [QP] "第 04 篇：QLoRA 原理" §3.4 (blockwise absmax), §4.3 (NF4 levels and
// block encoding), §5.2 (second-level quantization of the scales), §6.1
// (restore order); [CP] "QLoRA" concept page, "NF4 量化機制詳解" and "雙重量化".
#include "qlora_device.h"
#include "qlora_kernels.h"

namespace qlora {

// ---------------------------------------------------------------------------
// Kernel 1: per 64-weight block, absmax, x = w / absmax, nearest NF4 level,
// two indices per byte.  Eight lanes own one block (8 FP32 values each, two
// 16-byte loads); the block maximum is an exact max over the 8 lanes.
// The nearest level uses a 129-bucket table over x in [-1, 1]: bucket
// floor(64 x) + 64 is exact (a power-of-two scale), holds at most one
// decision threshold, and gives idx = base + (x >= threshold).
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void k_absmax_encode(const float* __restrict__ W,
                                                       int64_t n1,
                                                       uint8_t* __restrict__ codes,
                                                       float* __restrict__ absmax,
                                                       IndexLut lut) {
  __shared__ uint2 s_lut[kLutSize];
  for (int i = threadIdx.x; i < kLutSize; i += blockDim.x)
    s_lut[i] = make_uint2(__float_as_uint(lut.thr[i]), (uint32_t)lut.base[i]);
  __syncthreads();

  const int64_t items = n1 * 8;
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t it = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; it < items; it += stride) {
    const f32x4* p = reinterpret_cast<const f32x4*>(W + it * 8);
    f32x4 v0 = __builtin_nontemporal_load(p);
    f32x4 v1 = __builtin_nontemporal_load(p + 1);
    float w[8] = {v0.x, v0.y, v0.z, v0.w, v1.x, v1.y, v1.z, v1.w};
    float m = 0.0f;
#pragma unroll
    for (int e = 0; e < 8; ++e) m = fmaxf(m, fabsf(w[e]));
    m = fmaxf(m, __shfl_xor(m, 1, 8));
    m = fmaxf(m, __shfl_xor(m, 2, 8));
    m = fmaxf(m, __shfl_xor(m, 4, 8));
    uint32_t packed = 0;
    if (m == 0.0f) {
      packed = 0x77777777u;  // zero block: every element is the exact-zero level
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        float x = __fdiv_rn(w[e], m);
        int b = (int)__builtin_floorf(x * 64.0f) + 64;
        b = b < 0 ? 0 : (b > kLutSize - 1 ? kLutSize - 1 : b);  // finite x is in [-1, 1]
        uint2 ent = s_lut[b];
        uint32_t idx = ent.y + (x >= __uint_as_float(ent.x) ? 1u : 0u);
        packed |= idx << (4 * e);
      }
    }
    reinterpret_cast<uint32_t*>(codes)[it] = packed;
    if ((it & 7) == 0) absmax[it >> 3] = m;
  }
}

// ---------------------------------------------------------------------------
// Kernel 2: FP64 sum of each group of 256 absmax values by the stride-halving
// tree (j += j+128, then j += j+64, ... , j += j+1), one wavefront per group.
// Groups past the last real one are written as 0 up to the padded count.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void k_group_sums(const float* __restrict__ absmax, int64_t n1,
                                                    int64_t G, int64_t Gp,
                                                    double* __restrict__ part) {
  const int lane = threadIdx.x & 63;
  const int64_t g = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (g >= Gp) return;
  if (g >= G) {
    if (lane == 0) part[g] = 0.0;
    return;
  }
  double v[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    int64_t b = g * kGroup + lane + 64 * q;
    v[q] = (b < n1) ? (double)absmax[b] : 0.0;
  }
  v[0] = v[0] + v[2];  // half = 128
  v[1] = v[1] + v[3];
  v[0] = v[0] + v[1];  // half = 64
#pragma unroll
  for (int half = 32; half >= 1; half >>= 1) {
    double o = __shfl_down(v[0], half, 64);
    v[0] = v[0] + o;
  }
  if (lane == 0) part[g] = v[0];
}

// One level of the stride-halving tree over a power-of-two array in global
// memory: v[j] += v[j + half] for j < half.
__global__ __launch_bounds__(256) void k_tree_level(double* __restrict__ v, int64_t half) {
  int64_t j = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (j < half) v[j] = v[j] + v[j + half];
}

// The remaining levels (len <= kTreeLds, power of two) in one workgroup, then
// mean = FP32(S / n1).
__global__ __launch_bounds__(1024) void k_tree_final(const double* __restrict__ v, int64_t len,
                                                     int64_t n1, float* __restrict__ mean) {
  __shared__ double s[kTreeLds];
  for (int64_t j = threadIdx.x; j < len; j += blockDim.x) s[j] = v[j];
  __syncthreads();
  for (int64_t half = len / 2; half >= 1; half /= 2) {
    for (int64_t j = threadIdx.x; j < half; j += blockDim.x) s[j] = s[j] + s[j + half];
    __syncthreads();
  }
  if (threadIdx.x == 0) mean[0] = (float)(s[0] / (double)n1);
}

// ---------------------------------------------------------------------------
// Kernel 3: second level.  One wavefront per group of 256 scales: centred
// d = a - mean, s2 = max|d| / 448, code = FP8 E4M3FN(d / s2) (RNE, saturating);
// s2 == 0 stores code 0.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void k_scale_dq(const float* __restrict__ absmax, int64_t n1,
                                                  int64_t G, const float* __restrict__ mean_p,
                                                  uint8_t* __restrict__ scale_codes,
                                                  float* __restrict__ scale2) {
  const int lane = threadIdx.x & 63;
  const int64_t g = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (g >= G) return;
  const float mean = mean_p[0];
  float d[4];
  bool ok[4];
  float mg = 0.0f;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    int64_t b = g * kGroup + lane + 64 * q;
    ok[q] = b < n1;
    d[q] = ok[q] ? __fsub_rn(absmax[b], mean) : 0.0f;
    mg = fmaxf(mg, fabsf(d[q]));
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) mg = fmaxf(mg, __shfl_xor(mg, off, 64));
  const float s2 = __fdiv_rn(mg, 448.0f);
  if (lane == 0) scale2[g] = s2;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    if (!ok[q]) continue;
    uint32_t code = (s2 == 0.0f) ? 0u : f32_to_fp8e4m3_rne_sat(__fdiv_rn(d[q], s2));
    scale_codes[g * kGroup + lane + 64 * q] = (uint8_t)code;
  }
}

// ---------------------------------------------------------------------------
// Double dequantization to BF16: restored scale fp8(code) * s2 + mean,
// 16-entry BF16 table RNE(level_i * scale), byte-permute lookups of eight
// weights per lane.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void k_dequant_bf16(const uint8_t* __restrict__ codes,
                                                      const uint8_t* __restrict__ scale_codes,
                                                      const float* __restrict__ scale2,
                                                      const float* __restrict__ mean_p,
                                                      int64_t n1, uint16_t* __restrict__ out) {
  // One code dword (eight weights, 16 output bytes) per thread: eight
  // consecutive threads share a block (each builds its table), and a
  // wavefront reads 256 contiguous code bytes and writes 1 KB of contiguous
  // output, so every store fills whole cache lines.
  const float mean = mean_p[0];
  const int64_t nunits = n1 * 8;
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  const uint32_t* cw = reinterpret_cast<const uint32_t*>(codes);
  u32x4* ov = reinterpret_cast<u32x4*>(out);
  for (int64_t u = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; u < nunits; u += stride) {
    const int64_t b = u >> 3;
    const uint32_t c = __builtin_nontemporal_load(cw + u);
    const Nf4Table t = nf4_table(restored_scale(scale_codes[b], scale2[b >> 8], mean));
    __builtin_nontemporal_store(nf4_dequant8(c, t), ov + u);
  }
}

// ---------------------------------------------------------------------------
// Host launchers
// ---------------------------------------------------------------------------
int grid_for(int64_t work, int per_block, int max_blocks) {
  int64_t g = (work + per_block - 1) / per_block;
  if (g < 1) g = 1;
  if (g > max_blocks) g = max_blocks;
  return (int)g;
}

void launch_mean_tree(double* part, int64_t Gp, int64_t n1, float* mean, hipStream_t st) {
  int64_t len = Gp;
  while (len > kTreeLds) {
    int64_t half = len / 2;
    hipLaunchKernelGGL(k_tree_level, dim3((unsigned)((half + 255) / 256)), dim3(256), 0, st,
                       part, half);
    len = half;
  }
  hipLaunchKernelGGL(k_tree_final, dim3(1), dim3(1024), 0, st, part, len, n1, mean);
}

hipError_t launch_quantize(const float* W, int64_t n, uint8_t* codes, uint8_t* scale_codes,
                           float* scale2, float* mean, const QuantWorkspace& ws,
                           const IndexLut& lut, hipStream_t st) {
  const int64_t n1 = n / kBlock;
  const int64_t G = (n1 + kGroup - 1) / kGroup;
  int64_t Gp = 1;
  while (Gp < G) Gp *= 2;
  weight_kernel_begin(st);
  hipLaunchKernelGGL(k_absmax_encode, dim3(grid_for(n1 * 8, 256, 8192)), dim3(256), 0, st, W,
                     n1, codes, ws.absmax, lut);
  weight_kernel_end(st);
  hipLaunchKernelGGL(k_group_sums, dim3((unsigned)((Gp + 3) / 4)), dim3(256), 0, st, ws.absmax,
                     n1, G, Gp, ws.part);
  launch_mean_tree(ws.part, Gp, n1, mean, st);
  hipLaunchKernelGGL(k_scale_dq, dim3((unsigned)((G + 3) / 4)), dim3(256), 0, st, ws.absmax, n1,
                     G, mean, scale_codes, scale2);
  return hipGetLastError();
}

hipError_t launch_dequant(const uint8_t* codes, const uint8_t* scale_codes, const float* scale2,
                          const float* mean, int64_t n, uint16_t* out, hipStream_t st) {
  const int64_t n1 = n / kBlock;
  weight_kernel_begin(st);
  hipLaunchKernelGGL(k_dequant_bf16, dim3(grid_for(n1 * 8, 256, 8192)), dim3(256), 0, st, codes,
                     scale_codes, scale2, mean, n1, out);
  weight_kernel_end(st);
  return hipGetLastError();
}

}  // namespace qlora
