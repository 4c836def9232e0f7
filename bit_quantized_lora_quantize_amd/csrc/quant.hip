// quant.hip -- NF4 blockwise quantization with double quantization of the
// block scales, and double dequantization to BF16 (gfx950).
//
// [QP] "第 04 篇：QLoRA 原理" §3.4 (blockwise absmax), §4.3 (NF4 levels and
// block encoding), §5.2 (second-level quantization of the scales), §6.1
// (restore order); [CP] "QLoRA" concept page, "NF4 量化機制詳解" and "雙重量化".
#include "qlora_device.h"
#include "qlora_kernels.h"

namespace qlora {

// x = w / m for |w| <= m with m in [2^-64, 2^64]: Newton-Raphson division by
// fused multiply-add (Markstein, "IA-64 and Elementary Functions", 2000):
// a refined reciprocal r1 of m, then two correction steps of the quotient.
// These are the steps of the IEEE single-precision division on this GPU
// when neither operand needs scaling; in this range only quotients of
// magnitude below 2^-126 could need it, and those fall in the bucket next
// to 0 whose code does not depend on their exact value (the decision
// thresholds nearest 0 are -0.0455 and 0.0398).
__device__ __forceinline__ float div_for_code(float w, float m) {
  const float r = __builtin_amdgcn_rcpf(m);
  const float r1 = __builtin_fmaf(__builtin_fmaf(-m, r, 1.0f), r, r);
  const float q0 = __fmul_rn(w, r1);
  const float q1 = __builtin_fmaf(__builtin_fmaf(-m, q0, w), r1, q0);
  return __builtin_fmaf(__builtin_fmaf(-m, q1, w), r1, q1);
}

// ---------------------------------------------------------------------------
// First level and group sums: per 64-weight block, absmax, x = w / absmax,
// nearest NF4 level, two indices per byte; per group of kGroup = 256 blocks,
// the FP64 sum of the block absmax values.  One workgroup of 512 threads per
// group (2048 items of 8 weights), every load of the group issued before
// its first encode through a descriptor over the group's bytes (items past
// n1 read zero and are not stored).  Eight lanes own one block (8 FP32
// values each, two 16-byte loads); the block maximum is an exact max over
// the 8 lanes.  The nearest level uses a 129-bucket table over x in
// [-1, 1]: bucket floor(64 x) + 64 is exact (a power-of-two scale), holds at
// most one decision threshold, and gives idx = base + (x >= threshold).
// The group's absmax values also go to LDS, and wavefront 0 forms the
// group's sum by the stride-halving tree (j += j + 128, then j += j + 64,
// ..., j += j + 1; blocks past n1 count 0).  Workgroups of the padding
// groups G .. Gp - 1 write 0.
// ---------------------------------------------------------------------------
constexpr int kEncodeThreads = 512;
constexpr int kEncodeItems = kGroup * 8 / kEncodeThreads;   // items per thread

__global__ __launch_bounds__(kEncodeThreads) void k_absmax_encode(QuantList a, IndexLut lut) {
  __shared__ uint2 s_lut[kLutSize];
  __shared__ float s_am[kGroup];
  const int di = group_index(a.count, (int)blockIdx.x, [&](int i) { return a.d[i].enc_begin; });
  const QuantItem& d = a.d[di];
  const float* __restrict__ W = d.W;
  const int64_t n1 = d.n1, G = d.G;
  uint8_t* __restrict__ codes = d.codes;
  float* __restrict__ absmax = d.absmax;
  double* __restrict__ part = d.part;
  const int64_t g = (int64_t)blockIdx.x - d.enc_begin;
  const int t = threadIdx.x;
  if (g >= G) {
    if (t == 0) part[g] = 0.0;
    return;
  }
  // the decision table first: its loads are waited for before any weight
  // load is in flight
  if (t < kLutSize) s_lut[t] = make_uint2(__float_as_uint(lut.thr[t]), (uint32_t)lut.base[t]);
  const int64_t items = n1 * 8;
  const int64_t c0 = g * (kGroup * 8);
  const int64_t cbytes = (items - c0 < kGroup * 8 ? items - c0 : kGroup * 8) * 32;
  const uint64_t wb = reinterpret_cast<uint64_t>(W + c0 * 8);
  const __amdgpu_buffer_rsrc_t rw = __builtin_amdgcn_make_buffer_rsrc(
      reinterpret_cast<void*>(((uint64_t)(uint32_t)__builtin_amdgcn_readfirstlane((int)(wb >> 32)) << 32) |
                              (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)wb)),
      0, __builtin_amdgcn_readfirstlane((int)cbytes), 0x00020000);
  f32x4 v[kEncodeItems][2];
#pragma unroll
  for (int k = 0; k < kEncodeItems; ++k) {
    const uint32_t off = (uint32_t)(t + kEncodeThreads * k) * 32u;
    v[k][0] = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(rw, off, 0, 0));
    v[k][1] = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(rw, off + 16, 0, 0));
  }
  __syncthreads();
#pragma unroll
  for (int k = 0; k < kEncodeItems; ++k) {
    const int64_t it = c0 + t + kEncodeThreads * k;
    const float w[8] = {v[k][0].x, v[k][0].y, v[k][0].z, v[k][0].w,
                        v[k][1].x, v[k][1].y, v[k][1].z, v[k][1].w};
    float m = 0.0f;
#pragma unroll
    for (int e = 0; e < 8; ++e) m = fmaxf(m, fabsf(w[e]));
    m = fmaxf(m, __shfl_xor(m, 1, 8));
    m = fmaxf(m, __shfl_xor(m, 2, 8));
    m = fmaxf(m, __shfl_xor(m, 4, 8));
    uint32_t packed = 0;
    // the block's lanes take the same branch (m is the block maximum)
    const bool fast = m >= 0x1p-64f && m <= 0x1p64f;
    if (m == 0.0f) {
      packed = 0x77777777u;  // zero block: every element is the exact-zero level
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        float x = fast ? div_for_code(w[e], m) : __fdiv_rn(w[e], m);
        int b = (int)__builtin_floorf(x * 64.0f) + 64;
        b = b < 0 ? 0 : (b > kLutSize - 1 ? kLutSize - 1 : b);  // finite x is in [-1, 1]
        uint2 ent = s_lut[b];
        uint32_t idx = ent.y + (x >= __uint_as_float(ent.x) ? 1u : 0u);
        packed |= idx << (4 * e);
      }
    }
    if (it < items) {
      reinterpret_cast<uint32_t*>(codes)[it] = packed;
      if ((t & 7) == 0) absmax[it >> 3] = m;
    }
    if ((t & 7) == 0) s_am[(t >> 3) + (kEncodeThreads / 8) * k] = m;   // 0 past n1
  }
  __syncthreads();
  if (t < 64) {
    double d[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int64_t b = g * kGroup + t + 64 * q;
      d[q] = (b < n1) ? (double)s_am[t + 64 * q] : 0.0;
    }
    d[0] = d[0] + d[2];  // half = 128
    d[1] = d[1] + d[3];
    d[0] = d[0] + d[1];  // half = 64
#pragma unroll
    for (int half = 32; half >= 1; half >>= 1) {
      double o = __shfl_down(d[0], half, 64);
      d[0] = d[0] + o;
    }
    if (t == 0) part[g] = d[0];
  }
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

// Mean and second level.  Wavefront 0 of every workgroup adds the len group
// sums (len a power of two, <= kTreeLds) by the stride-halving tree, the
// same additions in the same order as k_tree_final: element j sits in lane
// j % 64, register j / 64, so the levels with half >= 64 add registers
// within a lane and the last six add across lanes.  Every workgroup thus
// holds the same mean (workgroup 0 stores it).  Then each wavefront encodes
// kScaleGroups groups, g = kScaleGroups (4 blockIdx + w) + i: centred
// d = a - mean, s2 = max|d| / 448, code = FP8 E4M3FN(d / s2) (RNE,
// saturating); s2 == 0 stores code 0.  The groups' absmax values are loaded
// before the tree.
constexpr int kScaleGroups = 4;
constexpr int kTreeRegs = kTreeLds / 64;

__global__ __launch_bounds__(256) void k_mean_scale_dq(QuantList a) {
  __shared__ float s_mean;
  const int di = group_index(a.count, (int)blockIdx.x, [&](int i) { return a.d[i].scale_begin; });
  const QuantItem& d = a.d[di];
  const double* __restrict__ part = d.part;
  const float* __restrict__ absmax = d.absmax;
  const int64_t len = d.len, n1 = d.n1, G = d.G;
  float* __restrict__ mean_out = d.mean;
  uint8_t* __restrict__ scale_codes = d.scale_codes;
  float* __restrict__ scale2 = d.scale2;
  const int64_t wg = (int64_t)blockIdx.x - d.scale_begin;
  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int64_t g0 = (wg * 4 + w) * kScaleGroups;
  float am[kScaleGroups][4];
#pragma unroll
  for (int i = 0; i < kScaleGroups; ++i)
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int64_t b = (g0 + i) * kGroup + lane + 64 * q;
      am[i][q] = (g0 + i < G && b < n1) ? absmax[b] : 0.0f;
    }
  if (w == 0) {
    double v[kTreeRegs];
#pragma unroll
    for (int i = 0; i < kTreeRegs; ++i) v[i] = (lane + 64 * i < len) ? part[lane + 64 * i] : 0.0;
#pragma unroll
    for (int h = kTreeRegs / 2; h >= 1; h /= 2) {
      if (len >= 128 * h) {
#pragma unroll
        for (int i = 0; i < h; ++i) v[i] = v[i] + v[i + h];
      }
    }
#pragma unroll
    for (int half = 32; half >= 1; half >>= 1) {
      const double o = __shfl_down(v[0], half, 64);
      if (len >= 2 * half) v[0] = v[0] + o;
    }
    if (lane == 0) {
      const float mean = (float)(v[0] / (double)n1);
      s_mean = mean;
      if (wg == 0) mean_out[0] = mean;
    }
  }
  __syncthreads();
  const float mean = s_mean;
#pragma unroll
  for (int i = 0; i < kScaleGroups; ++i) {
    const int64_t g = g0 + i;
    if (g >= G) break;
    float dv[4];
    float mg = 0.0f;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const bool ok = (g * kGroup + lane + 64 * q) < n1;
      dv[q] = ok ? __fsub_rn(am[i][q], mean) : 0.0f;
      mg = fmaxf(mg, fabsf(dv[q]));
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) mg = fmaxf(mg, __shfl_xor(mg, off, 64));
    const float s2 = __fdiv_rn(mg, 448.0f);
    if (lane == 0) scale2[g] = s2;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int64_t b = g * kGroup + lane + 64 * q;
      if (b >= n1) continue;
      const uint32_t code = (s2 == 0.0f) ? 0u : f32_to_fp8e4m3_rne_sat(__fdiv_rn(dv[q], s2));
      scale_codes[b] = (uint8_t)code;
    }
  }
}

// ---------------------------------------------------------------------------
// Double dequantization to BF16: restored scale fp8(code) * s2 + mean,
// 16-entry BF16 table RNE(level_i * scale), byte-permute lookups of eight
// weights per lane.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void k_dequant_bf16(DequantList a) {
  // One code dword (eight weights, 16 output bytes) per thread: eight
  // consecutive threads share a block (each builds its table), and a
  // wavefront reads 256 contiguous code bytes and writes 1 KB of contiguous
  // output, so every store fills whole cache lines.  A tensor's workgroups
  // stride over its units.
  const int di = group_index(a.count, (int)blockIdx.x, [&](int i) { return a.d[i].begin; });
  const DequantItem& d = a.d[di];
  const uint8_t* __restrict__ scale_codes = d.scale_codes;
  const float* __restrict__ scale2 = d.scale2;
  const float mean = d.mean[0];
  const int64_t nunits = d.n1 * 8;
  const int64_t stride = (int64_t)d.wgs * blockDim.x;
  const uint32_t* cw = reinterpret_cast<const uint32_t*>(d.codes);
  u32x4* ov = reinterpret_cast<u32x4*>(d.out);
  for (int64_t u = (int64_t)(blockIdx.x - d.begin) * blockDim.x + threadIdx.x; u < nunits;
       u += stride) {
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

QuantItem quant_item(const float* W, int64_t n, uint8_t* codes, uint8_t* scale_codes,
                     float* scale2, float* mean, const QuantWorkspace& ws) {
  QuantItem d{};
  d.W = W;
  d.n1 = n / kBlock;
  d.G = (d.n1 + kGroup - 1) / kGroup;
  d.Gp = 1;
  while (d.Gp < d.G) d.Gp *= 2;
  d.codes = codes;
  d.scale_codes = scale_codes;
  d.scale2 = scale2;
  d.mean = mean;
  d.absmax = ws.absmax;
  d.part = ws.part;
  return d;
}

hipError_t launch_quantize_list(QuantList& a, const IndexLut& lut, hipStream_t st) {
  // encode with the group sums (Gp workgroups per tensor), the tree levels
  // above kTreeLds one launch each, then the last levels fused with the
  // second-level encode
  int enc = 0, sc = 0;
  for (int i = 0; i < a.count; ++i) {
    QuantItem& d = a.d[i];
    d.enc_begin = enc;
    d.scale_begin = sc;
    enc += (int)d.Gp;
    sc += (int)((d.G + 4 * kScaleGroups - 1) / (4 * kScaleGroups));
    d.len = d.Gp;
  }
  a.enc_wgs = enc;
  a.scale_wgs = sc;
  weight_kernel_begin(st);
  hipLaunchKernelGGL(k_absmax_encode, dim3((unsigned)enc), dim3(kEncodeThreads), 0, st, a, lut);
  weight_kernel_end(st);
  for (int i = 0; i < a.count; ++i) {
    QuantItem& d = a.d[i];
    while (d.len > kTreeLds) {
      const int64_t half = d.len / 2;
      hipLaunchKernelGGL(k_tree_level, dim3((unsigned)((half + 255) / 256)), dim3(256), 0, st,
                         d.part, half);
      d.len = half;
    }
  }
  hipLaunchKernelGGL(k_mean_scale_dq, dim3((unsigned)sc), dim3(256), 0, st, a);
  return hipGetLastError();
}

hipError_t launch_quantize(const float* W, int64_t n, uint8_t* codes, uint8_t* scale_codes,
                           float* scale2, float* mean, const QuantWorkspace& ws,
                           const IndexLut& lut, hipStream_t st) {
  QuantList a{};
  a.count = 1;
  a.d[0] = quant_item(W, n, codes, scale_codes, scale2, mean, ws);
  return launch_quantize_list(a, lut, st);
}

hipError_t launch_dequant_list(DequantList& a, hipStream_t st) {
  int wgs = 0;
  for (int i = 0; i < a.count; ++i) {
    DequantItem& d = a.d[i];
    d.wgs = grid_for(d.n1 * 8, 256, 8192);
    d.begin = wgs;
    wgs += d.wgs;
  }
  a.wgs = wgs;
  weight_kernel_begin(st);
  hipLaunchKernelGGL(k_dequant_bf16, dim3((unsigned)wgs), dim3(256), 0, st, a);
  weight_kernel_end(st);
  return hipGetLastError();
}

hipError_t launch_dequant(const uint8_t* codes, const uint8_t* scale_codes, const float* scale2,
                          const float* mean, int64_t n, uint16_t* out, hipStream_t st) {
  DequantList a{};
  a.count = 1;
  a.d[0] = DequantItem{codes, scale_codes, scale2, mean, n / kBlock, out, 0, 0};
  return launch_dequant_list(a, st);
}

}  // namespace qlora
