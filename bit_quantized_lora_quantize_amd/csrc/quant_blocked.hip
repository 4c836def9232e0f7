// quant_blocked.hip -- NF4 double quantization and dequantization at general
// block sizes, for any element count (gfx950).
//
// [QP] "第 04 篇：QLoRA 原理" §5.5: the first-level block size B1 trades
// scale metadata (about 8 / B1 bits per weight after double quantization)
// against error (a smaller block localizes the range and outliers); the
// second-level group size B2 makes the same trade for the scales.  §3.4:
// blocks are runs of the flattened tensor.  The layer format (B1 = 64,
// B2 = 256, rows a multiple of 64) has its own kernels; these take B1 a
// power of two in 32..4096, B2 a power of two in 16..1024 and any n: a
// short last block takes the absmax of the elements it has, a short last
// group likewise, and for odd n the unused high nibble of the last byte is 0.
// Arithmetic and decisions are those of the layer format: IEEE division by
// the absmax, nearest level with ties to the lower index, centred scales in
// FP8 E4M3FN against the group's max / 448, the mean by the stride-halving
// FP64 tree (groups of B2, then the padded group sums).
#include "qlora_device.h"
#include "qlora_kernels.h"

namespace qlora {

// ---------------------------------------------------------------------------
// First level.  A block is handled by a group of L = min(B1 / 8, 64) lanes,
// each lane taking C = max(1, B1 / 512) chunks of eight consecutive elements
// (chunk c of lane l covers elements 8 (c L + l) .. + 8 of the block), so
// every load instruction of a wavefront reads contiguous memory.  Groups are
// aligned within a wavefront and iterate together, so the max reduction
// (xor shuffles below L) never reads an inactive lane.
// ---------------------------------------------------------------------------
template <int C>
__global__ __launch_bounds__(256) void k_absmax_encode_blocked(const float* __restrict__ W,
                                                               int64_t n, int64_t B1, int L,
                                                               uint8_t* __restrict__ codes,
                                                               float* __restrict__ absmax,
                                                               IndexLut lut) {
  __shared__ uint2 s_lut[kLutSize];
  for (int i = threadIdx.x; i < kLutSize; i += blockDim.x)
    s_lut[i] = make_uint2(__float_as_uint(lut.thr[i]), (uint32_t)lut.base[i]);
  __syncthreads();

  const int64_t n1 = (n + B1 - 1) / B1;
  const int64_t gl = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int l = (int)(gl % L);
  const int64_t stride = (int64_t)gridDim.x * blockDim.x / L;
  for (int64_t b = gl / L; b < n1; b += stride) {
    float w[C][8];
    float m = 0.0f;
#pragma unroll
    for (int c = 0; c < C; ++c) {
      const int64_t e = b * B1 + 8 * ((int64_t)c * L + l);
      if (e + 8 <= n) {
        const f32x4* p = reinterpret_cast<const f32x4*>(W + e);
        const f32x4 v0 = __builtin_nontemporal_load(p);
        const f32x4 v1 = __builtin_nontemporal_load(p + 1);
        w[c][0] = v0.x; w[c][1] = v0.y; w[c][2] = v0.z; w[c][3] = v0.w;
        w[c][4] = v1.x; w[c][5] = v1.y; w[c][6] = v1.z; w[c][7] = v1.w;
      } else {
#pragma unroll
        for (int j = 0; j < 8; ++j) w[c][j] = (e + j < n) ? W[e + j] : 0.0f;
      }
#pragma unroll
      for (int j = 0; j < 8; ++j) m = fmaxf(m, fabsf(w[c][j]));
    }
    for (int o = 1; o < L; o <<= 1) m = fmaxf(m, __shfl_xor(m, o, 64));
#pragma unroll
    for (int c = 0; c < C; ++c) {
      const int64_t e = b * B1 + 8 * ((int64_t)c * L + l);
      if (e >= n) continue;
      uint32_t packed = 0;
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        uint32_t idx = 7u;  // zero block: the exact-zero level
        if (m != 0.0f) {
          const float x = __fdiv_rn(w[c][j], m);
          int bk = (int)__builtin_floorf(x * 64.0f) + 64;
          bk = bk < 0 ? 0 : (bk > kLutSize - 1 ? kLutSize - 1 : bk);
          const uint2 ent = s_lut[bk];
          idx = ent.y + (x >= __uint_as_float(ent.x) ? 1u : 0u);
        }
        if (e + j < n) packed |= idx << (4 * j);
      }
      if (e + 8 <= n) {
        reinterpret_cast<uint32_t*>(codes)[e >> 3] = packed;
      } else {
        // short tail: the bytes that hold at least one element
        for (int j = 0; j < 4; ++j)
          if (e + 2 * j < n) codes[(e >> 1) + j] = (uint8_t)(packed >> (8 * j));
      }
    }
    if (l == 0) absmax[b] = m;
  }
}

// ---------------------------------------------------------------------------
// Mean: FP64 sum of each group of B2 scales by the stride-halving tree, one
// wavefront per group.  A lane holds Q = max(1, B2 / 64) values, v[q] =
// a[g B2 + lane + 64 q]; the levels above 32 pair registers of one lane,
// the rest pair lanes.  Groups past the last real one are written as 0.
// ---------------------------------------------------------------------------
template <int Q>
__global__ __launch_bounds__(256) void k_group_sums_blocked(const float* __restrict__ absmax,
                                                            int64_t n1, int64_t B2, int64_t G,
                                                            int64_t Gp, double* __restrict__ part) {
  const int lane = threadIdx.x & 63;
  const int64_t g = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (g >= Gp) return;
  if (g >= G) {
    if (lane == 0) part[g] = 0.0;
    return;
  }
  double v[Q];
#pragma unroll
  for (int q = 0; q < Q; ++q) {
    const int64_t j = lane + 64 * q;
    const int64_t b = g * B2 + j;
    v[q] = (j < B2 && b < n1) ? (double)absmax[b] : 0.0;
  }
#pragma unroll
  for (int h = Q / 2; h >= 1; h /= 2)
#pragma unroll
    for (int q = 0; q < h; ++q) v[q] = __dadd_rn(v[q], v[q + h]);
  const int top = B2 < 64 ? (int)B2 : 64;
  for (int half = top / 2; half >= 1; half >>= 1) v[0] = __dadd_rn(v[0], __shfl_down(v[0], half, 64));
  if (lane == 0) part[g] = v[0];
}

// ---------------------------------------------------------------------------
// Second level: one wavefront per group of B2 scales; d = a - mean, s2 =
// max|d| / 448, code = FP8 E4M3FN(d / s2) (RNE, saturating), 0 when s2 = 0.
// ---------------------------------------------------------------------------
template <int Q>
__global__ __launch_bounds__(256) void k_scale_dq_blocked(const float* __restrict__ absmax,
                                                          int64_t n1, int64_t B2, int64_t G,
                                                          const float* __restrict__ mean_p,
                                                          uint8_t* __restrict__ scale_codes,
                                                          float* __restrict__ scale2) {
  const int lane = threadIdx.x & 63;
  const int64_t g = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (g >= G) return;
  const float mean = mean_p[0];
  float d[Q];
  bool ok[Q];
  float mg = 0.0f;
#pragma unroll
  for (int q = 0; q < Q; ++q) {
    const int64_t j = lane + 64 * q;
    const int64_t b = g * B2 + j;
    ok[q] = j < B2 && b < n1;
    d[q] = ok[q] ? __fsub_rn(absmax[b], mean) : 0.0f;
    mg = fmaxf(mg, fabsf(d[q]));
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) mg = fmaxf(mg, __shfl_xor(mg, off, 64));
  const float s2 = __fdiv_rn(mg, 448.0f);
  if (lane == 0) scale2[g] = s2;
#pragma unroll
  for (int q = 0; q < Q; ++q) {
    if (!ok[q]) continue;
    const uint32_t code = (s2 == 0.0f) ? 0u : f32_to_fp8e4m3_rne_sat(__fdiv_rn(d[q], s2));
    scale_codes[g * B2 + lane + 64 * q] = (uint8_t)code;
  }
}

// ---------------------------------------------------------------------------
// Dequantization: one code dword (eight weights, one block since B1 >= 32)
// per thread; the short tail reads its bytes and writes its elements singly.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void k_dequant_blocked(const uint8_t* __restrict__ codes,
                                                         const uint8_t* __restrict__ scale_codes,
                                                         const float* __restrict__ scale2,
                                                         const float* __restrict__ mean_p,
                                                         int64_t n, int sh1, int sh2,
                                                         uint16_t* __restrict__ out) {
  const float mean = mean_p[0];
  const int64_t units = (n + 7) / 8;
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t u = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; u < units; u += stride) {
    const int64_t e = 8 * u;
    const int64_t b = e >> sh1;
    const Nf4Table t = nf4_table(restored_scale(scale_codes[b], scale2[b >> sh2], mean));
    if (e + 8 <= n) {
      const uint32_t c = __builtin_nontemporal_load(reinterpret_cast<const uint32_t*>(codes) + u);
      __builtin_nontemporal_store(nf4_dequant8(c, t), reinterpret_cast<u32x4*>(out) + u);
    } else {
      uint32_t c = 0;
      for (int j = 0; j < 4; ++j)
        if (e + 2 * j < n) c |= (uint32_t)codes[(e >> 1) + j] << (8 * j);
      const u32x4 v = nf4_dequant8(c, t);
      const uint32_t wv[4] = {v.x, v.y, v.z, v.w};
      for (int j = 0; j < 8; ++j)
        if (e + j < n) out[e + j] = (uint16_t)(wv[j >> 1] >> (16 * (j & 1)));
    }
  }
}

static int log2i(int64_t v) {
  int s = 0;
  while ((int64_t(1) << s) < v) ++s;
  return s;
}

template <int Q>
static void launch_second_level(const BlockedQuant& q, int64_t n1, int64_t G, int64_t Gp,
                                hipStream_t st) {
  hipLaunchKernelGGL(k_group_sums_blocked<Q>, dim3((unsigned)((Gp + 3) / 4)), dim3(256), 0, st,
                     q.absmax, n1, q.group, G, Gp, q.part);
  launch_mean_tree(q.part, Gp, n1, q.mean, st);
  hipLaunchKernelGGL(k_scale_dq_blocked<Q>, dim3((unsigned)((G + 3) / 4)), dim3(256), 0, st,
                     q.absmax, n1, q.group, G, q.mean, q.scale_codes, q.scale2);
}

hipError_t launch_quantize_blocked(const BlockedQuant& q, const IndexLut& lut, hipStream_t st) {
  const int64_t n1 = (q.n + q.block - 1) / q.block;
  const int64_t G = (n1 + q.group - 1) / q.group;
  int64_t Gp = 1;
  while (Gp < G) Gp *= 2;
  const int C = q.block > 512 ? (int)(q.block / 512) : 1;
  const int L = (int)(q.block / (8 * C));
  const int grid = grid_for(n1 * L, 256, 8192);
  switch (C) {
    case 1:
      hipLaunchKernelGGL(k_absmax_encode_blocked<1>, dim3(grid), dim3(256), 0, st, q.W, q.n,
                         q.block, L, q.codes, q.absmax, lut);
      break;
    case 2:
      hipLaunchKernelGGL(k_absmax_encode_blocked<2>, dim3(grid), dim3(256), 0, st, q.W, q.n,
                         q.block, L, q.codes, q.absmax, lut);
      break;
    case 4:
      hipLaunchKernelGGL(k_absmax_encode_blocked<4>, dim3(grid), dim3(256), 0, st, q.W, q.n,
                         q.block, L, q.codes, q.absmax, lut);
      break;
    default:
      hipLaunchKernelGGL(k_absmax_encode_blocked<8>, dim3(grid), dim3(256), 0, st, q.W, q.n,
                         q.block, L, q.codes, q.absmax, lut);
      break;
  }
  switch (q.group <= 64 ? 1 : (int)(q.group / 64)) {
    case 1: launch_second_level<1>(q, n1, G, Gp, st); break;
    case 2: launch_second_level<2>(q, n1, G, Gp, st); break;
    case 4: launch_second_level<4>(q, n1, G, Gp, st); break;
    case 8: launch_second_level<8>(q, n1, G, Gp, st); break;
    default: launch_second_level<16>(q, n1, G, Gp, st); break;
  }
  return hipGetLastError();
}

hipError_t launch_dequant_blocked(const uint8_t* codes, const uint8_t* scale_codes,
                                  const float* scale2, const float* mean, int64_t n,
                                  int64_t block, int64_t group, uint16_t* out, hipStream_t st) {
  hipLaunchKernelGGL(k_dequant_blocked, dim3(grid_for((n + 7) / 8, 256, 8192)), dim3(256), 0, st,
                     codes, scale_codes, scale2, mean, n, log2i(block), log2i(group), out);
  return hipGetLastError();
}

}  // namespace qlora
