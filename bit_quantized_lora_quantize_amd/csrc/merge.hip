// merge.hip -- LoRA merge into the restored base weight (gfx950).
//
// [QP] "第 04 篇：QLoRA 原理" §12.3: an adapter is merged by adding s B A to
// the base weight; merging into a 4-bit base restores it, adds the update
// and quantizes again, which rounds once more.  This kernel forms the merged
// weight at FP32 from the restored BF16 weight (the double-dequantized value
// of §2.3 / §6.1) and the rank-r update:
//   Wm[n][k] = RN_fp32( Wh[n][k] + s * sum_i B[n][i] A[i][k] ),
// the right-hand side evaluated in FP64 with the rank index ascending, each
// product and sum rounded on its own.  The products of BF16 values are exact
// in FP64, so the sum is exact but for extreme exponent spreads; one FP32
// rounding remains.  The requantization is the ordinary quantize path.
//
// Mapping: one workgroup per (four rows n, 2048 columns), eight consecutive
// columns of each of the four rows per thread: each rank index brings one
// 16-byte load of A and eight conversions to FP64, shared by the four rows
// (B[n][*] is uniform across the workgroup).  A product of two BF16 values
// is exact in FP64, so the fused multiply-add used for the rank sum rounds
// exactly as a separate product and sum would.
#include "qlora_device.h"
#include "qlora_kernels.h"

namespace qlora {

constexpr int kMergeCols = 8;
constexpr int kMergeRows = 4;
constexpr int kMergeWgCols = 256 * kMergeCols;

__global__ __launch_bounds__(256) void k_merge(MergeArgs a) {
  const int64_t tiles = (a.d_in + kMergeWgCols - 1) / kMergeWgCols;
  const int64_t n0 = (blockIdx.x / tiles) * kMergeRows;
  const int64_t k0 = (blockIdx.x % tiles) * kMergeWgCols + kMergeCols * threadIdx.x;
  if (k0 >= a.d_in) return;                          // d_in is a multiple of 64
  const int rows = a.d_out - n0 < kMergeRows ? (int)(a.d_out - n0) : kMergeRows;
  double acc[kMergeRows][kMergeCols];
#pragma unroll
  for (int r = 0; r < kMergeRows; ++r)
#pragma unroll
    for (int j = 0; j < kMergeCols; ++j) acc[r][j] = 0.0;
  const uint16_t* brow = a.B + n0 * a.r;
  for (int64_t i = 0; i < a.r; ++i) {
    const u32x4 av = *reinterpret_cast<const u32x4*>(a.A + i * a.d_in + k0);
    const uint32_t aw[4] = {av.x, av.y, av.z, av.w};
    double x[kMergeCols];
#pragma unroll
    for (int j = 0; j < kMergeCols; ++j)
      x[j] = (double)__uint_as_float((j & 1) ? (aw[j >> 1] & 0xFFFF0000u) : (aw[j >> 1] << 16));
#pragma unroll
    for (int r = 0; r < kMergeRows; ++r) {
      // rows past d_out multiply by zero and are never stored
      const double bv = r < rows ? (double)__uint_as_float((uint32_t)brow[r * a.r + i] << 16) : 0.0;
#pragma unroll
      for (int j = 0; j < kMergeCols; ++j) acc[r][j] = __fma_rn(bv, x[j], acc[r][j]);
    }
  }
  const float lv[16] = {QLORA_NF4_LEVELS};
#pragma unroll
  for (int r = 0; r < kMergeRows; ++r) {
    if (r >= rows) break;
    const int64_t e0 = (n0 + r) * a.d_in + k0;       // flat index, row-major
    const int64_t b = e0 / kBlock;                   // first-level block (same for all 8)
    const float scale = restored_scale(a.scodes[b], a.scale2[b >> 8], a.mean[0]);
    const uint32_t cw = *reinterpret_cast<const uint32_t*>(a.codes + (e0 >> 1));
    float out[kMergeCols];
#pragma unroll
    for (int j = 0; j < kMergeCols; ++j) {
      const uint32_t idx = (cw >> (4 * j)) & 15u;    // element 2m in the low nibble of byte m
      const float wh = bf16lo_to_f32(pack_bf16x2(__fmul_rn(lv[idx], scale), 0.0f) & 0xFFFFu);
      out[j] = (float)__dadd_rn((double)wh, __dmul_rn((double)a.scale, acc[r][j]));
    }
    float4* dst = reinterpret_cast<float4*>(a.out + e0);
    dst[0] = make_float4(out[0], out[1], out[2], out[3]);
    dst[1] = make_float4(out[4], out[5], out[6], out[7]);
  }
}

hipError_t launch_merge(const MergeArgs& a, hipStream_t st) {
  const int64_t tiles = (a.d_in + kMergeWgCols - 1) / kMergeWgCols;
  const int64_t wgs = (a.d_out + kMergeRows - 1) / kMergeRows * tiles;
  if (wgs > 0x7FFFFFFF) return hipErrorInvalidValue;
  hipLaunchKernelGGL(k_merge, dim3((unsigned)wgs), dim3(256), 0, st, a);
  return hipGetLastError();
}

}  // namespace qlora
