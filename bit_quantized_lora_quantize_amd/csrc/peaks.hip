// peaks.hip -- measurement aid, not part of libqlora: two microbenchmarks
// that give the peaks this GPU actually reaches, reported beside the
// published figures (8 TB/s HBM, 2.5 PFLOP/s dense BF16 MFMA).  Built as
// libqlora_peaks.so; only the benchmark loads it.
//
//   qlora_peak_stream_read  every byte of a device buffer read once with
//                           16-byte loads, four in flight per thread; the
//                           result feeds a store that never happens, so the
//                           loads cannot be dropped;
//   qlora_peak_mfma         back-to-back v_mfma_f32_32x32x16_bf16 on register
//                           operands, four independent accumulators per
//                           wavefront, no memory traffic in the loop.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kThreads = 256;
constexpr int kUnroll = 4;

__global__ __launch_bounds__(kThreads) void k_stream_read(const u32x4* __restrict__ p, int64_t n16,
                                                          uint32_t* sink) {
  const int64_t stride = (int64_t)gridDim.x * kThreads;
  int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  u32x4 acc = {0u, 0u, 0u, 0u};
  for (; i + (kUnroll - 1) * stride < n16; i += kUnroll * stride) {
    u32x4 v[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) v[u] = p[i + u * stride];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) acc ^= v[u];
  }
  for (; i < n16; i += stride) acc ^= p[i];
  if ((acc.x & acc.y & acc.z & acc.w) == 0xFFFFFFFFu) sink[blockIdx.x] = acc.x;  // never true for the zero buffer
}

__global__ __launch_bounds__(kThreads) void k_mfma(float* sink, int iters) {
  const uint32_t t = threadIdx.x;
  u32x4 ai = {t, t + 1u, t + 2u, t + 3u}, bi = {t ^ 5u, t ^ 6u, t ^ 7u, t ^ 8u};
  ai &= 0x3F803F80u;                      // small BF16 values (0 or 1)
  bi &= 0x3F803F80u;
  const bf16x8 a = __builtin_bit_cast(bf16x8, ai), b = __builtin_bit_cast(bf16x8, bi);
  f32x16 c0 = {}, c1 = {}, c2 = {}, c3 = {};
  for (int i = 0; i < iters; ++i) {
    c0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c0, 0, 0, 0);
    c1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c1, 0, 0, 0);
    c2 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c2, 0, 0, 0);
    c3 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c3, 0, 0, 0);
  }
  float s = 0.0f;
#pragma unroll
  for (int e = 0; e < 16; ++e) s += c0[e] + c1[e] + c2[e] + c3[e];
  if (s == -1.0f) sink[blockIdx.x * kThreads + t] = s;     // sums of products of 0/1: never -1
}

}  // namespace

extern "C" {

// Reads bytes (a multiple of 16, 16-byte aligned) of `buf` once; sink holds
// at least `workgroups` words.  Returns a hipError_t value.
int qlora_peak_stream_read(const void* buf, int64_t bytes, uint32_t* sink, int workgroups,
                           void* stream) {
  if (!buf || !sink || bytes <= 0 || (bytes & 15) || workgroups < 1) return (int)hipErrorInvalidValue;
  hipLaunchKernelGGL(k_stream_read, dim3(workgroups), dim3(kThreads), 0,
                     static_cast<hipStream_t>(stream), static_cast<const u32x4*>(buf), bytes / 16,
                     sink);
  return (int)hipGetLastError();
}

// workgroups x 4 wavefronts, each iters x 4 MFMAs of 32 x 32 x 16 (2 x 16384
// FLOP each); sink holds at least workgroups x 256 floats.
int qlora_peak_mfma(float* sink, int workgroups, int iters, void* stream) {
  if (!sink || workgroups < 1 || iters < 1) return (int)hipErrorInvalidValue;
  hipLaunchKernelGGL(k_mfma, dim3(workgroups), dim3(kThreads), 0, static_cast<hipStream_t>(stream),
                     sink, iters);
  return (int)hipGetLastError();
}

}  // extern "C"
