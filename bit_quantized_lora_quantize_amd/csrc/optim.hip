// optim.hip -- the optimizer step on the LoRA factors (gfx950).
//
// [QP] "第 04 篇：QLoRA 原理" §7.3: AdamW keeps a first and a second moment
// per trainable parameter, in 32-bit (the paged variant changes where the
// states live, not what they are); §10.2: the gradients may be clipped by
// their global norm before the step.  Only the LoRA factors train, so the
// step touches A and B alone.
//
// Global norm: S = sum over tensors (list order, FP64) of S_t, each S_t the
// FP64 sum of the squared gradients (exact squares of FP32 values) taken in
// groups of 256 by the stride-halving tree and then by the same tree over
// the group sums padded with zeros to a power of two -- the same fixed
// order as the scale mean of the quantizer, so the result does not depend
// on the launch shape.
//
// AdamW (decoupled weight decay), per element, FP32, every operation
// rounded on its own in this order:
//   g  = g * c                          (c: clip coefficient, 1 without)
//   p  = p - lrwd * p                   (lrwd = lr * wd)
//   m  = b1 * m + ob1 * g               (ob1 = 1 - b1)
//   v  = b2 * v + ob2 * (g * g)         (ob2 = 1 - b2)
//   p  = p - lr * ((m / bc1) / (sqrt(v / bc2) + eps))
//   p16 = RNE_bf16(p)                   (optional compute copy)
// with bc_i = 1 - b_i^t; the scalar terms come in from the host.
#include "qlora_device.h"
#include "qlora_kernels.h"

namespace qlora {

namespace {

// Up to kOptBatch tensors of one sum-of-squares launch.  Tensor t owns
// part[poff[t] .. poff[t] + gp[t]) and the workgroups [blk_end[t-1],
// blk_end[t]) of the group launch (four groups per workgroup).
struct SumsqBatch {
  const float* g[kOptBatch];
  int64_t n[kOptBatch];
  int64_t gp[kOptBatch];
  int64_t poff[kOptBatch];
  uint32_t blk_end[kOptBatch];
  int count;
};

// Up to kOptBatch tensors of one AdamW launch; tensor t owns workgroups
// [blk_end[t-1], blk_end[t]), kAdamwChunk elements each.  Bit t of vec: all
// of tensor t's arrays allow 16-byte (BF16 copy: 8-byte) accesses.
struct AdamwBatch {
  AdamwDesc d[kOptBatch];
  uint32_t blk_end[kOptBatch];
  uint32_t vec;
  int count;
};

// The tensor of a batch that workgroup `blk` belongs to: the number of
// tensors that end at or before it.  Unused slots hold UINT32_MAX, so the
// count needs no loop bound; the unrolled form issues every load at once.
__device__ __forceinline__ int batch_slot(const uint32_t* blk_end, uint32_t blk) {
  int t = 0;
#pragma unroll
  for (int j = 0; j < kOptBatch - 1; ++j) t += blk >= blk_end[j] ? 1 : 0;
  return t;
}

}  // namespace

// FP64 sums of squares of groups of 256 (stride-halving tree), one
// wavefront per group; groups past a tensor's last real one get 0 up to its
// power-of-two count.
__global__ __launch_bounds__(256) void k_sumsq_groups(SumsqBatch b, double* __restrict__ part) {
  const int t = batch_slot(b.blk_end, blockIdx.x);
  const uint32_t first = t ? b.blk_end[t - 1] : 0u;
  const int lane = threadIdx.x & 63;
  const int64_t grp = (int64_t)(blockIdx.x - first) * 4 + (threadIdx.x >> 6);
  const int64_t n = b.n[t];
  const int64_t G = (n + 255) / 256;
  if (grp >= b.gp[t]) return;
  double* out = part + b.poff[t];
  if (grp >= G) {
    if (lane == 0) out[grp] = 0.0;
    return;
  }
  const float* g = b.g[t];
  double v[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int64_t i = grp * 256 + lane + 64 * q;
    const double x = (i < n) ? (double)g[i] : 0.0;
    v[q] = __dmul_rn(x, x);   // exact: a square of an FP32 value fits FP64
  }
  v[0] = __dadd_rn(v[0], v[2]);  // half = 128
  v[1] = __dadd_rn(v[1], v[3]);
  v[0] = __dadd_rn(v[0], v[1]);  // half = 64
#pragma unroll
  for (int half = 32; half >= 1; half >>= 1) v[0] = __dadd_rn(v[0], __shfl_down(v[0], half, 64));
  if (lane == 0) out[grp] = v[0];
}

// One tree level over one tensor's group sums: v[j] += v[j + half], j < half.
__global__ __launch_bounds__(256) void k_sumsq_level(double* __restrict__ v, int64_t half) {
  const int64_t j = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (j < half) v[j] = __dadd_rn(v[j], v[j + half]);
}

// The remaining levels (at most kTreeLds values) of every tensor of a batch,
// one workgroup per tensor; sums[t] = the tree's sum.
__global__ __launch_bounds__(1024) void k_sumsq_final(SumsqBatch b, const double* __restrict__ part,
                                                      double* __restrict__ sums) {
  __shared__ double s[kTreeLds];
  const int t = blockIdx.x;
  const double* v = part + b.poff[t];
  const int64_t len = b.gp[t] < kTreeLds ? b.gp[t] : kTreeLds;
  for (int64_t j = threadIdx.x; j < len; j += blockDim.x) s[j] = v[j];
  __syncthreads();
  for (int64_t half = len / 2; half >= 1; half /= 2) {
    for (int64_t j = threadIdx.x; j < half; j += blockDim.x) s[j] = __dadd_rn(s[j], s[j + half]);
    __syncthreads();
  }
  if (threadIdx.x == 0) sums[t] = s[0];
}

// acc += t[0] + t[1] + ... (in that order).  The tensor sums are staged in
// LDS by the whole workgroup, 1024 at a time, and added by one thread.
__global__ __launch_bounds__(256) void k_sumsq_accumulate(const double* __restrict__ t, int count,
                                                          double* acc) {
  __shared__ double s[1024];
  double a = 0.0;
  if (threadIdx.x == 0) a = acc[0];
  for (int c0 = 0; c0 < count; c0 += 1024) {
    const int len = count - c0 < 1024 ? count - c0 : 1024;
    for (int i = threadIdx.x; i < len; i += blockDim.x) s[i] = t[c0 + i];
    __syncthreads();
    if (threadIdx.x == 0)
      for (int i = 0; i < len; ++i) a = __dadd_rn(a, s[i]);
    __syncthreads();
  }
  if (threadIdx.x == 0) acc[0] = a;
}

int64_t sumsq_part_len(int64_t n) {
  const int64_t G = (n + 255) / 256;
  int64_t Gp = 1;
  while (Gp < G) Gp *= 2;
  return Gp;
}

hipError_t launch_sumsq(const float* const* grads, const int64_t* n, int count, double* acc,
                        double* part, double* sums, hipStream_t st) {
  int64_t off = 0;
  for (int b0 = 0; b0 < count; b0 += kOptBatch) {
    SumsqBatch b{};
    b.count = std::min(kOptBatch, count - b0);
    std::fill(b.blk_end, b.blk_end + kOptBatch, UINT32_MAX);
    uint32_t blocks = 0;
    for (int j = 0; j < b.count; ++j) {
      b.g[j] = grads[b0 + j];
      b.n[j] = n[b0 + j];
      b.gp[j] = sumsq_part_len(b.n[j]);
      b.poff[j] = off;
      off += b.gp[j];
      blocks += (uint32_t)((b.gp[j] + 3) / 4);
      b.blk_end[j] = blocks;
    }
    hipLaunchKernelGGL(k_sumsq_groups, dim3(blocks), dim3(256), 0, st, b, part);
    for (int j = 0; j < b.count; ++j) {
      for (int64_t len = b.gp[j]; len > kTreeLds; len /= 2) {
        const int64_t half = len / 2;
        hipLaunchKernelGGL(k_sumsq_level, dim3((unsigned)((half + 255) / 256)), dim3(256), 0, st,
                           part + b.poff[j], half);
      }
    }
    hipLaunchKernelGGL(k_sumsq_final, dim3(b.count), dim3(1024), 0, st, b, part, sums + b0);
  }
  hipLaunchKernelGGL(k_sumsq_accumulate, dim3(1), dim3(256), 0, st, sums, count, acc);
  return hipGetLastError();
}

// Clip coefficient from the accumulated sum of squares: norm = FP32(sqrt(S)),
// c = min(1, max_norm / (norm + 1e-6)) in FP32; 1 when no norm is given.
__device__ __forceinline__ float clip_coef(const double* sumsq, float max_norm) {
  if (!sumsq) return 1.0f;
  const float norm = (float)__dsqrt_rn(sumsq[0]);
  const float c = __fdiv_rn(max_norm, __fadd_rn(norm, 1e-6f));
  return c < 1.0f ? c : 1.0f;
}

// Correctly rounded FP32 square root.  The FP32 hardware square root is
// faithful (within one ulp), not correctly rounded.  The FP64 root is
// correctly rounded, and rounding it once more to FP32 keeps that: double
// rounding cannot hurt a square root when the wider format carries at least
// 2p + 2 bits (here 53 >= 2 * 24 + 2; S. A. Figueroa, "When is double
// rounding innocuous?", SIGNUM Newsletter 30(3), 1995).
__device__ __forceinline__ float sqrt_rn_f32(float x) { return (float)__dsqrt_rn((double)x); }

// Each thread updates four consecutive elements, so a wavefront streams 1 KB
// of every FP32 array per access.
__global__ __launch_bounds__(256) void k_adamw(AdamwBatch b, AdamwScalars h, const double* sumsq) {
  const int t = batch_slot(b.blk_end, blockIdx.x);
  const uint32_t first = t ? b.blk_end[t - 1] : 0u;
  const AdamwDesc d = b.d[t];
  const int64_t i0 = (int64_t)(blockIdx.x - first) * kAdamwChunk + 4 * (int64_t)threadIdx.x;
  if (i0 >= d.n) return;
  const int cnt = d.n - i0 < 4 ? (int)(d.n - i0) : 4;
  const bool vec = ((b.vec >> t) & 1u) && cnt == 4;
  float g[4], p[4], m[4], v[4];
  if (vec) {
    const f32x4 g4 = *reinterpret_cast<const f32x4*>(d.grad + i0);
    const f32x4 p4 = *reinterpret_cast<const f32x4*>(d.param + i0);
    const f32x4 m4 = *reinterpret_cast<const f32x4*>(d.m + i0);
    const f32x4 v4 = *reinterpret_cast<const f32x4*>(d.v + i0);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      g[e] = g4[e];
      p[e] = p4[e];
      m[e] = m4[e];
      v[e] = v4[e];
    }
  } else {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const bool ok = e < cnt;
      g[e] = ok ? d.grad[i0 + e] : 0.0f;
      p[e] = ok ? d.param[i0 + e] : 0.0f;
      m[e] = ok ? d.m[i0 + e] : 0.0f;
      v[e] = ok ? d.v[i0 + e] : 0.0f;
    }
  }
  const float c = clip_coef(sumsq, h.max_norm);
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const float ge = __fmul_rn(g[e], c);
    float pe = __fsub_rn(p[e], __fmul_rn(h.lrwd, p[e]));
    const float me = __fadd_rn(__fmul_rn(h.b1, m[e]), __fmul_rn(h.ob1, ge));
    const float ve = __fadd_rn(__fmul_rn(h.b2, v[e]), __fmul_rn(h.ob2, __fmul_rn(ge, ge)));
    const float mh = __fdiv_rn(me, h.bc1);
    const float den = __fadd_rn(sqrt_rn_f32(__fdiv_rn(ve, h.bc2)), h.eps);
    p[e] = __fsub_rn(pe, __fmul_rn(h.lr, __fdiv_rn(mh, den)));
    m[e] = me;
    v[e] = ve;
  }
  if (vec) {
    *reinterpret_cast<f32x4*>(d.param + i0) = f32x4{p[0], p[1], p[2], p[3]};
    *reinterpret_cast<f32x4*>(d.m + i0) = f32x4{m[0], m[1], m[2], m[3]};
    *reinterpret_cast<f32x4*>(d.v + i0) = f32x4{v[0], v[1], v[2], v[3]};
    if (d.p16)
      *reinterpret_cast<uint2*>(d.p16 + i0) = make_uint2(pack_bf16x2(p[0], p[1]),
                                                         pack_bf16x2(p[2], p[3]));
  } else {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      if (e >= cnt) break;
      d.param[i0 + e] = p[e];
      d.m[i0 + e] = m[e];
      d.v[i0 + e] = v[e];
      if (d.p16) d.p16[i0 + e] = (uint16_t)(pack_bf16x2(p[e], 0.0f) & 0xFFFFu);
    }
  }
}

static bool aligned_to(const void* p, uintptr_t a) {
  return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0;
}

hipError_t launch_adamw(const AdamwDesc* d, int count, const AdamwScalars& h,
                        const double* sumsq, hipStream_t st) {
  for (int b0 = 0; b0 < count; b0 += kOptBatch) {
    AdamwBatch b{};
    b.count = std::min(kOptBatch, count - b0);
    std::fill(b.blk_end, b.blk_end + kOptBatch, UINT32_MAX);
    uint32_t blocks = 0;
    for (int j = 0; j < b.count; ++j) {
      const AdamwDesc& t = d[b0 + j];
      b.d[j] = t;
      blocks += (uint32_t)((t.n + kAdamwChunk - 1) / kAdamwChunk);
      b.blk_end[j] = blocks;
      const bool v16 = aligned_to(t.param, 16) && aligned_to(t.grad, 16) &&
                       aligned_to(t.m, 16) && aligned_to(t.v, 16) &&
                       (!t.p16 || aligned_to(t.p16, 8));
      if (v16) b.vec |= 1u << j;
    }
    hipLaunchKernelGGL(k_adamw, dim3(blocks), dim3(256), 0, st, b, h, sumsq);
  }
  return hipGetLastError();
}

}  // namespace qlora
