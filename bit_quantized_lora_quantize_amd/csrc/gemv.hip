// gemv.hip -- forward of the NF4 LoRA linear layer for M <= 16 tokens
// (gfx950).  HBM-bound: every packed weight byte is read once.
//
// [QP] "第 04 篇：QLoRA 原理" §2.3 / §6.1: the kernel reads the 4-bit codes and
// the quantization state, unpacks, restores the scales, looks up the NF4
// levels, converts to BF16 and multiplies, without writing a BF16 copy of W.
//
// Mapping.  A workgroup of four wavefronts owns 64 output rows (16 per
// wavefront) and a K range.  K advances in 256-wide super-steps: lane
// (n = l%16, g = l/16) owns the whole 64-weight block g of row n, so it
// restores that block's scale once and builds its 16-entry BF16 table once
// (nf4_table), then feeds eight v_mfma_f32_16x16x32_bf16 with eight weights
// each.  The MFMA pairs A lane (m, g) with B lane (n, g), so lane group g of
// the X operand reads the same 64 columns, already permuted within each
// eight (Xp) to match the table lookup's output order.  M is padded to 16
// rows with zeros.
#include "qlora_device.h"
#include "qlora_kernels.h"

namespace qlora {

// Global data of one 256-wide super-step for one lane, held in registers
// between its loads and its MFMAs.
struct StepData {
  u32x4 c0, c1;   // 32 bytes of codes: the lane's block
  u32x4 x[8];     // X operand for the eight MFMAs
  uint32_t sc;    // FP8 scale code
  float s2;       // second-level scale (0 for a block past d_in)
  float mu;       // scale mean (0 for a block past d_in)
};

// Buffer descriptor of a workgroup-uniform range, in scalar registers.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t gemv_rsrc(const void* base, int64_t bytes) {
  const int32_t n = bytes > 0x7FFFFFFF ? 0x7FFFFFFF : (bytes < 0 ? 0 : (int32_t)bytes);
  const uint64_t b = reinterpret_cast<uint64_t>(base);
  const uint64_t bu = ((uint64_t)(uint32_t)__builtin_amdgcn_readfirstlane((int)(b >> 32)) << 32) |
                      (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)b);
  return __builtin_amdgcn_make_buffer_rsrc(reinterpret_cast<void*>(bu), 0,
                                           __builtin_amdgcn_readfirstlane(n), 0x00020000);
}

struct GemvLane {
  __amdgpu_buffer_rsrc_t codes, scodes, s2, x;
  uint32_t vc, vs, vx;   // lane byte offsets (step 0)
  int64_t blk0;          // first-level block index of the lane's row, step 0
  int64_t nblk;
  int g;
};

// Super-step ss (lane block kb = 4 ss + g).  Rows past d_out and X rows past
// M read as zero (descriptor bounds); a block past d_in gets s2 = 0, so its
// restored scale, table and products are zero whatever codes it reads.
__device__ __forceinline__ void load_step(const GemvLane& L, int64_t ss, float mean, StepData& s) {
  const uint32_t so_c = (uint32_t)(ss * 128), so_x = (uint32_t)(ss * 512);
  s.c0 = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(L.codes, L.vc, so_c, 0));
  s.c1 = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(L.codes, L.vc + 16, so_c, 0));
  s.sc = __builtin_amdgcn_raw_buffer_load_b8(L.scodes, L.vs, (uint32_t)(ss * 4), 0);
  const int64_t kb = ss * 4 + L.g;
  const uint32_t grp = (uint32_t)((L.blk0 + ss * 4) >> 8);
  const float s2 = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(L.s2, grp * 4, 0, 0));
  s.s2 = kb < L.nblk ? s2 : 0.0f;
  s.mu = kb < L.nblk ? mean : 0.0f;
#pragma unroll
  for (int j = 0; j < 8; ++j)
    s.x[j] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(L.x, L.vx + 16 * j, so_x, 0));
}

__device__ __forceinline__ f32x4 compute_step(const StepData& s, f32x4 acc) {
  // a masked block has s2 = 0 and mean 0: restored scale, table and
  // products are zero
  const Nf4Table t = nf4_table(restored_scale(s.sc, s.s2, s.mu));
  const uint32_t cw[8] = {s.c0.x, s.c0.y, s.c0.z, s.c0.w, s.c1.x, s.c1.y, s.c1.z, s.c1.w};
#pragma unroll
  for (int j = 0; j < 8; ++j) acc = mfma16(s.x[j], nf4_dequant8_perm(cw[j], t), acc);
  return acc;
}

constexpr int kGemvDepth = 3;   // super-steps in flight per lane

__global__ __launch_bounds__(256) void k_gemv(GemvArgs a) {
  const int wg = blockIdx.x;
  int di = 0;
  while (di + 1 < a.count && wg >= a.d[di + 1].wg_begin) ++di;
  const GemvDesc& d = a.d[di];
  const int local = wg - d.wg_begin;
  const int split = local % d.ksplit;
  const int tile = local / d.ksplit;

  const int lane = threadIdx.x & 63, w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int r16 = lane & 15, g = lane >> 4;
  const int M = a.M;
  const int64_t n = (int64_t)tile * 64 + 16 * w + r16;  // B-operand row and output column
  const int64_t nblk = d.d_in / kBlock;
  const int64_t nss = (nblk + 3) / 4;
  const int64_t ss0 = (int64_t)split * d.ss_per_split;
  int64_t ss1 = ss0 + d.ss_per_split;
  if (ss1 > nss) ss1 = nss;
  const float mean = d.mean[0];

  GemvLane L;
  L.codes = gemv_rsrc(d.codes, d.d_out * (d.d_in / 2));
  L.scodes = gemv_rsrc(d.scodes, d.d_out * nblk);
  L.s2 = gemv_rsrc(d.scale2, ((d.d_out * nblk + kGroup - 1) / kGroup) * 4);
  L.x = gemv_rsrc(d.Xp, (int64_t)M * d.d_in * 2);
  L.vc = (uint32_t)(n * (d.d_in / 2) + 32 * g);
  L.vs = (uint32_t)(n * nblk + g);
  L.vx = (uint32_t)((int64_t)r16 * d.d_in * 2 + 128 * g);
  L.blk0 = n * nblk + g;
  L.nblk = nblk;
  L.g = g;

  // Ring of kGemvDepth steps: the loads of step ss + D - 1 are issued before
  // the MFMAs of step ss.  Prologue and steady loop load unconditionally
  // (steps past ss1 read in bounds or zero and are never used), which keeps
  // the compiler's wait counts exact; the last steps run in a guarded tail.
  constexpr int D = kGemvDepth;
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  const int nsteps = (int)(ss1 - ss0);
  {
    StepData st[D];
#pragma unroll
    for (int i = 0; i < D - 1; ++i) load_step(L, ss0 + i, mean, st[i]);
    int i = 0;
    for (; i + 2 * D - 1 <= nsteps; i += D) {
#pragma unroll
      for (int j = 0; j < D; ++j) {
        load_step(L, ss0 + i + j + D - 1, mean, st[(j + D - 1) % D]);
        acc = compute_step(st[j], acc);
      }
    }
    for (; i < nsteps; i += D) {
#pragma unroll
      for (int j = 0; j < D; ++j) {
        if (i + j < nsteps) {
          if (i + j + D - 1 < nsteps) load_step(L, ss0 + i + j + D - 1, mean, st[(j + D - 1) % D]);
          acc = compute_step(st[j], acc);
        }
      }
    }
  }

  // ---- split-K: partials, then the last workgroup of this tile reduces ----
  if (d.ksplit > 1) {
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int m = 4 * g + v;
      if (m < M && n < d.d_out) d.part[((int64_t)split * 16 + m) * d.d_out + n] = acc[v];
    }
    __shared__ int s_last;
    __threadfence();
    __syncthreads();
    if (threadIdx.x == 0) {
      const uint32_t prev = atomicAdd(&d.counters[tile], 1u);
      s_last = (prev == (uint32_t)(d.ksplit - 1));
    }
    __syncthreads();
    if (!s_last) return;
    __threadfence();
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int m = 4 * g + v;
      float tot = 0.0f;
      if (m < M && n < d.d_out) {
        tot = __hip_atomic_load(&d.part[(int64_t)m * d.d_out + n], __ATOMIC_RELAXED,
                                __HIP_MEMORY_SCOPE_AGENT);
        for (int s = 1; s < d.ksplit; ++s)
          tot = __fadd_rn(tot, __hip_atomic_load(&d.part[((int64_t)s * 16 + m) * d.d_out + n],
                                                 __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT));
      }
      acc[v] = tot;
    }
    if (threadIdx.x == 0) d.counters[tile] = 0u;
  }

  // ---- LoRA term: acc += [T_hi | T_lo] [B | B]^T, two MFMAs per 32 ranks ----
  const bool bvec = (d.r % 8) == 0 && ((uintptr_t)d.B % 16) == 0;
  const bool tvec = (d.r % 4) == 0 && ((uintptr_t)d.t_part % 16) == 0;
  for (int64_t k0 = 0; k0 < d.r; k0 += 32) {
    const int64_t kk = k0 + 8 * g;
    float t[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) t[e] = 0.0f;
    if (r16 < M && kk < d.r) {
      for (int s = 0; s < d.t_splits; ++s) {
        const float* tp = d.t_part + ((int64_t)s * M + r16) * d.r + kk;
        float v8[8];
        if (tvec && kk + 8 <= d.r) {
          const float4 a0 = reinterpret_cast<const float4*>(tp)[0];
          const float4 a1 = reinterpret_cast<const float4*>(tp)[1];
          v8[0] = a0.x; v8[1] = a0.y; v8[2] = a0.z; v8[3] = a0.w;
          v8[4] = a1.x; v8[5] = a1.y; v8[6] = a1.z; v8[7] = a1.w;
        } else {
#pragma unroll
          for (int e = 0; e < 8; ++e) v8[e] = (kk + e < d.r) ? tp[e] : 0.0f;
        }
#pragma unroll
        for (int e = 0; e < 8; ++e) t[e] = (s == 0) ? v8[e] : __fadd_rn(t[e], v8[e]);
      }
    }
    float hi[8], lo[8], tv[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      tv[e] = __fmul_rn(d.t_scale, t[e]);
      split_bf16(tv[e], hi[e], lo[e]);
    }
    // T itself, once per problem: the first wavefront of tile 0 (of the
    // split that reached this epilogue)
    if (d.t_out && tile == 0 && w == 0 && r16 < M) {
#pragma unroll
      for (int e = 0; e < 8; ++e)
        if (kk + e < d.r) d.t_out[(int64_t)r16 * d.r + kk + e] = tv[e];
    }
    u32x4 ah, al;
    ah.x = pack_bf16x2(hi[0], hi[1]); ah.y = pack_bf16x2(hi[2], hi[3]);
    ah.z = pack_bf16x2(hi[4], hi[5]); ah.w = pack_bf16x2(hi[6], hi[7]);
    al.x = pack_bf16x2(lo[0], lo[1]); al.y = pack_bf16x2(lo[2], lo[3]);
    al.z = pack_bf16x2(lo[4], lo[5]); al.w = pack_bf16x2(lo[6], lo[7]);
    u32x4 bw = {0u, 0u, 0u, 0u};
    if (n < d.d_out && kk < d.r) {
      const uint16_t* brow = d.B + n * d.r;
      if (bvec && kk + 8 <= d.r) {
        bw = *reinterpret_cast<const u32x4*>(brow + kk);
      } else {
        uint32_t h[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) h[e] = (kk + e < d.r) ? brow[kk + e] : 0u;
        bw.x = h[0] | (h[1] << 16); bw.y = h[2] | (h[3] << 16);
        bw.z = h[4] | (h[5] << 16); bw.w = h[6] | (h[7] << 16);
      }
    }
    acc = mfma16(ah, bw, acc);
    acc = mfma16(al, bw, acc);
  }

#pragma unroll
  for (int v = 0; v < 4; ++v) {
    const int m = 4 * g + v;
    if (m < M && n < d.d_out) {
      f32x2 p = {acc[v], 0.0f};
      d.Y[(int64_t)m * d.d_out + n] =
          (uint16_t)(__builtin_bit_cast(uint32_t, __builtin_convertvector(p, bf16x2)) & 0xFFFFu);
    }
  }
}

hipError_t launch_gemv(const GemvArgs& a, int total_wgs, hipStream_t st) {
  weight_kernel_begin(st);
  hipLaunchKernelGGL(k_gemv, dim3(total_wgs), dim3(256), 0, st, a);
  weight_kernel_end(st);
  return hipGetLastError();
}

}  // namespace qlora
