// gemv.hip -- forward of the NF4 LoRA linear layer for M <= 16 tokens
// (gfx950).  HBM-bound: every packed weight byte is read once.
//
// [QP] "第 04 篇：QLoRA 原理" §2.3 / §6.1: the kernel reads the 4-bit codes and
// the quantization state, unpacks, restores the scales, looks up the NF4
// levels, converts to BF16 and multiplies, without writing a BF16 copy of W.
//
// Mapping.  A workgroup of four wavefronts owns kGemvRows output rows and a
// K range; wavefront w holds kSets = kGemvRows / 64 sets of 16 rows (rows
// 16 (kSets w + t) + l%16 of the tile).  K advances in 256-wide super-steps:
// lane (n = l%16, g = l/16) owns the whole 64-weight block g of its row in
// each set, so it restores that block's scale once and builds its 16-entry
// BF16 table once (nf4_table), then feeds eight v_mfma_f32_16x16x32_bf16 with
// eight weights each.  The MFMA pairs A lane (m, g) with B lane (n, g), so
// lane group g of the X operand reads the same 64 columns.  The workgroup
// stages its K slice of X in LDS once, permuted within each eight to match
// the table lookup's output order, and every wavefront reads its X fragments
// there once per step for all of its sets.  M is padded to 16 rows with a
// zero row.  Each workgroup writes the FP32 partial sums of its K split.
// The first workgroups of the launch form T = t_scale X A^T instead, one
// 16-rank block each over the whole of K.  A second, small kernel adds the
// splits in order, applies the LoRA term and rounds Y, so that no workgroup
// waits on another and no device-wide fence (an L2 write-back and
// invalidate on this chip) is needed.
#include "qlora_device.h"
#include "qlora_kernels.h"

#include <algorithm>

namespace qlora {

constexpr int kSets = kGemvRows / 64;   // 16-row sets per wavefront

// Codes and scales of one 256-wide super-step for one lane, held in
// registers between their loads and the MFMAs.
struct StepData {
  u32x4 c[kSets][2];     // 32 bytes of codes per set: the lane's block
  uint32_t sc[kSets];    // FP8 scale codes
  float s2[kSets];       // second-level scales as loaded
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
  __amdgpu_buffer_rsrc_t codes, scodes, s2;   // codes, scodes based at the tile's first row
  uint32_t vc[kSets], vs[kSets];              // lane byte offsets (step 0)
  int64_t blk0[kSets];                        // first-level block of the lane, step 0
};

// Super-step ss.  Rows past d_out read as zero (descriptor bounds).  Blocks
// past d_in read whatever lies there; compute_step gives them scale zero.
__device__ __forceinline__ void load_step(const GemvLane& L, int64_t ss, StepData& s) {
  const uint32_t so_c = (uint32_t)(ss * 128), so_s = (uint32_t)(ss * 4);
#pragma unroll
  for (int t = 0; t < kSets; ++t) {
    s.c[t][0] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(L.codes, L.vc[t], so_c, 0));
    s.c[t][1] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(L.codes, L.vc[t] + 16, so_c, 0));
    s.sc[t] = __builtin_amdgcn_raw_buffer_load_b8(L.scodes, L.vs[t], so_s, 0);
    const uint32_t grp = (uint32_t)((L.blk0[t] + ss * 4) >> 8);
    s.s2[t] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(L.s2, grp * 4, 0, 0));
  }
}

// The 8 kSets MFMAs of a step.  X fragment j (columns 64 g + 8 j of the
// step, permuted within each eight) comes from the lane's staged row; the
// weights of set t come from its block's table.  A block past d_in (ok
// false) gets scale 0, so its table and products are zero whatever codes it
// read.
__device__ __forceinline__ void compute_step(const StepData& s, bool ok, float mean,
                                             const uint8_t* xrow, f32x4 (&acc)[kSets]) {
  if constexpr (kSets == 1) {
    // one set: X fragments read as they are used, four at a time
    const Nf4Table tab = nf4_table(restored_scale(s.sc[0], ok ? s.s2[0] : 0.0f, ok ? mean : 0.0f));
    const uint32_t cw[8] = {s.c[0][0].x, s.c[0][0].y, s.c[0][0].z, s.c[0][0].w,
                            s.c[0][1].x, s.c[0][1].y, s.c[0][1].z, s.c[0][1].w};
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      u32x4 xf[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) xf[j] = *reinterpret_cast<const u32x4*>(xrow + 64 * h + 16 * j);
#pragma unroll
      for (int j = 0; j < 4; ++j) acc[0] = mfma16(xf[j], nf4_dequant8_perm(cw[4 * h + j], tab), acc[0]);
    }
  } else {
    u32x4 xf[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) xf[j] = *reinterpret_cast<const u32x4*>(xrow + 16 * j);
#pragma unroll
    for (int t = 0; t < kSets; ++t) {
      const Nf4Table tab = nf4_table(restored_scale(s.sc[t], ok ? s.s2[t] : 0.0f, ok ? mean : 0.0f));
      const uint32_t cw[8] = {s.c[t][0].x, s.c[t][0].y, s.c[t][0].z, s.c[t][0].w,
                              s.c[t][1].x, s.c[t][1].y, s.c[t][1].z, s.c[t][1].w};
#pragma unroll
      for (int j = 0; j < 8; ++j) acc[t] = mfma16(xf[j], nf4_dequant8_perm(cw[j], tab), acc[t]);
    }
  }
}

// Four 16-byte pieces of row `arow` of A (element offset) at columns
// col + 8 j; columns past din read as zero.
__device__ __forceinline__ void load_a_half(__amdgpu_buffer_rsrc_t ra, uint32_t arow, uint32_t col,
                                            uint32_t din, u32x4 (&av)[4]) {
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const uint32_t cj = col + 8 * j;
    const uint32_t off = cj < din ? (arow + cj) * 2 : 0x80000000u;
    av[j] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(ra, off, 0, 0));
  }
}

// ---- LoRA down-projection, one 16-rank block per workgroup:
// T[m][i] = t_scale * sum_k X[m][k] A[i][k] for i in 16 b .. 16 b + 15.
// Wavefront w takes the w-th quarter of the 256-wide super-steps; lane
// (l%16, g = l/16) reads X row l%16 and A row 16 b + l%16 at columns 64 g +
// 8 j of each super-step (both in natural order, so the MFMA sees the same
// column set in both operands), with the next half step's loads in flight
// while the current one multiplies.  The four wavefront sums are added in
// order 0..3 through LDS.  Rows past M or r and columns past d_in read as
// zero.  The forward (weight-streaming launch) and the backward's recompute
// (k_lora_down) run this same code, so both get the same T.
__device__ __forceinline__ void load_half(__amdgpu_buffer_rsrc_t r, uint32_t row, uint32_t col,
                                          uint32_t din, u32x4 (&v)[4]) {
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const uint32_t cj = col + 8 * j;
    const uint32_t off = cj < din ? (row + cj) * 2 : 0x80000000u;
    v[j] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0));
  }
}

__device__ __forceinline__ void lora_down_block(const GemvDesc& d, int M, int b, float* red) {
  const int lane = threadIdx.x & 63, w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int r16 = lane & 15, g = lane >> 4;
  const uint32_t din = (uint32_t)d.d_in;
  const __amdgpu_buffer_rsrc_t rx = gemv_rsrc(d.XA, (int64_t)M * d.d_in * 2);  // rows past M: zero
  const __amdgpu_buffer_rsrc_t ra = gemv_rsrc(d.A, d.r * d.d_in * 2);          // rows past r: zero
  const uint32_t xrow = (uint32_t)r16 * din, arow = (uint32_t)(16 * b + r16) * din;
  const int nss = (int)((d.d_in / kBlock + 3) / 4);
  const int qn = (nss + 3) / 4;
  const int q0 = w * qn < nss ? w * qn : nss;
  const int q1 = q0 + qn < nss ? q0 + qn : nss;
  const int nh = 2 * (q1 - q0);                       // half steps of this wavefront
  const uint32_t col0 = (uint32_t)(q0 * 256 + 64 * g);

  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  u32x4 x0[4], a0[4], x1[4], a1[4];
  if (nh > 0) {
    load_half(rx, xrow, col0, din, x0);
    load_half(ra, arow, col0, din, a0);
  }
  for (int h = 0; h < nh; h += 2) {
    const uint32_t col = col0 + 128 * h;              // super-step q0 + h / 2
    load_half(rx, xrow, col + 32, din, x1);
    load_half(ra, arow, col + 32, din, a1);
#pragma unroll
    for (int j = 0; j < 4; ++j) acc = mfma16(x0[j], a0[j], acc);
    if (h + 2 < nh) {
      load_half(rx, xrow, col + 256, din, x0);
      load_half(ra, arow, col + 256, din, a0);
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) acc = mfma16(x1[j], a1[j], acc);
  }
  // accumulator lane (r16, g): rows m = 4 g + v, rank 16 b + r16
#pragma unroll
  for (int v = 0; v < 4; ++v) red[(w * 16 + 4 * g + v) * 16 + r16] = acc[v];
  __syncthreads();
  if (w == 0) {
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int m = 4 * g + v, i = 16 * b + r16;
      float sum = red[(4 * g + v) * 16 + r16];
#pragma unroll
      for (int ww = 1; ww < 4; ++ww) sum = __fadd_rn(sum, red[(ww * 16 + 4 * g + v) * 16 + r16]);
      if (m < M && i < d.r) d.t_buf[(int64_t)m * d.r + i] = __fmul_rn(d.t_scale, sum);
    }
  }
}

// Workgroup -> (problem, 16-rank block) of the LoRA down-projection part of a
// launch (the first t_wgs workgroups).
__device__ __forceinline__ void lora_down_dispatch(const GemvArgs& a, int wg, float* red) {
  int di = 0;
  while (di + 1 < a.count && wg >= a.d[di + 1].tb_begin) ++di;
  lora_down_block(a.d[di], a.M, wg - a.d[di].tb_begin, red);
}

__global__ __launch_bounds__(256) void k_lora_down(GemvArgs a) {
  __shared__ float red[4 * 16 * 16];
  lora_down_dispatch(a, blockIdx.x, red);
}

#ifndef QLORA_GEMV_DEPTH
#define QLORA_GEMV_DEPTH 3
#endif
constexpr int kGemvDepth = QLORA_GEMV_DEPTH;   // super-steps in flight per lane
constexpr int kStageBatch = 4;  // 16-byte X chunks per thread per staging round

__global__ __launch_bounds__(256)
void k_gemv(GemvArgs a) {
  extern __shared__ __attribute__((aligned(16))) uint8_t xs[];
  if ((int)blockIdx.x < a.t_wgs) {       // LoRA down-projection blocks first
    lora_down_dispatch(a, blockIdx.x, reinterpret_cast<float*>(xs));
    return;
  }
  const int wg = blockIdx.x - a.t_wgs;
  int di = 0;
  while (di + 1 < a.count && wg >= a.d[di + 1].wg_begin) ++di;
  const GemvDesc& d = a.d[di];
  const int local = wg - d.wg_begin;
  const int split = local % d.ksplit;
  const int tile = local / d.ksplit;

  const int lane = threadIdx.x & 63, w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int r16 = lane & 15, g = lane >> 4;
  const int M = a.M;
  const int64_t row0 = (int64_t)tile * kGemvRows;        // first row of the tile
  const int64_t nblk = d.d_in / kBlock;
  const int64_t nss = (nblk + 3) / 4;
  const int64_t ss0 = (int64_t)split * d.ss_per_split;
  int64_t ss1 = ss0 + d.ss_per_split;
  if (ss1 > nss) ss1 = nss;
  const float mean = d.mean[0];

  // X rows of the split staged in LDS, permuted within each eight, at a
  // padded row stride; row M is zero and serves the rows past M, and columns
  // past d_in are zero (d_in is a multiple of 64, so chunks of eight never
  // straddle it).  Loads go out kStageBatch at a time; a chunk outside the
  // data gets an offset past the descriptor and reads zero.  Staged before
  // the weight loads start, so that every pass into the main loop finds the
  // same loads in flight.
  const int64_t kl = (int64_t)d.ss_per_split * 256;
  const int64_t ld = kl * 2 + 16;                       // staged row, bytes
  {
    const __amdgpu_buffer_rsrc_t rx = gemv_rsrc(d.X, (int64_t)M * d.d_in * 2);
    // 32-bit index math: (M + 1) * per_row is below 2^16 (the LDS limit)
    const uint32_t per_row = (uint32_t)(kl / 8);        // 16-byte chunks
    const uint32_t nchunk = (uint32_t)(M + 1) * per_row;
    const uint32_t col0 = (uint32_t)(ss0 * 256), din = (uint32_t)d.d_in;
    for (uint32_t base = 0; base < nchunk; base += 256 * kStageBatch) {
      u32x4 v[kStageBatch];
      uint32_t dst[kStageBatch];
#pragma unroll
      for (int u = 0; u < kStageBatch; ++u) {
        const uint32_t i = base + 256 * u + threadIdx.x;
        const uint32_t row = i / per_row, c = i - row * per_row, col = col0 + 8 * c;
        const bool in = row < (uint32_t)M && col < din;
        const uint32_t off = in ? (row * din + col) * 2 : 0x80000000u;
        v[u] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rx, off, 0, 0));
        dst[u] = i < nchunk ? row * (uint32_t)ld + 16 * c : 0xFFFFFFFFu;
      }
#pragma unroll
      for (int u = 0; u < kStageBatch; ++u)
        if (dst[u] != 0xFFFFFFFFu) *reinterpret_cast<u32x4*>(xs + dst[u]) = perm8_bf16(v[u]);
    }
  }
  __syncthreads();

  GemvLane L;
  L.codes = gemv_rsrc(d.codes + row0 * (d.d_in / 2), (d.d_out - row0) * (d.d_in / 2));
  L.scodes = gemv_rsrc(d.scodes + row0 * nblk, (d.d_out - row0) * nblk);
  L.s2 = gemv_rsrc(d.scale2, ((d.d_out * nblk + kGroup - 1) / kGroup) * 4);
#pragma unroll
  for (int t = 0; t < kSets; ++t) {
    const int64_t rl = 16 * (kSets * w + t) + r16;           // row within the tile
    L.vc[t] = (uint32_t)(rl * (d.d_in / 2) + 32 * g);
    L.vs[t] = (uint32_t)(rl * nblk + g);
    L.blk0[t] = (row0 + rl) * nblk + g;
  }

  // Ring of kGemvDepth steps: the loads of step ss + D - 1 are issued before
  // the MFMAs of step ss.  The prologue and the steady loop load
  // unconditionally (steps past ss1 read in bounds or zero and are never
  // used), which keeps the compiler's wait counts exact; the last steps run
  // in a guarded tail.
  constexpr int D = kGemvDepth;
  const int nsteps = (int)(ss1 - ss0);
  StepData st[D];
#pragma unroll
  for (int i = 0; i < D - 1; ++i) {
    load_step(L, ss0 + i, st[i]);
    __builtin_amdgcn_sched_barrier(0);   // issue order = use order
  }

  const uint8_t* xrow = xs + (r16 < M ? r16 : M) * ld + 128 * g;   // step 0 of this lane
  const int64_t kb0 = ss0 * 4 + g;                                  // lane block, step 0

  f32x4 acc[kSets];
#pragma unroll
  for (int t = 0; t < kSets; ++t) acc[t] = f32x4{0.f, 0.f, 0.f, 0.f};
  {
    int i = 0;
    for (; i + 2 * D - 1 <= nsteps; i += D) {
#pragma unroll
      for (int j = 0; j < D; ++j) {
        load_step(L, ss0 + i + j + D - 1, st[(j + D - 1) % D]);
        __builtin_amdgcn_sched_barrier(0);   // loads issued ahead of the step's math
        compute_step(st[j], kb0 + 4 * (i + j) < nblk, mean, xrow + 512 * (i + j), acc);
      }
    }
    for (; i < nsteps; i += D) {
#pragma unroll
      for (int j = 0; j < D; ++j) {
        if (i + j < nsteps) {
          if (i + j + D - 1 < nsteps) load_step(L, ss0 + i + j + D - 1, st[(j + D - 1) % D]);
          compute_step(st[j], kb0 + 4 * (i + j) < nblk, mean, xrow + 512 * (i + j), acc);
        }
      }
    }
  }

  // ---- partial sums of the split: part[split][m][n] ----
#pragma unroll
  for (int t = 0; t < kSets; ++t) {
    const int64_t n = row0 + 16 * (kSets * w + t) + r16;
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int m = 4 * g + v;
      if (m < M && n < d.d_out) d.part[((int64_t)split * 16 + m) * d.d_out + n] = acc[t][v];
    }
  }

}

// Finish: one workgroup per 64 output columns of a problem; wavefront w
// takes columns 16 w .. 16 w + 15, lane (n = l%16, g = l/16) rows 4 g .. 4 g
// + 3 as in the MFMA accumulator.
//   acc = sum_s part[s]                      (s ascending)
//   acc += [T_hi | T_lo] [B | B]^T           (two MFMAs per 32 ranks)
//   Y   = RNE_bf16(acc)
// Partials are loaded kFinBatch splits at a time, so the sum does not wait on
// one load after another.
constexpr int kFinBatch = 4;

__global__ __launch_bounds__(256) void k_gemv_finish(GemvArgs a) {
  const int wg = blockIdx.x;
  int di = 0;
  while (di + 1 < a.count && wg >= a.d[di + 1].fin_begin) ++di;
  const GemvDesc& d = a.d[di];
  const int ct = wg - d.fin_begin;                 // 64-column tile
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int r16 = lane & 15, g = lane >> 4;
  const int M = a.M;
  const int64_t n = (int64_t)ct * 64 + 16 * w + r16;
  const int ks = d.ksplit;

  const bool col_ok = n < d.d_out;
  const bool bvec = (d.r % 8) == 0 && ((uintptr_t)d.B % 16) == 0;
  const bool tvec = (d.r % 4) == 0;
  // T (lane row l%16, ranks kk .. kk+7) and B (column n, same ranks) of one
  // 32-rank chunk
  auto load_tb = [&](int64_t k0, float (&t8)[8], u32x4& bw) {
    const int64_t kk = k0 + 8 * g;
    const float* tp = d.t_buf + (int64_t)r16 * d.r + kk;
    if (r16 < M && tvec && kk + 8 <= d.r) {
      const float4 t0 = reinterpret_cast<const float4*>(tp)[0];
      const float4 t1 = reinterpret_cast<const float4*>(tp)[1];
      t8[0] = t0.x; t8[1] = t0.y; t8[2] = t0.z; t8[3] = t0.w;
      t8[4] = t1.x; t8[5] = t1.y; t8[6] = t1.z; t8[7] = t1.w;
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e) t8[e] = (r16 < M && kk + e < d.r) ? tp[e] : 0.0f;
    }
    bw = u32x4{0u, 0u, 0u, 0u};
    if (col_ok && kk < d.r) {
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
  };
  auto apply_tb = [&](const float (&t8)[8], const u32x4& bw, f32x4& acc) {
    float hi[8], lo[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) split_bf16(t8[e], hi[e], lo[e]);
    u32x4 ah, al;
    ah.x = pack_bf16x2(hi[0], hi[1]); ah.y = pack_bf16x2(hi[2], hi[3]);
    ah.z = pack_bf16x2(hi[4], hi[5]); ah.w = pack_bf16x2(hi[6], hi[7]);
    al.x = pack_bf16x2(lo[0], lo[1]); al.y = pack_bf16x2(lo[2], lo[3]);
    al.z = pack_bf16x2(lo[4], lo[5]); al.w = pack_bf16x2(lo[6], lo[7]);
    acc = mfma16(ah, bw, acc);
    acc = mfma16(al, bw, acc);
  };

  // the first two rank chunks' loads go out with the partial loads
  float t0[8], t1[8];
  u32x4 b0, b1;
  load_tb(0, t0, b0);
  if (d.r > 32) load_tb(32, t1, b1);

  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  for (int s0 = 0; s0 < ks; s0 += kFinBatch) {
    float v[kFinBatch][4];
#pragma unroll
    for (int u = 0; u < kFinBatch; ++u)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int m = 4 * g + q;
        v[u][q] = (s0 + u < ks && m < M && col_ok)
                      ? d.part[((int64_t)(s0 + u) * 16 + m) * d.d_out + n] : 0.0f;
      }
#pragma unroll
    for (int u = 0; u < kFinBatch; ++u)
#pragma unroll
      for (int q = 0; q < 4; ++q)
        if (s0 + u < ks) acc[q] = (s0 + u == 0) ? v[u][q] : __fadd_rn(acc[q], v[u][q]);
  }

  apply_tb(t0, b0, acc);
  if (d.r > 32) apply_tb(t1, b1, acc);
  for (int64_t k0 = 64; k0 < d.r; k0 += 32) {
    load_tb(k0, t0, b0);
    apply_tb(t0, b0, acc);
  }

#pragma unroll
  for (int v = 0; v < 4; ++v) {
    const int m = 4 * g + v;
    if (m < M && col_ok) {
      f32x2 p = {acc[v], 0.0f};
      d.Y[(int64_t)m * d.d_out + n] =
          (uint16_t)(__builtin_bit_cast(uint32_t, __builtin_convertvector(p, bf16x2)) & 0xFFFFu);
    }
  }
}

hipError_t launch_lora_down(const GemvArgs& a, hipStream_t st) {
  hipLaunchKernelGGL(k_lora_down, dim3(a.t_wgs), dim3(256), 0, st, a);
  return hipGetLastError();
}

hipError_t launch_gemv(const GemvArgs& a, int total_wgs, int fin_wgs, hipStream_t st) {
  // staged X: (M + 1) rows of the largest split, padded
  int64_t lds = 0;
  for (int i = 0; i < a.count; ++i)
    lds = std::max<int64_t>(lds, gemv_lds_bytes(a.M, a.d[i].ss_per_split));
  static hipError_t attr = hipFuncSetAttribute(reinterpret_cast<const void*>(&k_gemv),
                                               hipFuncAttributeMaxDynamicSharedMemorySize,
                                               kGemvMaxLds);
  if (attr != hipSuccess) return attr;
  if (lds > kGemvMaxLds) return hipErrorInvalidValue;
  weight_kernel_begin(st);
  hipLaunchKernelGGL(k_gemv, dim3(a.t_wgs + total_wgs), dim3(256), (unsigned)lds, st, a);
  weight_kernel_end(st);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(k_gemv_finish, dim3(fin_wgs), dim3(256), 0, st, a);
  return hipGetLastError();
}

}  // namespace qlora
