// gemv.hip -- forward of the NF4 LoRA linear layer for M <= 16 tokens
// (gfx950), for up to kMaxGroup layers per launch.  HBM-bound on the packed
// weights: every packed byte is read once.
//
// [QP] "第 04 篇：QLoRA 原理" §2.3 / §6.1: the kernel reads the 4-bit codes and
// the quantization state, unpacks, restores the scales, looks up the NF4
// levels, converts to BF16 and multiplies, without writing a BF16 copy of W.
//
// A call is two launches.
//
// Weight streaming and T (k_gemv): kGemvWgs workgroups of four wavefronts,
// four on every compute unit, each layer a block of them in proportion to
// its work, and workgroup j of the block a contiguous range of the layer's
// list of T tasks and weight units (qlora_kernels.h), so every workgroup has
// about the same work and the long K of one layer does not leave the
// others' workgroups idle.  A T task (t_task) is a short burst of BF16 loads
// straight into MFMAs.  In the weight units, wavefront v owns rows
// 16 v .. 16 v + 15 of the current tile; lane (n = l%16, g = l/16) owns the
// whole 64-weight block g of its row in each super-step, restores that
// block's scale once and builds its 16-entry BF16 table once (nf4_table),
// then feeds eight v_mfma_f32_16x16x32_bf16 with eight weights each.  The
// MFMA pairs A lane (m, g) with B lane (n, g), so lane group g of the X
// operand reads the same 64 columns.  Codes and scales of a step (into
// registers) and its X rows (straight into LDS) are loaded kRing - 1 steps
// ahead, in the order they are used, so a wait never holds a later step's
// loads.  At the end of a tile (or of the range) the workgroup writes its
// FP32 partial of that tile.
//
// Finish (k_gemv_finish, one workgroup per 64 output columns): adds a
// tile's partials in slot order, forms T from the chunk partials in chunk
// order, applies the LoRA term by MFMA and rounds Y.  No workgroup waits on
// another and no device-wide fence is needed.
#include "qlora_device.h"
#include "qlora_kernels.h"

#include <algorithm>

namespace qlora {

// Buffer descriptor of a workgroup-uniform range, in scalar registers.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t gemv_rsrc(const void* base, int64_t bytes) {
  const int32_t n = bytes > 0x7FFFFFFF ? 0x7FFFFFFF : (bytes < 0 ? 0 : (int32_t)bytes);
  const uint64_t b = reinterpret_cast<uint64_t>(base);
  const uint64_t bu = ((uint64_t)(uint32_t)__builtin_amdgcn_readfirstlane((int)(b >> 32)) << 32) |
                      (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)b);
  return __builtin_amdgcn_make_buffer_rsrc(reinterpret_cast<void*>(bu), 0,
                                           __builtin_amdgcn_readfirstlane(n), 0x00020000);
}

// Offset beyond every buffer descriptor: the load returns zero without
// memory traffic.
constexpr uint32_t kOutOfRange = 0x80000000u;

// --------------------------------------------------------------- T tasks
// T task t of a layer, by the four wavefronts of a workgroup: rank block
// rb = t % ceil(r / 16), chunk c = t / ceil(r / 16).  The chunk's columns
// are kTParts consecutive equal parts (32 x tchunk_ss columns each, the last
// ones shorter or empty at d_in); wavefront w sums parts 2 w and 2 w + 1,
// each by MFMA over its 32-wide k steps in order, lane (r16, g) reading XA
// row r16 and A row 16 rb + r16 at columns k + 8 g (rows past M or r read
// zero), kTRound steps of both parts per round of loads.  The parts are
// then added in part order through `red` (kTParts x 256 floats of LDS).
// Ends with a barrier: `red` may be reused at once.
constexpr int kTParts = 8;
constexpr int kTRound = 4;
static_assert(kTParts * 256 * 4 <= kGemvRing * 16 * 512, "T reduction buffer inside the X ring");

__device__ __forceinline__ void t_task(const GemvDesc& d, int M, int t, int w, int lane,
                                       float* red) {
  const int nrb = (int)((d.r + 15) / 16);
  const int rb = t % nrb, c = t / nrb;
  const int r16 = lane & 15, g = lane >> 4;
  const uint32_t din = (uint32_t)d.d_in;
  const __amdgpu_buffer_rsrc_t rx = gemv_rsrc(d.XA, (int64_t)M * d.d_in * 2);
  const __amdgpu_buffer_rsrc_t ra = gemv_rsrc(d.A, d.r * d.d_in * 2);
  const uint32_t xrow = (uint32_t)r16 * din, arow = (uint32_t)(16 * rb + r16) * din;
  const uint32_t q = (uint32_t)d.tchunk_ss * 32u;               // part width
  const uint32_t c0 = (uint32_t)c * q * kTParts;
  uint32_t k0[2], k1[2];
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const uint32_t b = c0 + q * (2 * w + h);
    k0[h] = b < din ? b : din;
    k1[h] = b + q < din ? b + q : din;                          // d_in: a multiple of 64
  }
  f32x4 acc[2] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
  for (uint32_t kb = 0; kb < q; kb += 32 * kTRound) {
    u32x4 x[2][kTRound], v[2][kTRound];
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int j = 0; j < kTRound; ++j) {
        const uint32_t k = k0[h] + kb + 32 * j;
        const bool in = k < k1[h];
        x[h][j] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(
                                                rx, in ? (xrow + k + 8 * g) * 2 : kOutOfRange, 0, 0));
        v[h][j] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(
                                                ra, in ? (arow + k + 8 * g) * 2 : kOutOfRange, 0, 0));
      }
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int j = 0; j < kTRound; ++j) acc[h] = mfma16(x[h][j], v[h][j], acc[h]);
  }
  // accumulator lane (r16, g): rows m = 4 g + e, rank 16 rb + r16
#pragma unroll
  for (int h = 0; h < 2; ++h)
#pragma unroll
    for (int e = 0; e < 4; ++e) red[((2 * w + h) * 16 + 4 * g + e) * 16 + r16] = acc[h][e];
  __syncthreads();
  {
    const int m = threadIdx.x >> 4, i = threadIdx.x & 15;
    float sum = red[threadIdx.x];
#pragma unroll
    for (int p = 1; p < kTParts; ++p) sum = __fadd_rn(sum, red[p * 256 + threadIdx.x]);
    if (m < M && 16 * rb + i < d.r) d.tpart[((int64_t)c * M + m) * d.r + 16 * rb + i] = sum;
  }
  __syncthreads();
}

// The T tasks alone: one workgroup per task.
__global__ __launch_bounds__(256) void k_gemv_tasks(GemvArgs a) {
  __shared__ float red[kTParts * 256];
  const int task = blockIdx.x;
  const int di = group_index(a.count, task, [&](int i) { return a.d[i].task_begin; });
  const GemvDesc& d = a.d[di];
  t_task(d, a.M, task - d.task_begin, __builtin_amdgcn_readfirstlane(threadIdx.x >> 6),
         threadIdx.x & 63, red);
}

// ------------------------------------------------------ weight streaming
// Codes and scales of one step for one lane.
struct StepData {
  u32x4 c[2];       // the 32 code bytes of the lane's block
  uint32_t sc;      // FP8 scale code
  float s2;         // second-level scale
};

// Loop-invariant addressing of one layer for one lane, and the per-tile
// descriptors of the weight cursor.
struct LayerLanes {
  __amdgpu_buffer_rsrc_t rc, rs;   // codes and scale codes from the cursor's tile
  __amdgpu_buffer_rsrc_t r2, rx;   // second-level scales; X
  uint32_t vc, vs;                 // lane offsets inside a tile (codes, scale codes)
  int64_t blk;                     // lane's first-level block at the cursor's tile, step 0
};

__device__ __forceinline__ void tile_rsrc(const GemvDesc& d, int tile, int rl, int g,
                                          LayerLanes& L) {
  const int64_t half = d.d_in / 2, nblk = d.d_in / kBlock;
  const int64_t row0 = (int64_t)tile * kGemvRows;
  L.rc = gemv_rsrc(d.codes + row0 * half, (d.d_out - row0) * half);
  L.rs = gemv_rsrc(d.scodes + row0 * nblk, (d.d_out - row0) * nblk);
  L.blk = (row0 + rl) * nblk + g;
}

// Loads of step ss at the cursor's tile.  Rows past d_out read as zero
// (descriptor bounds); blocks past d_in read whatever lies there and get
// scale zero in the compute.  A step past the range (valid false) loads
// from offsets beyond every descriptor, which return zero without memory
// traffic: the loads are issued on every path, so the compiler's wait
// counts stay exact.
constexpr int kRing = kGemvRing;   // steps of weights (registers) and X (LDS): loaded kRing - 1 ahead
__device__ __forceinline__ void load_step(const LayerLanes& L, int ss, bool valid, StepData& s) {
  const uint32_t so_c = valid ? (uint32_t)ss * 128u : kOutOfRange;
  const uint32_t so_s = valid ? (uint32_t)ss * 4u : kOutOfRange;
  s.c[0] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(L.rc, L.vc, so_c, 0));
  s.c[1] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(L.rc, L.vc + 16, so_c, 0));
  s.sc = __builtin_amdgcn_raw_buffer_load_b8(L.rs, L.vs, so_s, 0);
  const uint32_t grp = (uint32_t)((L.blk + (int64_t)ss * 4) >> 8);
  s.s2 = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(L.r2, grp * 4u,
                                                                        valid ? 0u : kOutOfRange, 0));
}

// X of super-step ss straight into its LDS slot (16 rows of 512 bytes, the
// rows past M zero): wavefront w issues two loads, each filling rows
// 4 w + 2 i and 4 w + 2 i + 1, lane l landing at byte 16 l.  Piece c (columns
// 8 c .. 8 c + 7) of row R sits at position c ^ (R & 15) of the row, so that
// the sixteen rows' fragment reads of one MFMA hit distinct banks.  Pieces
// past M, d_in or the range read zero.
constexpr int kXRowBytes = 512;
constexpr int kXSlotBytes = 16 * kXRowBytes;
__device__ __forceinline__ void dma_x(__amdgpu_buffer_rsrc_t rx, uint32_t din, int M, int ss,
                                      bool valid, int w, int lane, uint8_t* slot) {
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int row0 = 4 * w + 2 * i;
    const int R = row0 + (lane >> 5);
    const uint32_t c = (uint32_t)((lane & 31) ^ (R & 15));
    const uint32_t col = (uint32_t)ss * 256u + 8u * c;
    const bool in = valid && R < M && col < din;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(
        rx, (__attribute__((address_space(3))) void*)(slot + row0 * kXRowBytes), 16,
        in ? ((uint32_t)R * din + col) * 2 : kOutOfRange, 0, 0, 0);
  }
}

// Wait until at most N vector-memory operations of this wavefront are
// outstanding (loads straight into LDS count as such; the compiler's fence
// at a barrier does not track them).
template <int N>
__device__ __forceinline__ void wait_vmem() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
}

// The eight MFMAs of a step: X fragment j (columns 64 g + 8 j of the step)
// from the lane's staged row, the weights (natural element order) from its
// block's table.  A block past d_in (ok false) gets scale 0.
__device__ __forceinline__ void compute_step(const StepData& s, bool ok, float mean,
                                             const uint8_t* xrow, int swz, int g, f32x4& acc) {
  const Nf4Table tab = nf4_table(restored_scale(s.sc, ok ? s.s2 : 0.0f, ok ? mean : 0.0f));
  const uint32_t cw[8] = {s.c[0].x, s.c[0].y, s.c[0].z, s.c[0].w,
                          s.c[1].x, s.c[1].y, s.c[1].z, s.c[1].w};
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    u32x4 xf[4];
#pragma unroll
    for (int j = 0; j < 4; ++j)
      xf[j] = *reinterpret_cast<const u32x4*>(xrow + 16 * ((8 * g + 4 * h + j) ^ swz));
#pragma unroll
    for (int j = 0; j < 4; ++j) acc = mfma16(xf[j], nf4_dequant8(cw[4 * h + j], tab), acc);
  }
}

// Barrier between the steps of the ring.  The only LDS writes inside the
// loop are loads straight into LDS, which each wavefront has waited for
// (wait_vmem) right before; a plain s_barrier then orders them for every
// wavefront.  (__syncthreads would add a fence that waits for every such
// load in flight, the later steps' included, and so shorten the ring to one
// step.)  The empty asm and sched_barrier keep the compiler from moving
// memory operations or other instructions across it.
__device__ __forceinline__ void ring_barrier() {
  __builtin_amdgcn_sched_barrier(0);
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
  __builtin_amdgcn_sched_barrier(0);
}

__global__ __launch_bounds__(256) void k_gemv(GemvArgs a) {
  extern __shared__ __attribute__((aligned(16))) uint8_t xs[];
  const int wg = blockIdx.x;
  const int di = group_index(a.count, wg, [&](int i) { return a.d[i].wg_begin; });
  const GemvDesc& d = a.d[di];
  const int j = wg - d.wg_begin;                    // workgroup within the layer
  const int c0 = gemv_unit_begin(j, d.uq, d.urem), c1 = gemv_unit_begin(j + 1, d.uq, d.urem);
  const int M = a.M;
  const int lane = threadIdx.x & 63, w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  // the T tasks that start in the range, then its weight units
  for (int t = (c0 + d.tcost - 1) / d.tcost; t < d.n_tasks && t * d.tcost < c1; ++t)
    t_task(d, M, t, w, lane, reinterpret_cast<float*>(xs));
  const int u0 = (c0 > d.toff ? c0 : d.toff) - d.toff;
  const int u1 = (c1 > d.toff ? c1 : d.toff) - d.toff;
  if (u0 >= u1) return;
  const int r16 = lane & 15, g = lane >> 4;
  const int rl = 16 * w + r16;                       // lane's row in the tile
  const int nss = d.nss;
  const int64_t half = d.d_in / 2, nblk = d.d_in / kBlock;
  const uint32_t din = (uint32_t)d.d_in;

  const float mean = d.mean[0];                     // loaded before the ring's loads
  LayerLanes L;
  L.r2 = gemv_rsrc(d.scale2, ((d.d_out * nblk + kGroup - 1) / kGroup) * 4);
  L.rx = gemv_rsrc(d.X, (int64_t)M * d.d_in * 2);
  L.vc = (uint32_t)(rl * half + 32 * g);
  L.vs = (uint32_t)(rl * nblk + g);

  // cursors: computed step (tile tc, step sc); loaded X and weights (step sw
  // of tile tw, kRing - 1 ahead)
  int tc = u0 / nss, sc = u0 % nss;
  int tw = tc, sw = sc;
  tile_rsrc(d, tw, rl, g, L);
  StepData st[kRing];
#pragma unroll
  for (int i = 0; i < kRing - 1; ++i) {
    dma_x(L.rx, din, M, sw, u0 + i < u1, w, lane, xs + i * kXSlotBytes);
    load_step(L, sw, u0 + i < u1, st[i]);
    if (++sw == nss) { sw = 0; tile_rsrc(d, ++tw, rl, g, L); }
  }

  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  const int xrow = r16 * kXRowBytes;                // lane's row; rows past M are zero
  const int swz = r16 & 15;
  int tile_first = tc * nss;                        // first unit of the current tile
  // unrolled by the ring depth, so that every ring index is static; every
  // load is issued (past the range: zero, no traffic), only the compute of
  // steps past the range is skipped
  for (int ub = u0; ub < u1; ub += kRing) {
#pragma unroll
    for (int k = 0; k < kRing; ++k) {
      const int u = ub + k;
      // this step's X: its own loads done (at most the weights of this step
      // and the loads of the kRing - 2 later steps still in flight), then
      // every wavefront's (and every wavefront is done with the slot the
      // next loads overwrite)
      wait_vmem<4 + 6 * (kRing - 2)>();
      ring_barrier();
      dma_x(L.rx, din, M, sw, u + kRing - 1 < u1, w, lane,
            xs + ((k + kRing - 1) % kRing) * kXSlotBytes);
      load_step(L, sw, u + kRing - 1 < u1, st[(k + kRing - 1) % kRing]);
      __builtin_amdgcn_sched_barrier(0);            // loads issued before the step's math
      if (u < u1) {
        const bool ok = (int64_t)sc * 4 + g < nblk;
        compute_step(st[k], ok, mean, xs + k * kXSlotBytes + xrow, swz, g, acc);
        // end of the tile's run in this workgroup: write the partial
        if (sc + 1 == nss || u + 1 == u1) {
          const int slot = j - gemv_wg_of(d.toff + tile_first, d.uq, d.urem);
          const int64_t n = (int64_t)tc * kGemvRows + rl;
#pragma unroll
          for (int v = 0; v < 4; ++v) {
            const int m = 4 * g + v;
            if (m < M && n < d.d_out) d.part[((int64_t)slot * M + m) * d.d_out + n] = acc[v];
          }
          acc = f32x4{0.f, 0.f, 0.f, 0.f};
        }
      }
      if (++sc == nss) {
        sc = 0;
        ++tc;
        tile_first += nss;
      }
      if (++sw == nss) {
        sw = 0;
        tile_rsrc(d, ++tw, rl, g, L);
      }
    }
  }
}

// Finish: one workgroup per 64 output columns of a layer; wavefront w takes
// columns 16 w .. 16 w + 15, lane (n = l%16, g = l/16) rows 4 g .. 4 g + 3
// as in the MFMA accumulator.
//   acc = sum_s part[s]                      (slots of the tile, in order)
//   T   = t_scale * sum_c tpart[c]            (chunks in order; the workgroup
//                                             shares the work and keeps T in
//                                             LDS as its BF16 hi and lo parts)
//   acc += [T_hi | T_lo] [B | B]^T           (two MFMAs per 32 ranks)
//   Y   = RNE_bf16(acc)
// Every global load is issued before the first wait; loads that no lane of
// a wavefront needs are skipped by wavefront-uniform branches, and a lane
// whose element does not exist reads at an offset past its buffer
// descriptor (zero, no traffic).  kVecB: B rows are read 16
// bytes at a time (r % 8 == 0, B 16-byte aligned), else element by element.
constexpr int kFinMaxT = 16 * 256;             // M x r at most
template <bool kVecB>
__global__ __launch_bounds__(256) void k_gemv_finish(GemvArgs a) {
  __shared__ uint32_t thl[kFinMaxT];           // (hi | lo << 16) of T[m][i] at m * rp + i
  const int wg = blockIdx.x;
  const int di = group_index(a.count, wg, [&](int i) { return a.d[i].fin_begin; });
  const GemvDesc& d = a.d[di];
  const int ct = wg - d.fin_begin;                 // 64-column tile
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int wu = __builtin_amdgcn_readfirstlane(w);
  const int r16 = lane & 15, g = lane >> 4;
  const int M = a.M;
  const uint32_t dout = (uint32_t)d.d_out;
  const uint32_t n = (uint32_t)ct * 64u + 16u * w + r16;
  const bool col_ok = n < dout;
  const int ufirst = d.toff + ct * d.nss;
  const int s0 = gemv_wg_of(ufirst, d.uq, d.urem);
  const int ns = gemv_wg_of(ufirst + d.nss - 1, d.uq, d.urem) - s0 + 1;
  const int r = (int)d.r, rp = (r + 31) & ~31;
  const __amdgpu_buffer_rsrc_t rb = gemv_rsrc(d.B, d.d_out * d.r * 2);
  const __amdgpu_buffer_rsrc_t rpart = gemv_rsrc(d.part, (int64_t)kGemvMaxSlots * M * d.d_out * 4);
  const __amdgpu_buffer_rsrc_t rtp = gemv_rsrc(d.tpart, (int64_t)d.tchunks * M * d.r * 4);

  // B fragments (column n, ranks 32 c + 8 g ..), the tile's partials, then
  // the chunk partials of T for the elements e = m * r + i this thread adds
  // (kTGroup per pass)
  constexpr int kRankChunks = 256 / 32;
  u32x4 bw[kRankChunks];
#pragma unroll
  for (int c = 0; c < kRankChunks; ++c) {
    const uint32_t kk = 32u * c + 8u * g;
    if (kVecB) {
      const uint32_t off = col_ok && kk < (uint32_t)r ? (n * r + kk) * 2 : kOutOfRange;
      bw[c] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rb, off, 0, 0));
    } else {
      uint32_t h[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const uint32_t off = col_ok && kk + e < (uint32_t)r ? (n * r + kk + e) * 2 : kOutOfRange;
        h[e] = __builtin_amdgcn_raw_buffer_load_b16(rb, off, 0, 0);
      }
      bw[c] = u32x4{h[0] | (h[1] << 16), h[2] | (h[3] << 16), h[4] | (h[5] << 16),
                    h[6] | (h[7] << 16)};
    }
  }
  float pv[kGemvMaxSlots][4];
#pragma unroll
  for (int s = 0; s < kGemvMaxSlots; ++s)
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int m = 4 * g + v;
      pv[s][v] = 0.0f;
      if (s >= ns || v >= M) continue;             // uniform: no loads issued
      const uint32_t off = m < M && col_ok ? ((uint32_t)(s * M + m) * dout + n) * 4 : kOutOfRange;
      pv[s][v] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rpart, off, 0, 0));
    }

  // T to LDS, scaled and split into BF16 hi + lo (ranks in [r, rp) zero)
  constexpr int kTGroup = 2;
  const int te = M * r;
  for (int e0 = 0; e0 < te; e0 += 256 * kTGroup) {
    float tv[kGemvMaxChunks][kTGroup];
#pragma unroll
    for (int c = 0; c < kGemvMaxChunks; ++c)
#pragma unroll
      for (int q = 0; q < kTGroup; ++q) {
        const int e = e0 + threadIdx.x + 256 * q;
        tv[c][q] = 0.0f;
        // uniform: no loads issued by a wavefront with no element here
        if (c >= d.tchunks || e0 + 256 * q + 64 * wu >= te) continue;
        const uint32_t off = e < te ? (uint32_t)(c * te + e) * 4 : kOutOfRange;
        tv[c][q] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rtp, off, 0, 0));
      }
#pragma unroll
    for (int q = 0; q < kTGroup; ++q) {
      const int e = e0 + threadIdx.x + 256 * q;
      if (e < te) {
        float sum = tv[0][q];
#pragma unroll
        for (int c = 1; c < kGemvMaxChunks; ++c)
          if (c < d.tchunks) sum = __fadd_rn(sum, tv[c][q]);
        const int m = e / r, i = e - m * r;
        const float t = __fmul_rn(d.t_scale, sum);
        if (ct == 0 && d.T_save) d.T_save[e] = t;
        float hi, lo;
        split_bf16(t, hi, lo);
        thl[m * rp + i] = (__float_as_uint(hi) >> 16) | (pack_bf16x2(lo, 0.0f) << 16);
      }
    }
  }
  for (int e = threadIdx.x; e < M * (rp - r); e += 256) {
    const int m = e / (rp - r), i = r + e - m * (rp - r);
    thl[m * rp + i] = 0u;
  }

  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int s = 0; s < kGemvMaxSlots; ++s)
#pragma unroll
    for (int v = 0; v < 4; ++v)
      if (s < ns) acc[v] = s == 0 ? pv[s][v] : __fadd_rn(acc[v], pv[s][v]);
  __syncthreads();

#pragma unroll
  for (int c = 0; c < kRankChunks; ++c) {
    const int kk = 32 * c + 8 * g;
    if (32 * c >= r) break;
    // A operand: T of row r16 (zero past M), ranks kk .. kk + 7
    u32x4 ah = {0u, 0u, 0u, 0u}, al = {0u, 0u, 0u, 0u};
    if (r16 < M) {
      const uint32_t* tr = thl + r16 * rp + kk;
      uint32_t h[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) h[e] = tr[e];
      ah = u32x4{(h[0] & 0xFFFFu) | (h[1] << 16), (h[2] & 0xFFFFu) | (h[3] << 16),
                 (h[4] & 0xFFFFu) | (h[5] << 16), (h[6] & 0xFFFFu) | (h[7] << 16)};
      al = u32x4{(h[0] >> 16) | (h[1] & 0xFFFF0000u), (h[2] >> 16) | (h[3] & 0xFFFF0000u),
                 (h[4] >> 16) | (h[5] & 0xFFFF0000u), (h[6] >> 16) | (h[7] & 0xFFFF0000u)};
    }
    acc = mfma16(ah, bw[c], acc);
    acc = mfma16(al, bw[c], acc);
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

hipError_t launch_gemv_tasks(const GemvArgs& a, hipStream_t st) {
  if (a.tasks == 0) return hipSuccess;
  hipLaunchKernelGGL(k_gemv_tasks, dim3(a.tasks), dim3(256), 0, st, a);
  return hipGetLastError();
}

hipError_t launch_gemv(const GemvArgs& a, hipStream_t st) {
  weight_kernel_begin(st);
  hipLaunchKernelGGL(k_gemv, dim3(a.wgs), dim3(256), (unsigned)gemv_lds_bytes(a.M), st, a);
  weight_kernel_end(st);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (a.vec_b)
    hipLaunchKernelGGL(k_gemv_finish<true>, dim3(a.fin_wgs), dim3(256), 0, st, a);
  else
    hipLaunchKernelGGL(k_gemv_finish<false>, dim3(a.fin_wgs), dim3(256), 0, st, a);
  return hipGetLastError();
}

}  // namespace qlora
