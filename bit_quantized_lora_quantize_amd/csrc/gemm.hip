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
// 256 x 256; K step 32 (half a quantization block).  Each wavefront owns a
// 128 x 128 sub-tile: 4 x 4 tiles of v_mfma_f32_32x32x16_bf16 with 256 FP32
// accumulators per lane, two K slices of 16 per step.
//
// Pipeline (three LDS buffers, two register stages).  During step s the
// matrix cores consume buffer s%3 while the same wavefronts
//   * read the operand fragments of the next K slice into the second
//     fragment register set (slice 1 of step s, then slice 0 of step s+1,
//     whose buffer was completed one barrier earlier),
//   * restore step s+2 into buffer (s+2)%3 from registers loaded two steps
//     earlier (activations copied, weights looked up in the block's
//     16-entry table), and
//   * issue the global loads of step s+4 into the freed register stage.
// One barrier per step; no wavefront waits on LDS data written in the same
// step.  The restore work (about four VALU instructions per MFMA) is spread
// between the MFMAs of the step.
//
// Forward   Y[m][n]  = sum_k X[m][k] Wh[n][k]   (+ LoRA: T_hi/T_lo x B^T)
//   LDS  As[m][k] = X permuted within each eight; Bs[n][k] = table lookups in
//        the same permuted order (nf4_dequant8_perm).  Both fragments are
//        16-byte LDS reads.
// Backward  dX[m][c] = sum_n dY[m][n] Wh[n][c]  (+ LoRA: U_hi/U_lo x A)
//   LDS  As[m][k] = dY; Bs[k][c] = restored weight rows as stored (row n of
//        W, columns permuted within each eight).  The B fragments (eight
//        consecutive k of one column per lane) come from two transposing LDS
//        reads (ds_read_b64_tr_b16); the column permutation is undone when
//        the result is stored.
// LoRA term: extra K steps over [hi(0..RP) | lo(0..RP)], RP = r rounded up
// to 32, from the rank-r activations split into two BF16 terms beforehand.
// They run before the weight steps, so with LoRA dropout ([QP §6.3]) the
// backward clears the dropped positions of that term in the accumulators
// before the base term is added.
//
// Workgroup order: consecutive workgroup ids are spread over the 8 XCDs, so
// ids are remapped for each XCD to own a contiguous run of output tiles
// (same activation rows, neighbouring weight rows) in its own L2.
#include "qlora_device.h"
#include "qlora_kernels.h"

namespace qlora {

constexpr int BM = 256, BN = 256, BK = 32;
constexpr int kNumBuf = 3;
constexpr int LDA = BK + 8;                  // As[m][k], forward Bs[n][k] row (BF16 elements)
constexpr int LDT = BN + 16;                 // backward Bs[k][c] row: 136 dwords, = 8 mod 32
constexpr int kABytes = BM * LDA * 2;
constexpr int kBFwdBytes = BN * LDA * 2;
constexpr int kBBwdBytes = BK * LDT * 2;
template <bool BWD>
constexpr int buf_bytes() { return kABytes + (BWD ? kBBwdBytes : kBFwdBytes); }
template <bool BWD>
constexpr int lds_bytes() { return kNumBuf * buf_bytes<BWD>(); }
constexpr int kXcds = 8;
// VALU instructions placed after each MFMA of the two halves of a step
#ifndef QLORA_GEMM_V1
#define QLORA_GEMM_V1 3
#endif
#ifndef QLORA_GEMM_V2
#define QLORA_GEMM_V2 5
#endif

typedef short v4i16 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) v4i16 lds_v4i16;

// Buffer descriptor of a workgroup-uniform range, read through scalar
// registers so that every load using it is a single instruction.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, int64_t bytes) {
  const int32_t n = bytes > 0x7FFFFFFF ? 0x7FFFFFFF : (bytes < 0 ? 0 : (int32_t)bytes);
  const uint64_t b = reinterpret_cast<uint64_t>(base);
  const uint64_t bu = ((uint64_t)(uint32_t)__builtin_amdgcn_readfirstlane((int)(b >> 32)) << 32) |
                      (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)b);
  return __builtin_amdgcn_make_buffer_rsrc(reinterpret_cast<void*>(bu), 0,
                                           __builtin_amdgcn_readfirstlane(n), 0x00020000);
}
__device__ __forceinline__ u32x4 ld128(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
  return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, 0));
}

// Global data of one K step held in registers between load and restore.
struct Stage {
  u32x4 x[4];     // activation rows of the thread: 4 x 8 BF16
  u32x4 c;        // 32 packed NF4 codes: one weight row segment
  uint32_t sc;    // FP8 code of the segment's block scale
  float s2;       // its FP32 second-level scale
};

struct Frags {
  u32x4 a[4], b[4];
};

// Per-thread constants of a tile.
struct Tile {
  int64_t m0, n0, K, NOUT;
  int nk;                          // NF4 K steps
  __amdgpu_buffer_rsrc_t act;      // activations from row m0
  __amdgpu_buffer_rsrc_t s2;       // whole second-level scale array
  uint32_t vx;                     // activation byte offset of pass 0
  uint32_t sx;                     // activation byte stride between passes (64 rows)
  // forward weights (tile rows n0 ..)
  __amdgpu_buffer_rsrc_t codes, scodes;
  uint32_t vc, vs;                 // byte offsets of the thread's row
  int64_t blk0;                    // block index of the row's first block
  // backward weights: row segment (k0 + nl, columns c0 + 32 * cg ..)
  int nl, cg;
  float mu;
  // LDS offsets (bytes, relative to a buffer)
  uint32_t wa, wb;                 // restore stores
  uint32_t ra, rb;                 // fragment reads
  // activations loaded straight into LDS (unpadded 64-byte rows, 16-byte
  // pieces swizzled): global offset of the lane's piece in pass 0, the
  // LoRA-step store offset, and the fragment read offset of slice 0
  uint32_t vd, wad, rad;
};

// ------------------------------------------------------------------ loads
// VEC: activation rows 16-byte aligned (K % 8 == 0); always so in the
// forward direction (K = d_in, a multiple of 64).  WIDE (backward): the
// packed weights exceed what one buffer descriptor reaches with 32-bit
// offsets, so each step builds descriptors based at its own rows; otherwise
// one descriptor per tile serves every step through its scalar offset.
template <bool BWD, bool VEC, bool DMA, bool WIDE>
__device__ __forceinline__ void load_step(const GemmArgs& p, const Tile& t, int step,
                                          bool with_scale, Stage& g) {
  const uint32_t k0 = (uint32_t)step * BK;
  if (DMA) {
    // activations go straight to LDS (dma_act)
  } else if (!BWD || VEC) {
#pragma unroll
    for (int q = 0; q < 4; ++q) g.x[q] = ld128(t.act, t.vx + q * t.sx, k0 * 2);
  } else {
    // unaligned rows (backward, d_out % 8 != 0): element loads, zero past K
    const int64_t kc = (int64_t)k0 + 8 * ((threadIdx.x & 63) >> 4);
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      uint32_t e2[8];
#pragma unroll
      for (int e = 0; e < 8; ++e)
        e2[e] = (kc + e < t.K) ? (uint32_t)__builtin_amdgcn_raw_buffer_load_b16(
                                     t.act, t.vx + q * t.sx + (k0 + e) * 2, 0, 0)
                               : 0u;
      g.x[q] = u32x4{e2[0] | (e2[1] << 16), e2[2] | (e2[3] << 16), e2[4] | (e2[5] << 16),
                     e2[6] | (e2[7] << 16)};
    }
  }
  if (!BWD) {
    g.c = ld128(t.codes, t.vc, k0 / 2);
    if (with_scale) {
      g.sc = __builtin_amdgcn_raw_buffer_load_b8(t.scodes, t.vs, k0 / 64, 0);
      const int64_t blk = t.blk0 + k0 / 64;
      g.s2 = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(t.s2, (uint32_t)(blk >> 8) * 4, 0, 0));
    }
  } else if (!WIDE) {
    // row k0 + nl of W, columns c0 + 32 cg .. +32
    const uint32_t nb = (uint32_t)(p.d_in / kBlock);
    g.c = ld128(t.codes, (uint32_t)(t.nl * (p.d_in / 2) + 16 * t.cg), k0 * (uint32_t)(p.d_in / 2));
    g.sc = __builtin_amdgcn_raw_buffer_load_b8(t.scodes, (uint32_t)t.nl * nb + (uint32_t)(t.cg >> 1),
                                               k0 * nb, 0);
    const int64_t blk = ((int64_t)k0 + t.nl) * nb + t.n0 / kBlock + (t.cg >> 1);
    g.s2 = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(t.s2, (uint32_t)(blk >> 8) * 4, 0, 0));
  } else {
    const int64_t row = (int64_t)k0;
    const int64_t nb = p.d_in / kBlock;
    const uint8_t* cbase = p.codes + row * (p.d_in / 2) + t.n0 / 2;
    const int64_t cbytes = p.d_out * (p.d_in / 2) - (row * (p.d_in / 2) + t.n0 / 2);
    const __amdgpu_buffer_rsrc_t rc = make_rsrc(cbase, cbytes);
    g.c = ld128(rc, (uint32_t)(t.nl * (p.d_in / 2) + 16 * t.cg), 0);
    const uint8_t* sbase = p.scodes + row * nb + t.n0 / kBlock;
    const int64_t sbytes = p.d_out * nb - (row * nb + t.n0 / kBlock);
    const __amdgpu_buffer_rsrc_t rs = make_rsrc(sbase, sbytes);
    g.sc = __builtin_amdgcn_raw_buffer_load_b8(rs, (uint32_t)(t.nl * nb + (t.cg >> 1)), 0, 0);
    const int64_t blk = (row + t.nl) * nb + t.n0 / kBlock + (t.cg >> 1);
    g.s2 = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(t.s2, (uint32_t)(blk >> 8) * 4, 0, 0));
  }
}

// Activations of a step straight into LDS: each of a wavefront's four
// 16-byte-per-lane buffer loads fills 1 KB of the buffer's activation
// region, rows 64 q + 16 w .. +16 of 64 bytes each, lane l landing at byte
// 16 l.  Lane l loads row 64 q + 16 w + l / 4, piece (l % 4) ^ ((l / 8) % 4)
// of the step's 32 columns, so that piece c of row m sits at byte
// 64 m + 16 (c ^ ((m / 2) % 4)) and the fragment reads are free of bank
// conflicts.  Rows past M read zero (bounds-checked loads).
__device__ __forceinline__ void dma_act(const Tile& t, int step, uint8_t* buf, int wu) {
  const uint32_t k0 = (uint32_t)step * BK;
#pragma unroll
  for (int q = 0; q < 4; ++q)
    __builtin_amdgcn_raw_ptr_buffer_load_lds(
        t.act, (__attribute__((address_space(3))) void*)(buf + (64 * q + 16 * wu) * 64), 16,
        t.vd + q * t.sx, k0 * 2, 0, 0);
}

// Wait until at most N vector-memory operations of this wavefront are
// outstanding (the loads straight into LDS count as such).  Every barrier
// after such loads carries its own wait: the compiler's fence at
// __syncthreads does not track them through every control-flow shape.
// Operations issued after the awaited ones (spill stores included) only make
// a count stricter.
template <int N>
__device__ __forceinline__ void wait_vmem() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
}

// ---------------------------------------------------------------- restore
// Activations: pass q of the thread covers row 64 q + 16 w + (lane & 15),
// columns 8 (lane >> 4) .. +8 of the step.
// EDGE: the step may be the last, partial one (backward K = d_out).
template <bool BWD, bool EDGE = true>
__device__ __forceinline__ void restore_act(const Tile& t, int step, const Stage& g, uint8_t* buf,
                                            int lane) {
  u32x4 v[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) v[q] = g.x[q];
  if (BWD && EDGE) {
    // last, partial step: contraction columns at or past K are zero
    const int64_t kc = (int64_t)step * BK + 8 * (lane >> 4);
    if ((int64_t)(step + 1) * BK > t.K && kc >= t.K) {
#pragma unroll
      for (int q = 0; q < 4; ++q) v[q] = u32x4{0u, 0u, 0u, 0u};
    }
  }
#pragma unroll
  for (int q = 0; q < 4; ++q)
    *reinterpret_cast<u32x4*>(buf + t.wa + q * 64 * LDA * 2) = BWD ? v[q] : perm8_bf16(v[q]);
}

template <bool BWD>
__device__ __forceinline__ void restore_table(const Tile& t, int step, const Stage& g,
                                              Nf4Table& tab) {
  float scale = restored_scale(g.sc, g.s2, t.mu);
  if (BWD && (int64_t)step * BK + t.nl >= t.K) scale = 0.0f;  // rows past d_out
  tab = nf4_table(scale);
}

// Eight weights (codes dword j of the segment) looked up and stored.  The
// forward with activations loaded straight into LDS keeps both operands in
// natural order; otherwise the weights take the lookup's own order (the
// activations are permuted to match on their way into LDS, the backward
// undoes the column order at the store).
template <bool NATURAL>
__device__ __forceinline__ void restore_dq(const Tile& t, int j, const Stage& g,
                                           const Nf4Table& tab, uint8_t* buf) {
  const uint32_t cw = j == 0 ? g.c.x : j == 1 ? g.c.y : j == 2 ? g.c.z : g.c.w;
  *reinterpret_cast<u32x4*>(buf + kABytes + t.wb + 16 * j) =
      NATURAL ? nf4_dequant8(cw, tab) : nf4_dequant8_perm(cw, tab);
}

template <bool BWD, bool DMA>
__device__ __forceinline__ void restore_w(const Tile& t, int step, const Stage& g, Nf4Table& tab,
                                          bool new_table, uint8_t* buf) {
  if (new_table) restore_table<BWD>(t, step, g, tab);
#pragma unroll
  for (int j = 0; j < 4; ++j) restore_dq<!BWD && DMA>(t, j, g, tab, buf);
}

// -------------------------------------------------------------- fragments
template <bool BWD, bool DMA>
__device__ __forceinline__ void read_frags(const Tile& t, const uint8_t* buf, int ks, Frags& f) {
  if (DMA) {
    // swizzled 64-byte rows: slice ks of row m is piece (2 ks + h) ^ ((m / 2) % 4)
    const uint32_t ra = t.rad ^ (32u * (uint32_t)ks);
#pragma unroll
    for (int i = 0; i < 4; ++i)
      f.a[i] = *reinterpret_cast<const u32x4*>(buf + ra + 32 * 64 * i);
  } else {
#pragma unroll
    for (int i = 0; i < 4; ++i)
      f.a[i] = *reinterpret_cast<const u32x4*>(buf + t.ra + (32 * i * LDA + 16 * ks) * 2);
  }
  if (!BWD) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
      f.b[i] = *reinterpret_cast<const u32x4*>(buf + kABytes + t.rb + (32 * i * LDA + 16 * ks) * 2);
  } else {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint8_t* pb = buf + kABytes + t.rb + (16 * ks * LDT + 32 * i) * 2;
      const v4i16 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16*)(pb));
      const v4i16 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16*)(pb + 4 * LDT * 2));
      const uint2 l2 = __builtin_bit_cast(uint2, lo), h2 = __builtin_bit_cast(uint2, hi);
      f.b[i] = u32x4{l2.x, l2.y, h2.x, h2.y};
    }
  }
}

__device__ __forceinline__ void mma_slice(const Frags& f, f32x16 (&acc)[4][4]) {
#pragma unroll
  for (int mt = 0; mt < 4; ++mt)
#pragma unroll
    for (int nt = 0; nt < 4; ++nt) acc[mt][nt] = mfma32(f.a[mt], f.b[nt], acc[mt][nt]);
}

// Interleave of half a steady-state step: each of its 16 MFMAs is followed
// by up to V VALU instructions and one LDS access; with VMEM, the global
// loads sit between the first eight.
template <int V, bool VMEM>
__device__ __forceinline__ void half_schedule() {
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);   // MFMA
    if (VMEM && i < 8) __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);  // VMEM read
    __builtin_amdgcn_sched_group_barrier(0x002, V, 0);   // VALU
    __builtin_amdgcn_sched_group_barrier(0x300, 1, 0);   // DS read / write
  }
}

// Steady-state K step s (s + 4 < nk).  Register stages hold the global data
// of three steps: gl receives step s+4 (issued first, so that the newest
// loads in flight are always a step old), gr holds step s+2, restored into
// bw during this step.  Buffer bc is consumed (fragments of slice 0 already
// in f0) and slice 0 of step s+1 is read from bn.  The three buffers and the
// stages are distinct.  The step runs as two halves of 16 MFMAs, each with
// about half the restore work.
template <bool BWD, bool VEC, bool DMA, bool WIDE, bool EVEN>
__device__ __forceinline__ void k_step_full(const GemmArgs& p, const Tile& t, int s,
                                            const uint8_t* __restrict__ bc,
                                            const uint8_t* __restrict__ bn,
                                            uint8_t* __restrict__ bw, const Stage& gr,
                                            Stage& gl, Nf4Table& tab, Frags& f0, Frags& f1,
                                            f32x16 (&acc)[4][4], int lane, int wu) {
  // even steps open a quantization block (forward); every backward step
  // holds new rows
  constexpr bool kTable = BWD || EVEN;
  constexpr int kFirst = kTable ? 1 : 2;   // lookups in the first half
  if (DMA) {
    // activations of step s + 2 straight into bw, ahead of this step's other loads
    dma_act(t, s + 2, bw, wu);
    __builtin_amdgcn_sched_barrier(0);
  }
  load_step<BWD, VEC, DMA, WIDE>(p, t, s + 4, kTable, gl);
  read_frags<BWD, DMA>(t, bc, 1, f1);
  mma_slice(f0, acc);
  if (!DMA) restore_act<BWD, false>(t, s + 2, gr, bw, lane);   // s + 2 < nk - 1: a full step
  if (kTable) restore_table<BWD>(t, s + 2, gr, tab);
#pragma unroll
  for (int j = 0; j < kFirst; ++j) restore_dq<!BWD && DMA>(t, j, gr, tab, bw);
  half_schedule<QLORA_GEMM_V1, true>();
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int j = kFirst; j < 4; ++j) restore_dq<!BWD && DMA>(t, j, gr, tab, bw);
  read_frags<BWD, DMA>(t, bn, 0, f0);
  mma_slice(f1, acc);
  half_schedule<QLORA_GEMM_V2, false>();
  // the activations of step s + 2 (loads started at the top of this step)
  // must be in LDS before the barrier, since the next step reads slice 0 of
  // step s + 2; only the weight loads issued after them (three with a new
  // table, else one) may stay in flight
  if (DMA) wait_vmem<kTable ? 3 : 1>();
  __syncthreads();
}

// Generic K step (any s < nk): the same work with the load, restore and
// next-step read skipped past the end.
template <bool BWD, bool VEC, bool DMA, bool WIDE, bool EVEN>
__device__ __forceinline__ void k_step(const GemmArgs& p, const Tile& t, int s,
                                       const uint8_t* bc, const uint8_t* bn, uint8_t* bw,
                                       const Stage& gr, Stage& gl, Nf4Table& tab, Frags& f0,
                                       Frags& f1, f32x16 (&acc)[4][4], int lane, int wu) {
  constexpr bool kTable = BWD || EVEN;
  if (DMA && s + 2 < t.nk) dma_act(t, s + 2, bw, wu);
  if (s + 4 < t.nk) load_step<BWD, VEC, DMA, WIDE>(p, t, s + 4, kTable, gl);
  read_frags<BWD, DMA>(t, bc, 1, f1);
  mma_slice(f0, acc);
  if (s + 2 < t.nk) {
    if (!DMA) restore_act<BWD>(t, s + 2, gr, bw, lane);
    restore_w<BWD, DMA>(t, s + 2, gr, tab, kTable, bw);
  }
  if (s + 1 < t.nk) read_frags<BWD, DMA>(t, bn, 0, f0);
  mma_slice(f1, acc);
  if (DMA) wait_vmem<0>();   // this step's loads straight into LDS, whatever was issued
  __syncthreads();
}

// LoRA extension steps: As[m][j] = ext[m][e0 + j]; forward Bs[n][j] =
// B[n][kappa], backward Bs[j][c] = A[kappa][c], with kappa = (e0 + j) mod
// RP and zero where kappa >= r.  Loaded into registers one step ahead of
// the LDS store.
struct ExtStage {
  u32x4 a[4];   // ext rows, same thread mapping as the activation restore
  u32x4 b[4];   // factor: forward row n = tid, 32 columns; backward row nl, 32 columns
};

template <bool BWD>
__device__ __forceinline__ void ext_load(const GemmArgs& p, const Tile& t, int64_t e0, int64_t RP,
                                         int tid, int lane, ExtStage& E) {
  const int w = tid >> 6;
  const __amdgpu_buffer_rsrc_t re = make_rsrc(p.ext + t.m0 * 2 * RP, (p.M - t.m0) * 2 * RP * 2);
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int row = 64 * q + 16 * w + (lane & 15);
    E.a[q] = ld128(re, (uint32_t)((row * 2 * RP + e0 + 8 * (lane >> 4)) * 2), 0);
  }
  const u32x4 z = {0u, 0u, 0u, 0u};
  if (!BWD) {
    const __amdgpu_buffer_rsrc_t rb = make_rsrc(p.lw + t.n0 * p.r, (p.d_out - t.n0) * p.r * 2);
    const bool vec = (p.r % 8) == 0 && (reinterpret_cast<uintptr_t>(p.lw) & 15u) == 0;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int64_t kap = (e0 + 8 * j) % RP;
      u32x4 v = z;
      if (vec) {
        if (kap < p.r) v = ld128(rb, (uint32_t)((tid * p.r + kap) * 2), 0);
      } else {
        uint32_t h[8];
#pragma unroll
        for (int e = 0; e < 8; ++e)
          h[e] = (kap + e < p.r) ? (uint32_t)__builtin_amdgcn_raw_buffer_load_b16(
                                       rb, (uint32_t)((tid * p.r + kap + e) * 2), 0, 0)
                                 : 0u;
        v = u32x4{h[0] | (h[1] << 16), h[2] | (h[3] << 16), h[4] | (h[5] << 16),
                  h[6] | (h[7] << 16)};
      }
      E.b[j] = v;
    }
  } else {
    const int64_t kap = (e0 + t.nl) % RP;
    const __amdgpu_buffer_rsrc_t ra = make_rsrc(p.lw + t.n0, (p.r * p.d_in - t.n0) * 2);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      u32x4 v = z;
      if (kap < p.r) v = ld128(ra, (uint32_t)((kap * p.d_in + 32 * t.cg + 8 * j) * 2), 0);
      E.b[j] = v;
    }
  }
}

template <bool BWD, bool DMA>
__device__ __forceinline__ void ext_store(const Tile& t, const ExtStage& E, uint8_t* buf) {
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    if (DMA)
      *reinterpret_cast<u32x4*>(buf + t.wad + q * 64 * 64) = E.a[q];   // swizzled 64-byte rows
    else
      *reinterpret_cast<u32x4*>(buf + t.wa + q * 64 * LDA * 2) = E.a[q];
  }
  // forward: both operands in natural order (the permutation within eights
  // belongs to the NF4 steps only); backward: factor columns in the order
  // of the restored weights, undone at the store
#pragma unroll
  for (int j = 0; j < 4; ++j)
    *reinterpret_cast<u32x4*>(buf + kABytes + t.wb + 16 * j) = BWD ? perm8_bf16(E.b[j]) : E.b[j];
}

template <bool BWD, bool VEC, bool DROP, bool DMA, bool WIDE>
__global__ __launch_bounds__(256) void k_gemm(GemmArgs p) {
  extern __shared__ __attribute__((aligned(16))) uint8_t lds[];

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int wm = w & 1, wn = w >> 1;
  const int r32 = lane & 31, h = lane >> 5;

  Tile t;
  t.NOUT = BWD ? p.d_in : p.d_out;
  t.K = BWD ? p.d_out : p.d_in;
  const int tiles_n = (int)((t.NOUT + BN - 1) / BN);
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
  t.n0 = (int64_t)(id % tiles_n) * BN;
  t.m0 = (int64_t)(id / tiles_n) * BM;
  t.nk = (int)((t.K + BK - 1) / BK);
  t.mu = p.mean[0];

  t.act = make_rsrc(p.act + t.m0 * t.K, (p.M - t.m0) * t.K * 2);
  t.vx = (uint32_t)(((16 * w + (lane & 15)) * t.K + 8 * (lane >> 4)) * 2);
  t.sx = (uint32_t)(64 * t.K * 2);
  const int64_t nb = p.d_in / kBlock;
  t.s2 = make_rsrc(p.scale2, ((p.d_out * nb + kGroup - 1) / kGroup) * 4);
  if (!BWD) {
    t.codes = make_rsrc(p.codes + t.n0 * (p.d_in / 2), (p.d_out - t.n0) * (p.d_in / 2));
    t.scodes = make_rsrc(p.scodes + t.n0 * nb, (p.d_out - t.n0) * nb);
    t.vc = (uint32_t)(tid * (p.d_in / 2));
    t.vs = (uint32_t)(tid * nb);
    t.blk0 = (t.n0 + tid) * nb;
    t.nl = 0;
    t.cg = 0;
    t.wb = (uint32_t)(tid * LDA * 2);
    t.rb = (uint32_t)(((128 * wn + r32) * LDA + 8 * h) * 2);
  } else {
    t.nl = tid & 31;
    t.cg = tid >> 5;
    if (!WIDE) {
      // whole rows of W from column c0 on; each step adds its rows as the
      // scalar offset
      t.codes = make_rsrc(p.codes + t.n0 / 2, p.d_out * (p.d_in / 2) - t.n0 / 2);
      t.scodes = make_rsrc(p.scodes + t.n0 / kBlock, p.d_out * nb - t.n0 / kBlock);
    }
    t.wb = (uint32_t)((t.nl * LDT + 32 * t.cg) * 2);
    // transposing read: lane group g = lane / 16 covers columns
    // 16 (g & 1) .. +16 and contraction rows 8 (g >> 1) .. +4 (first read)
    const int g = lane >> 4, j = lane & 15;
    t.rb = (uint32_t)(((8 * (g >> 1) + (j >> 2)) * LDT + 128 * wn + 16 * (g & 1) + 4 * (j & 3)) * 2);
  }
  t.wa = (uint32_t)(((16 * w + (lane & 15)) * LDA + 8 * (lane >> 4)) * 2);
  t.ra = (uint32_t)(((128 * wm + r32) * LDA + 8 * h) * 2);
  {
    // activation pieces straight into LDS: lane l of pass q holds row
    // 64 q + 16 w + l / 4, piece (l % 4) ^ ((l / 8) % 4); the LoRA-step store
    // and the fragment reads use the same swizzle
    const int lr = lane >> 2;
    t.vd = (uint32_t)(((16 * w + lr) * t.K + 8 * ((lane & 3) ^ ((lr >> 1) & 3))) * 2);
    const int er = lane & 15, ec = lane >> 4;
    t.wad = (uint32_t)((16 * w + er) * 64 + 16 * (ec ^ ((er >> 1) & 3)));
    t.rad = (uint32_t)((128 * wm + r32) * 64 + 16 * (h ^ ((r32 >> 1) & 3)));
  }
  const int wu = __builtin_amdgcn_readfirstlane(w);

  f32x16 acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f32x16{};

  // Global data of step j sits in register stage j % 3; step j is staged in
  // LDS buffer j % 3.
  Stage g0, g1, g2;
  Nf4Table tab;
  Frags f0, f1;
  const int nk = t.nk;
  uint8_t* const b0 = lds;
  uint8_t* const b1 = lds + buf_bytes<BWD>();
  uint8_t* const b2 = lds + 2 * buf_bytes<BWD>();

  // Steps 0 and 1 of the weights are loaded first; their latency is covered
  // by the LoRA term, which runs as the first K steps (over [hi | lo] of
  // the rank-r activations, buffers 0 and 1 alternating, each step's global
  // data loaded one step ahead).  Loads are unconditional: steps past K read
  // zeros (buffer loads are bounds-checked) and are never consumed.
  load_step<BWD, VEC, DMA, WIDE>(p, t, 0, true, g0);
  load_step<BWD, VEC, DMA, WIDE>(p, t, 1, BWD, g1);
  {
    const int64_t RP = (p.r + 31) / 32 * 32;
    const int ne = (int)(2 * RP / BK);
    ExtStage E;
    ext_load<BWD>(p, t, 0, RP, tid, lane, E);
    for (int e = 0; e < ne; ++e) {
      uint8_t* be = (e & 1) ? b1 : b0;
      ext_store<BWD, DMA>(t, E, be);
      if (e + 1 < ne) ext_load<BWD>(p, t, (int64_t)(e + 1) * BK, RP, tid, lane, E);
      __syncthreads();
      read_frags<BWD, DMA>(t, be, 0, f0);
      read_frags<BWD, DMA>(t, be, 1, f1);
      mma_slice(f0, acc);
      mma_slice(f1, acc);
    }
    __syncthreads();
  }
  if constexpr (DROP) {
    // LoRA dropout (backward): the accumulators hold the LoRA term alone
    // here; clear it at dropped (token, input) positions.  One keep word per
    // 32 x 32 tile: rows 32 i .. +32 of the wavefront's 128 (bit = row in
    // the tile, 8 (v / 4) + 4 h + v % 4 for element v) at the lane's column
    // 32 j + (permuted lane column).
    const int cj = (r32 & ~7) | (2 * (r32 & 3) + ((r32 >> 2) & 1));
    uint32_t kw[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int64_t m = t.m0 + 128 * wm + 32 * i;
        const int64_t c = t.n0 + 128 * wn + 32 * j + cj;
        kw[i][j] = (m < p.M && c < t.NOUT) ? p.keep[c * p.keep_ld + m / 32] : 0u;
      }
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const uint32_t bit = (kw[i][j] >> (8 * (v >> 2) + 4 * h + (v & 3))) & 1u;
          acc[i][j][v] = bit ? acc[i][j][v] : 0.0f;
        }
  }
  // weights: steps 0 and 1 restored, 2 and 3 in flight
  if (DMA) {
    // activations of steps 0 and 1 straight into their buffers, then the
    // weight loads of steps 2 and 3; both activation steps land before the
    // barrier, the weight loads (3 + 3 backward, 3 + 1 forward) may still be
    // in flight
    dma_act(t, 0, b0, wu);
    dma_act(t, 1, b1, wu);
    __builtin_amdgcn_sched_barrier(0);
  } else {
    restore_act<BWD>(t, 0, g0, b0, lane);
    restore_act<BWD>(t, 1, g1, b1, lane);
  }
  restore_w<BWD, DMA>(t, 0, g0, tab, true, b0);
  restore_w<BWD, DMA>(t, 1, g1, tab, BWD, b1);
  load_step<BWD, VEC, DMA, WIDE>(p, t, 2, true, g2);
  load_step<BWD, VEC, DMA, WIDE>(p, t, 3, BWD, g0);
  __builtin_amdgcn_sched_barrier(0);
  if (DMA) wait_vmem<3 + (BWD ? 3 : 1)>();
  __syncthreads();
  read_frags<BWD, DMA>(t, b0, 0, f0);

  // steady state: six steps per iteration (s = 0 mod 6), so that stage,
  // buffer and table parity are fixed for each of them.  A full step only
  // needs the next step to exist (it reads slice 0 of step s + 1): its
  // loads and restores for steps s + 2 and s + 4 past K read zeros or
  // in-bounds data that no step consumes, into buffers and registers already
  // consumed.  Activations copied through registers take the generic step
  // from two steps before the last one on, so that the last, partial step
  // clears its columns past K.
  constexpr int kMargin = DMA ? 7 : 10;   // iteration s runs while s + kMargin <= nk
  int s = 0;
  for (; s + kMargin <= nk; s += 6) {
    k_step_full<BWD, VEC, DMA, WIDE, true>(p, t, s + 0, b0, b1, b2, g2, g1, tab, f0, f1, acc, lane, wu);
    k_step_full<BWD, VEC, DMA, WIDE, false>(p, t, s + 1, b1, b2, b0, g0, g2, tab, f0, f1, acc, lane, wu);
    k_step_full<BWD, VEC, DMA, WIDE, true>(p, t, s + 2, b2, b0, b1, g1, g0, tab, f0, f1, acc, lane, wu);
    k_step_full<BWD, VEC, DMA, WIDE, false>(p, t, s + 3, b0, b1, b2, g2, g1, tab, f0, f1, acc, lane, wu);
    k_step_full<BWD, VEC, DMA, WIDE, true>(p, t, s + 4, b1, b2, b0, g0, g2, tab, f0, f1, acc, lane, wu);
    k_step_full<BWD, VEC, DMA, WIDE, false>(p, t, s + 5, b2, b0, b1, g1, g0, tab, f0, f1, acc, lane, wu);
  }
  for (; s < nk; s += 6) {
    k_step<BWD, VEC, DMA, WIDE, true>(p, t, s + 0, b0, b1, b2, g2, g1, tab, f0, f1, acc, lane, wu);
    if (s + 1 < nk) k_step<BWD, VEC, DMA, WIDE, false>(p, t, s + 1, b1, b2, b0, g0, g2, tab, f0, f1, acc, lane, wu);
    if (s + 2 < nk) k_step<BWD, VEC, DMA, WIDE, true>(p, t, s + 2, b2, b0, b1, g1, g0, tab, f0, f1, acc, lane, wu);
    if (s + 3 < nk) k_step<BWD, VEC, DMA, WIDE, false>(p, t, s + 3, b0, b1, b2, g2, g1, tab, f0, f1, acc, lane, wu);
    if (s + 4 < nk) k_step<BWD, VEC, DMA, WIDE, true>(p, t, s + 4, b1, b2, b0, g0, g2, tab, f0, f1, acc, lane, wu);
    if (s + 5 < nk) k_step<BWD, VEC, DMA, WIDE, false>(p, t, s + 5, b2, b0, b1, g1, g0, tab, f0, f1, acc, lane, wu);
  }

  // ---- epilogue: RNE to BF16, staged through LDS so that the global stores
  // are 16-byte row segments.  Accumulator element v of lane l holds row
  // 8*(v/4) + 4*(l/32) + v%4 and column l%32 of its 32 x 32 tile; in the
  // backward direction tile column j holds W column 8 (j/8) + sigma(j%8),
  // sigma = (0 2 4 6 1 3 5 7), the order of nf4_dequant8_perm.  Each
  // wavefront stages its 128 x 128 tile in two halves of 64 rows in a region
  // of its own (the last K step ended with a barrier). ----
  const int cj = BWD ? ((r32 & ~7) | (2 * (r32 & 3) + ((r32 >> 2) & 1))) : r32;
  constexpr int EPI_LD = 136;  // staged row, BF16 elements
  uint16_t* ep = reinterpret_cast<uint16_t*>(lds) + w * 64 * EPI_LD;
  const bool out_vec = (t.NOUT % 8) == 0;
#pragma unroll
  for (int half = 0; half < 2; ++half) {
#pragma unroll
    for (int mt2 = 0; mt2 < 2; ++mt2)
#pragma unroll
      for (int nt = 0; nt < 4; ++nt)
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int row = 32 * mt2 + 8 * (v >> 2) + 4 * h + (v & 3);
          f32x2 pr = {acc[2 * half + mt2][nt][v], 0.0f};
          ep[row * EPI_LD + 32 * nt + cj] = (uint16_t)(
              __builtin_bit_cast(uint32_t, __builtin_convertvector(pr, bf16x2)) & 0xFFFFu);
        }
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int idx = i * 64 + lane, row = idx >> 4, ch = idx & 15;
      const u32x4 v = *reinterpret_cast<const u32x4*>(ep + row * EPI_LD + 8 * ch);
      const int64_t m = t.m0 + 128 * wm + 64 * half + row;
      const int64_t n = t.n0 + 128 * wn + 8 * ch;
      if (m < p.M) {
        uint16_t* dst = p.out + m * t.NOUT + n;
        if (out_vec && n + 8 <= t.NOUT) {
          *reinterpret_cast<u32x4*>(dst) = v;
        } else {
          const uint32_t wv[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
          for (int e = 0; e < 8; ++e)
            if (n + e < t.NOUT) dst[e] = (uint16_t)(wv[e >> 1] >> (16 * (e & 1)));
        }
      }
    }
  }
}

template <bool BWD, bool VEC, bool DROP, bool DMA, bool WIDE = false>
static hipError_t launch_gemm(const GemmArgs& a, hipStream_t st) {
  static hipError_t attr = hipFuncSetAttribute(
      reinterpret_cast<const void*>(&k_gemm<BWD, VEC, DROP, DMA, WIDE>),
      hipFuncAttributeMaxDynamicSharedMemorySize, lds_bytes<BWD>());
  if (attr != hipSuccess) return attr;
  const int64_t NOUT = BWD ? a.d_in : a.d_out;
  const int64_t tiles = ((NOUT + BN - 1) / BN) * ((a.M + BM - 1) / BM);
  weight_kernel_begin(st);
  hipLaunchKernelGGL((k_gemm<BWD, VEC, DROP, DMA, WIDE>), dim3((unsigned)tiles), dim3(256),
                     lds_bytes<BWD>(), st, a);
  weight_kernel_end(st);
  return hipGetLastError();
}

hipError_t launch_gemm_fwd(const GemmArgs& a, hipStream_t st) {
  // K = d_in is a multiple of 64: every step's activations are whole rows
  return launch_gemm<false, true, false, true>(a, st);
}
template <bool WIDE>
static hipError_t launch_gemm_bwd_t(const GemmArgs& a, hipStream_t st) {
  // dY rows are 16-byte aligned exactly when d_out % 8 == 0; activations go
  // straight to LDS when every K step is whole (d_out % 32 == 0), else
  // through registers, which clear the columns past K of the last step
  const bool vec = (a.d_out % 8) == 0;
  const bool dma = (a.d_out % BK) == 0;
  if (a.keep) {
    if (dma) return launch_gemm<true, true, true, true, WIDE>(a, st);
    return vec ? launch_gemm<true, true, true, false, WIDE>(a, st)
               : launch_gemm<true, false, true, false, WIDE>(a, st);
  }
  if (dma) return launch_gemm<true, true, false, true, WIDE>(a, st);
  return vec ? launch_gemm<true, true, false, false, WIDE>(a, st)
             : launch_gemm<true, false, false, false, WIDE>(a, st);
}

// Largest packed-code size (bytes) that one descriptor per tile serves.  A
// test build sets it to 0 so that every backward takes the per-step path.
#ifndef QLORA_WIDE_CODE_BYTES
#define QLORA_WIDE_CODE_BYTES 0x7FFFFFFF
#endif

hipError_t launch_gemm_bwd(const GemmArgs& a, hipStream_t st) {
  // one descriptor over the packed codes reaches them all with 32-bit
  // offsets when they stay below 2^31 bytes (every weight of the 7B and 65B
  // models: at most 90 MB)
  const bool wide = a.d_out * (a.d_in / 2) > int64_t(QLORA_WIDE_CODE_BYTES);
  return wide ? launch_gemm_bwd_t<true>(a, st) : launch_gemm_bwd_t<false>(a, st);
}

}  // namespace qlora
