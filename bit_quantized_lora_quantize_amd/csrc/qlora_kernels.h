// qlora_kernels.h -- launch interfaces between the host library (api.cpp) and
// the HIP kernels of libqlora.  Internal; not part of the public C ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <algorithm>

#include "qlora.h"

namespace qlora {

// Event pair around the next weight-kernel launch: only in the timing build
// (QLORA_TIMING_HOOK, libqlora_timed.so) that benchmarks use to time single
// kernels; the library itself keeps no state and these are empty.
#ifdef QLORA_TIMING_HOOK
void weight_kernel_begin(hipStream_t st);
void weight_kernel_end(hipStream_t st);
#else
inline void weight_kernel_begin(hipStream_t) {}
inline void weight_kernel_end(hipStream_t) {}
#endif

// ----------------------------------------------------------- quantization
constexpr int kLutSize = 129;     // buckets floor(64 x) + 64 for x in [-1, 1]
constexpr int64_t kTreeLds = 4096; // top tree levels done in one workgroup

// Nearest-level decision table for x in [-1, 1]: bucket b covers
// [(b-64)/64, (b-63)/64) and idx = base[b] + (x >= thr[b]).
struct IndexLut {
  float thr[kLutSize];
  uint8_t base[kLutSize];
};

struct QuantWorkspace {
  float* absmax;  // [n1]
  double* part;   // [Gp] group sums, Gp = next power of two >= G
};

hipError_t launch_quantize(const float* W, int64_t n, uint8_t* codes, uint8_t* scale_codes,
                           float* scale2, float* mean, const QuantWorkspace& ws,
                           const IndexLut& lut, hipStream_t st);
// The top of the mean's tree: part[0..Gp) (Gp a power of two) summed by the
// stride-halving tree, mean = FP32(sum / n1).
void launch_mean_tree(double* part, int64_t Gp, int64_t n1, float* mean, hipStream_t st);
// Workgroups for `work` items at `per_block` per workgroup, in [1, max_blocks].
int grid_for(int64_t work, int per_block, int max_blocks);

// General block sizes: first-level blocks of `block` elements (a power of
// two, 32..4096), second-level groups of `group` scales (a power of two,
// 16..1024), any n >= 1 (short last block and group).  Workspace: absmax
// FP32 [n1], part FP64 [power of two >= ceil(n1 / group)].
struct BlockedQuant {
  const float* W;
  int64_t n, block, group;
  uint8_t* codes;
  uint8_t* scale_codes;
  float* scale2;
  float* mean;
  float* absmax;
  double* part;
};
hipError_t launch_quantize_blocked(const BlockedQuant& q, const IndexLut& lut, hipStream_t st);
hipError_t launch_dequant_blocked(const uint8_t* codes, const uint8_t* scale_codes,
                                  const float* scale2, const float* mean, int64_t n,
                                  int64_t block, int64_t group, uint16_t* out, hipStream_t st);
hipError_t launch_dequant(const uint8_t* codes, const uint8_t* scale_codes, const float* scale2,
                          const float* mean, int64_t n, uint16_t* out, hipStream_t st);

// ------------------------------------------------------------- rank-r work
constexpr int kMaxGroup = 8;
// Index of the problem of a grouped launch that workgroup (or task) x
// belongs to: the number of problems i >= 1 with begin(i) <= x, begin
// nondecreasing.  All the begins are read at once (independent loads of
// the kernel arguments), not one after another.
template <typename Begin>
__device__ __forceinline__ int group_index(int count, int x, Begin begin) {
  int di = 0;
#pragma unroll
  for (int i = 1; i < kMaxGroup; ++i) {
    const int b = begin(i);
    di += (i < count && x >= b) ? 1 : 0;
  }
  return di;
}

// Quantize / dequantize of up to kMaxGroup tensors per launch (one list),
// each with the arithmetic of a single call.  Encode workgroups: Gp per
// tensor from enc_begin; second-level workgroups from scale_begin;
// dequantize workgroups: wgs per tensor from begin.
struct QuantItem {
  const float* W;
  int64_t n1, G, Gp;
  int64_t len;            // tree length left for the last launch (<= kTreeLds)
  uint8_t* codes;
  uint8_t* scale_codes;
  float* scale2;
  float* mean;
  float* absmax;          // workspace [n1]
  double* part;           // workspace [Gp]
  int enc_begin, scale_begin;
};
struct QuantList {
  QuantItem d[kMaxGroup];
  int count;
  int enc_wgs, scale_wgs;
};
// One QuantItem of a tensor of n weights (its len and begins are set by
// launch_quantize_list).
QuantItem quant_item(const float* W, int64_t n, uint8_t* codes, uint8_t* scale_codes,
                     float* scale2, float* mean, const QuantWorkspace& ws);
hipError_t launch_quantize_list(QuantList& a, const IndexLut& lut, hipStream_t st);

struct DequantItem {
  const uint8_t* codes;
  const uint8_t* scale_codes;
  const float* scale2;
  const float* mean;
  int64_t n1;
  uint16_t* out;
  int wgs, begin;
};
struct DequantList {
  DequantItem d[kMaxGroup];
  int count;
  int wgs;
};
hipError_t launch_dequant_list(DequantList& a, hipStream_t st);

// Small-M rank-r product (M <= 16), up to kMaxGroup problems per launch, as
// kRankSmallSplits partial sums over consecutive quarters of K:
//   part[s][m][n] = sum_{k in quarter s} P[m][k] Q[n][k],
// P [M][K] BF16, Q [N][ldq] BF16, part FP32 [kRankSmallSplits][M][N].
// v = scale * (((part[0] + part[1]) + part[2]) + part[3]) is formed by the
// consumer (weight-streaming epilogue or launch_rank_finish) in that order,
// so every path gets the same bits.  One 4-wavefront workgroup per
// 16-column block, problem and quarter; wavefronts take consecutive parts
// of the quarter and add their sums in wavefront order.  The first
// workgroup of a problem also clears zero[0 .. zero_count) (split-K counters
// of the following weight-streaming launch).
constexpr int kRankSmallSplits = 4;
struct RankSmallDesc {
  const uint16_t* P;
  const uint16_t* Q;
  int64_t K, ldq, N;
  float* part;
  uint32_t* zero;
  int64_t zero_count;
  int wg_begin;     // first workgroup of this problem (set by the launcher)
};
struct RankSmallArgs {
  RankSmallDesc d[kMaxGroup];
  int count;
  int64_t M;
};
hipError_t launch_rank_small(const RankSmallArgs& a, hipStream_t st);

// Large-M rank-r product in one pass, no partials:
//   v[m][n] = scale * sum_k P[m][k] Q[n][k],  P [M][K], Q [N][ldq], N <= 256.
// Outputs, each optional (NULL skips): out FP32 [M][N]; hl BF16 [M][2 rp],
// hi | lo split of v with zeros for n in [N, rp) (rp a multiple of 32,
// rp >= N); ht / lt the transposed hi / lo BF16 copies, element (n, m) at
// frag_index(n, m, ldt), with zeros for m in [M, ldt) and n in [N, round_up(N,
// 32)) (ldt a multiple of 16, >= M; round_up(N, 32) * ldt elements).
// Fragment order of the transposed rank-r copies (the token contraction's
// MFMA row operand): 32-row x 16-token chunks of 1 KB, chunk (i / 32, k / 16)
// at chunk index (i / 32) * (ldt / 16) + k / 16, and inside a chunk the
// 16-byte piece of lane (i % 32) + 32 ((k / 8) % 2) holding tokens k & ~7 ..
// +8, so a wavefront reads one chunk with one contiguous 1 KB load.
__host__ __device__ inline int64_t frag_index(int64_t i, int64_t k, int64_t ldt) {
  return (((i >> 5) * (ldt >> 4) + (k >> 4)) * 64 + (i & 31) + 32 * ((k >> 3) & 1)) * 8 + (k & 7);
}

struct RankRowsArgs {
  const uint16_t* P;
  const uint16_t* Q;
  int64_t M, N, K, ldq;
  float scale;
  float* out;
  uint16_t* hl;
  int64_t rp;
  uint16_t* ht;
  uint16_t* lt;
  int64_t ldt;
  // optional keep bits of P (row-major words, bit k % 32 of word
  // [m * K / 32 + k / 32]; K a multiple of 32): P elements with bit 0 count as
  // zero.  Only launch_rank_split (k_rank_part) takes them.
  const uint32_t* pmask = nullptr;
  // Q given as stored [K][ldq] (element (n, k) at Q[k * ldq + n]) instead of
  // [N][ldq]: only launch_rank_split takes it, with N, ldq and K multiples
  // of 8, P, Q 16-byte aligned and no keep bits.
  bool q_kn = false;
};
hipError_t launch_rank_rows(const RankRowsArgs& a, hipStream_t st);
// The same product (same outputs) through K-split partials part
// [rank_k_splits(M, K)][M][N] FP32 and k_rank_finish (splits added in order);
// K or ldq not a multiple of 8, or unaligned P / Q, take launch_rank_rows.
// extra (optional): one more finish problem with the same M, run in the same
// finish launch.
struct FinishDesc;
hipError_t launch_rank_split(const RankRowsArgs& a, float* part, hipStream_t st,
                             const FinishDesc* extra = nullptr);
// K splits of launch_rank_split: about 512 workgroups of 64 rows; each split
// a multiple of 128 columns.  *kper receives the split length.
#ifndef QLORA_RANK_TARGET_WGS
#define QLORA_RANK_TARGET_WGS 512
#endif
inline int rank_k_splits(int64_t M, int64_t K, int64_t* kper) {
  const int64_t rb = (M + 63) / 64;
  const int64_t maxs = (K + 127) / 128;
  int64_t ks = (QLORA_RANK_TARGET_WGS + rb - 1) / rb;
  ks = ks < 1 ? 1 : (ks > maxs ? maxs : ks);
  int64_t per = ((K + ks - 1) / ks + 127) / 128 * 128;
  if (per < 128) per = 128;
  *kper = per;
  return (int)((K + per - 1) / per);
}

// Finish of split partials: v[m][n] = scale * sum_s part[s][m][n] (s
// ascending).  out (optional) = v, FP32 [M][N]; ht/lt (optional) = the
// transposed hi/lo BF16 pair of v in fragment order (as for RankRowsArgs).
// Up to kMaxGroup independent problems per launch.
struct FinishDesc {
  const float* part;
  float* out;
  uint16_t* ht;
  uint16_t* lt;
  int64_t M, N, ldt;
  float scale;
  int splits;
  int wg_begin;
  uint16_t* hl;   // optional row-major split: hl[m][n] = hi, hl[m][rp + n] = lo, zero for n in [N, rp)
  int64_t rp;
};
struct FinishArgs {
  FinishDesc d[kMaxGroup];
  int count;
};
hipError_t launch_rank_finish(const FinishArgs& a, hipStream_t st);
// Single-problem convenience form.
hipError_t launch_rank_finish(const float* part, int splits, int64_t M, int64_t N, float scale,
                              float* out, uint16_t* ht, uint16_t* lt, int64_t ldt,
                              uint16_t* hl, int64_t rp, hipStream_t st);

// The same finish for many rows (one workgroup per 16 rows x 64 columns,
// coalesced partial reads and transposed writes through LDS); identical
// outputs.  The list form runs up to kMaxGroup problems with the same M in
// one launch.
hipError_t launch_rank_finish_rows(const float* part, int splits, int64_t M, int64_t N,
                                   float scale, float* out, uint16_t* ht, uint16_t* lt,
                                   int64_t ldt, uint16_t* hl, int64_t rp, hipStream_t st);
hipError_t launch_rank_finish_rows(const FinishDesc* d, int count, hipStream_t st);

// Transpose of a BF16 matrix in[rows][cols] into out[cols][ldo]:
// out[c][i] = in[i][c] for i < rows, and 0 for i in [rows, ldo).
hipError_t launch_transpose_bf16(const uint16_t* in, int64_t rows, int64_t cols, uint16_t* out,
                                 int64_t ldo, hipStream_t st);

// Token contractions out = P^T Q over the M tokens: part[s][i][c] = sum
// over tokens m in split s of P[m][i] * Q[m][c], then out = sum_s part[s]
// (s ascending), out[c][i] if transposed else out[i][c].  P is given
// transposed as a hi + lo BF16 pair in fragment order (frag_index, ldp >= M
// a multiple of 16, round_up(R, 32) rows, zero-padded); Q BF16 [M][N]
// (16-byte aligned); R <= 256; m_per_split a multiple of 128.  Up to two
// problems with the same M, R and ldp run in one contraction launch and one
// finish launch.
struct GramProblem {
  const uint16_t* Pt_hi;
  const uint16_t* Pt_lo;
  const uint16_t* Q;
  int64_t N, m_per_split;
  int splits;
  float* part;   // [splits][R][N]
  float* out;
  bool transposed;
  // optional keep bits of Q (row-major words [M][N / 32], N a multiple of
  // 32): Q elements with bit 0 count as zero
  const uint32_t* qmask = nullptr;
};
hipError_t launch_grams(const GramProblem* p, int count, int64_t ldp, int64_t M, int64_t R,
                        hipStream_t st);

// ------------------------------------------------- optimizer step
// Tensors are handled in batches of up to kOptBatch per launch (descriptors
// passed by value), so a step over many small adapter tensors costs a few
// launches rather than a few per tensor.
constexpr int kOptBatch = 32;
constexpr int64_t kOptMaxElems = int64_t(1) << 32;  // per tensor
constexpr int kAdamwChunk = 1024;                   // elements per workgroup

// acc[0] += sum over tensors t (in order) of the FP64 sum of grads[t][i]^2
// (groups of 256 by the stride-halving tree, then the tree over the group
// sums padded to a power of two).  part: FP64, sum over t of that power of
// two (sumsq_part_len); sums: FP64 [count].  grads and n are host arrays.
int64_t sumsq_part_len(int64_t n);
hipError_t launch_sumsq(const float* const* grads, const int64_t* n, int count, double* acc,
                        double* part, double* sums, hipStream_t st);
struct AdamwDesc {
  float* param;       // FP32 master [n]
  uint16_t* p16;      // optional BF16 copy [n]
  const float* grad;  // [n]
  float* m;           // first moment [n]
  float* v;           // second moment [n]
  int64_t n;
};
struct AdamwScalars {
  float lr, lrwd, b1, ob1, b2, ob2, bc1, bc2, eps, max_norm;
};
// One AdamW step over `count` tensors (host array of descriptors, n > 0);
// sumsq (device, may be NULL: no clipping) gives the clip coefficient.
hipError_t launch_adamw(const AdamwDesc* d, int count, const AdamwScalars& h,
                        const double* sumsq, hipStream_t st);

// ------------------------------------------------- LoRA dropout mask
// Xm = X with the dropped elements cleared (may be NULL) and the keep bits
// keep[k * ldw + m / 32] (may be NULL); d even, X rows 4-byte aligned.
struct DropoutArgs {
  const uint16_t* X;
  uint16_t* Xm;
  uint32_t* keep;
  int64_t M, d, ldw;      // ldw = ceil(M / 32)
  uint32_t thr;           // keep when the generator word >= thr
  uint32_t key_lo, key_hi, off_lo, off_hi;
};
hipError_t launch_dropout(const DropoutArgs& a, hipStream_t st);
// The same mask as keep bits only, in two layouts (either may be NULL):
// keep [d][ldw] (bit m % 32 of word [k][m / 32], as launch_dropout) and
// rbits [M][d / 32] (bit k % 32 of word [m][k / 32]), d a multiple of 32.
// X and Xm are not used.
hipError_t launch_dropout_bits(const DropoutArgs& a, uint32_t* rbits, hipStream_t st);

// ------------------------------------------------- LoRA merge
// out[n][k] = RN_fp32(Wh[n][k] + scale * sum_i B[n][i] A[i][k]) (FP64
// evaluation), Wh the restored BF16 weight of the quantized state.
struct MergeArgs {
  const uint8_t* codes;
  const uint8_t* scodes;
  const float* scale2;
  const float* mean;
  const uint16_t* A;      // [r][d_in]
  const uint16_t* B;      // [d_out][r]
  float* out;             // [d_out][d_in]
  int64_t d_out, d_in, r;
  float scale;
};
hipError_t launch_merge(const MergeArgs& a, hipStream_t st);

// ------------------------------------------------- small-M forward (GEMV)
// Y[m][n] = RNE_bf16( sum_k X[m][k] Wh[n][k] + sum_i T[m][i] B[n][i] ),
// T = t_scale * XA A^T, for m < M <= 16, up to kMaxGroup layers per launch.
//
// Work.  A weight unit is one 64-row tile of one layer's weight times one
// 256-wide K super-step; a layer's units are listed tile by tile,
// super-step by super-step.  A T task forms one partial of T over a chunk
// of tchunk_ss super-steps for 16 ranks: tpart[c][m][i] = sum over the
// chunk's columns k of XA[m][k] A[i][k]; a layer has ceil(r / 16) x tchunks
// of them.  Each layer's work is one list: its T tasks first, each counted
// as tcost units, then its weight units (toff = n_tasks x tcost onwards).
//
// The weight-streaming launch gives layer i a block of wgs_i workgroups
// (wg_begin ..), the blocks sized in proportion to the layers' work so that
// the launch has kGemvWgs workgroups, four on every compute unit, each with
// about the same work.  Workgroup j of a layer takes the contiguous range
// gemv_unit_begin(j) .. gemv_unit_begin(j + 1) of the layer's list (uq or
// uq + 1 units, the first urem workgroups one more): the T tasks that start
// in it, then its weight units, writing one FP32 partial per tile it
// touches into slot j - gemv_wg_of(toff + first unit of the tile) of that
// tile (part[slot][m][n], at most kGemvMaxSlots slots per tile).
//
// The finish launch (one workgroup per 64 output columns) adds a tile's
// slots in order, forms T = t_scale * (((tpart[0] + tpart[1]) + ...) in
// chunk order, adds the LoRA term, rounds Y and, from the workgroup of the
// first columns, writes T_save.  The backward's recompute of T runs the same
// T tasks (launch_gemv_tasks) and k_rank_finish adds the same partials in
// the same order: both get the same bits.
#ifndef QLORA_GEMV_WGS
#define QLORA_GEMV_WGS 1024
#endif
constexpr int kGemvRows = 64;                       // rows per tile (16 per wavefront)
constexpr int kGemvWgs = QLORA_GEMV_WGS;            // workgroups of one launch
constexpr int kGemvMaxSlots = 16;                   // partials per tile, at most
constexpr int kGemvMaxChunks = 16;                  // T chunks per layer, at most
struct GemvDesc {
  const uint8_t* codes;
  const uint8_t* scodes;
  const float* scale2;
  const float* mean;
  const uint16_t* X;      // [M][d_in], 16-byte aligned: the base product's input
  const uint16_t* XA;     // LoRA branch input [M][d_in] (X, or X with dropped
                          // elements cleared), 16-byte aligned
  const uint16_t* A;      // [r][d_in], 16-byte aligned
  const uint16_t* B;      // [d_out][r]
  float* T_save;          // T FP32 [M][r] or NULL
  uint16_t* Y;            // [M][d_out]
  float* part;            // [kGemvMaxSlots][M][d_out]
  float* tpart;           // [tchunks][M][r]
  int64_t d_out, d_in, r;
  float t_scale;
  int tiles;              // 64-row tiles
  int nss;                // 256-wide super-steps of K
  int units;              // weight units: tiles * nss
  int tchunks;            // T chunks
  int tchunk_ss;          // super-steps per T chunk
  int n_tasks;            // T tasks: ceil(r / 16) * tchunks
  int tcost;              // units a T task counts for
  int toff;               // n_tasks * tcost
  int task_begin;         // first T task of this layer (T tasks alone)
  int wgs;                // workgroups of this layer in the streaming launch
  int wg_begin;           // its first workgroup there
  int uq, urem;           // (toff + units) / wgs and (toff + units) % wgs
  int fin_begin;          // first finish workgroup of this layer
};
struct GemvArgs {
  GemvDesc d[kMaxGroup];
  int count;
  int M;
  int wgs;                // workgroups of the weight-streaming launch
  int tasks;              // workgroups of a T-tasks-alone launch
  int fin_wgs;            // workgroups of the finish launch
  bool vec_b;             // every B 16-byte aligned with r % 8 == 0
};
// First unit of workgroup j of a list split over workgroups with
// q = units / wgs, rem = units % wgs (the first rem get one unit more), and
// the workgroup of unit u.  Lists hold fewer than 2^31 units.
__host__ __device__ inline int gemv_unit_begin(int j, int q, int rem) {
  return j * q + (j < rem ? j : rem);
}
__host__ __device__ inline int gemv_wg_of(int u, int q, int rem) {
  const int big = rem * (q + 1);
  return u < big ? (int)((unsigned)u / (unsigned)(q + 1))
                 : rem + (int)((unsigned)(u - big) / (unsigned)q);
}
// LDS of the weight-streaming launch: a ring of kGemvRing staged X
// super-steps of 16 rows x 512 bytes (rows past M zero), which also holds a
// T task's reduction buffer.
#ifndef QLORA_GEMV_RING
#define QLORA_GEMV_RING 4
#endif
constexpr int kGemvRing = QLORA_GEMV_RING;
inline int64_t gemv_lds_bytes(int64_t M) {
  (void)M;
  return (int64_t)kGemvRing * 16 * 512;
}
hipError_t launch_gemv(const GemvArgs& a, hipStream_t st);
// The T tasks of `a` alone (one workgroup per task; no weight streaming).
hipError_t launch_gemv_tasks(const GemvArgs& a, hipStream_t st);

// ------------------------------------------------- large-M fused GEMM
// Forward: Y = RNE_bf16(X Wh^T + [T_hi T_lo] [B B]^T), dequant tiles in LDS.
// Backward: dX = RNE_bf16(dY Wh + [U_hi U_lo] [A A]), W tiles written
// transposed into LDS.
struct GemmArgs {
  const uint8_t* codes;
  const uint8_t* scodes;
  const float* scale2;
  const float* mean;
  const uint16_t* act;    // X [M][d_in] (forward) or dY [M][d_out] (backward)
  const uint16_t* ext;    // T or U split into BF16 terms: [M][2*RP], hi | lo, RP = r rounded up to 32
  const uint16_t* lw;     // B [d_out][r] (forward) or A [r][d_in] (backward)
  uint16_t* out;          // Y [M][d_out] or dX [M][d_in]
  int64_t M, d_out, d_in, r;
  // backward with LoRA dropout: keep bit of (m, c) is bit m % 32 of
  // keep[c * keep_ld + m / 32]; the LoRA term of dX is cleared where it is 0
  const uint32_t* keep;
  int64_t keep_ld;
};
hipError_t launch_gemm_fwd(const GemmArgs& a, hipStream_t st);
hipError_t launch_gemm_bwd(const GemmArgs& a, hipStream_t st);

// ------------------------------------------------- host-side checks
// qlora_linear_fwd's argument checks for a workspace of ws_bytes bytes (not
// dereferenced): QLORA_ERR_WORKSPACE when the call needs more.
int linear_fwd_check(const qlora_nf4_t* q, const uint16_t* X, int64_t M, const uint16_t* A,
                     const uint16_t* B, int64_t r, uint16_t* Y, float* T_save, size_t ws_bytes);

}  // namespace qlora
