/*
 * qlora.h -- C ABI of libqlora: the frozen-base NF4 LoRA linear layer on an
 * AMD CDNA4 (gfx950) GPU.
 *
 * Sources of the operations (the pages):
 *   [QP]  "第 04 篇：QLoRA 原理" (jupiter-lab.pages.dev, QLoRA principles)
 *   [CP]  "QLoRA" concept page (compassingai.com), sections
 *         "NF4 量化機制詳解" (NF4 steps) and "雙重量化" (double quantization).
 *
 * Conventions for every entry point
 *   - Every array argument is a DEVICE pointer to caller-owned memory.  The
 *     library allocates nothing, frees nothing and keeps no state between
 *     calls (the one exception is the fixed device array that
 *     qlora_linear_fwd_noalloc works in); it never synchronizes.  Work is
 *     enqueued on `stream` (a
 *     hipStream_t; NULL means the null stream) and the call returns at once.
 *   - All matrices are dense row-major.  BF16 values are passed as their
 *     uint16_t bit patterns.
 *   - Arguments are checked on the host before anything is enqueued; on any
 *     error the call returns a negative qlora_status and enqueues nothing.
 *     A failing kernel launch returns QLORA_ERR_HIP (work enqueued before it
 *     on the same call may have run).  Non-finite inputs are a precondition
 *     violation and are not detected.
 *   - Pointers marked (16B) must be 16-byte aligned.
 *   - Calls that share a workspace buffer must be ordered (same stream or
 *     explicit events); calls on different buffers may overlap freely.
 */
#ifndef QLORA_H
#define QLORA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  QLORA_OK = 0,
  QLORA_ERR_NULL = -1,       /* a required pointer is NULL                  */
  QLORA_ERR_SHAPE = -2,      /* a size is out of its documented range        */
  QLORA_ERR_ALIGN = -3,      /* a (16B) pointer is not 16-byte aligned       */
  QLORA_ERR_WORKSPACE = -4,  /* workspace smaller than qlora_workspace_bytes */
  QLORA_ERR_HIP = -5,        /* the HIP runtime reported an error            */
  QLORA_ERR_SCRATCH = -6     /* the call needs more than the library's fixed
                                device scratch (qlora_linear_fwd_noalloc)    */
} qlora_status;

/* Block sizes fixed by the method: 64 weights share one first-level scale
 * ([QP §3.4], [CP, NF4 量化機制詳解] step 1), 256 first-level scales share one
 * second-level FP32 scale ([QP §5.2], [CP, 雙重量化]). */
#define QLORA_BLOCK 64
#define QLORA_GROUP 256

/*
 * NF4 + double-quantized weight W[d_out, d_in] ([QP §2.1, §5.2, §6.1]).
 * n = d_out*d_in weights, flattened row-major; n1 = n/64 blocks;
 * G = ceil(n1/256) groups.  Requires d_in % 64 == 0 (no block straddles a
 * row), d_out >= 1.
 *   codes        uint8[n/2] (16B)  4-bit level indices, two per byte; element
 *                                  2j in the low nibble of byte j [QP §2.1].
 *   scale_codes  uint8[n1]         OCP FP8 E4M3FN codes of the centred block
 *                                  scales, (absmax_b - mean) / scale2[b/256].
 *   scale2       float[G]          second-level scales: the group's largest
 *                                  |absmax - mean| divided by 448.
 *   scale_mean   float[1]          mean of all n1 block absmax values.
 * The restored weight of element e in block b is
 *   RNE_bf16(codebook[idx_e] * (fp8(scale_codes[b]) * scale2[b/256] + mean))
 * with every FP32 operation rounded separately (no fused multiply-add), and
 * codebook = the 16 NF4 levels printed in [QP §4.3].
 */
typedef struct {
  int64_t d_out;
  int64_t d_in;
  uint8_t *codes;
  uint8_t *scale_codes;
  float *scale2;
  float *scale_mean;
} qlora_nf4_t;

/* Byte sizes of the four buffers of an NF4 weight (host only, no GPU use).
 * Returns QLORA_ERR_SHAPE for d_out < 1, d_in < 64 or d_in % 64 != 0, and
 * QLORA_ERR_NULL when an output pointer is NULL. */
int qlora_nf4_sizes(int64_t d_out, int64_t d_in, size_t *codes_bytes,
                    size_t *scale_codes_bytes, size_t *scale2_bytes,
                    size_t *scale_mean_bytes);

/* Operations for qlora_workspace_bytes. */
#define QLORA_OP_QUANTIZE 0
#define QLORA_OP_FWD 1
#define QLORA_OP_BWD 2
#define QLORA_OP_FWD_DROPOUT 3
#define QLORA_OP_BWD_DROPOUT 4

/* Device workspace (bytes) that one call of `op` needs for these sizes
 * (M and r are ignored for QLORA_OP_QUANTIZE).  Host only.  Returns 0 for
 * sizes the call would reject. */
size_t qlora_workspace_bytes(int op, int64_t d_out, int64_t d_in, int64_t M,
                             int64_t r);

/*
 * Quantize W (FP32 [d_out, d_in], (16B)) into `q` ([QP §3.4, §4.3, §5.2];
 * [CP, NF4 量化機制詳解; 雙重量化]):
 *   1. absmax a_b of each 64-element block;
 *   2. x = w / a_b (IEEE FP32 division); a zero block gives x = 0;
 *   3. index of the nearest NF4 level, ties to the lower index;
 *   4. two indices per byte;
 *   5. mean of the a_b (FP64 sum in a fixed stride-halving tree: pairs
 *      (j, j+128), (j, j+64), ... within each group of 256, then the same
 *      tree over the group sums padded with zeros to a power of two; the
 *      FP64 quotient by n1 is rounded to FP32);
 *   6. per group: scale2 = max |a_b - mean| / 448 and FP8 E4M3FN codes of
 *      (a_b - mean) / scale2, round to nearest even, saturating at 448;
 *      a group whose scale2 is 0 stores code 0.
 * Deterministic: repeated calls give identical bytes.
 * q->codes (16B), q->scale_codes, q->scale2, q->scale_mean are outputs.
 * workspace (16B) >= qlora_workspace_bytes(QLORA_OP_QUANTIZE, ...).
 */
int qlora_quantize_nf4(const float *W, const qlora_nf4_t *q, void *workspace,
                       size_t workspace_bytes, void *stream);

/*
 * Double dequantization ([QP §2.3, §6.1]): W_bf16[d_out, d_in] (16B) gets the
 * restored weights of `q` as BF16 bit patterns, bit-exact with the formula
 * under qlora_nf4_t.  Needs no workspace.
 */
int qlora_dequant_bf16(const qlora_nf4_t *q, uint16_t *W_bf16, void *stream);

/*
 * LoRA merge into the base ([QP §12.3]; restored weight as in
 * qlora_dequant_bf16): the merged weight
 *     Wm[n][k] = RN_fp32( Wh[n][k] + s * sum_i B[n][i] A[i][k] ),
 * s = lora_alpha / r (FP32), with the right-hand side evaluated in FP64
 * (rank index ascending, every product and sum rounded on its own) and
 * rounded once to FP32.  When q_out is not NULL the merged weight is then
 * quantized into q_out exactly as qlora_quantize_nf4 would (the second
 * rounding that the merge into a 4-bit base implies).
 *   q        quantized base (input)
 *   A        BF16 [r, d_in]  (16B)    1 <= r <= 256
 *   B        BF16 [d_out, r]          any alignment
 *   W_merged FP32 [d_out, d_in] (16B) output
 *   q_out    NULL, or a quantized state of the same shape (output; may not
 *            alias q or W_merged)
 * workspace (16B) >= qlora_workspace_bytes(QLORA_OP_QUANTIZE, d_out, d_in,
 * 0, 0) when q_out is given (unused otherwise).  Deterministic.
 */
int qlora_merge_nf4(const qlora_nf4_t *q, const uint16_t *A, const uint16_t *B,
                    int64_t r, float lora_alpha, float *W_merged,
                    const qlora_nf4_t *q_out, void *workspace,
                    size_t workspace_bytes, void *stream);

/*
 * Forward of the LoRA linear layer on the frozen NF4 base
 * ([QP §1.2, §2.2, §2.3, §6.3]; column-vector form y = W x + (alpha/r) B A x,
 * written here for token rows):
 *     Y = X Wh^T + s (X A^T) B^T,      s = lora_alpha / r (FP32),
 * where Wh is the restored BF16 weight.  Products take BF16 inputs and
 * accumulate in FP32; Y is rounded once to BF16.  The rank-r intermediate
 * T = s X A^T is formed in FP32 and enters the second product as the sum of
 * two BF16 terms (hi + lo), so it carries about 16 significant bits.  T is
 * deliberately not a BF16 tensor: one BF16 rounding of T (and of U in the
 * backward) would spend most of the 2e-3 relative error allowed for dA and
 * dB, so it is saved and handed to the backward as FP32.
 *   X       BF16 [M, d_in]  (16B)        M >= 0 tokens (M = 0: no work)
 *   A       BF16 [r, d_in]  (16B)        1 <= r <= 256
 *   B       BF16 [d_out, r]              any alignment
 *   Y       BF16 [M, d_out] (16B)        output
 *   T_save  FP32 [M, r]     (16B) or NULL: receives T for the backward.
 * workspace (16B) >= qlora_workspace_bytes(QLORA_OP_FWD, d_out, d_in, M, r).
 * Sizes per call: d_out <= 2^21, d_in <= 2^21 and M <= 2^21 tokens (the
 * kernels' device byte offsets are 32-bit within a tile or split), else
 * QLORA_ERR_SHAPE; the same holds for the backward.
 * M <= 16 runs a weight-streaming kernel (HBM-bound); larger M runs the
 * fused dequant-GEMM on the matrix cores.  No full BF16 copy of W is made.
 */
int qlora_linear_fwd(const qlora_nf4_t *q, const uint16_t *X, int64_t M,
                     const uint16_t *A, const uint16_t *B, int64_t r,
                     float lora_alpha, uint16_t *Y, float *T_save,
                     void *workspace, size_t workspace_bytes, void *stream);

/*
 * Backward of the same layer for the upstream gradient dY ([QP §2.4, §6.4,
 * §6.5]; [CP, 推論與訓練的精度關係]): gradients reach X, A and B; the frozen
 * base takes part in dX but gets no gradient of its own.
 *     U  = s dY B                 (FP32, [M, r])
 *     dX = dY Wh + U A            (BF16 out, FP32 accumulation)
 *     dA = U^T X                  (FP32 [r, d_in])
 *     dB = s dY^T (X A^T) = dY^T T (FP32 [d_out, r])
 * U and T enter the products as hi + lo BF16 pairs as in the forward.
 *   X, A, B, r, lora_alpha as in qlora_linear_fwd; dY BF16 [M, d_out] (16B).
 *   T_saved FP32 [M, r] (16B) from qlora_linear_fwd, or NULL to recompute.
 *   dX      BF16 [M, d_in] (16B) or NULL to skip the input gradient.
 *   dA      FP32 [r, d_in] (16B), dB FP32 [d_out, r] (16B): overwritten
 *           (M = 0 writes zeros).
 * workspace (16B) >= qlora_workspace_bytes(QLORA_OP_BWD, d_out, d_in, M, r).
 * dA and dB are reduced over tokens in a fixed order: results are
 * deterministic.
 */
int qlora_linear_bwd(const qlora_nf4_t *q, const uint16_t *X,
                     const uint16_t *dY, int64_t M, const uint16_t *A,
                     const uint16_t *B, int64_t r, float lora_alpha,
                     const float *T_saved, uint16_t *dX, float *dA, float *dB,
                     void *workspace, size_t workspace_bytes, void *stream);

/*
 * qlora_linear_fwd without a workspace argument, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc).  The workspace comes from a fixed device
 * array inside the library, QLORA_STATIC_SCRATCH_BYTES bytes on each GPU the
 * library runs on, held until the process ends; the call itself allocates
 * nothing.  Same arguments, checks, kernels and results (bit for bit) as
 * qlora_linear_fwd.  A call whose workspace (qlora_workspace_bytes(
 * QLORA_OP_FWD, ...)) exceeds the array returns QLORA_ERR_SCRATCH and
 * enqueues nothing; every projection shape of the LLaMA-7B and -65B layers
 * fits at r <= 64 for any M up to 40000 tokens.  Every call on one GPU
 * shares that GPU's array:
 * calls that may overlap on one GPU (other streams, unordered host threads)
 * race and must not be issued.  Nothing in the array needs to start at zero.
 */
#define QLORA_STATIC_SCRATCH_BYTES (32u << 20)
int qlora_linear_fwd_noalloc(const qlora_nf4_t *q, const uint16_t *X, int64_t M,
                             const uint16_t *A, const uint16_t *B, int64_t r,
                             float lora_alpha, uint16_t *Y, float *T_save,
                             void *stream);

/*
 * Forward of up to QLORA_MAX_GROUP layers that share the token count M, in
 * one pass: the same operation as qlora_linear_fwd for every item (each with
 * its own weight, LoRA factors, outputs and workspace sized by
 * qlora_workspace_bytes(QLORA_OP_FWD, ...)).  For M <= 16 all items run in
 * one weight-streaming launch (which also forms every T) and one finish
 * launch, so the projections of a decoder layer stream their packed weights
 * back to back; the K split of each weight is chosen over the whole group,
 * so an item's Y may differ from a single call's by FP32 summation order
 * (T does not).  For larger M the items run one after another.  Items must
 * not share outputs or workspace.
 * Returns the first failing item's status (nothing enqueued on argument
 * errors).
 */
#define QLORA_MAX_GROUP 8
typedef struct {
  qlora_nf4_t w;
  const uint16_t *X;
  const uint16_t *A;
  const uint16_t *B;
  int64_t r;
  float lora_alpha;
  uint16_t *Y;
  float *T_save;
  void *workspace;
  size_t workspace_bytes;
} qlora_fwd_item;

int qlora_linear_fwd_many(int count, const qlora_fwd_item *items, int64_t M,
                          void *stream);

/*
 * Quantize (dequantize) up to QLORA_MAX_GROUP tensors in one call: the same
 * operation as qlora_quantize_nf4 (qlora_dequant_bf16) for every item, with
 * the same results bit for bit, in two launches (one) for the whole list
 * when no tensor has more than 2^20 first-level blocks, so the projections
 * of a layer pay the launch and call overhead once.  Each item has its own
 * input, output and (quantize) workspace sized by
 * qlora_workspace_bytes(QLORA_OP_QUANTIZE, ...); items must not share any
 * of them.  Returns the first failing item's status (nothing enqueued on
 * argument errors) or QLORA_ERR_SHAPE when count is not in
 * 1 .. QLORA_MAX_GROUP.
 */
typedef struct {
  const float *W;           /* FP32 [q.d_out, q.d_in] (16B) */
  qlora_nf4_t q;            /* output state */
  void *workspace;          /* (16B) */
  size_t workspace_bytes;
} qlora_quant_item;

int qlora_quantize_nf4_many(int count, const qlora_quant_item *items, void *stream);

typedef struct {
  qlora_nf4_t q;            /* input state */
  uint16_t *W_bf16;         /* BF16 [q.d_out, q.d_in] (16B) output */
} qlora_dequant_item;

int qlora_dequant_bf16_many(int count, const qlora_dequant_item *items, void *stream);

/*
 * General block sizes ([QP §5.5]: the first-level block size B1 trades
 * scale metadata, about 8 / B1 bits per weight after double quantization,
 * against error; the second-level group size B2 makes the same trade for
 * the scales).  The same quantization as qlora_quantize_nf4 over a flat
 * array of n >= 1 values with
 *   block  B1: a power of two, 32 <= B1 <= 4096 (the layer format uses 64),
 *   group  B2: a power of two, 16 <= B2 <= 1024 (the layer format uses 256),
 * and no divisibility requirement: a short last block takes the absmax of
 * the elements it has, a short last group likewise.  With n1 = ceil(n/B1)
 * and G = ceil(n1/B2):
 *   codes        uint8[ceil(n/2)] (16B); for odd n the high nibble of the
 *                last byte is 0.
 *   scale_codes  uint8[n1];  scale2 float[G];  scale_mean float[1].
 * With B1 = 64, B2 = 256 and n % 64 == 0 the bytes equal those of
 * qlora_quantize_nf4 for the same values.  n <= 2^40.
 */
typedef struct {
  int64_t n;
  int64_t block;
  int64_t group;
  uint8_t *codes;
  uint8_t *scale_codes;
  float *scale2;
  float *scale_mean;
} qlora_nf4_blocked_t;

/* Buffer sizes of the blocked format (host only); QLORA_ERR_SHAPE for an
 * unsupported n, block or group. */
int qlora_nf4_blocked_sizes(int64_t n, int64_t block, int64_t group,
                            size_t *codes_bytes, size_t *scale_codes_bytes,
                            size_t *scale2_bytes);

/* Workspace of qlora_quantize_nf4_blocked (host only); 0 when unsupported. */
size_t qlora_quantize_blocked_workspace_bytes(int64_t n, int64_t block,
                                              int64_t group);

/* Quantize W (FP32 [n], (16B)) into q.  workspace (16B) >=
 * qlora_quantize_blocked_workspace_bytes(n, block, group). */
int qlora_quantize_nf4_blocked(const float *W, const qlora_nf4_blocked_t *q,
                               void *workspace, size_t workspace_bytes,
                               void *stream);

/* Double dequantization of q to BF16 [n] (16B). */
int qlora_dequant_bf16_blocked(const qlora_nf4_blocked_t *q, uint16_t *W_bf16,
                               void *stream);

/*
 * LoRA dropout in training mode ([QP §6.3]: the LoRA branch takes D(x)
 * instead of x, the base branch x; inference has no dropout):
 *     D(X) = keep * X / (1 - p),
 * keep drawn per element of X [M, d_in] from a counter-based generator, so
 * the backward regenerates the forward's mask from the same parameters:
 * element (m, k) takes output word m % 4 of Philox4x32-10 (Salmon, Moraes,
 * Dror, Shaw, SC'11) at counter (k, floor(m / 4), offset_lo, offset_hi)
 * under key (seed_lo, seed_hi), and is kept when that word is at least
 * floor(p * 2^32).  Use a new offset (or seed) for every layer and step.
 */
typedef struct {
  float p;          /* drop probability, 0 <= p < 1 (else QLORA_ERR_SHAPE) */
  uint64_t seed;    /* generator key                                       */
  uint64_t offset;  /* counter words 2 and 3                               */
  /* Optional saved mask of a layer call with M > 16 tokens (ignored for
   * M <= 16 and by qlora_dropout_mask), device memory (16B):
   *   keep_rows  [M, d_in / 32] words: bit (k % 32) of word [m][k / 32]
   *   keep_cols  [d_in, ceil(M / 32)] words: bit (m % 32) of word [k][m / 32]
   * (bits of rows m >= M are 0).  When both are non-NULL,
   * qlora_linear_fwd_dropout writes them, and qlora_linear_bwd_dropout reads
   * them instead of regenerating the mask, so the generator runs once per
   * training step; they must then hold the mask of the same M, d_in, p,
   * seed and offset.  NULL: nothing written, the backward regenerates. */
  uint32_t *keep_rows;
  uint32_t *keep_cols;
} qlora_dropout_t;

/*
 * The mask alone: X_kept = X with the dropped elements set to +0 (kept ones
 * unchanged; the 1 / (1 - p) is not applied) and, if keep_bits is not NULL,
 * keep_bits[k * ceil(M/32) + m/32] bit (m % 32) = keep of element (m, k)
 * (bits of rows m >= M are 0).
 *   X, X_kept  BF16 [M, d] (16B), d % 8 == 0, d <= 2^21, M <= 2^21;
 *   X_kept or keep_bits may be NULL (not both; X may be NULL without X_kept).
 */
int qlora_dropout_mask(const uint16_t *X, int64_t M, int64_t d,
                       const qlora_dropout_t *drop, uint16_t *X_kept,
                       uint32_t *keep_bits, void *stream);

/*
 * qlora_linear_fwd with LoRA dropout:
 *     Y = X Wh^T + s (D(X) A^T) B^T,   T = s D(X) A^T (saved in T_save).
 * The kernels form keep * X (exact) and fold 1 / (1 - p) into the scale:
 * s' = FP32(FP32(lora_alpha / r) / FP32(1 - p)).  With p = 0 the results
 * equal qlora_linear_fwd's bit for bit.  Same arguments and limits as
 * qlora_linear_fwd, plus `drop` (host pointer, not NULL); workspace (16B) >=
 * qlora_workspace_bytes(QLORA_OP_FWD_DROPOUT, d_out, d_in, M, r).
 */
int qlora_linear_fwd_dropout(const qlora_nf4_t *q, const uint16_t *X,
                             int64_t M, const uint16_t *A, const uint16_t *B,
                             int64_t r, float lora_alpha,
                             const qlora_dropout_t *drop, uint16_t *Y,
                             float *T_save, void *workspace,
                             size_t workspace_bytes, void *stream);

/*
 * Backward of qlora_linear_fwd_dropout for the same X and `drop` (the mask
 * is regenerated, or read from drop->keep_rows / keep_cols when both are
 * given and M > 16):
 *     U  = s dY B
 *     dX = dY Wh + keep * (U A) / (1 - p)
 *     dA = U^T D(X),   dB = dY^T T   with T = s D(X) A^T.
 * Arguments and limits as qlora_linear_bwd, plus `drop`; T_saved (if given)
 * must come from qlora_linear_fwd_dropout with the same `drop`; workspace
 * (16B) >= qlora_workspace_bytes(QLORA_OP_BWD_DROPOUT, d_out, d_in, M, r).
 * With p = 0 the results equal qlora_linear_bwd's bit for bit.
 */
int qlora_linear_bwd_dropout(const qlora_nf4_t *q, const uint16_t *X,
                             const uint16_t *dY, int64_t M, const uint16_t *A,
                             const uint16_t *B, int64_t r, float lora_alpha,
                             const qlora_dropout_t *drop, const float *T_saved,
                             uint16_t *dX, float *dA, float *dB,
                             void *workspace, size_t workspace_bytes,
                             void *stream);

/*
 * Optimizer step on the LoRA factors ([QP §7.3]: AdamW with one first and
 * one second moment per trainable parameter, 32-bit; [QP §10.2]: optional
 * clipping by the global gradient norm).  Only A and B train.
 *
 * Tensors are processed in batches of up to 32 per kernel launch, so a step
 * over many small adapter tensors costs a few launches.  One tensor of the
 * step (all arrays device memory, any 4-byte alignment; 16-byte aligned
 * arrays, 8-byte for the BF16 copy, take wider accesses, same results):
 */
typedef struct {
  float *param;          /* FP32 master values [n], updated in place        */
  uint16_t *param_bf16;  /* BF16 copy [n] written after the step (RNE), or  */
                         /* NULL                                            */
  const float *grad;     /* FP32 gradient [n]                               */
  float *m;              /* first moment [n], updated in place              */
  float *v;              /* second moment [n], updated in place             */
  int64_t n;             /* element count, 0 <= n <= 2^32                   */
} qlora_adamw_param;

/*
 * acc[0] += sum over the listed tensors (in list order, FP64) of the sum of
 * their squared gradients, each taken in groups of 256 by the stride-halving
 * tree (pairs (j, j+128), (j, j+64), ..., (j, j+1)) and then by the same tree
 * over the group sums padded with zeros to a power of two.  acc is one FP64
 * device value the caller zeroes before the first call of a step; several
 * calls accumulate in call order.  workspace (16B-aligned device memory)
 * >= qlora_sumsq_workspace_bytes(count, params) for the same list (about
 * 8 bytes per 128 elements plus 8 per tensor; 0 for an invalid list).
 * QLORA_ERR_SHAPE for count < 0 or n outside [0, 2^32]; QLORA_ERR_NULL for
 * a missing acc, workspace or gradient (n > 0); QLORA_ERR_ALIGN,
 * QLORA_ERR_WORKSPACE.
 */
int qlora_grad_sumsq(int count, const qlora_adamw_param *params, double *acc,
                     void *workspace, size_t workspace_bytes, void *stream);
size_t qlora_sumsq_workspace_bytes(int count, const qlora_adamw_param *params);

/*
 * AdamW with decoupled weight decay, step number `step` >= 1 (bias
 * corrections bc_i = 1 - beta_i^step, evaluated in FP64 on the host and
 * rounded to FP32).  With grad_sumsq (device FP64 from qlora_grad_sumsq) the
 * gradients are first scaled by c = min(1, max_grad_norm / (norm + 1e-6)),
 * norm = FP32(sqrt(sumsq)); with NULL, c = 1.  Per element, FP32, each
 * operation rounded on its own in this order:
 *   g = g * c;   p = p - (lr * wd) * p;
 *   m = b1 * m + (1 - b1) * g;   v = b2 * v + (1 - b2) * (g * g);
 *   p = p - lr * ((m / bc1) / (sqrt(v / bc2) + eps));   p_bf16 = RNE_bf16(p).
 * The square root is correctly rounded.  Tensors with n = 0 are skipped.
 * QLORA_ERR_SHAPE for step < 1, count < 0, n outside [0, 2^32] or beta
 * outside [0, 1); QLORA_ERR_NULL for a missing array (n > 0).
 */
int qlora_adamw_step(int count, const qlora_adamw_param *params, float lr,
                     float beta1, float beta2, float eps, float weight_decay,
                     int64_t step, const double *grad_sumsq,
                     float max_grad_norm, void *stream);

/* Static English text for a qlora_status value. */
const char *qlora_status_string(int status);

/* ABI version: (major << 16) | minor. */
int qlora_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* QLORA_H */
