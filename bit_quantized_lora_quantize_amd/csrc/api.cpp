// api.cpp -- host side of libqlora's C ABI: argument checks, workspace
// planning and kernel launch sequences.  The operations are stated in
// include/qlora.h with their sources on the pages.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdint>
#include <cstring>
#include <vector>

#include "qlora.h"
#include "qlora_device.h"
#include "qlora_kernels.h"

using namespace qlora;

// ------------------------------------------------------------ timing aid
// Only in the timing build (libqlora_timed.so): an event pair the caller
// arms for the next weight-kernel launch.  Process-wide, not thread-safe.
#ifdef QLORA_TIMING_HOOK
#include "qlora_timing.h"
namespace {
hipEvent_t g_ev_start = nullptr, g_ev_stop = nullptr;
bool g_ev_armed = false;
}  // namespace

namespace qlora {
void weight_kernel_begin(hipStream_t st) {
  if (g_ev_armed && g_ev_start) (void)hipEventRecord(g_ev_start, st);
}
void weight_kernel_end(hipStream_t st) {
  if (!g_ev_armed) return;
  if (g_ev_stop) (void)hipEventRecord(g_ev_stop, st);
  g_ev_armed = false;
  g_ev_start = g_ev_stop = nullptr;
}
}  // namespace qlora

extern "C" int qlora_time_next_weight_kernel(void* start_event, void* stop_event) {
  g_ev_start = static_cast<hipEvent_t>(start_event);
  g_ev_stop = static_cast<hipEvent_t>(stop_event);
  g_ev_armed = g_ev_start != nullptr || g_ev_stop != nullptr;
  return QLORA_OK;
}
#endif

namespace {

constexpr int64_t kMaxRank = 256;
constexpr int64_t kSmallM = 16;      // M <= 16 streams the weight (GEMV path)
// Layer sizes and token counts per call: every device byte offset the kernels
// form within one tile, split or transposed copy then stays below 2^31.
constexpr int64_t kMaxLinearDim = int64_t(1) << 21;
constexpr int64_t kMaxTokens = int64_t(1) << 21;

inline bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
inline int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }
inline int64_t round_up(int64_t a, int64_t b) { return cdiv(a, b) * b; }

// Sequential carving of a workspace into 256-byte aligned pieces; with a null
// base it only measures.
struct Carver {
  char* base;
  size_t off = 0;
  explicit Carver(void* b) : base(static_cast<char*>(b)) {}
  template <class T>
  T* take(int64_t count) {
    off = (off + 255) & ~size_t(255);
    T* p = base ? reinterpret_cast<T*>(base + off) : nullptr;
    off += size_t(std::max<int64_t>(count, 0)) * sizeof(T);
    return p;
  }
};

bool shape_ok(int64_t d_out, int64_t d_in) {
  return d_out >= 1 && d_in >= kBlock && d_in % kBlock == 0 && d_out <= (int64_t(1) << 31) &&
         d_in <= (int64_t(1) << 31) && d_out * d_in <= (int64_t(1) << 40);
}

int check_nf4(const qlora_nf4_t* q) {
  if (!q) return QLORA_ERR_NULL;
  if (!shape_ok(q->d_out, q->d_in)) return QLORA_ERR_SHAPE;
  if (!q->codes || !q->scale_codes || !q->scale2 || !q->scale_mean) return QLORA_ERR_NULL;
  if (!aligned16(q->codes) || (reinterpret_cast<uintptr_t>(q->scale2) & 3u) ||
      (reinterpret_cast<uintptr_t>(q->scale_mean) & 3u))
    return QLORA_ERR_ALIGN;
  return QLORA_OK;
}

// --------------------------------------------------------------- plans
struct QuantPlan {
  int64_t n, n1, G, Gp;
  float* absmax;
  double* part;
  size_t bytes;
};

QuantPlan plan_quant(int64_t d_out, int64_t d_in, void* ws) {
  QuantPlan p{};
  p.n = d_out * d_in;
  p.n1 = p.n / kBlock;
  p.G = cdiv(p.n1, kGroup);
  p.Gp = 1;
  while (p.Gp < p.G) p.Gp *= 2;
  Carver c(ws);
  p.absmax = c.take<float>(p.n1);
  p.part = c.take<double>(p.Gp);
  p.bytes = c.off + 256;
  return p;
}

// Small-M forward: T chunks of at least 4 super-steps (1024 columns: one
// round of loads per T task), at most kGemvMaxChunks of them.
int64_t gemv_nss(int64_t d_in) { return cdiv(d_in / kBlock, 4); }
int64_t gemv_tchunk_ss(int64_t d_in) {
  return std::max<int64_t>(4, cdiv(gemv_nss(d_in), kGemvMaxChunks));
}
int64_t gemv_tchunks(int64_t d_in) { return cdiv(gemv_nss(d_in), gemv_tchunk_ss(d_in)); }

struct FwdPlan {
  bool small;
  float* t_buf;       // [M][r] when T_save is NULL (large M)
  uint16_t* t_hl;     // [M][2 rp] BF16 hi | lo of T (large M)
  int64_t rp;         // r rounded up to 32
  float* gemv_part;   // [kGemvMaxSlots][M][d_out] (small M)
  float* gemv_tpart;  // [gemv_tchunks(d_in)][M][r] (small M)
  float* r_part;      // [rank_k_splits(M, d_in)][M][r] (large M)
  size_t bytes;
};

FwdPlan plan_fwd(int64_t d_out, int64_t d_in, int64_t M, int64_t r, void* ws) {
  FwdPlan p{};
  p.small = M <= kSmallM;
  Carver c(ws);
  p.rp = round_up(r, 32);
  if (!p.small) {
    int64_t kper;
    p.t_buf = c.take<float>(M * r);
    p.t_hl = c.take<uint16_t>(M * 2 * p.rp);
    p.r_part = c.take<float>((int64_t)rank_k_splits(M, d_in, &kper) * M * r);
  } else {
    p.gemv_part = c.take<float>((int64_t)kGemvMaxSlots * M * d_out);
    p.gemv_tpart = c.take<float>(gemv_tchunks(d_in) * M * r);
  }
  p.bytes = c.off + 256;
  return p;
}

struct BwdPlan {
  float* t_buf;       // [M][r]
  float* r_part;      // rank-r partials: [kRankSmallSplits][M][r] (small M), else
                      // [max K splits of T and U][M][r]
  float* t_part;      // small M: T chunk partials [gemv_tchunks(d_in)][M][r]
  int64_t ldbt;       // row stride of B^T
  uint16_t* bt;       // [r][ldbt]
  int64_t rp;         // r rounded up to 32
  uint16_t* u_hl;     // [M][2 rp] BF16 hi | lo of U
  int64_t ldp;        // token stride of the transposed hi/lo copies
  uint16_t *ut_hi, *ut_lo, *tt_hi, *tt_lo;  // [round_up(r, 32)][ldp], fragment order
  int ms_a, ms_b;     // token splits of dA and dB
  int64_t mper_a, mper_b;
  float* da_part;     // [ms_a][r][d_in]
  float* db_part;     // [ms_b][r][d_out]
  size_t bytes;
};

// Token split of dA / dB: about QLORA_GRAM_TARGET_WGS workgroups (256
// columns x one split each, one 64-column tile per wavefront); a split is a
// multiple of QLORA_GRAM_SPLIT_TOKENS tokens (whole pairs of 64-token blocks).
// Longer splits mean fewer FP32 partials for the finish to add: at 4096
// tokens, four splits of 1024 measured faster overall than eight of 512.
#ifndef QLORA_GRAM_TARGET_WGS
#define QLORA_GRAM_TARGET_WGS 512
#endif
#ifndef QLORA_GRAM_SPLIT_TOKENS
#define QLORA_GRAM_SPLIT_TOKENS 1024
#endif
int token_splits(int64_t M, int64_t N, int64_t r, int64_t* per) {
  (void)r;
  const int64_t cgroups = cdiv(N, 256);
  const int64_t ms = std::max<int64_t>(
      1, std::min<int64_t>(cdiv(QLORA_GRAM_TARGET_WGS, cgroups), cdiv(M, QLORA_GRAM_SPLIT_TOKENS)));
  *per = round_up(cdiv(std::max<int64_t>(M, 1), ms), QLORA_GRAM_SPLIT_TOKENS);
  return (int)std::max<int64_t>(1, cdiv(M, *per));
}

BwdPlan plan_bwd(int64_t d_out, int64_t d_in, int64_t M, int64_t r, void* ws) {
  BwdPlan p{};
  Carver c(ws);
  p.t_buf = c.take<float>(M * r);
  p.ldbt = round_up(d_out, 64);
  p.bt = c.take<uint16_t>(r * p.ldbt);
  p.rp = round_up(r, 32);
  p.u_hl = c.take<uint16_t>(M * 2 * p.rp);
  if (M <= kSmallM) {
    p.r_part = c.take<float>(kRankSmallSplits * M * r);
    p.t_part = c.take<float>(gemv_tchunks(d_in) * M * r);
  } else {
    int64_t kper;
    const int64_t ks = std::max(rank_k_splits(M, d_in, &kper), rank_k_splits(M, d_out, &kper));
    p.r_part = c.take<float>(ks * M * r);
  }
  p.ldp = round_up(std::max<int64_t>(M, 1), 16);
  // fragment-ordered transposed copies: round_up(r, 32) rows
  const int64_t rf = round_up(r, 32);
  p.ut_hi = c.take<uint16_t>(rf * p.ldp);
  p.ut_lo = c.take<uint16_t>(rf * p.ldp);
  p.tt_hi = c.take<uint16_t>(rf * p.ldp);
  p.tt_lo = c.take<uint16_t>(rf * p.ldp);
  p.ms_a = token_splits(M, d_in, r, &p.mper_a);
  p.ms_b = token_splits(M, d_out, r, &p.mper_b);
  p.da_part = c.take<float>((int64_t)p.ms_a * r * d_in);
  p.db_part = c.take<float>((int64_t)p.ms_b * r * d_out);
  p.bytes = c.off + 256;
  return p;
}

// General block sizes: supported parameters and the workspace.
bool blocked_ok(int64_t n, int64_t block, int64_t group) {
  const auto pow2 = [](int64_t v) { return v > 0 && (v & (v - 1)) == 0; };
  return n >= 1 && n <= (int64_t(1) << 40) && pow2(block) && block >= 32 && block <= 4096 &&
         pow2(group) && group >= 16 && group <= 1024;
}

struct BlockedPlan {
  float* absmax;
  double* part;
  size_t bytes;
};

BlockedPlan plan_blocked(int64_t n, int64_t block, int64_t group, void* ws) {
  BlockedPlan p{};
  const int64_t n1 = cdiv(n, block), G = cdiv(n1, group);
  int64_t Gp = 1;
  while (Gp < G) Gp *= 2;
  Carver c(ws);
  p.absmax = c.take<float>(n1);
  p.part = c.take<double>(Gp);
  p.bytes = c.off + 256;
  return p;
}

int check_blocked(const qlora_nf4_blocked_t* q) {
  if (!q) return QLORA_ERR_NULL;
  if (!blocked_ok(q->n, q->block, q->group)) return QLORA_ERR_SHAPE;
  if (!q->codes || !q->scale_codes || !q->scale2 || !q->scale_mean) return QLORA_ERR_NULL;
  if (!aligned16(q->codes) || (reinterpret_cast<uintptr_t>(q->scale2) & 3u) ||
      (reinterpret_cast<uintptr_t>(q->scale_mean) & 3u))
    return QLORA_ERR_ALIGN;
  return QLORA_OK;
}

// LoRA dropout buffers, after the region of the plan they extend.  Small M
// (weight-streaming path): the masked LoRA input xm [M][d_in].  Larger M:
// the row-major keep words rbits [M][d_in / 32], applied by the rank-r
// kernels as they load X (no masked copy).  Backward: also the keep words
// of the input-gradient GEMM, keep [d_in][ldw].
struct DropPlan {
  uint16_t* xm;
  uint32_t* rbits;
  uint32_t* keep;
  int64_t ldw;
  size_t bytes;
};

DropPlan plan_drop(size_t base_bytes, int64_t M, int64_t d_in, bool with_bits, void* ws) {
  DropPlan d{};
  Carver c(ws);
  c.off = base_bytes;
  if (M <= kSmallM) d.xm = c.take<uint16_t>(M * d_in);
  else d.rbits = c.take<uint32_t>(M * (d_in / 32));
  d.ldw = cdiv(std::max<int64_t>(M, 1), 32);
  if (with_bits) d.keep = c.take<uint32_t>(d_in * d.ldw);
  d.bytes = c.off + 256;
  return d;
}

// Generator parameters of a dropout request; QLORA_ERR_SHAPE unless
// 0 <= p < 1.  thr = floor(p 2^32) (exact in FP64).
int dropout_params(const qlora_dropout_t* drop, DropoutArgs* a) {
  if (!drop) return QLORA_ERR_NULL;
  if (!(drop->p >= 0.0f && drop->p < 1.0f)) return QLORA_ERR_SHAPE;
  if (!aligned16(drop->keep_rows) || !aligned16(drop->keep_cols)) return QLORA_ERR_ALIGN;
  *a = DropoutArgs{};
  a->thr = (uint32_t)std::floor((double)drop->p * 4294967296.0);
  a->key_lo = (uint32_t)drop->seed;
  a->key_hi = (uint32_t)(drop->seed >> 32);
  a->off_lo = (uint32_t)drop->offset;
  a->off_hi = (uint32_t)(drop->offset >> 32);
  return QLORA_OK;
}

// ------------------------------------------------ nearest-level table
// Decision thresholds between adjacent NF4 levels: t_i is the smallest FP32
// value above the exact midpoint, so x >= t_i <=> x > midpoint, and a value
// exactly on a midpoint keeps the lower index.
IndexLut make_lut() {
  const float c[16] = {QLORA_NF4_LEVELS};
  float t[15];
  for (int i = 0; i < 15; ++i) {
    const double mid = ((double)c[i] + (double)c[i + 1]) / 2.0;
    const float f = (float)mid;
    t[i] = ((double)f > mid) ? f : std::nextafter(f, INFINITY);
  }
  IndexLut lut;
  for (int b = 0; b < kLutSize; ++b) {
    const double lo = (b - 64) / 64.0, hi = lo + 1.0 / 64.0;
    int base = 0;
    float thr = 2.0f;  // never reached: x <= 1
    for (int i = 0; i < 15; ++i) {
      if ((double)t[i] <= lo) ++base;
      else if ((double)t[i] < hi) thr = t[i];
    }
    lut.thr[b] = thr;
    lut.base[b] = (uint8_t)base;
  }
  return lut;
}

const IndexLut& lut() {
  static const IndexLut l = make_lut();
  return l;
}

inline int hip_status(hipError_t e) { return e == hipSuccess ? QLORA_OK : QLORA_ERR_HIP; }

// ------------------------------------------------------------- rank-r products
// v = scale * P Q^T (P [M][K], Q [N][ldq]) with the outputs of RankRowsArgs;
// small M and large M use different kernels, each deterministic, and the
// forward and the backward call the same one for the same M.  Both go
// through FP32 partials (part, [splits][M][N]) and the finish kernel, which
// adds the splits in order: kRankSmallSplits K quarters for small M, the K
// splits of rank_k_splits for large M.
int rank_product(const RankRowsArgs& ra, float* part, hipStream_t st) {
  if (ra.M > kSmallM) return hip_status(launch_rank_split(ra, part, st));
  RankSmallArgs a{};
  a.count = 1;
  a.M = ra.M;
  a.d[0] = RankSmallDesc{ra.P, ra.Q, ra.K, ra.ldq, ra.N, part, nullptr, 0, 0};
  int s = hip_status(launch_rank_small(a, st));
  if (s) return s;
  return hip_status(launch_rank_finish(part, kRankSmallSplits, ra.M, ra.N, ra.scale, ra.out,
                                       ra.ht, ra.lt, ra.ldt, ra.hl, ra.rp, st));
}

struct FwdItemArgs {
  const qlora_nf4_t* q;
  const uint16_t* X;
  const uint16_t* A;
  const uint16_t* B;
  int64_t r;
  float alpha;
  uint16_t* Y;
  float* T_save;
  void* ws;
  size_t ws_bytes;
  const uint16_t* XA;  // LoRA branch input: X, or X after dropout
  float sc;            // LoRA scale: alpha / r, or alpha / r / (1 - p)
  const uint32_t* xmask = nullptr;   // large M with dropout: keep words of XA = X
};

// Descriptors and work partition of the small-M forward for a group (see
// qlora_kernels.h): the kGemvWgs workgroups of the weight-streaming launch
// are shared among the layers in proportion to their work (largest
// remainders first), at least one each, and so that every range holds at
// least ceil(nss / (kGemvMaxSlots - 1)) units: a tile then spans at most
// kGemvMaxSlots workgroups.  A T task counts for half its chunk's
// super-steps in units: its loads go straight into MFMAs (its time is
// about one round trip to memory per four super-steps), while a weight
// unit's time is mostly the restore of its 16384 weights.
int gemv_task_cost(int64_t d_in) { return (int)std::max<int64_t>(1, gemv_tchunk_ss(d_in) / 2); }

void small_gemv_args(const FwdItemArgs* items, int count, int64_t M, GemvArgs* ga) {
  *ga = GemvArgs{};
  ga->count = count;
  ga->M = (int)M;
  ga->vec_b = true;
  int64_t U = 0;
  int tasks = 0, fin = 0;
  int64_t cost[kMaxGroup];
  for (int i = 0; i < count; ++i) {
    const FwdItemArgs& f = items[i];
    const qlora_nf4_t* q = f.q;
    const FwdPlan p = plan_fwd(q->d_out, q->d_in, M, f.r, f.ws);
    GemvDesc& d = ga->d[i];
    d.codes = q->codes;
    d.scodes = q->scale_codes;
    d.scale2 = q->scale2;
    d.mean = q->scale_mean;
    d.X = f.X;
    d.XA = f.XA;
    d.A = f.A;
    d.B = f.B;
    d.T_save = f.T_save;
    d.Y = f.Y;
    d.part = p.gemv_part;
    d.tpart = p.gemv_tpart;
    d.d_out = q->d_out;
    d.d_in = q->d_in;
    d.r = f.r;
    d.t_scale = f.sc;
    // d_out, d_in <= 2^21: fewer than 2^28 units and 2^12 tasks
    d.tiles = (int)cdiv(q->d_out, kGemvRows);
    d.nss = (int)gemv_nss(q->d_in);
    d.units = d.tiles * d.nss;
    d.tchunks = (int)gemv_tchunks(q->d_in);
    d.tchunk_ss = (int)gemv_tchunk_ss(q->d_in);
    d.n_tasks = (int)cdiv(f.r, 16) * d.tchunks;
    d.tcost = gemv_task_cost(q->d_in);
    d.toff = d.n_tasks * d.tcost;
    d.task_begin = tasks;
    d.fin_begin = fin;
    cost[i] = (int64_t)d.toff + d.units;
    U += cost[i];
    tasks += d.n_tasks;
    fin += (int)cdiv(q->d_out, 64);
    if (f.r % 8 != 0 || !aligned16(f.B)) ga->vec_b = false;
  }
  int64_t given = 0;
  int64_t rem[kMaxGroup];
  for (int i = 0; i < count; ++i) {
    const int64_t share = (int64_t)kGemvWgs * cost[i];
    ga->d[i].wgs = (int)(share / U);
    rem[i] = share % U;
    given += ga->d[i].wgs;
  }
  for (int64_t left = kGemvWgs - given; left > 0; --left) {
    int best = 0;
    for (int i = 1; i < count; ++i)
      if (rem[i] > rem[best]) best = i;
    ++ga->d[best].wgs;
    rem[best] = -1;
  }
  int wg = 0;
  for (int i = 0; i < count; ++i) {
    GemvDesc& d = ga->d[i];
    const int64_t cap = cost[i] / cdiv(d.nss, kGemvMaxSlots - 1);
    d.wgs = (int)std::max<int64_t>(1, std::min<int64_t>(d.wgs, cap));
    d.uq = (int)(cost[i] / d.wgs);
    d.urem = (int)(cost[i] % d.wgs);
    d.wg_begin = wg;
    wg += d.wgs;
  }
  ga->wgs = wg;
  ga->tasks = tasks;
  ga->fin_wgs = fin;
}

int check_fwd_item(const FwdItemArgs& f, int64_t M) {
  int s = check_nf4(f.q);
  if (s) return s;
  if (f.q->d_out > kMaxLinearDim || f.q->d_in > kMaxLinearDim) return QLORA_ERR_SHAPE;
  if (M < 0 || M > kMaxTokens) return QLORA_ERR_SHAPE;
  if (f.r < 1 || f.r > kMaxRank) return QLORA_ERR_SHAPE;
  if (M == 0) return QLORA_OK;
  if (!f.X || !f.A || !f.B || !f.Y) return QLORA_ERR_NULL;
  if (!aligned16(f.X) || !aligned16(f.A) || !aligned16(f.Y) || !aligned16(f.T_save) ||
      !aligned16(f.ws))
    return QLORA_ERR_ALIGN;
  if (!f.ws) return QLORA_ERR_NULL;
  if (f.ws_bytes < plan_fwd(f.q->d_out, f.q->d_in, M, f.r, nullptr).bytes)
    return QLORA_ERR_WORKSPACE;
  return QLORA_OK;
}

// Forward of up to kMaxGroup layers sharing the token count M.
int fwd_group(const FwdItemArgs* items, int count, int64_t M, hipStream_t st) {
  if (count < 1 || count > kMaxGroup) return QLORA_ERR_SHAPE;
  for (int i = 0; i < count; ++i) {
    int s = check_fwd_item(items[i], M);
    if (s) return s;
  }
  if (M == 0) return QLORA_OK;

  if (M > kSmallM) {
    for (int i = 0; i < count; ++i) {
      const FwdItemArgs& f = items[i];
      const qlora_nf4_t* q = f.q;
      FwdPlan p = plan_fwd(q->d_out, q->d_in, M, f.r, f.ws);
      float* T = f.T_save ? f.T_save : p.t_buf;
      RankRowsArgs ra{f.XA,   f.A,     M,       f.r,     q->d_in, q->d_in, f.sc,
                      T,      p.t_hl,  p.rp,    nullptr, nullptr, 0,        f.xmask};
      int s = rank_product(ra, p.r_part, st);
      if (s) return s;
      GemmArgs g{q->codes, q->scale_codes, q->scale2, q->scale_mean, f.X, p.t_hl, f.B, f.Y,
                 M,        q->d_out,      q->d_in,  f.r};
      s = hip_status(launch_gemm_fwd(g, st));
      if (s) return s;
    }
    return QLORA_OK;
  }

  // Small M: one weight-streaming launch for the whole group (whose first
  // workgroups also form the partials of T = s X A^T) and one finish launch.
  GemvArgs ga;
  small_gemv_args(items, count, M, &ga);
  return hip_status(launch_gemv(ga, st));
}

// Argument checks shared by both backward entry points.
int check_bwd(const qlora_nf4_t* q, const uint16_t* X, const uint16_t* dY, int64_t M,
              const uint16_t* A, const uint16_t* B, int64_t r, const float* T_saved,
              const uint16_t* dX, const float* dA, const float* dB, const void* ws) {
  int s = check_nf4(q);
  if (s) return s;
  if (M < 0 || M > kMaxTokens || r < 1 || r > kMaxRank) return QLORA_ERR_SHAPE;
  if (q->d_out > kMaxLinearDim || q->d_in > kMaxLinearDim) return QLORA_ERR_SHAPE;
  if (!dA || !dB || !ws) return QLORA_ERR_NULL;
  if (M > 0 && (!X || !dY || !A || !B)) return QLORA_ERR_NULL;
  if (!aligned16(X) || !aligned16(dY) || !aligned16(A) || !aligned16(T_saved) ||
      !aligned16(dX) || !aligned16(dA) || !aligned16(dB) || !aligned16(ws))
    return QLORA_ERR_ALIGN;
  return QLORA_OK;
}

// The backward after the checks.  XA is the LoRA branch's input (X, or X
// after dropout), sc the LoRA scale, keep the dropout keep words of the
// input gradient's LoRA term (NULL: none).
int bwd_impl(const qlora_nf4_t* q, const uint16_t* XA, const uint32_t* xmask,
             const uint32_t* keep, int64_t keep_ld, const uint16_t* dY, int64_t M,
             const uint16_t* A, const uint16_t* B, int64_t r, float sc, const float* T_saved,
             uint16_t* dX, float* dA, float* dB, const BwdPlan& p, hipStream_t st) {
  int s = QLORA_OK;
  const int64_t d_out = q->d_out, d_in = q->d_in;
  if (M == 0) {
    s = hip_status(hipMemsetAsync(dA, 0, size_t(r * d_in) * sizeof(float), st));
    if (!s) s = hip_status(hipMemsetAsync(dB, 0, size_t(d_out * r) * sizeof(float), st));
    return s;
  }
  // T = s XA A^T (unless saved by the forward), and its transposed hi/lo copy
  // (the same kernels and summation order as the forward, so a recomputed T
  // equals a saved one bit for bit)
  const float* T = T_saved;
  // large M with a saved T: its transposed copies are formed in the finish
  // launch of U below
  bool t_with_u = false;
  FinishDesc t_copy{};
  if (T && M > kSmallM) {
    t_with_u = true;
    t_copy = FinishDesc{T, nullptr, p.tt_hi, p.tt_lo, M, r, p.ldp, 1.0f, 1, 0, nullptr, 0};
  } else if (!T && M > kSmallM) {
    RankRowsArgs ra{XA, A, M, r, d_in, d_in, sc, p.t_buf, nullptr, 0, p.tt_hi, p.tt_lo, p.ldp,
                    xmask};
    s = rank_product(ra, p.r_part, st);
    if (s) return s;
    T = p.t_buf;
  } else if (!T) {
    // the forward's T tasks alone, then the chunk partials added in the same
    // order and scaled as in the forward's finish (same bits), with the
    // transposed copies
    GemvArgs ga{};
    ga.count = 1;
    ga.M = (int)M;
    GemvDesc& d = ga.d[0];
    d.XA = XA;
    d.A = A;
    d.tpart = p.t_part;
    d.d_in = d_in;
    d.d_out = d_out;
    d.r = r;
    d.tchunks = (int)gemv_tchunks(d_in);
    d.tchunk_ss = (int)gemv_tchunk_ss(d_in);
    d.n_tasks = (int)cdiv(r, 16) * d.tchunks;
    ga.tasks = d.n_tasks;
    s = hip_status(launch_gemv_tasks(ga, st));
    if (s) return s;
    s = hip_status(launch_rank_finish(p.t_part, d.tchunks, M, r, sc, p.t_buf, p.tt_hi, p.tt_lo,
                                      p.ldp, nullptr, 0, st));
    if (s) return s;
    T = p.t_buf;
  } else {
    s = hip_status(launch_rank_finish(T, 1, M, r, 1.0f, nullptr, p.tt_hi, p.tt_lo, p.ldp,
                                      nullptr, 0, st));
    if (s) return s;
  }
  // U = s dY B.  For large M with whole 16-byte pieces of dY's and B's rows,
  // the K-split kernel stages B as stored; otherwise through B^T, so that
  // the contraction over d_out is contiguous.  Same products, same bits.
  const bool b_as_stored = M > kSmallM && d_out % 8 == 0 && r % 8 == 0 && aligned16(B);
  if (!b_as_stored) {
    s = hip_status(launch_transpose_bf16(B, d_out, r, p.bt, p.ldbt, st));
    if (s) return s;
  }
  {
    RankRowsArgs ra{dY, b_as_stored ? B : p.bt, M, r, d_out, b_as_stored ? r : p.ldbt, sc, nullptr,
                    p.u_hl, p.rp, p.ut_hi, p.ut_lo, p.ldp};
    ra.q_kn = b_as_stored;
    s = t_with_u ? hip_status(launch_rank_split(ra, p.r_part, st, &t_copy))
                 : rank_product(ra, p.r_part, st);
  }
  if (s) return s;
  // dX = dY Wh + U A (the U A term cleared at dropped positions)
  if (dX) {
    GemmArgs g{q->codes, q->scale_codes, q->scale2, q->scale_mean, dY, p.u_hl, A, dX,
               M,        d_out,          d_in,      r,            keep, keep_ld};
    s = hip_status(launch_gemm_bwd(g, st));
    if (s) return s;
  }
  // dA = U^T XA ; dB = (T^T dY)^T, both contractions in one launch and
  // both finishes in another
  const GramProblem gp[2] = {
      {p.ut_hi, p.ut_lo, XA, d_in, p.mper_a, p.ms_a, p.da_part, dA, false, xmask},
      {p.tt_hi, p.tt_lo, dY, d_out, p.mper_b, p.ms_b, p.db_part, dB, true, nullptr}};
  return hip_status(launch_grams(gp, 2, p.ldp, M, r, st));
}

}  // namespace

namespace qlora {
// qlora_linear_fwd's argument checks for a workspace of ws_bytes bytes (not
// dereferenced): QLORA_ERR_WORKSPACE when the call needs more.  Host only.
int linear_fwd_check(const qlora_nf4_t* q, const uint16_t* X, int64_t M, const uint16_t* A,
                     const uint16_t* B, int64_t r, uint16_t* Y, float* T_save, size_t ws_bytes) {
  // a stand-in address that passes the workspace's null and alignment checks
  void* const ws = reinterpret_cast<void*>(uintptr_t(256));
  FwdItemArgs f{q, X, A, B, r, 0.0f, Y, T_save, ws, ws_bytes, X, 0.0f};
  return check_fwd_item(f, M);
}
}  // namespace qlora

// ===================================================================== ABI
extern "C" {

const char* qlora_status_string(int status) {
  switch (status) {
    case QLORA_OK: return "ok";
    case QLORA_ERR_NULL: return "a required pointer is NULL";
    case QLORA_ERR_SHAPE: return "a size is out of range";
    case QLORA_ERR_ALIGN: return "a pointer is not 16-byte aligned";
    case QLORA_ERR_WORKSPACE: return "workspace too small";
    case QLORA_ERR_HIP: return "HIP runtime error";
    case QLORA_ERR_SCRATCH: return "the call needs more than the library's fixed device scratch";
    default: return "unknown status";
  }
}

int qlora_abi_version(void) { return (1 << 16) | 1; }

int qlora_nf4_sizes(int64_t d_out, int64_t d_in, size_t* codes_bytes, size_t* scale_codes_bytes,
                    size_t* scale2_bytes, size_t* scale_mean_bytes) {
  if (!codes_bytes || !scale_codes_bytes || !scale2_bytes || !scale_mean_bytes)
    return QLORA_ERR_NULL;
  if (!shape_ok(d_out, d_in)) return QLORA_ERR_SHAPE;
  const int64_t n = d_out * d_in, n1 = n / kBlock;
  *codes_bytes = size_t(n / 2);
  *scale_codes_bytes = size_t(n1);
  *scale2_bytes = size_t(cdiv(n1, kGroup)) * sizeof(float);
  *scale_mean_bytes = sizeof(float);
  return QLORA_OK;
}

size_t qlora_workspace_bytes(int op, int64_t d_out, int64_t d_in, int64_t M, int64_t r) {
  if (!shape_ok(d_out, d_in)) return 0;
  if (op == QLORA_OP_QUANTIZE) return plan_quant(d_out, d_in, nullptr).bytes;
  if (M < 0 || r < 1 || r > kMaxRank) return 0;
  if (op == QLORA_OP_FWD) return plan_fwd(d_out, d_in, M, r, nullptr).bytes;
  if (op == QLORA_OP_BWD) return plan_bwd(d_out, d_in, M, r, nullptr).bytes;
  if (op == QLORA_OP_FWD_DROPOUT)
    return plan_drop(plan_fwd(d_out, d_in, M, r, nullptr).bytes, M, d_in, false, nullptr).bytes;
  if (op == QLORA_OP_BWD_DROPOUT)
    return plan_drop(plan_bwd(d_out, d_in, M, r, nullptr).bytes, M, d_in, true, nullptr).bytes;
  return 0;
}

int qlora_quantize_nf4(const float* W, const qlora_nf4_t* q, void* ws, size_t ws_bytes,
                       void* stream) {
  int s = check_nf4(q);
  if (s) return s;
  if (!W || !ws) return QLORA_ERR_NULL;
  if (!aligned16(W) || !aligned16(ws)) return QLORA_ERR_ALIGN;
  QuantPlan p = plan_quant(q->d_out, q->d_in, ws);
  if (ws_bytes < p.bytes) return QLORA_ERR_WORKSPACE;
  QuantWorkspace w{p.absmax, p.part};
  return hip_status(launch_quantize(W, p.n, q->codes, q->scale_codes, q->scale2, q->scale_mean, w,
                                    lut(), static_cast<hipStream_t>(stream)));
}

int qlora_dequant_bf16(const qlora_nf4_t* q, uint16_t* W_bf16, void* stream) {
  int s = check_nf4(q);
  if (s) return s;
  if (!W_bf16) return QLORA_ERR_NULL;
  if (!aligned16(W_bf16)) return QLORA_ERR_ALIGN;
  return hip_status(launch_dequant(q->codes, q->scale_codes, q->scale2, q->scale_mean,
                                   q->d_out * q->d_in, W_bf16, static_cast<hipStream_t>(stream)));
}

int qlora_quantize_nf4_many(int count, const qlora_quant_item* items, void* stream) {
  if (count < 1 || count > kMaxGroup) return QLORA_ERR_SHAPE;
  if (!items) return QLORA_ERR_NULL;
  QuantList a{};
  a.count = count;
  for (int i = 0; i < count; ++i) {
    const qlora_quant_item& it = items[i];
    int s = check_nf4(&it.q);
    if (s) return s;
    if (!it.W || !it.workspace) return QLORA_ERR_NULL;
    if (!aligned16(it.W) || !aligned16(it.workspace)) return QLORA_ERR_ALIGN;
    const QuantPlan p = plan_quant(it.q.d_out, it.q.d_in, it.workspace);
    if (it.workspace_bytes < p.bytes) return QLORA_ERR_WORKSPACE;
    a.d[i] = quant_item(it.W, p.n, it.q.codes, it.q.scale_codes, it.q.scale2, it.q.scale_mean,
                        QuantWorkspace{p.absmax, p.part});
  }
  return hip_status(launch_quantize_list(a, lut(), static_cast<hipStream_t>(stream)));
}

int qlora_dequant_bf16_many(int count, const qlora_dequant_item* items, void* stream) {
  if (count < 1 || count > kMaxGroup) return QLORA_ERR_SHAPE;
  if (!items) return QLORA_ERR_NULL;
  DequantList a{};
  a.count = count;
  for (int i = 0; i < count; ++i) {
    const qlora_dequant_item& it = items[i];
    int s = check_nf4(&it.q);
    if (s) return s;
    if (!it.W_bf16) return QLORA_ERR_NULL;
    if (!aligned16(it.W_bf16)) return QLORA_ERR_ALIGN;
    a.d[i] = DequantItem{it.q.codes, it.q.scale_codes, it.q.scale2, it.q.scale_mean,
                         it.q.d_out * it.q.d_in / kBlock, it.W_bf16, 0, 0};
  }
  return hip_status(launch_dequant_list(a, static_cast<hipStream_t>(stream)));
}

size_t qlora_sumsq_workspace_bytes(int count, const qlora_adamw_param* params) {
  if (count < 0 || (count > 0 && !params)) return 0;
  int64_t len = 0;
  for (int i = 0; i < count; ++i) {
    if (params[i].n < 0 || params[i].n > kOptMaxElems) return 0;
    len += sumsq_part_len(params[i].n);
  }
  Carver c(nullptr);
  c.take<double>(std::max<int64_t>(len, 1));
  c.take<double>(std::max(count, 1));
  return c.off + 256;
}

int qlora_grad_sumsq(int count, const qlora_adamw_param* params, double* acc, void* ws,
                     size_t ws_bytes, void* stream) {
  if (count < 0) return QLORA_ERR_SHAPE;
  if (count == 0) return QLORA_OK;
  if (!params || !acc || !ws) return QLORA_ERR_NULL;
  if (!aligned16(ws)) return QLORA_ERR_ALIGN;
  int64_t len = 0;
  for (int i = 0; i < count; ++i) {
    if (params[i].n < 0 || params[i].n > kOptMaxElems) return QLORA_ERR_SHAPE;
    if (params[i].n > 0 && !params[i].grad) return QLORA_ERR_NULL;
    len += sumsq_part_len(params[i].n);
  }
  if (ws_bytes < qlora_sumsq_workspace_bytes(count, params)) return QLORA_ERR_WORKSPACE;
  Carver c(ws);
  double* part = c.take<double>(std::max<int64_t>(len, 1));
  double* sums = c.take<double>(count);
  std::vector<const float*> g(count);
  std::vector<int64_t> n(count);
  for (int i = 0; i < count; ++i) {
    g[i] = params[i].grad;
    n[i] = params[i].n;
  }
  return hip_status(launch_sumsq(g.data(), n.data(), count, acc, part, sums,
                                 static_cast<hipStream_t>(stream)));
}

int qlora_adamw_step(int count, const qlora_adamw_param* params, float lr, float beta1,
                     float beta2, float eps, float weight_decay, int64_t step,
                     const double* grad_sumsq, float max_grad_norm, void* stream) {
  if (count < 0 || step < 1) return QLORA_ERR_SHAPE;
  if (!(beta1 >= 0.0f && beta1 < 1.0f && beta2 >= 0.0f && beta2 < 1.0f)) return QLORA_ERR_SHAPE;
  if (count == 0) return QLORA_OK;
  if (!params) return QLORA_ERR_NULL;
  std::vector<AdamwDesc> d;
  d.reserve(count);
  for (int i = 0; i < count; ++i) {
    const qlora_adamw_param& t = params[i];
    if (t.n < 0 || t.n > kOptMaxElems) return QLORA_ERR_SHAPE;
    if (t.n == 0) continue;
    if (!t.param || !t.grad || !t.m || !t.v) return QLORA_ERR_NULL;
    d.push_back(AdamwDesc{t.param, t.param_bf16, t.grad, t.m, t.v, t.n});
  }
  if (d.empty()) return QLORA_OK;
  AdamwScalars h{};
  h.lr = lr;
  h.lrwd = lr * weight_decay;
  h.b1 = beta1;
  h.ob1 = 1.0f - beta1;
  h.b2 = beta2;
  h.ob2 = 1.0f - beta2;
  h.bc1 = (float)(1.0 - std::pow((double)beta1, (double)step));
  h.bc2 = (float)(1.0 - std::pow((double)beta2, (double)step));
  h.eps = eps;
  h.max_norm = max_grad_norm;
  return hip_status(launch_adamw(d.data(), (int)d.size(), h, grad_sumsq,
                                 static_cast<hipStream_t>(stream)));
}

int qlora_merge_nf4(const qlora_nf4_t* q, const uint16_t* A, const uint16_t* B, int64_t r,
                    float lora_alpha, float* W_merged, const qlora_nf4_t* q_out, void* ws,
                    size_t ws_bytes, void* stream) {
  int s = check_nf4(q);
  if (s) return s;
  if (q->d_out > kMaxLinearDim || q->d_in > kMaxLinearDim) return QLORA_ERR_SHAPE;
  if (r < 1 || r > kMaxRank) return QLORA_ERR_SHAPE;
  if (!A || !B || !W_merged) return QLORA_ERR_NULL;
  if (!aligned16(A) || !aligned16(W_merged)) return QLORA_ERR_ALIGN;
  QuantPlan p{};
  if (q_out) {
    s = check_nf4(q_out);
    if (s) return s;
    if (q_out->d_out != q->d_out || q_out->d_in != q->d_in) return QLORA_ERR_SHAPE;
    if (!ws) return QLORA_ERR_NULL;
    if (!aligned16(ws)) return QLORA_ERR_ALIGN;
    p = plan_quant(q->d_out, q->d_in, ws);
    if (ws_bytes < p.bytes) return QLORA_ERR_WORKSPACE;
  }
  hipStream_t st = static_cast<hipStream_t>(stream);
  const MergeArgs m{q->codes, q->scale_codes, q->scale2, q->scale_mean, A, B, W_merged,
                    q->d_out, q->d_in, r, lora_alpha / (float)r};
  s = hip_status(launch_merge(m, st));
  if (s || !q_out) return s;
  QuantWorkspace w{p.absmax, p.part};
  return hip_status(launch_quantize(W_merged, p.n, q_out->codes, q_out->scale_codes,
                                    q_out->scale2, q_out->scale_mean, w, lut(), st));
}

int qlora_linear_fwd(const qlora_nf4_t* q, const uint16_t* X, int64_t M, const uint16_t* A,
                     const uint16_t* B, int64_t r, float lora_alpha, uint16_t* Y, float* T_save,
                     void* ws, size_t ws_bytes, void* stream) {
  FwdItemArgs f{q, X, A, B, r, lora_alpha, Y, T_save, ws, ws_bytes, X, lora_alpha / (float)r};
  return fwd_group(&f, 1, M, static_cast<hipStream_t>(stream));
}

int qlora_linear_fwd_many(int count, const qlora_fwd_item* items, int64_t M, void* stream) {
  if (!items) return QLORA_ERR_NULL;
  if (count < 1 || count > kMaxGroup) return QLORA_ERR_SHAPE;
  FwdItemArgs f[kMaxGroup];
  for (int i = 0; i < count; ++i) {
    const qlora_fwd_item& it = items[i];
    f[i] = FwdItemArgs{&it.w, it.X, it.A, it.B, it.r, it.lora_alpha, it.Y, it.T_save,
                       it.workspace, it.workspace_bytes, it.X,
                       it.r > 0 ? it.lora_alpha / (float)it.r : 0.0f};
  }
  return fwd_group(f, count, M, static_cast<hipStream_t>(stream));
}

int qlora_linear_bwd(const qlora_nf4_t* q, const uint16_t* X, const uint16_t* dY, int64_t M,
                     const uint16_t* A, const uint16_t* B, int64_t r, float lora_alpha,
                     const float* T_saved, uint16_t* dX, float* dA, float* dB, void* ws,
                     size_t ws_bytes, void* stream) {
  int s = check_bwd(q, X, dY, M, A, B, r, T_saved, dX, dA, dB, ws);
  if (s) return s;
  const BwdPlan p = plan_bwd(q->d_out, q->d_in, M, r, ws);
  if (ws_bytes < p.bytes) return QLORA_ERR_WORKSPACE;
  return bwd_impl(q, X, nullptr, nullptr, 0, dY, M, A, B, r, lora_alpha / (float)r, T_saved, dX,
                  dA, dB, p, static_cast<hipStream_t>(stream));
}

int qlora_linear_fwd_dropout(const qlora_nf4_t* q, const uint16_t* X, int64_t M,
                             const uint16_t* A, const uint16_t* B, int64_t r, float lora_alpha,
                             const qlora_dropout_t* drop, uint16_t* Y, float* T_save, void* ws,
                             size_t ws_bytes, void* stream) {
  DropoutArgs da;
  int s = dropout_params(drop, &da);
  if (s) return s;
  FwdItemArgs f{q, X, A, B, r, lora_alpha, Y, T_save, ws, ws_bytes, X, 0.0f};
  s = check_fwd_item(f, M);
  if (s) return s;
  if (M == 0) return QLORA_OK;
  const int64_t d_in = q->d_in;
  const DropPlan dp = plan_drop(plan_fwd(q->d_out, d_in, M, r, nullptr).bytes, M, d_in, false, ws);
  if (ws_bytes < dp.bytes) return QLORA_ERR_WORKSPACE;
  hipStream_t st = static_cast<hipStream_t>(stream);
  da.X = X;
  da.Xm = dp.xm;
  da.M = M;
  da.d = d_in;
  da.ldw = dp.ldw;
  if (M <= kSmallM) {
    // the masked copy (M rows) for the weight-streaming launch's T
    s = hip_status(launch_dropout(da, st));
    f.XA = dp.xm;
  } else {
    // keep words only (also into the caller's saved-mask buffers when
    // given); T's kernel clears the dropped elements as it loads X
    const bool save = drop->keep_rows && drop->keep_cols;
    uint32_t* rows = save ? drop->keep_rows : dp.rbits;
    da.keep = save ? drop->keep_cols : nullptr;
    s = hip_status(launch_dropout_bits(da, rows, st));
    f.XA = X;
    f.xmask = rows;
  }
  if (s) return s;
  f.sc = (lora_alpha / (float)r) / (1.0f - drop->p);
  return fwd_group(&f, 1, M, st);
}

int qlora_linear_bwd_dropout(const qlora_nf4_t* q, const uint16_t* X, const uint16_t* dY,
                             int64_t M, const uint16_t* A, const uint16_t* B, int64_t r,
                             float lora_alpha, const qlora_dropout_t* drop, const float* T_saved,
                             uint16_t* dX, float* dA, float* dB, void* ws, size_t ws_bytes,
                             void* stream) {
  DropoutArgs da;
  int s = dropout_params(drop, &da);
  if (s) return s;
  s = check_bwd(q, X, dY, M, A, B, r, T_saved, dX, dA, dB, ws);
  if (s) return s;
  const int64_t d_in = q->d_in;
  const BwdPlan p = plan_bwd(q->d_out, d_in, M, r, ws);
  const DropPlan dp = plan_drop(p.bytes, M, d_in, true, ws);
  if (ws_bytes < dp.bytes) return QLORA_ERR_WORKSPACE;
  hipStream_t st = static_cast<hipStream_t>(stream);
  // the forward's saved mask (M > 16), else the mask regenerated
  const bool saved = M > kSmallM && drop->keep_rows && drop->keep_cols;
  if (M > 0 && !saved) {
    da.X = X;
    da.Xm = dp.xm;
    da.keep = dp.keep;
    da.M = M;
    da.d = d_in;
    da.ldw = dp.ldw;
    s = hip_status(M <= kSmallM ? launch_dropout(da, st) : launch_dropout_bits(da, dp.rbits, st));
    if (s) return s;
  }
  const float sc = (lora_alpha / (float)r) / (1.0f - drop->p);
  if (M <= kSmallM)
    return bwd_impl(q, dp.xm, nullptr, dp.keep, dp.ldw, dY, M, A, B, r, sc, T_saved, dX, dA, dB,
                    p, st);
  if (saved)
    return bwd_impl(q, X, drop->keep_rows, drop->keep_cols, dp.ldw, dY, M, A, B, r, sc, T_saved,
                    dX, dA, dB, p, st);
  return bwd_impl(q, X, dp.rbits, dp.keep, dp.ldw, dY, M, A, B, r, sc, T_saved, dX, dA, dB, p,
                  st);
}

int qlora_nf4_blocked_sizes(int64_t n, int64_t block, int64_t group, size_t* codes_bytes,
                            size_t* scale_codes_bytes, size_t* scale2_bytes) {
  if (!codes_bytes || !scale_codes_bytes || !scale2_bytes) return QLORA_ERR_NULL;
  if (!blocked_ok(n, block, group)) return QLORA_ERR_SHAPE;
  const int64_t n1 = cdiv(n, block);
  *codes_bytes = size_t(cdiv(n, 2));
  *scale_codes_bytes = size_t(n1);
  *scale2_bytes = size_t(cdiv(n1, group)) * sizeof(float);
  return QLORA_OK;
}

size_t qlora_quantize_blocked_workspace_bytes(int64_t n, int64_t block, int64_t group) {
  if (!blocked_ok(n, block, group)) return 0;
  return plan_blocked(n, block, group, nullptr).bytes;
}

int qlora_quantize_nf4_blocked(const float* W, const qlora_nf4_blocked_t* q, void* ws,
                               size_t ws_bytes, void* stream) {
  int s = check_blocked(q);
  if (s) return s;
  if (!W || !ws) return QLORA_ERR_NULL;
  if (!aligned16(W) || !aligned16(ws)) return QLORA_ERR_ALIGN;
  const BlockedPlan p = plan_blocked(q->n, q->block, q->group, ws);
  if (ws_bytes < p.bytes) return QLORA_ERR_WORKSPACE;
  const BlockedQuant bq{W, q->n, q->block, q->group, q->codes, q->scale_codes, q->scale2,
                        q->scale_mean, p.absmax, p.part};
  return hip_status(launch_quantize_blocked(bq, lut(), static_cast<hipStream_t>(stream)));
}

int qlora_dequant_bf16_blocked(const qlora_nf4_blocked_t* q, uint16_t* W_bf16, void* stream) {
  int s = check_blocked(q);
  if (s) return s;
  if (!W_bf16) return QLORA_ERR_NULL;
  if (!aligned16(W_bf16)) return QLORA_ERR_ALIGN;
  return hip_status(launch_dequant_blocked(q->codes, q->scale_codes, q->scale2, q->scale_mean,
                                           q->n, q->block, q->group, W_bf16,
                                           static_cast<hipStream_t>(stream)));
}

int qlora_dropout_mask(const uint16_t* X, int64_t M, int64_t d, const qlora_dropout_t* drop,
                       uint16_t* X_kept, uint32_t* keep_bits, void* stream) {
  DropoutArgs da;
  int s = dropout_params(drop, &da);
  if (s) return s;
  if (M < 0 || M > kMaxTokens || d < 0 || d > kMaxLinearDim || d % 8) return QLORA_ERR_SHAPE;
  if (M == 0 || d == 0) return QLORA_OK;
  if (!X_kept && !keep_bits) return QLORA_ERR_NULL;
  if (X_kept && !X) return QLORA_ERR_NULL;
  if (!aligned16(X) || !aligned16(X_kept) || !aligned16(keep_bits)) return QLORA_ERR_ALIGN;
  da.X = X;
  da.Xm = X_kept;
  da.keep = keep_bits;
  da.M = M;
  da.d = d;
  da.ldw = cdiv(M, 32);
  return hip_status(launch_dropout(da, static_cast<hipStream_t>(stream)));
}

}  // extern "C"
