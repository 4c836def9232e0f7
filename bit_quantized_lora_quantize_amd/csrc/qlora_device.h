// qlora_device.h -- device helpers shared by the libqlora kernels (gfx950).
//
// Sources (the pages): "第 04 篇：QLoRA 原理" [QP], "QLoRA" concept page [CP].
// Compiled with -ffp-contract=off: every FP32 product and sum below is rounded
// on its own, as the restored-weight formula requires.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace qlora {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kBlock = 64;   // weights per first-level scale  [QP §3.4]
constexpr int kGroup = 256;  // first-level scales per FP32 second-level scale [QP §5.2]

// The 16 NF4 levels printed in [QP §4.3], index 0..15.
#define QLORA_NF4_LEVELS                                                      \
  -1.0000000f, -0.6961928f, -0.5250731f, -0.3949175f, -0.2844414f,            \
      -0.1847734f, -0.0910500f, 0.0000000f, 0.0795803f, 0.1609302f,           \
      0.2461123f, 0.3379152f, 0.4407098f, 0.5626170f, 0.7229568f, 1.0000000f

// ---------------------------------------------------------------- FP8 E4M3FN
// OCP 8-bit float: sign, 4 exponent bits (bias 7), 3 mantissa bits, no
// infinities; exponent 0 holds subnormals m * 2^-9; largest finite 448.
// gfx950's v_cvt_f32_fp8 decodes this format exactly (every value is a small
// integer times a power of two); it reads the low byte of `code`.  The
// encoder below never produces the NaN codes 0x7F / 0xFF.
__device__ __forceinline__ float fp8e4m3_to_f32(uint32_t code) {
  return __builtin_amdgcn_cvt_f32_fp8((int)code, 0);
}

// Round-to-nearest-even encode with saturation at 448; sign bit = sign of y.
__device__ __forceinline__ uint32_t f32_to_fp8e4m3_rne_sat(float y) {
  uint32_t u = __float_as_uint(y);
  uint32_t sign = (u >> 24) & 0x80u;
  uint32_t a = u & 0x7FFFFFFFu;
  float af = __uint_as_float(a);
  uint32_t code;
  if (!(af < 448.0f)) {
    code = 0x7Eu;
  } else if (af < 0x1p-6f) {              // subnormal range: multiples of 2^-9
    code = (uint32_t)__builtin_rintf(af * 512.0f);  // exact scaling, RNE; 8 == 2^-6
  } else {
    uint32_t e = (a >> 23) - 127u + 7u;   // 1..15
    uint32_t q = (a >> 20) & 7u, rem = a & 0xFFFFFu;
    if (rem > 0x80000u || (rem == 0x80000u && (q & 1u))) ++q;
    code = (e << 3) + q;                  // q == 8 carries into the exponent
    if (code > 0x7Eu) code = 0x7Eu;
  }
  return code | sign;
}

// Restored first-level scale: fp8(code) * s2 + mean, two FP32 roundings.
__device__ __forceinline__ float restored_scale(uint32_t code, float s2, float mean) {
  return __fadd_rn(__fmul_rn(fp8e4m3_to_f32(code), s2), mean);
}

// Two FP32 values -> packed BF16 pair (RNE, hardware v_cvt_pk_bf16_f32); a in
// the low half.
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  f32x2 v = {a, b};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2));
}

__device__ __forceinline__ float bf16lo_to_f32(uint32_t p) { return __uint_as_float(p << 16); }
__device__ __forceinline__ float bf16hi_to_f32(uint32_t p) { return __uint_as_float(p & 0xFFFF0000u); }

// ------------------------------------------------------- NF4 block table
// The 16 restored weights of one block, RNE_bf16(level_i * scale), stored as
// four 8-byte byte tables for v_perm_b32: low bytes and high bytes of the
// BF16 patterns, for the negative half (levels 0..7) and the positive half
// (levels 8..15).
struct Nf4Table {
  uint32_t ln0, ln1, lp0, lp1;  // low bytes: levels 0-3, 4-7, 8-11, 12-15
  uint32_t hn0, hn1, hp0, hp1;  // high bytes, same grouping
};

__device__ __forceinline__ Nf4Table nf4_table(float scale) {
  const float c[16] = {QLORA_NF4_LEVELS};
  uint32_t q[8];
#pragma unroll
  for (int i = 0; i < 8; ++i)
    q[i] = pack_bf16x2(__fmul_rn(c[2 * i], scale), __fmul_rn(c[2 * i + 1], scale));
  Nf4Table t;
  // q[2i] holds levels 4i, 4i+1; q[2i+1] holds 4i+2, 4i+3.  Bytes 0,2 are the
  // low bytes and 1,3 the high bytes of the two BF16 patterns.
  t.ln0 = __builtin_amdgcn_perm(q[1], q[0], 0x06040200u);
  t.hn0 = __builtin_amdgcn_perm(q[1], q[0], 0x07050301u);
  t.ln1 = __builtin_amdgcn_perm(q[3], q[2], 0x06040200u);
  t.hn1 = __builtin_amdgcn_perm(q[3], q[2], 0x07050301u);
  t.lp0 = __builtin_amdgcn_perm(q[5], q[4], 0x06040200u);
  t.hp0 = __builtin_amdgcn_perm(q[5], q[4], 0x07050301u);
  t.lp1 = __builtin_amdgcn_perm(q[7], q[6], 0x06040200u);
  t.hp1 = __builtin_amdgcn_perm(q[7], q[6], 0x07050301u);
  return t;
}

// Look up four 4-bit indices held one per byte (values 0..15) in `n`.
// v_perm_b32 picks byte `sel` (0..7) of its 8-byte source and returns 0xFF
// for selectors >= 13.  The index bit 3 is moved to bit 4, so the
// negative-half selector is in range (0..7) exactly when the index is < 8 and
// the positive-half selector (bit 4 flipped) exactly when it is >= 8; the
// out-of-range side reads 0xFF and the AND keeps the in-range byte.
__device__ __forceinline__ void nf4_lookup4(uint32_t n, const Nf4Table& t,
                                            uint32_t& lo, uint32_t& hi) {
  uint32_t sn = n + (n & 0x08080808u);
  uint32_t sp = sn ^ 0x10101010u;
  lo = __builtin_amdgcn_perm(t.ln1, t.ln0, sn) & __builtin_amdgcn_perm(t.lp1, t.lp0, sp);
  hi = __builtin_amdgcn_perm(t.hn1, t.hn0, sn) & __builtin_amdgcn_perm(t.hp1, t.hp0, sp);
}

// Eight packed indices (element e in bits 4e..4e+3 of `codes`) -> eight BF16
// restored weights in the order [e0 e2 e4 e6 e1 e3 e5 e7], two per dword.
// Contractions that use this order must permute the other operand the same
// way (QLORA_PERM8).
__device__ __forceinline__ u32x4 nf4_dequant8_perm(uint32_t codes, const Nf4Table& t) {
  uint32_t le, he, lo, ho;
  nf4_lookup4(codes & 0x0F0F0F0Fu, t, le, he);          // e0 e2 e4 e6
  nf4_lookup4((codes >> 4) & 0x0F0F0F0Fu, t, lo, ho);   // e1 e3 e5 e7
  u32x4 r;
  r.x = __builtin_amdgcn_perm(he, le, 0x05010400u);     // (e0, e2)
  r.y = __builtin_amdgcn_perm(he, le, 0x07030602u);     // (e4, e6)
  r.z = __builtin_amdgcn_perm(ho, lo, 0x05010400u);     // (e1, e3)
  r.w = __builtin_amdgcn_perm(ho, lo, 0x07030602u);     // (e5, e7)
  return r;
}

// Same lookup, natural element order: (e0,e1), (e2,e3), (e4,e5), (e6,e7).
// The indices are put in element order before the lookups (two byte
// permutes of the even and odd nibbles), so each lookup yields the low and
// high bytes of four consecutive weights and one permute per dword pairs them.
__device__ __forceinline__ u32x4 nf4_dequant8(uint32_t codes, const Nf4Table& t) {
  const uint32_t ev = codes & 0x0F0F0F0Fu;            // e0 e2 e4 e6
  const uint32_t od = (codes >> 4) & 0x0F0F0F0Fu;     // e1 e3 e5 e7
  uint32_t l03, h03, l47, h47;
  nf4_lookup4(__builtin_amdgcn_perm(od, ev, 0x05010400u), t, l03, h03);   // e0 e1 e2 e3
  nf4_lookup4(__builtin_amdgcn_perm(od, ev, 0x07030602u), t, l47, h47);   // e4 e5 e6 e7
  u32x4 r;
  r.x = __builtin_amdgcn_perm(h03, l03, 0x05010400u);
  r.y = __builtin_amdgcn_perm(h03, l03, 0x07030602u);
  r.z = __builtin_amdgcn_perm(h47, l47, 0x05010400u);
  r.w = __builtin_amdgcn_perm(h47, l47, 0x07030602u);
  return r;
}

// Permute eight BF16 values (natural order, two per dword) into the
// [e0 e2 e4 e6 e1 e3 e5 e7] order of nf4_dequant8_perm.
__device__ __forceinline__ u32x4 perm8_bf16(u32x4 v) {
  u32x4 r;
  r.x = __builtin_amdgcn_perm(v.y, v.x, 0x05040100u);  // e0 (x lo), e2 (y lo)
  r.y = __builtin_amdgcn_perm(v.w, v.z, 0x05040100u);  // e4, e6
  r.z = __builtin_amdgcn_perm(v.y, v.x, 0x07060302u);  // e1, e3
  r.w = __builtin_amdgcn_perm(v.w, v.z, 0x07060302u);  // e5, e7
  return r;
}

// --------------------------------------------------------------- MFMA
// v_mfma_f32_16x16x32_bf16: D[16x16] += A[16x32] B[32x16].  Lane l holds row
// (A) / column (B) l%16 and the eight contraction indices of group l/16; the
// accumulator lane l holds D[4*(l/16) + v][l%16], v = 0..3.
__device__ __forceinline__ f32x4 mfma16(u32x4 a, u32x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                 __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

typedef float f32x16 __attribute__((ext_vector_type(16)));

// v_mfma_f32_32x32x16_bf16: D[32x32] += A[32x16] B[16x32].  Lane l holds row
// (A) / column (B) l%32 and the eight contraction indices of group l/32; the
// accumulator element v of lane l holds D[8*(v/4) + 4*(l/32) + v%4][l%32].
__device__ __forceinline__ f32x16 mfma32(u32x4 a, u32x4 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                 __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

// FP32 value -> (hi, lo) BF16 pair with hi + lo = v to about 16 bits.
__device__ __forceinline__ void split_bf16(float v, float& hi, float& lo) {
  f32x2 p = {v, 0.0f};
  uint32_t h = __builtin_bit_cast(uint32_t, __builtin_convertvector(p, bf16x2)) & 0xFFFFu;
  hi = __uint_as_float(h << 16);
  lo = __fsub_rn(v, hi);
}

}  // namespace qlora
