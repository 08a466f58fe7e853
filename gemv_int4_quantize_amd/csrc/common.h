// Device helpers shared by the gfx950 kernels of the W4A16 library.
//
// Packed layout: code k = 8c + j of a row sits in bits 4j..4j+3 of int32 word c.
// Weight operand of the matmul: bf16_rne((q - z) * s) (fp32 arithmetic), the
// dequantize-then-bf16-matmul reference path of "Re-write HQQ Fused Gemm
// Transpose" (pytorch/ao #185).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace w4 {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kWave = 64;

__device__ __forceinline__ float f16_bits_to_f32(uint32_t h) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)h);
}

__device__ __forceinline__ uint16_t f32_to_f16_bits(float x) {
  // fp32 -> fp16, round to nearest even (v_cvt_f16_f32 under the default round mode)
  return __builtin_bit_cast(uint16_t, (_Float16)x);
}

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t b) {
  return __uint_as_float(b << 16);
}

// Two fp32 values -> one dword holding bf16_rne(lo) | bf16_rne(hi) << 16.
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
  bf16x2 v = {(__bf16)lo, (__bf16)hi};
  return __builtin_bit_cast(uint32_t, v);
}

// fma(f16 operand taken from the low / high half of `h`, a, b) with one rounding.
// v_fma_mix_f32 converts the fp16 half exactly (fp16 denormals are kept), so a
// nibble masked into bits 0..3 (value q * 2^-24) or 4..7 (q * 2^-20) of a half
// becomes an exact fp32 operand with no separate conversion instruction.
__device__ __forceinline__ float fma_mix_lo(uint32_t h, float a, float b) {
  float d;
  asm("v_fma_mix_f32 %0, %1, %2, %3 op_sel_hi:[1,0,0]" : "=v"(d) : "v"(h), "v"(a), "v"(b));
  return d;
}
__device__ __forceinline__ float fma_mix_hi(uint32_t h, float a, float b) {
  float d;
  asm("v_fma_mix_f32 %0, %1, %2, %3 op_sel:[1,0,0] op_sel_hi:[1,0,0]" : "=v"(d) : "v"(h), "v"(a), "v"(b));
  return d;
}

// Per-group constants of the in-register dequantization:
//   s24 = s * 2^24, s20 = s * 2^20, nzs = -(z * s) (exact in fp32: 11-bit x 11-bit).
// Then fma(q * 2^-24, s24, nzs) = fp32((q - z) * s) whenever q - z is exact in fp32
// (always, except for a nonzero |z| < 2^-10, where it differs by at most one fp32
// ulp before the bf16 rounding).
struct DqConst {
  float s24, s20, nzs;
};

__device__ __forceinline__ DqConst dq_const(uint32_t s_bits, uint32_t z_bits) {
  const float s = f16_bits_to_f32(s_bits);
  const float z = f16_bits_to_f32(z_bits);
  DqConst c;
  c.s24 = s * 16777216.0f;
  c.s20 = s * 1048576.0f;
  c.nzs = -(z * s);
  return c;
}

// Dequantization constants from raw fp16 bits, three v_fma_mix_f32 (exact):
// s * 2^24, s * 2^20 and -(z * s).  The operands go in as fp16 values, whose upper
// register half the instruction ignores, so a 16-bit load feeds them with no masking.
__device__ __forceinline__ DqConst dq_const_mix(uint16_t s_bits, uint16_t z_bits) {
  const _Float16 s = __builtin_bit_cast(_Float16, s_bits), z = __builtin_bit_cast(_Float16, z_bits);
  DqConst c;
  asm("v_fma_mix_f32 %0, %1, %2, 0 op_sel_hi:[1,0,0]" : "=v"(c.s24) : "v"(s), "v"(16777216.0f));
  asm("v_fma_mix_f32 %0, %1, %2, 0 op_sel_hi:[1,0,0]" : "=v"(c.s20) : "v"(s), "v"(1048576.0f));
  asm("v_fma_mix_f32 %0, -%1, %2, 0 op_sel_hi:[1,1,0]" : "=v"(c.nzs) : "v"(z), "v"(s));
  return c;
}

// One iteration covers 2048 columns: 64 lanes x one 16-byte chunk (32 codes) per row.
constexpr int kIterCols = 2048;

// One packed word (8 codes along K) -> 4 dwords of bf16 pairs in K order:
// out[i] = (w[2i], w[2i+1]).  17 VALU instructions.
__device__ __forceinline__ void dq_word_bf16(uint32_t w, const DqConst& c, uint32_t out[4]) {
  const uint32_t a = w & 0x000F000Fu;  // q0 | q4
  const uint32_t b = w & 0x00F000F0u;  // q1 | q5  (x16)
  const uint32_t t = w >> 8;
  const uint32_t d = t & 0x000F000Fu;  // q2 | q6
  const uint32_t e = t & 0x00F000F0u;  // q3 | q7  (x16)
  const float v0 = fma_mix_lo(a, c.s24, c.nzs);
  const float v4 = fma_mix_hi(a, c.s24, c.nzs);
  const float v1 = fma_mix_lo(b, c.s20, c.nzs);
  const float v5 = fma_mix_hi(b, c.s20, c.nzs);
  const float v2 = fma_mix_lo(d, c.s24, c.nzs);
  const float v6 = fma_mix_hi(d, c.s24, c.nzs);
  const float v3 = fma_mix_lo(e, c.s20, c.nzs);
  const float v7 = fma_mix_hi(e, c.s20, c.nzs);
  out[0] = pack_bf16x2(v0, v1);
  out[1] = pack_bf16x2(v2, v3);
  out[2] = pack_bf16x2(v4, v5);
  out[3] = pack_bf16x2(v6, v7);
}

// The 8 dequantized fp32 values of one word (before bf16 rounding), K order.
__device__ __forceinline__ void dq_word_f32(uint32_t w, const DqConst& c, float v[8]) {
  const uint32_t a = w & 0x000F000Fu;
  const uint32_t b = w & 0x00F000F0u;
  const uint32_t t = w >> 8;
  const uint32_t d = t & 0x000F000Fu;
  const uint32_t e = t & 0x00F000F0u;
  v[0] = fma_mix_lo(a, c.s24, c.nzs);
  v[4] = fma_mix_hi(a, c.s24, c.nzs);
  v[1] = fma_mix_lo(b, c.s20, c.nzs);
  v[5] = fma_mix_hi(b, c.s20, c.nzs);
  v[2] = fma_mix_lo(d, c.s24, c.nzs);
  v[6] = fma_mix_hi(d, c.s24, c.nzs);
  v[3] = fma_mix_lo(e, c.s20, c.nzs);
  v[7] = fma_mix_hi(e, c.s20, c.nzs);
}

// Two fp32 values -> one dword holding fp16_rne(lo) | fp16_rne(hi) << 16 (v_cvt_pk_f16_f32:
// src0 to the low half, round to nearest even; checked on gfx950 against per-value
// conversion over ties, subnormals and overflow).
__device__ __forceinline__ uint32_t pack_f16x2(float lo, float hi) {
  uint32_t d;
  asm("v_cvt_pk_f16_f32 %0, %1, %2" : "=v"(d) : "v"(lo), "v"(hi));
  return d;
}

// One packed word -> 4 dwords of fp16 pairs in K order, each fp16_rne(fp32((q - z) * s)):
// the fp32 values of dq_word_bf16, rounded to fp16.  17 VALU instructions.
__device__ __forceinline__ void dq_word_f16(uint32_t w, const DqConst& c, uint32_t out[4]) {
  float v[8];
  dq_word_f32(w, c, v);
  out[0] = pack_f16x2(v[0], v[1]);
  out[1] = pack_f16x2(v[2], v[3]);
  out[2] = pack_f16x2(v[4], v[5]);
  out[3] = pack_f16x2(v[6], v[7]);
}

// Weight operand of one packed word in the activation dtype (bf16 or fp16 pairs).
template <bool F16>
__device__ __forceinline__ void dq_word_op(uint32_t w, const DqConst& c, uint32_t out[4]) {
  if constexpr (F16) dq_word_f16(w, c, out);
  else dq_word_bf16(w, c, out);
}

// Two words of consecutive rows (contraction index) -> 8 operand pairs, pair j holding column
// j of both rows (the transposed operand layout).
template <bool F16>
__device__ __forceinline__ void dq_rows_op(uint32_t w0, const DqConst& c0, uint32_t w1, const DqConst& c1,
                                           uint32_t out[8]) {
  float v0[8], v1[8];
  dq_word_f32(w0, c0, v0);
  dq_word_f32(w1, c1, v1);
#pragma unroll
  for (int j = 0; j < 8; ++j) out[j] = F16 ? pack_f16x2(v0[j], v1[j]) : pack_bf16x2(v0[j], v1[j]);
}

// acc += a.lo * b.lo + a.hi * b.hi on fp16 pairs, fp32 accumulate (v_dot2_f32_f16).
__device__ __forceinline__ float dot2_f16(uint32_t a, uint32_t b, float acc) {
  typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
  return __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2, a), __builtin_bit_cast(f16x2, b), acc, false);
}

// acc += a.lo * b.lo + a.hi * b.hi on bf16 pairs, fp32 accumulate (v_dot2_f32_bf16).
__device__ __forceinline__ float dot2_bf16(uint32_t a, uint32_t b, float acc) {
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, a), __builtin_bit_cast(bf16x2, b), acc,
                                         false);
}

template <bool F16>
__device__ __forceinline__ float dot2_op(uint32_t a, uint32_t b, float acc) {
  if constexpr (F16) return dot2_f16(a, b, acc);
  else return dot2_bf16(a, b, acc);
}

typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));

// One 32x32x16 MFMA on operand bits (eight bf16 or fp16 values per lane), fp32 accumulate.
template <bool F16>
__device__ __forceinline__ f32x16 mfma_op(const u32x4& a, const u32x4& b, const f32x16& c) {
  if constexpr (F16)
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a), __builtin_bit_cast(f16x8, b), c, 0, 0,
                                                  0);
  else
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b), c, 0,
                                                   0, 0);
}

// Meta-data addressing: one (scale, zero) per row-group.
//   GLOBAL:    index 0
//   ROWWISE:   index n
//   GROUPWISE: index n * (K / g) + k / g
enum MetaKind { META_GLOBAL = 0, META_ROW = 1, META_GROUP = 2 };

}  // namespace w4
