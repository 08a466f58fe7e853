// Device side of the matmul output epilogue (struct Epi in launch.h): fp32
// accumulator + bias in the output dtype, rounded once to fp32 / fp16 / bf16 (round
// to nearest even), stored into the output segment that holds the column.  Sources:
// "[Kernel] Adding bias epilogue support for cutlass_scaled_mm" (vLLM #5560: the bias
// takes the output dtype); "Add fused QKV HQQ triton_mm test" (pytorch/ao #306: one
// fused Q/K/V product, here written to separate Q, K and V outputs).
#pragma once

#include "common.h"
#include "launch.h"

namespace w4 {

// Column c's store target: the segment base at row 0, its row stride and the bias.
struct EpiCol {
  char* p;
  int64_t ld;
  float b;
};

__device__ __forceinline__ EpiCol epi_col(const Epi& e, int64_t c) {
  int s = 0;
#pragma unroll
  for (int i = 1; i < kMaxSegs; ++i) s += c >= e.c0[i] ? 1 : 0;
  const int esz = e.dt == W4_DT_F32 ? 4 : 2;
  EpiCol r;
  r.p = static_cast<char*>(e.y[s]) + (c - e.c0[s]) * esz;
  r.ld = e.ld[s] * esz;
  r.b = 0.0f;
  if (e.bias != nullptr) {
    if (e.dt == W4_DT_F32) r.b = static_cast<const float*>(e.bias)[c];
    else if (e.dt == W4_DT_BF16) r.b = bf16_bits_to_f32(static_cast<const uint16_t*>(e.bias)[c]);
    else r.b = f16_bits_to_f32(static_cast<const uint16_t*>(e.bias)[c]);
  }
  return r;
}

// Store acc (+ the column's bias) at row m of column `col`.
__device__ __forceinline__ void epi_put(const Epi& e, const EpiCol& col, int64_t m, float acc) {
  const float v = acc + col.b;
  char* q = col.p + m * col.ld;
  if (e.dt == W4_DT_F32) *reinterpret_cast<float*>(q) = v;
  else if (e.dt == W4_DT_BF16) *reinterpret_cast<uint16_t*>(q) = (uint16_t)(pack_bf16x2(v, 0.0f) & 0xFFFFu);
  else *reinterpret_cast<uint16_t*>(q) = f32_to_f16_bits(v);
}

// Bytes per element when four consecutive columns of a plain one-segment output can go
// out as one store: 4 (fp32 rows 16-byte aligned: 16-byte stores), 2 (bf16 / fp16 rows
// 8-byte aligned: 8-byte stores), else 0 (per-element stores).  outc = output columns.
__device__ __forceinline__ int epi_wide(const Epi& e, int64_t outc) {
  if (e.nseg != 1 || (outc & 3) != 0 || (e.ld[0] & 3) != 0) return 0;
  const uintptr_t p = reinterpret_cast<uintptr_t>(e.y[0]);
  if (e.dt == W4_DT_F32) return (p & 15) == 0 ? 4 : 0;
  return (p & 7) == 0 ? 2 : 0;
}

// Columns c4 .. c4 + 3 of such an output: row 0, row stride (bytes) and the four biases
// (converted exactly to fp32 from the output dtype).
struct EpiQuad {
  char* y;
  int64_t ld;
  float b[4];
  int dt;
  bool ok;  // the four columns lie inside the output
};

__device__ __forceinline__ EpiQuad epi_quad(const Epi& e, int64_t c4, int64_t outc) {
  EpiQuad q;
  const int esz = e.dt == W4_DT_F32 ? 4 : 2;
  q.ok = c4 < outc;
  q.dt = e.dt;
  q.y = static_cast<char*>(e.y[0]) + c4 * esz;
  q.ld = e.ld[0] * esz;
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    float b = 0.0f;
    if (e.bias != nullptr && q.ok) {
      if (e.dt == W4_DT_F32) b = static_cast<const float*>(e.bias)[c4 + u];
      else if (e.dt == W4_DT_BF16) b = bf16_bits_to_f32(static_cast<const uint16_t*>(e.bias)[c4 + u]);
      else b = f16_bits_to_f32(static_cast<const uint16_t*>(e.bias)[c4 + u]);
    }
    q.b[u] = b;
  }
  return q;
}

// Four consecutive columns of one row (+ their biases) -> one store: 16 bytes of fp32, or
// 8 bytes of bf16 / fp16 pairs each rounded to nearest even (the values epi_put stores,
// bit for bit).  Non-temporal: the output is not read again by the kernel.
__device__ __forceinline__ void epi_store4(const EpiQuad& q, int64_t m, const float (&v)[4]) {
  typedef float f32x4v __attribute__((ext_vector_type(4)));
  char* p = q.y + m * q.ld;
  if (q.dt == W4_DT_F32) {
    const f32x4v o = {v[0] + q.b[0], v[1] + q.b[1], v[2] + q.b[2], v[3] + q.b[3]};
    __builtin_nontemporal_store(o, reinterpret_cast<f32x4v*>(p));
  } else if (q.dt == W4_DT_BF16) {
    const u32x2 o = {pack_bf16x2(v[0] + q.b[0], v[1] + q.b[1]), pack_bf16x2(v[2] + q.b[2], v[3] + q.b[3])};
    __builtin_nontemporal_store(o, reinterpret_cast<u32x2*>(p));
  } else {
    const u32x2 o = {pack_f16x2(v[0] + q.b[0], v[1] + q.b[1]), pack_f16x2(v[2] + q.b[2], v[3] + q.b[3])};
    __builtin_nontemporal_store(o, reinterpret_cast<u32x2*>(p));
  }
}

// One 32x32 result block of v_mfma_f32_32x32x16 (register r of lane l: row row0 +
// 8 (r / 4) + 4 (l / 32) + (r % 4), column l % 32 of the block) + bias, stored four
// columns at a time.  A 4x4 transpose within each lane quad (two DPP quad-permute
// exchanges) leaves lane (k, s) of a half-wave with row s of every 4-row group for the
// quad's columns 4k .. 4k + 3, the columns of q.  Every lane of the wave must call it
// (DPP); rows past M are skipped.  row0 includes the 4 (l / 32) term.
__device__ __forceinline__ void epi_put_block_wide(const EpiQuad& q, const f32x16& acc, int64_t row0, int64_t M,
                                                   int lane) {
  const int s = lane & 3;
#pragma unroll
  for (int g = 0; g < 4; ++g) {
    float v[4], p[4];
#pragma unroll
    for (int t = 0; t < 4; ++t) v[t] = acc[g * 4 + t];
    // rows of the lane pair (s, s ^ 2): keep the diagonal 2x2 blocks, swap the others
#pragma unroll
    for (int t = 0; t < 4; ++t)
      p[t] = __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v[t ^ 2]), 0x4E, 0xF, 0xF, false));
#pragma unroll
    for (int t = 0; t < 4; ++t) v[t] = ((s & 2) == 0) == (t < 2) ? v[t] : p[t];
    // within the 2x2 blocks, lane pair (s, s ^ 1)
#pragma unroll
    for (int t = 0; t < 4; ++t)
      p[t] = __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v[t ^ 1]), 0xB1, 0xF, 0xF, false));
#pragma unroll
    for (int t = 0; t < 4; ++t) v[t] = (s & 1) == (t & 1) ? v[t] : p[t];
    const int64_t m = row0 + g * 8 + s;
    if (q.ok && m < M) epi_store4(q, m, v);
  }
}

}  // namespace w4
