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

}  // namespace w4
