// Quantize-and-pack and dequantize kernels for gfx950.
//
// Method: Objective 1 of "Quantized LLM Inference with Triton Kernels"
// (anaaaiva/llm-quantization): FP16 -> INT4 with one scale and zero per group
// (global, rowwise or groupwise along K), packed 8 codes per INT32 word.
// Per group:  s = fp16_rne((max - min) / 15)  (1 if that is 0 or not finite),
//             z = fp16_rne((0 - min) / s),
//             q = clamp(rint(w / s + z), 0, 15),
// every step in IEEE fp32 (correctly rounded division, no contraction).
// Integer zero points, in the AWQ style of the W4A16 AWQ g = 128 workload of "Modify
// small-batched weight only quantization" (TensorRT-LLM #2213):
//             z = clamp(rint((0 - min) / s), 0, 15)  (an integer, exact in fp16),
//             q = clamp(rint(w / s) + z, 0, 15),
// so that q - z is an integer and the dequantized weight is exactly (q - z) * s.
//
// The kernels are HBM streams: each lane reads the 8 elements of one output word
// with 16-byte loads (32 for fp32) and writes one int32 word.
#include "common.h"
#include "launch.h"

namespace w4 {

// 8 consecutive elements of W starting at element `off`, widened to fp32 (exact).
template <int DT>
__device__ __forceinline__ void load8(const void* W, int64_t off, float v[8]) {
  if constexpr (DT == W4_DT_F32) {
    const f32x4* p = reinterpret_cast<const f32x4*>(static_cast<const float*>(W) + off);
    const f32x4 a = p[0];
    const f32x4 b = p[1];
    v[0] = a[0]; v[1] = a[1]; v[2] = a[2]; v[3] = a[3];
    v[4] = b[0]; v[5] = b[1]; v[6] = b[2]; v[7] = b[3];
  } else {
    const u32x4 u = *reinterpret_cast<const u32x4*>(static_cast<const uint16_t*>(W) + off);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      if constexpr (DT == W4_DT_F16) {
        v[2 * i] = f16_bits_to_f32(u[i] & 0xFFFFu);
        v[2 * i + 1] = f16_bits_to_f32(u[i] >> 16);
      } else {
        v[2 * i] = __uint_as_float(u[i] << 16);
        v[2 * i + 1] = __uint_as_float(u[i] & 0xFFFF0000u);
      }
    }
  }
}

struct QParams {
  float s, z;        // fp32 values of the fp16 scale and zero
  uint16_t sb, zb;   // their fp16 bits
};

__device__ __forceinline__ QParams qparams(float lo, float hi, bool intz) {
  const float s32 = (hi - lo) / 15.0f;
  uint16_t sb = f32_to_f16_bits(s32);
  float s = f16_bits_to_f32(sb);
  if (!(s != 0.0f) || !__builtin_isfinite(s)) {
    sb = 0x3C00;  // 1.0
    s = 1.0f;
  }
  // IEEE 0 - lo is +0 when lo is +0 or -0 and -lo otherwise.  Written as a select: the
  // backend turns `0.0f - lo` into a negate modifier, which yields -0 for lo == +0.
  const float nlo = lo == 0.0f ? 0.0f : -lo;
  const float z32 = nlo / s;
  uint16_t zb = intz ? f32_to_f16_bits(__builtin_fminf(__builtin_fmaxf(__builtin_rintf(z32), 0.0f), 15.0f))
                     : f32_to_f16_bits(z32);
  if (!intz && (zb & 0x7FFFu) == 0x7C00u) {
    // The zero point overflowed fp16: the group's range is below 15 |min| / 65504, tiny next
    // to its offset (reachable with fp32 weights only).  It is quantized as a constant
    // group: s = 1, z = fp16(0 - min).
    sb = 0x3C00;
    s = 1.0f;
    zb = f32_to_f16_bits(nlo);
  }
  QParams p;
  p.s = s;
  p.z = f16_bits_to_f32(zb);
  p.sb = sb;
  p.zb = zb;
  return p;
}

__device__ __forceinline__ uint32_t code4(float w, const QParams& p, bool intz) {
  // fp16 zero: rint(w / s + z); integer zero: rint(w / s) + z (the add is then exact)
  const float r = intz ? __builtin_rintf(w / p.s) + p.z : __builtin_rintf(w / p.s + p.z);  // half to even
  return (uint32_t)__builtin_fminf(__builtin_fmaxf(r, 0.0f), 15.0f);
}

// The 8 codes of one word, bit-identical to code4 but mostly without the division.
// Fast path: t = fma(w, rcp(s), z) (z = 0 for integer zeros, where the boundaries are those
// of rint(w / s)).  With rcp within 2^-22 relative of 1 / s (v_rcp_f32 is 1 ulp), t differs
// from the exact sequence RN(RN(w / s) + z) by at most |w / s| 2^-21.7 plus one ulp of t,
// which is below d = (|t| + 2 |z| + 17) 2^-20 (|w / s| <= |t| + |z| + tiny).  Rounding and
// clamping are monotone, so the codes can differ only if t lies within d of a half-integer;
// a lane holding such a value takes its 8 codes from code4 (the correctly rounded division).
// Then the codes, exact integers in [0, 15], go into bytes (v_cvt_pk_u8_f32): even codes in
// one word, odd codes in another, merged with one shift-or.
__device__ __forceinline__ uint32_t pack8(const float v[8], const QParams& p, bool intz) {
  const float y = __builtin_amdgcn_rcpf(p.s);
  const float zf = intz ? 0.0f : p.z;
  const float lim = 0.5f - (2.0f * __builtin_fabsf(zf) + 17.0f) * 0x1p-20f;
  float r[8];
  // the largest |t - rint(t)| + |t| 2^-20 of the word against lim: one max per value
  // instead of a compare and a flag merge (a NaN term, from an infinite t, is ignored by
  // the max as it fails the compare)
  float m = 0.0f;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const float t = __builtin_fmaf(v[j], y, zf);
    r[j] = __builtin_rintf(t);
    const float f = t - r[j];
    m = __builtin_fmaxf(m, __builtin_fmaf(__builtin_fabsf(t), 0x1p-20f, __builtin_fabsf(f)));
  }
  if (m >= lim) {
    uint32_t w = 0;
#pragma unroll
    for (int j = 0; j < 8; ++j) w |= code4(v[j], p, intz) << (4 * j);
    return w;
  }
  uint32_t even = 0, odd = 0;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const float c = __builtin_fminf(__builtin_fmaxf(intz ? r[j] + p.z : r[j], 0.0f), 15.0f);
    if (j & 1) odd = __builtin_amdgcn_cvt_pk_u8_f32(c, j >> 1, odd);
    else even = __builtin_amdgcn_cvt_pk_u8_f32(c, j >> 1, even);
  }
  return even | (odd << 4);
}

// Groups of T * WPL words (T lanes, T | 64, WPL consecutive words per lane: 2, or 4 / 8
// for groups of 256 / 512 words, which a wave then holds in registers).  Two words per lane
// halve the per-element share of the reduction and of the scale / zero arithmetic, and at
// g = 16 a lane holds a whole group.  Groups tile the rows exactly, so group index =
// global lane index / T.
// One word of W as loaded (8 elements: one 16-byte load, two for fp32), widened to fp32
// only when used, so the next word's load can be in flight meanwhile.
template <int DT>
struct RawWord {
  u32x4 a, b;
};
template <int DT>
__device__ __forceinline__ void load_raw(const void* W, int64_t off, RawWord<DT>& r) {
  if constexpr (DT == W4_DT_F32) {
    const u32x4* p = reinterpret_cast<const u32x4*>(static_cast<const float*>(W) + off);
    r.a = p[0];
    r.b = p[1];
  } else {
    r.a = *reinterpret_cast<const u32x4*>(static_cast<const uint16_t*>(W) + off);
  }
}
template <int DT>
__device__ __forceinline__ void widen(const RawWord<DT>& r, float v[8]) {
  if constexpr (DT == W4_DT_F32) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      v[i] = __uint_as_float(r.a[i]);
      v[4 + i] = __uint_as_float(r.b[i]);
    }
  } else {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      if constexpr (DT == W4_DT_F16) {
        v[2 * i] = f16_bits_to_f32(r.a[i] & 0xFFFFu);
        v[2 * i + 1] = f16_bits_to_f32(r.a[i] >> 16);
      } else {
        v[2 * i] = __uint_as_float(r.a[i] << 16);
        v[2 * i + 1] = __uint_as_float(r.a[i] & 0xFFFF0000u);
      }
    }
  }
}

template <int DT, int T, int WPL>
__global__ __launch_bounds__(256) void quant_small_kernel(const void* __restrict__ W, int32_t* __restrict__ packed,
                                                          uint16_t* __restrict__ scales,
                                                          uint16_t* __restrict__ zeros, int64_t total_lanes,
                                                          int intz) {
  // grid-stride over blocks of 256 lanes, the next block's words loaded while this one is
  // quantized; a lane past the end holds zeros (a group's lanes are all in or all out)
  const int64_t stride = (int64_t)gridDim.x * 256;
  auto fetch = [&](int64_t base, RawWord<DT> (&r)[WPL]) {
    const int64_t gl = base + threadIdx.x;
#pragma unroll
    for (int u = 0; u < WPL; ++u) {
      if (gl < total_lanes) {
        load_raw<DT>(W, (gl * WPL + u) * 8, r[u]);
      } else {
        r[u].a = u32x4{0u, 0u, 0u, 0u};
        r[u].b = u32x4{0u, 0u, 0u, 0u};
      }
    }
  };
  RawWord<DT> cur[WPL], nxt[WPL];
  int64_t base = (int64_t)blockIdx.x * 256;
  fetch(base, cur);
  for (; base < total_lanes; base += stride) {
    fetch(base + stride, nxt);
    const int64_t gl = base + threadIdx.x;
    const bool valid = gl < total_lanes;
    float v[WPL][8];
#pragma unroll
    for (int u = 0; u < WPL; ++u) widen<DT>(cur[u], v[u]);
    float lo = v[0][0], hi = v[0][0];
#pragma unroll
    for (int u = 0; u < WPL; ++u)
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        lo = __builtin_fminf(lo, v[u][j]);
        hi = __builtin_fmaxf(hi, v[u][j]);
      }
#pragma unroll
    for (int o = T / 2; o >= 1; o >>= 1) {
      lo = __builtin_fminf(lo, __shfl_xor(lo, o));
      hi = __builtin_fmaxf(hi, __shfl_xor(hi, o));
    }
    const QParams p = qparams(lo, hi, intz != 0);
    uint32_t word[WPL];
#pragma unroll
    for (int u = 0; u < WPL; ++u) word[u] = pack8(v[u], p, intz != 0);
    if (valid) {
      if constexpr (WPL == 2) {
        reinterpret_cast<u32x2*>(packed)[gl] = u32x2{word[0], word[1]};
      } else {
#pragma unroll
        for (int u = 0; u < WPL; u += 4)
          reinterpret_cast<u32x4*>(packed)[gl * (WPL / 4) + u / 4] = u32x4{word[u], word[u + 1], word[u + 2], word[u + 3]};
      }
      if ((threadIdx.x & (T - 1)) == 0) {
        scales[gl / T] = p.sb;
        zeros[gl / T] = p.zb;
      }
    }
#pragma unroll
    for (int u = 0; u < WPL; ++u) cur[u] = nxt[u];
  }
}

// One wave per group of `wpg` words (large groups, ROWWISE with long rows):
// pass 1 reduces min / max, pass 2 re-reads the group (an L2 hit) and packs.
template <int DT>
__global__ __launch_bounds__(256) void quant_large_kernel(const void* __restrict__ W, int32_t* __restrict__ packed,
                                                          uint16_t* __restrict__ scales,
                                                          uint16_t* __restrict__ zeros, int64_t num_groups,
                                                          int wpg, int intz) {
  const int lane = threadIdx.x & 63;
  const int64_t grp = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (grp >= num_groups) return;
  const int64_t w0 = grp * wpg;
  float lo = __builtin_inff(), hi = -__builtin_inff();
  for (int c = lane; c < wpg; c += kWave) {
    float v[8];
    load8<DT>(W, (w0 + c) * 8, v);
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      lo = __builtin_fminf(lo, v[j]);
      hi = __builtin_fmaxf(hi, v[j]);
    }
  }
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) {
    lo = __builtin_fminf(lo, __shfl_xor(lo, o));
    hi = __builtin_fmaxf(hi, __shfl_xor(hi, o));
  }
  const QParams p = qparams(lo, hi, intz != 0);
  for (int c = lane; c < wpg; c += kWave) {
    float v[8];
    load8<DT>(W, (w0 + c) * 8, v);
    packed[w0 + c] = (int32_t)pack8(v, p, intz != 0);
  }
  if (lane == 0) {
    scales[grp] = p.sb;
    zeros[grp] = p.zb;
  }
}

constexpr int kMinMaxBlocks = 1024;

__device__ __forceinline__ void block_minmax(float& lo, float& hi) {
  __shared__ float red_lo[4], red_hi[4];
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) {
    lo = __builtin_fminf(lo, __shfl_xor(lo, o));
    hi = __builtin_fmaxf(hi, __shfl_xor(hi, o));
  }
  const int wid = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 0) {
    red_lo[wid] = lo;
    red_hi[wid] = hi;
  }
  __syncthreads();
  lo = __builtin_fminf(__builtin_fminf(red_lo[0], red_lo[1]), __builtin_fminf(red_lo[2], red_lo[3]));
  hi = __builtin_fmaxf(__builtin_fmaxf(red_hi[0], red_hi[1]), __builtin_fmaxf(red_hi[2], red_hi[3]));
}

// GLOBAL pass 1: per-block min / max over a grid-stride range of words.
template <int DT>
__global__ __launch_bounds__(256) void minmax_partial_kernel(const void* __restrict__ W, int64_t total_words,
                                                             float* __restrict__ partial) {
  float lo = __builtin_inff(), hi = -__builtin_inff();
  for (int64_t gw = (int64_t)blockIdx.x * 256 + threadIdx.x; gw < total_words; gw += (int64_t)gridDim.x * 256) {
    float v[8];
    load8<DT>(W, gw * 8, v);
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      lo = __builtin_fminf(lo, v[j]);
      hi = __builtin_fmaxf(hi, v[j]);
    }
  }
  block_minmax(lo, hi);
  if (threadIdx.x == 0) {
    partial[2 * blockIdx.x] = lo;
    partial[2 * blockIdx.x + 1] = hi;
  }
}

// GLOBAL pass 2: every block folds the partials (min / max are exact, so every
// block derives the same scale and zero), then packs a grid-stride range.
template <int DT>
__global__ __launch_bounds__(256) void quant_global_kernel(const void* __restrict__ W, int32_t* __restrict__ packed,
                                                           uint16_t* __restrict__ scales,
                                                           uint16_t* __restrict__ zeros, int64_t total_words,
                                                           const float* __restrict__ partial, int nparts, int intz) {
  float lo = __builtin_inff(), hi = -__builtin_inff();
  for (int i = threadIdx.x; i < nparts; i += 256) {
    lo = __builtin_fminf(lo, partial[2 * i]);
    hi = __builtin_fmaxf(hi, partial[2 * i + 1]);
  }
  block_minmax(lo, hi);
  const QParams p = qparams(lo, hi, intz != 0);
  for (int64_t gw = (int64_t)blockIdx.x * 256 + threadIdx.x; gw < total_words; gw += (int64_t)gridDim.x * 256) {
    float v[8];
    load8<DT>(W, gw * 8, v);
    packed[gw] = (int32_t)pack8(v, p, intz != 0);
  }
  if (blockIdx.x == 0 && threadIdx.x == 0) {
    scales[0] = p.sb;
    zeros[0] = p.zb;
  }
}

// Dequantize: bf16_rne(fp32(q - z) * s), fp16_rne(fp32(q - z) * s) or fp32(q - z) * s,
// the exact two-op sequence (subtract, then multiply, each rounded) of the reference
// definition.  OUT: W4_DT_BF16, W4_DT_F16 or W4_DT_F32.
template <int OUT>
__global__ __launch_bounds__(256) void dequant_kernel(const int32_t* __restrict__ packed,
                                                      const uint16_t* __restrict__ scales,
                                                      const uint16_t* __restrict__ zeros, void* __restrict__ out,
                                                      int64_t total_words, int64_t words_per_row, int meta_kind,
                                                      int64_t groups_per_row, int words_per_group) {
  const int64_t gw = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (gw >= total_words) return;
  int64_t mi = 0;
  if (meta_kind != META_GLOBAL) {
    const int64_t n = gw / words_per_row;
    mi = meta_kind == META_ROW ? n : n * groups_per_row + (gw - n * words_per_row) / words_per_group;
  }
  const float s = f16_bits_to_f32(scales[mi]);
  const float z = f16_bits_to_f32(zeros[mi]);
  const uint32_t w = (uint32_t)packed[gw];
  float v[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const float qf = (float)((w >> (4 * j)) & 0xFu);
    const float d = qf - z;
    v[j] = d * s;
  }
  if constexpr (OUT == W4_DT_BF16) {
    u32x4 o;
#pragma unroll
    for (int i = 0; i < 4; ++i) o[i] = pack_bf16x2(v[2 * i], v[2 * i + 1]);
    __builtin_nontemporal_store(o, reinterpret_cast<u32x4*>(out) + gw);
  } else if constexpr (OUT == W4_DT_F16) {
    u32x4 o;
#pragma unroll
    for (int i = 0; i < 4; ++i)
      o[i] = (uint32_t)f32_to_f16_bits(v[2 * i]) | ((uint32_t)f32_to_f16_bits(v[2 * i + 1]) << 16);
    __builtin_nontemporal_store(o, reinterpret_cast<u32x4*>(out) + gw);
  } else {
    f32x4 a = {v[0], v[1], v[2], v[3]}, b = {v[4], v[5], v[6], v[7]};
    f32x4* p = reinterpret_cast<f32x4*>(out) + 2 * gw;
    __builtin_nontemporal_store(a, p);
    __builtin_nontemporal_store(b, p + 1);
  }
}

// ---------------------------------------------------------------- launchers

constexpr int64_t kQuantBlocks = 8192;  // grid of the grid-stride quantize kernel (measured: 2048 < 4096 < 8192 ~ 16384)

template <int DT, int WPL>
static hipError_t quant_small_dispatch(int T, const void* W, int32_t* packed, uint16_t* scales, uint16_t* zeros,
                                       int64_t total_words, int intz, hipStream_t st) {
  const int64_t lanes = total_words / WPL;
  const int64_t want = (lanes + 255) / 256;
  const dim3 grid((unsigned)(want < kQuantBlocks ? want : kQuantBlocks)), block(256);
  if constexpr (WPL > 2) {
    if (T != 64) return hipErrorInvalidValue;
    quant_small_kernel<DT, 64, WPL><<<grid, block, 0, st>>>(W, packed, scales, zeros, lanes, intz);
    return hipGetLastError();
  }
  switch (T) {
    case 1: quant_small_kernel<DT, 1, WPL><<<grid, block, 0, st>>>(W, packed, scales, zeros, lanes, intz); break;
    case 2: quant_small_kernel<DT, 2, WPL><<<grid, block, 0, st>>>(W, packed, scales, zeros, lanes, intz); break;
    case 4: quant_small_kernel<DT, 4, WPL><<<grid, block, 0, st>>>(W, packed, scales, zeros, lanes, intz); break;
    case 8: quant_small_kernel<DT, 8, WPL><<<grid, block, 0, st>>>(W, packed, scales, zeros, lanes, intz); break;
    case 16: quant_small_kernel<DT, 16, WPL><<<grid, block, 0, st>>>(W, packed, scales, zeros, lanes, intz); break;
    case 32: quant_small_kernel<DT, 32, WPL><<<grid, block, 0, st>>>(W, packed, scales, zeros, lanes, intz); break;
    case 64: quant_small_kernel<DT, 64, WPL><<<grid, block, 0, st>>>(W, packed, scales, zeros, lanes, intz); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

template <int DT>
static hipError_t quantize_dt(const void* W, int64_t N, int64_t K, int mode, int g, int intz, int32_t* packed,
                              uint16_t* scales, uint16_t* zeros, void* ws, hipStream_t st) {
  const int64_t total_words = N * (K / 8);
  if (mode == W4_MODE_GLOBAL) {
    float* partial = static_cast<float*>(ws);
    const int64_t want = (total_words + 255) / 256;
    const int nb = (int)(want < kMinMaxBlocks ? want : kMinMaxBlocks);
    minmax_partial_kernel<DT><<<nb, 256, 0, st>>>(W, total_words, partial);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const int64_t qb = (total_words + 255) / 256;
    const int qgrid = (int)(qb < 8192 ? qb : 8192);
    quant_global_kernel<DT><<<qgrid, 256, 0, st>>>(W, packed, scales, zeros, total_words, partial, nb, intz);
    return hipGetLastError();
  }
  const int64_t gsize = mode == W4_MODE_ROWWISE ? K : g;
  const int64_t wpg = gsize / 8;
  // power-of-two groups of up to 512 words: one pass with the group in registers
  if (wpg <= 128 && (wpg & (wpg - 1)) == 0 && wpg >= 2)
    return quant_small_dispatch<DT, 2>((int)(wpg / 2), W, packed, scales, zeros, total_words, intz, st);
  if (wpg == 256) return quant_small_dispatch<DT, 4>(64, W, packed, scales, zeros, total_words, intz, st);
  if (wpg == 512) return quant_small_dispatch<DT, 8>(64, W, packed, scales, zeros, total_words, intz, st);
  const int64_t ngroups = total_words / wpg;
  quant_large_kernel<DT><<<(unsigned)((ngroups + 3) / 4), 256, 0, st>>>(W, packed, scales, zeros, ngroups, (int)wpg,
                                                                         intz);
  return hipGetLastError();
}

hipError_t launch_quantize(const void* W, int dt, int64_t N, int64_t K, int mode, int g, int intz, int32_t* packed,
                           uint16_t* scales, uint16_t* zeros, void* ws, hipStream_t st) {
  switch (dt) {
    case W4_DT_F32: return quantize_dt<W4_DT_F32>(W, N, K, mode, g, intz, packed, scales, zeros, ws, st);
    case W4_DT_F16: return quantize_dt<W4_DT_F16>(W, N, K, mode, g, intz, packed, scales, zeros, ws, st);
    case W4_DT_BF16: return quantize_dt<W4_DT_BF16>(W, N, K, mode, g, intz, packed, scales, zeros, ws, st);
  }
  return hipErrorInvalidValue;
}

size_t quantize_workspace_bytes(int mode) { return mode == W4_MODE_GLOBAL ? 2 * sizeof(float) * kMinMaxBlocks : 0; }

hipError_t launch_dequantize(const int32_t* packed, const uint16_t* scales, const uint16_t* zeros, int64_t N,
                             int64_t K, int mode, int g, void* out, int out_dt, hipStream_t st) {
  const int64_t wpr = K / 8;
  const int64_t total_words = N * wpr;
  const int kind = mode == W4_MODE_GLOBAL ? META_GLOBAL : (mode == W4_MODE_ROWWISE ? META_ROW : META_GROUP);
  const int64_t gpr = mode == W4_MODE_GROUPWISE ? K / g : 1;
  const int wpgrp = mode == W4_MODE_GROUPWISE ? g / 8 : (int)wpr;
  const dim3 grid((unsigned)((total_words + 255) / 256)), block(256);
  if (out_dt == W4_DT_BF16)
    dequant_kernel<W4_DT_BF16><<<grid, block, 0, st>>>(packed, scales, zeros, out, total_words, wpr, kind, gpr, wpgrp);
  else if (out_dt == W4_DT_F16)
    dequant_kernel<W4_DT_F16><<<grid, block, 0, st>>>(packed, scales, zeros, out, total_words, wpr, kind, gpr, wpgrp);
  else
    dequant_kernel<W4_DT_F32><<<grid, block, 0, st>>>(packed, scales, zeros, out, total_words, wpr, kind, gpr, wpgrp);
  return hipGetLastError();
}

}  // namespace w4
