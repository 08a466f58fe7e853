// Mid-M forward matmul, 5 <= M <= 32:  Y[m][n] = sum_k X[m][k] * w[n][k] (+ bias[n]),
// w = bf16_rne((q - z) * s) (fp16 activations: fp16_rne), fp32 accumulation.
// Sources: Objective 2 of "Quantized LLM Inference with Triton Kernels" (Y = X_bf16 @
// W_int4^T); "Modify small-batched weight only quantization" (TensorRT-LLM #2213) for the
// batched-decode regime these sizes belong to.
//
// At these M the weight stream is the cost (M * 2 flops per 0.53 weight bytes), as in the
// decode GEMV, but the GEMV's per-row products (4 M dot instructions per packed word) would
// make the vector ALU the limit.  Here the products go to the matrix core and the vector ALU
// only dequantizes (17 instructions per word, whatever M is):
//   * v_mfma_f32_16x16x32_bf16 with the activations as the A operand (rows m, one MFMA per
//     16 rows of X) and 16 weight rows as B: lane l holds, for column n = l % 16 and quarter
//     q = l / 16, one packed word -- eight consecutive contraction values -- per MFMA.  One
//     16-byte load per lane (4 words of one row) feeds 4 MFMAs; a wave-wide load is 16 rows x
//     64 contiguous bytes.  Within a 128-column unit the contraction order is permuted (MFMA
//     j, quarter q <-> word 4 q + j), the same way on both operands;
//   * persistent row blocks of 16 waves, about one per CU, each block covering `rpb` rows
//     and one contiguous range of 128-column units (the whole row, or one of S splits);
//     wave w owns UP (1 or 2) consecutive units of that range and walks every 16-row group
//     of the block over them: its activation fragments (UP x 4 x MB 16-byte values per
//     lane) are loaded once, straight into registers, so nothing is staged in LDS and no
//     barrier is taken until the end;
//   * weights, scales and zeros through buffer loads: the 16 rows of a group are one scalar
//     resource, the per-lane offsets are fixed, rows past the end and units past the range
//     read zeros without a request; a two-slot register pipeline over the wave's (group,
//     unit) steps keeps the next step's loads in flight;
//   * each group's 16 x 16 (x MB) partial sum goes to LDS, one slot per wave; at the end the
//     block sums the waves' slots in wave order (deterministic) and stores through the
//     output epilogue, or, with S splits, into fp32 partial planes that the split-K
//     reduction finishes in split order.
#include <algorithm>
#include <atomic>
#include <type_traits>

#include "common.h"
#include "epilogue.h"
#include "launch.h"

namespace w4 {

namespace {

typedef __amdgpu_buffer_rsrc_t rsrc_t;
constexpr int kRsrcDword3 = 0x00020000;  // raw buffer, 32-bit data format (gfx9 class)

__device__ __forceinline__ rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, (int)bytes, kRsrcDword3);
}

constexpr int kWaves = 16;
constexpr int kUnitCols = 128;   // contraction columns per step (4 quarters x 4 words x 8)
// units per wave (activation fragments held in registers): 4 for one 16-row block of X, 2 for two
#ifndef W4_SKINNY_MAX_UNITS1
#define W4_SKINNY_MAX_UNITS1 4
#endif
constexpr int kMaxUnits1 = W4_SKINNY_MAX_UNITS1, kMaxUnits2 = 2;
constexpr uint32_t kOob = 0x80000000u;  // a buffer offset past every resource: reads zero
#ifndef W4_SKINNY_SLOTS
#define W4_SKINNY_SLOTS 4
#endif
constexpr int kSlots = W4_SKINNY_SLOTS;  // weight-load slots per wave
constexpr int kXScratch = 16 * 17 * 16;  // bytes of one wave's activation scratch

// One 16x16x32 MFMA on operand bits (eight bf16 or fp16 values per lane).
template <bool F16>
__device__ __forceinline__ f32x4 mfma16(const u32x4& a, const u32x4& b, const f32x4& c) {
  if constexpr (F16)
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, a), __builtin_bit_cast(f16x8, b), c, 0, 0,
                                                  0);
  else
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b), c, 0,
                                                   0, 0);
}

// Output argument: the general epilogue, or the fp32 bias and Y [M][N] (a smaller argument
// block for the common case).
struct PlainOut {
  const float* bias;
  float* Y;
};
template <bool GEN>
struct OutArg {
  typedef PlainOut type;
};
template <>
struct OutArg<true> {
  typedef Epi type;
};

// Per-lane state of one step: 4 packed words of one row and the (scale | zero << 16) fp16
// pair of the group(s) they belong to (GPC = 2 when g = 16).
template <int GPC>
struct Slot {
  u32x4 w;
  uint32_t sz[GPC];
};

// Dequantization constants from an LDS pair (fp16 scale in the low half, zero in the high
// half), three v_fma_mix_f32 (exact): s * 2^24, s * 2^20 and -(z * s).
__device__ __forceinline__ DqConst dq_const_pair(uint32_t sz) {
  DqConst c;
  asm("v_fma_mix_f32 %0, %1, %2, 0 op_sel_hi:[1,0,0]" : "=v"(c.s24) : "v"(sz), "v"(16777216.0f));
  asm("v_fma_mix_f32 %0, %1, %2, 0 op_sel_hi:[1,0,0]" : "=v"(c.s20) : "v"(sz), "v"(1048576.0f));
  asm("v_fma_mix_f32 %0, -%1, %1, 0 op_sel:[1,0,0] op_sel_hi:[1,1,0]" : "=v"(c.nzs) : "v"(sz));
  return c;
}

// f(std::integral_constant<int, 0>{}), ..., f(std::integral_constant<int, N - 1>{}): a loop
// body whose index is a compile-time constant (register arrays stay registers).
template <typename F, int... I>
__device__ __forceinline__ void unroll_seq(F&& f, std::integer_sequence<int, I...>) {
  (f(std::integral_constant<int, I>{}), ...);
}
template <int N, typename F>
__device__ __forceinline__ void unroll(F&& f) {
  unroll_seq(f, std::make_integer_sequence<int, N>{});
}

// MB: 16-row blocks of X (M <= 16 MB).  UP: units per wave.  D: load slots (steps in flight).
// part != nullptr: write the block's sums to partial plane blockIdx.y ([M][N] fp32) instead of
// the output.  meta_row: (scale, zero) pairs per weight row (K / g, 1 rowwise, 0 global);
// log2g: group shift (31 for rowwise / global).  log2gr: the block's groups are reduced in
// rounds of 2^log2gr groups, through two LDS buffers of [kWaves][M][16 << log2gr] partial sums.
// The block's (scale, zero) pairs are staged once into LDS after those buffers, a row of
// pairs every `ms` words (0 for global: one pair).
template <int MB, int UP, int GPC, bool GEN, bool F16, int D>
__global__ __launch_bounds__(kWaves * 64) void skinny_kernel(const uint16_t* __restrict__ X,
                                                             const int32_t* __restrict__ packed,
                                                             const uint16_t* __restrict__ scales,
                                                             const uint16_t* __restrict__ zeros,
                                                             int N, int K, int meta_row, int rpb, int units_per_split,
                                                             int lg, float* __restrict__ part,
                                                             const typename OutArg<GEN>::type ep) {
  static_assert(D % UP == 0, "a slot's unit is a compile-time constant");
  // lg packs M (bits 0-7), log2g (8-12) and log2gr (16-17): the fourteen argument dwords up to
  // and including it are what the build preloads into SGPRs at dispatch, so no wave waits on
  // an argument load before its first loads; part and the output come last (used at the end)
  const int M = lg & 255, log2g = (lg >> 8) & 31, log2gr = lg >> 16;
  extern __shared__ float outs[];  // [2][kWaves][M][RS]
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int n = lane & 15, q = lane >> 4;
  const int r0 = blockIdx.x * rpb, r1 = min(r0 + rpb, N);
  const int rows = r1 - r0;
  const int G = (rows + 15) >> 4;     // 16-row groups of this block
  const int RS = 16 << log2gr;        // rows per round
  const int rounds = (G + (1 << log2gr) - 1) >> log2gr;
  const int KW = K >> 3;              // packed words per row
  const int U = (K + kUnitCols - 1) / kUnitCols;
  const int u_begin = blockIdx.y * units_per_split;
  const int u_end = min(u_begin + units_per_split, U);
  const int wu0 = u_begin + wave * UP;               // this wave's first unit
  const int nu = max(0, min(UP, u_end - wu0));       // how many of its UP units are real
  const int nwv = min(kWaves, (u_end - u_begin + UP - 1) / UP);  // waves that hold sums

  // activation fragments: lane (row n + 16 mb, quarter q), unit t, MFMA j holds
  // X[m][128 u + 32 q + 8 j .. + 8]; rows past M, columns past K and units past the range are
  // zero.  In that layout a lane quad spans 4 rows, so they are loaded with each quad on 64
  // contiguous bytes of one row (lane l: row l / 4, 16-byte chunk l % 4 + 4 i of the unit)
  // and put in place through the wave's LDS scratch below
  u32x4 xl[UP][MB][4];
  {
    const rsrc_t xr = make_rsrc(X, (uint32_t)((size_t)M * K * 2));
    const int lr = lane >> 2, lc = lane & 3;
#pragma unroll
    for (int t = 0; t < UP; ++t)
#pragma unroll
      for (int mb = 0; mb < MB; ++mb)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int m = lr + 16 * mb;
          const int col = (wu0 + t) * kUnitCols + (lc + 4 * i) * 8;
          const bool ok = t < nu && m < M && col < K;
          const uint32_t off = ok ? (uint32_t)(((size_t)m * K + col) * 2) : kOob;
          xl[t][mb][i] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(xr, off, 0, 0));
        }
  }

  // the block's (scale, zero) pairs -> LDS with coalesced loads (lanes along a row's groups),
  // so that a step reads its lane's pair from LDS instead of two 2-byte loads whose lanes
  // span 16 rows; pad pairs past a row's last group are zero (the columns past K of a ragged
  // last unit dequantize to 0 against zero activations)
  const int kend = min(u_end * kUnitCols, K);
  const int g0 = meta_row > 0 ? (u_begin * kUnitCols) >> log2g : 0;
  const int ng = meta_row > 0 ? ((kend - 1) >> log2g) - g0 + 1 : 1;
  const int ms = meta_row > 0 ? ((ng + 8) | 1) : 0;
  // LDS: [round buffers | per-wave activation scratch, overlapped] [pairs]
  const size_t moff = max((size_t)2 * kWaves * M * RS, (size_t)kWaves * kXScratch / 4);
  uint32_t* const mlds = reinterpret_cast<uint32_t*>(outs + moff);
  {
    const int mrows = meta_row > 0 ? rows : 1, mw = meta_row > 0 ? ms : 1;
    for (int i = tid; i < mrows * mw; i += kWaves * 64) {
      const int r = i / mw, j = i - r * mw;
      uint32_t v = 0u;
      if (j < ng) {
        const size_t gi = (size_t)(r0 + r) * meta_row + g0 + j;
        v = (uint32_t)scales[gi] | ((uint32_t)zeros[gi] << 16);
      }
      mlds[i] = v;
    }
  }

  // round r's sums: every thread adds the waves' partial sums in wave order and stores them
  auto reduce = [&](int r) {
    const float* buf = outs + (size_t)(r & 1) * kWaves * M * RS;
    const int lo = r * RS, nr = min(RS, rows - lo);
    for (int u = tid; u < nr * M; u += kWaves * 64) {
      const int m = u / nr, lr = u - m * nr;
      float sum = 0.0f;
      for (int w = 0; w < nwv; ++w) sum += buf[((size_t)w * M + m) * RS + lr];
      const int col = r0 + lo + lr;
      if (part != nullptr) {
        part[((size_t)blockIdx.y * M + m) * N + col] = sum;
      } else if constexpr (!GEN) {
        ep.Y[(size_t)m * N + col] = sum + (ep.bias != nullptr ? ep.bias[col] : 0.0f);
      } else {
        epi_put(ep, epi_col(ep, col), m, sum);
      }
    }
  };
  // end of round r: the partial sums written (LDS) before the barrier, which carries no wait
  // for the weight loads in flight; the other buffer is still being read by no one (every
  // thread reduced round r - 1 before it reached this barrier)
  auto round_end = [&](int r) {
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    reduce(r);
  };

  // activation fragments into the MFMA layout through this wave's scratch (16 rows x 16
  // chunks, rows 17 chunks apart so that both the row-wise stores and the column-wise reads
  // spread over the banks); the wave's own LDS accesses complete in order
  u32x4 xf[UP][4][MB];
  {
    u32x4* const xs = reinterpret_cast<u32x4*>(outs) + wave * (kXScratch / 16);
    const int lr = lane >> 2, lc = lane & 3;
#pragma unroll
    for (int t = 0; t < UP; ++t)
#pragma unroll
      for (int mb = 0; mb < MB; ++mb) {
#pragma unroll
        for (int i = 0; i < 4; ++i) xs[lr * 17 + lc + 4 * i] = xl[t][mb][i];
#pragma unroll
        for (int j = 0; j < 4; ++j) xf[t][j][mb] = xs[n * 17 + 4 * q + j];
      }
  }
  __syncthreads();  // the staged pairs; every wave done with its scratch (round buffers next)

  if (nu == 0) {
    // no contraction units for this wave: it takes part in the rounds' barriers and sums
    for (int r = 0; r < rounds; ++r) round_end(r);
    return;
  }

  // weight offsets: fixed per lane; the group base is the scalar resource and the unit a
  // scalar offset.  Pair of lane (row n, quarter q), unit t, chunk half c: word
  // (16 g + n) ms + ((128 u) >> log2g) - g0 + ((32 q + 16 c) >> log2g) of the staged pairs
  const uint32_t wvo = (uint32_t)n * KW * 4 + q * 16;
  const uint32_t* mlane[UP][GPC];
#pragma unroll
  for (int t = 0; t < UP; ++t)
#pragma unroll
    for (int c = 0; c < GPC; ++c)
      mlane[t][c] = mlds + n * ms + (((wu0 + t) * kUnitCols) >> log2g) - g0 + ((q * 32 + c * 16) >> log2g);

  // loads of step (group g, unit t); a group past the block or a unit past the range gets a
  // zero-sized resource and reads zeros without a request (its pairs: those of the last group)
  auto load = [&](int g, int t, Slot<GPC>& sl) {
    const int row0 = r0 + g * 16;
    const bool ok = g < G && t < nu;
    const int nrow = ok ? min(16, r1 - row0) : 0;
    const int rb = ok ? row0 : r0;
    const rsrc_t pr = make_rsrc(packed + (size_t)rb * KW, (uint32_t)nrow * KW * 4);
    const int u = wu0 + t;
    // non-temporal (cache-policy operand 2: nt): each weight byte is read once per launch
    sl.w = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(pr, wvo, u * 64, 2));
    const int gm = min(g, G - 1) * 16 * ms;
#pragma unroll
    for (int c = 0; c < GPC; ++c) sl.sz[c] = mlane[t][c][gm];
  };

  f32x4 acc[MB];
#pragma unroll
  for (int mb = 0; mb < MB; ++mb) acc[mb] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};

  // step of unit T of group g: dequantize the 4 words, 4 MB MFMAs; after the last unit the
  // group's sums go to this wave's LDS slot (D layout of the MFMA: lane l holds rows
  // 4 (l / 16) + r, r = 0..3, of column l % 16), and after the last group of a round the
  // round is reduced
  auto compute = [&](const Slot<GPC>& sl, auto tc, int g) {
    constexpr int T = decltype(tc)::value;
    DqConst dc[GPC];
#pragma unroll
    for (int c = 0; c < GPC; ++c) dc[c] = dq_const_pair(sl.sz[c]);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      uint32_t b[4];
      dq_word_op<F16>(sl.w[j], dc[GPC == 2 ? j / 2 : 0], b);
      const u32x4 bv = {b[0], b[1], b[2], b[3]};
#pragma unroll
      for (int mb = 0; mb < MB; ++mb) acc[mb] = mfma16<F16>(xf[T][j][mb], bv, acc[mb]);
    }
    if constexpr (T == UP - 1) {
      const int r = g >> log2gr;
      float* o = outs + ((size_t)(r & 1) * kWaves + wave) * M * RS + (g - (r << log2gr)) * 16 + n;
#pragma unroll
      for (int mb = 0; mb < MB; ++mb)
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) {
          const int m = 16 * mb + 4 * q + rr;
          if (m < M) o[(size_t)m * RS] = acc[mb][rr];
        }
#pragma unroll
      for (int mb = 0; mb < MB; ++mb) acc[mb] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
      if (g - (r << log2gr) == (1 << log2gr) - 1 || g == G - 1) round_end(r);
    }
  };

  // D slots over the wave's steps (step s = group s / UP, unit s % UP), D - 1 steps of loads
  // in flight: each step issues the loads of the step D - 1 ahead into the slot just read,
  // so every step issues one step of loads (exact waits).  Loads past the last step read
  // nothing.  The wave raises its priority while it issues loads.
  const int steps = G * UP;
  Slot<GPC> S[D];
  unroll<D - 1>([&](auto ic) {
    constexpr int i = decltype(ic)::value;
    load(i / UP, i % UP, S[i]);
  });
  int s = 0;
  for (; s + D <= steps; s += D) {
    unroll<D>([&](auto ic) {
      constexpr int i = decltype(ic)::value;
      constexpr int ahead = i + D - 1;
      __builtin_amdgcn_s_setprio(2);
      load((s + ahead) / UP, ahead % UP, S[ahead % D]);
      __builtin_amdgcn_s_setprio(0);
      compute(S[i], std::integral_constant<int, i % UP>{}, (s + i) / UP);
    });
  }
  unroll<D - 1>([&](auto ic) {
    constexpr int i = decltype(ic)::value;
    if (s + i < steps) compute(S[i], std::integral_constant<int, i % UP>{}, (s + i) / UP);
  });
}

template <int MB, int UP, int GPC, bool GEN, bool F16>
hipError_t run(const MmArgs& a, const SkinnyPlan& p, float* part, hipStream_t st) {
  auto k = skinny_kernel<MB, UP, GPC, GEN, F16, kSlots>;
  static std::atomic<int> lds_set{64 * 1024};  // largest dynamic LDS size enabled so far
  if ((int)p.lds > lds_set.load()) {
    const hipError_t e = hipFuncSetAttribute((const void*)k, hipFuncAttributeMaxDynamicSharedMemorySize, (int)p.lds);
    if (e != hipSuccess) return e;
    lds_set.store((int)p.lds);
  }
  const int log2g = a.mode == W4_MODE_GROUPWISE ? 31 - __builtin_clz((unsigned)a.group) : 31;
  const int meta_row = a.mode == W4_MODE_GLOBAL ? 0 : a.mode == W4_MODE_ROWWISE ? 1 : (int)(a.K / a.group);
  typename OutArg<GEN>::type out;
  if constexpr (GEN) out = a.ep;
  else out = PlainOut{static_cast<const float*>(a.ep.bias), static_cast<float*>(a.ep.y[0])};
  const dim3 grid((unsigned)p.blocks, (unsigned)p.splits);
  k<<<grid, kWaves * 64, p.lds, st>>>(a.A, a.packed, a.scales, a.zeros, (int)a.N, (int)a.K, meta_row, p.rpb,
                                      p.units_per_split, (int)a.M | (log2g << 8) | (p.log2gr << 16),
                                      p.splits > 1 ? part : nullptr, out);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || p.splits == 1) return e;
  return launch_splitk_reduce(part, p.splits, a.M, 0, a.N, a.ep, st);
}

template <int MB, int UP, bool F16>
hipError_t run_g(const MmArgs& a, const SkinnyPlan& p, float* part, hipStream_t st) {
  const bool g16 = a.mode == W4_MODE_GROUPWISE && a.group == 16;  // two groups per 32-code lane chunk
  const Epi& e = a.ep;
  const bool plain = p.splits > 1 || (e.nseg == 1 && e.dt == W4_DT_F32 && e.ld[0] == a.N);
  if (plain) return g16 ? run<MB, UP, 2, false, F16>(a, p, part, st) : run<MB, UP, 1, false, F16>(a, p, part, st);
  return g16 ? run<MB, UP, 2, true, F16>(a, p, part, st) : run<MB, UP, 1, true, F16>(a, p, part, st);
}

template <int MB, int UP>
hipError_t run_f(const MmArgs& a, const SkinnyPlan& p, float* part, hipStream_t st) {
  return a.a_f16 ? run_g<MB, UP, true>(a, p, part, st) : run_g<MB, UP, false>(a, p, part, st);
}

}  // namespace

bool skinny_supported(const MmArgs& a) {
  if (a.transposed || a.M < kSkinnyMinM || a.M > kSkinnyMaxM) return false;
  // 32-bit buffer offsets: all of X, and 16 weight rows
  return a.K <= ((int64_t)1 << 24) && a.N <= ((int64_t)1 << 30) && (int64_t)a.M * a.K * 2 < ((int64_t)1 << 31);
}

SkinnyPlan skinny_plan(const MmArgs& a, const DeviceCaps& caps, bool allow_split) {
  SkinnyPlan p;
  const int64_t U = (a.K + kUnitCols - 1) / kUnitCols;
  p.MB = a.M <= 16 ? 1 : 2;
  const int64_t per_split = (int64_t)kWaves * (p.MB == 1 ? kMaxUnits1 : kMaxUnits2);  // units a block covers at most
  int64_t S = allow_split ? (U + per_split - 1) / per_split : 1;
  if (S == 1 && U > per_split) return p;  // unsplit, the rows are too long for one block
  const int64_t ub = (U + S - 1) / S;
  S = (U + ub - 1) / ub;
  p.UP = ub <= kWaves ? 1 : ub <= 2 * kWaves ? 2 : 4;
  p.splits = (int)S;
  p.units_per_split = (int)ub;
  // rows per block: a multiple of 16 that spreads the rows over about one block per CU per
  // split; the partial sums are reduced in rounds of up to 8 groups, as many as two LDS
  // buffers of [kWaves][M][16 per group] fp32 hold
  const int64_t cus = caps.cus > 0 ? caps.cus : 256;
  const size_t lds_cap = caps.lds > 0 ? caps.lds : 160 * 1024;
  const int64_t target = std::max<int64_t>(1, cus / S);
  // LDS words of the staged (scale, zero) pairs (the kernel's row stride (ng + 8) | 1)
  const int log2g = a.mode == W4_MODE_GROUPWISE ? 31 - __builtin_clz((unsigned)a.group) : 31;
  int64_t ngmax = 1;
  if (a.mode != W4_MODE_GLOBAL && a.mode != W4_MODE_ROWWISE)
    ngmax = ((ub * kUnitCols) >> log2g) + 2;
  const int64_t ms = a.mode == W4_MODE_GLOBAL ? 1 : ((ngmax + 8) | 1);
  int64_t rpb = ((a.N + target - 1) / target + 15) / 16 * 16;
  auto meta_bytes = [&](int64_t r) { return (size_t)(a.mode == W4_MODE_GLOBAL ? 1 : r * ms) * 4; };
  auto outs_bytes = [&](int g) { return (size_t)2 * kWaves * a.M * (16 << g) * 4; };
  // fewer rows per block when the pairs do not fit beside the smallest round buffers
  auto front = [&](int g) { return std::max(outs_bytes(g), (size_t)kWaves * kXScratch); };
  while (rpb > 16 && meta_bytes(rpb) + front(0) > lds_cap) rpb -= 16;
  if (meta_bytes(rpb) + front(0) > lds_cap) return p;
  int log2gr = 3;
  while (log2gr > 0 && ((rpb / 16) <= (1 << (log2gr - 1)) || meta_bytes(rpb) + front(log2gr) > lds_cap))
    --log2gr;
  p.rpb = (int)rpb;
  p.blocks = (int)((a.N + rpb - 1) / rpb);
  p.log2gr = log2gr;
  p.lds = std::max(outs_bytes(log2gr), (size_t)kWaves * kXScratch) + meta_bytes(rpb);
  p.ok = true;
  return p;
}

size_t skinny_split_bytes(const MmArgs& a, const SkinnyPlan& p) {
  return p.ok && p.splits > 1 ? (size_t)p.splits * a.M * a.N * sizeof(float) : 0;
}

const char* skinny_name(const MmArgs& a, const SkinnyPlan& p) {
  static thread_local char buf[48];
  const char* base = p.MB == 1 ? "skinny_m16" : "skinny_m32";
  if (p.splits == 1) return base;
  snprintf(buf, sizeof(buf), "%s_splitk%d", base, p.splits);
  return buf;
}

hipError_t launch_skinny(const MmArgs& a, const SkinnyPlan& p, float* part, hipStream_t st) {
  if (p.MB == 1) {
    if (p.UP == 4) return run_f<1, 4>(a, p, part, st);
    return p.UP == 1 ? run_f<1, 1>(a, p, part, st) : run_f<1, 2>(a, p, part, st);
  }
  return p.UP == 1 ? run_f<2, 1>(a, p, part, st) : run_f<2, 2>(a, p, part, st);
}

}  // namespace w4
