// MFMA W4A16 GEMM for gfx950, both directions on one packed buffer:
//   non-transposed  Y[m][n]  = sum_k X[m][k]  * w[n][k] (+ bias[n])
//   transposed      dX[m][k] = sum_n dY[m][n] * w[n][k] (+ bias[k])
// with w = bf16_rne((q - z) * s), bf16 MFMA operands and fp32 accumulation.
// Sources: Objective 2 of "Quantized LLM Inference with Triton Kernels"
// (Y = X_bf16 @ W_int4^T); "Re-write HQQ Fused Gemm Transpose" (pytorch/ao #185:
// the transposed product reads the same packed weights, scales and zeros);
// "[Kernel] Adding bias epilogue support for cutlass_scaled_mm" (vLLM #5560).
//
// This file holds the LDS-staged kernel, used for the transposed product and, in the
// non-transposed direction, only for contractions too long for the register-operand
// kernel of gemm_nt.hip; the tile / split-K planner for both; and the split-K reduction.
//
// Structure (one workgroup = WM x WN waves, output tile BM x BN, contraction step BK):
//   * the activation tile (X or dY, contraction along its rows) goes global -> LDS;
//   * the packed weight tile is loaded to registers, dequantized in registers with
//     v_fma_mix_f32 + v_cvt_pk_bf16_f32, and written to LDS as a bf16 tile whose
//     rows are output columns and whose BK columns are the contraction, so each MFMA
//     operand is one 16-byte LDS read in both directions.  Non-transposed, a packed
//     word already runs along the contraction; transposed, each thread dequantizes a
//     column of rows of one word and writes it across the contraction axis, into a
//     tile whose 16-byte chunks are XOR-swizzled by row / 16 (conflict-free writes and
//     operand reads);
//   * two or three LDS stages: the global loads of step k+1 (k+2) are in flight during
//     the MFMAs of step k; one barrier per step.  The transposed tiles use the interleaved
//     form (STAGES = 4): two LDS stages, loads two steps ahead, and the dequantization and
//     LDS writes of step k+1 cut into slices issued between the MFMAs of step k (with one
//     wave per SIMD at the 256 x 256 tile, nothing else would overlap that work);
//   * LDS rows are padded by 16 bytes so the rows read by one MFMA operand load fall
//     in distinct banks;
//   * v_mfma_f32_32x32x16_bf16 (on gfx950 it sustains twice the rate of the
//     16x16x32 form): lane l holds row (l % 32), contraction slots 8 (l / 32) .. +7
//     of A, column (l % 32) and the same slots of B; result register r of a 32x32
//     block is row 8 (r / 4) + 4 (l / 32) + (r % 4) of column l % 32.
#include "common.h"
#include "epilogue.h"
#include "launch.h"

#include <algorithm>
#include <type_traits>
#include <cstdio>
#include <cstdlib>

namespace w4 {

typedef __amdgpu_buffer_rsrc_t rsrc_t;

// raw buffer resource (gfx9-class dword 3: 32-bit data format); loads past `bytes` read 0
__device__ __forceinline__ rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, (int)bytes, 0x00020000);
}

// LDS rows hold BK contraction values plus 8 bf16 of padding: a row stride of
// (BK + 8) * 2 bytes puts the 16-byte operand reads of consecutive rows in distinct banks.
template <int BK>
constexpr int lds_row() { return BK + 8; }

// MPT: scale / zero pairs a thread loads per stage in the non-transposed mode: 1 when
// one group covers all of its words (rowwise, global, or g >= its span), else one per word.
// STAGES: 2 (loads of step k+1 in flight during step k), 3 (loads of step k+2), or 4 (two LDS
// stages, loads of step k+2, stores of step k+1 interleaved with the MFMAs of step k).
// F16: fp16 activations and weight operand (v_mfma_f32_32x32x16_f16), else bf16.
// DMA (transposed, STAGES = 4, N % BK == 0): the dY tile goes global -> LDS with direct
// loads instead of through the staging registers.
template <bool TRANS, int WM, int WN, int FM, int FN, int BK, int META, int MPT, int STAGES, bool F16, bool DMA>
__global__ __launch_bounds__(WM * WN * 64) void gemm_kernel(const uint16_t* __restrict__ A,
                                                            const int32_t* __restrict__ packed,
                                                            const uint16_t* __restrict__ scales,
                                                            const uint16_t* __restrict__ zeros,
                                                            const Epi ep,
                                                            int M, int N, int K, int log2g, int kt_per_slice,
                                                            int ct0, int pw, float* __restrict__ part) {
  constexpr int T = WM * WN * 64;
  constexpr int BM = WM * FM * 32;
  constexpr int BN = WN * FN * 32;
  constexpr int LR = lds_row<BK>();
  constexpr int SLOTS = BK / 8;                 // 16-byte units per activation row per stage
  constexpr int A_UNITS = BM * SLOTS / T;       // activation units per thread per stage
  static_assert(A_UNITS >= 1 && BM * SLOTS % T == 0, "activation tile split");
  constexpr int W_PER_T = BN * SLOTS / T;       // packed words per thread per stage
  static_assert(W_PER_T >= 1 && W_PER_T <= 8 && BN * SLOTS % T == 0, "weight tile split");

  constexpr int LST = STAGES == 4 ? 2 : STAGES;  // LDS stages (4: two, interleaved stores)
  static_assert(!DMA || (TRANS && STAGES == 4), "direct activation loads: interleaved transposed tiles");
  // activation rows: padded by 16 bytes, or (DMA) unpadded with the 16-byte chunk index
  // XOR-ed by (row >> ASH) % SLOTS, which keeps the 32 rows of a fragment read in
  // distinct banks (a direct load writes 64 consecutive 16-byte slots, so rows cannot
  // be padded)
  constexpr int LRA = DMA ? BK : LR;
  constexpr int ASH = SLOTS == 8 ? 2 : SLOTS == 4 ? 3 : 4;
  extern __shared__ __attribute__((aligned(16))) uint16_t smem[];
  uint16_t* As = smem;                          // [LST][BM][LRA]
  uint16_t* Bs = smem + LST * BM * LRA;         // [LST][BN][LR]
  // Transposed mode: the weight tile is written column-wise (rows 8 apart per lane), which
  // puts the lanes of one LDS write in the same banks; XOR-ing the 16-byte chunk index of
  // row k with (k / 16) spreads them while the 16 consecutive rows of an MFMA operand read
  // keep one swizzle value (so reads stay conflict-free).  Element offset e of row k.
  auto bswz = [](int k, int e) -> int {
    if constexpr (!TRANS) return e;
    else return ((((e >> 3) ^ (k >> 4)) & (BK / 8 - 1)) << 3) | (e & 7);
  };

  const int L = TRANS ? N : K;      // contraction length
  const int OUTC = TRANS ? K : N;   // output columns
  const int KW = K >> 3;            // packed words per weight row
  const int gpr = META == META_GROUP ? K >> log2g : 1;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave / WN, wn = wave % WN;
  const int m0 = blockIdx.y * BM;
  const int c0 = (blockIdx.x + ct0) * BN;
  // contraction steps of this workgroup: all of them, or one slice of a split-K launch
  const int KT_ALL = (L + BK - 1) / BK;
  const int KB = blockIdx.z * kt_per_slice;
  const int KT = min(KT_ALL - KB, kt_per_slice);

  // ---- staging registers: one stage of raw global data (two buffers alternate)
  struct Regs {
    u32x4 a[A_UNITS];
    uint32_t w[W_PER_T];
    uint16_t s[W_PER_T], z[W_PER_T];
    uint32_t sv[4], zv[4];  // transposed rowwise: the W_PER_T rows' pairs as loaded
  };
  // scale / zero bits of staged row i: transposed rowwise ones are split out of the loaded
  // words only where they are used, so the loads do not have to land when issued
  auto s_of = [](const Regs& R, int i) -> uint16_t {
    if constexpr (TRANS && META == META_ROW) return (uint16_t)(R.sv[i / 2] >> (16 * (i & 1)));
    else return R.s[i];
  };
  auto z_of = [](const Regs& R, int i) -> uint16_t {
    if constexpr (TRANS && META == META_ROW) return (uint16_t)(R.zv[i / 2] >> (16 * (i & 1)));
    else return R.z[i];
  };

  auto meta_index = [&](int n, int wcol) -> size_t {
    if constexpr (META == META_GLOBAL) return 0;
    else if constexpr (META == META_ROW) return (size_t)n;
    else return (size_t)n * gpr + ((wcol * 8) >> log2g);
  };

  // Transposed mode: buffer loads at per-thread offsets fixed for the whole contraction,
  // so a step adds one scalar to them.  Activations: one resource over the tile's rows
  // (rows past M read as zero).  Weights and scale / zero: a resource over the step's BK
  // contraction rows, rebuilt per step from scalars (rows past N read as zero: code 0,
  // scale 0, zero 0 dequantize to 0, against zeroed activation columns).
  constexpr int WCOLS = BN / 8;
  rsrc_t t_ar = make_rsrc(A, 0);
  uint32_t t_aoff[A_UNITS] = {};
  uint32_t t_woff = 0, t_moff = 0;
  uint16_t t_gs = 0, t_gz = 0;
  if constexpr (TRANS) {
    // N < 2^22 and K <= 2^21 (checked at the boundary) keep every offset below 2^32
    t_ar = make_rsrc(A + (size_t)m0 * L, (uint32_t)__builtin_amdgcn_readfirstlane(min(BM, M - m0)) * (uint32_t)L * 2u);
#pragma unroll
    for (int i = 0; i < A_UNITS; ++i) {
      const int u = tid + i * T;
      const int row = u / SLOTS;
      const int ch = DMA ? ((u % SLOTS) ^ ((row >> ASH) & (SLOTS - 1))) : u % SLOTS;
      t_aoff[i] = ((uint32_t)row * (uint32_t)L + (uint32_t)ch * 8u) * 2u;
    }
    const int wc = tid % WCOLS, rb = tid / WCOLS;
    const int wcol = min((c0 >> 3) + wc, KW - 1);
    t_woff = ((uint32_t)(rb * W_PER_T) * (uint32_t)KW + (uint32_t)wcol) * 4u;
    // groupwise: row rb * W_PER_T's pair of the word column's group; rowwise: that row's pair
    if constexpr (META == META_GROUP)
      t_moff = ((uint32_t)(rb * W_PER_T) * (uint32_t)gpr + (uint32_t)((wcol * 8) >> log2g)) * 2u;
    else
      t_moff = (uint32_t)(rb * W_PER_T) * 2u;
    if constexpr (META == META_GLOBAL) {
      t_gs = scales[0];
      t_gz = zeros[0];
    }
  }

  auto load_stage = [&](int kt, Regs& R) {
    const int l0 = (KB + kt) * BK;
    if constexpr (TRANS) {
      if constexpr (!DMA) {
#pragma unroll
        for (int i = 0; i < A_UNITS; ++i)
          R.a[i] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(t_ar, t_aoff[i] + (uint32_t)l0 * 2, 0, 0));
      }
      // uniform values, kept in scalar registers (a vector min / max here would make the
      // resource descriptor per-lane and every load a waterfall loop)
      const int rows = __builtin_amdgcn_readfirstlane(max(0, min(BK, N - l0)));
      const int nb = __builtin_amdgcn_readfirstlane(min(l0, N - 1));
      const rsrc_t pr = make_rsrc(packed + (size_t)nb * KW, (uint32_t)rows * (uint32_t)KW * 4u);
#pragma unroll
      for (int i = 0; i < W_PER_T; ++i)
        R.w[i] = __builtin_amdgcn_raw_buffer_load_b32(pr, t_woff + (uint32_t)(i * KW * 4), 0, 0);
      if constexpr (META == META_GROUP) {
        const rsrc_t sr = make_rsrc(scales + (size_t)nb * gpr, (uint32_t)(rows * gpr * 2));
        const rsrc_t zr = make_rsrc(zeros + (size_t)nb * gpr, (uint32_t)(rows * gpr * 2));
#pragma unroll
        for (int i = 0; i < W_PER_T; ++i) {
          R.s[i] = __builtin_amdgcn_raw_buffer_load_b16(sr, t_moff + (uint32_t)(i * gpr * 2), 0, 0);
          R.z[i] = __builtin_amdgcn_raw_buffer_load_b16(zr, t_moff + (uint32_t)(i * gpr * 2), 0, 0);
        }
      } else if constexpr (META == META_ROW) {
        // the W_PER_T consecutive rows' pairs in one load per array
        const rsrc_t sr = make_rsrc(scales + nb, (uint32_t)(rows * 2));
        const rsrc_t zr = make_rsrc(zeros + nb, (uint32_t)(rows * 2));
        uint32_t* sv = R.sv;
        uint32_t* zv = R.zv;
        if constexpr (W_PER_T == 8) {
          const u32x4 a = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(sr, t_moff, 0, 0));
          const u32x4 b = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(zr, t_moff, 0, 0));
#pragma unroll
          for (int q = 0; q < 4; ++q) { sv[q] = a[q]; zv[q] = b[q]; }
        } else if constexpr (W_PER_T == 4) {
          const u32x2 a = __builtin_bit_cast(u32x2, __builtin_amdgcn_raw_buffer_load_b64(sr, t_moff, 0, 0));
          const u32x2 b = __builtin_bit_cast(u32x2, __builtin_amdgcn_raw_buffer_load_b64(zr, t_moff, 0, 0));
          sv[0] = a[0]; sv[1] = a[1]; zv[0] = b[0]; zv[1] = b[1];
        } else if constexpr (W_PER_T == 2) {
          sv[0] = __builtin_amdgcn_raw_buffer_load_b32(sr, t_moff, 0, 0);
          zv[0] = __builtin_amdgcn_raw_buffer_load_b32(zr, t_moff, 0, 0);
        } else {
          sv[0] = __builtin_amdgcn_raw_buffer_load_b16(sr, t_moff, 0, 0);
          zv[0] = __builtin_amdgcn_raw_buffer_load_b16(zr, t_moff, 0, 0);
        }
      } else {
#pragma unroll
        for (int i = 0; i < W_PER_T; ++i) {
          R.s[i] = t_gs;
          R.z[i] = t_gz;
        }
      }
      return;
    }
#pragma unroll
    for (int i = 0; i < A_UNITS; ++i) {
      const int u = tid + i * T;
      const int row = u / SLOTS, slot = u % SLOTS;
      const int m = min(m0 + row, M - 1);
      const int l = min(l0 + slot * 8, L - 8);  // past the end of the contraction: zeroed at store
      R.a[i] = *reinterpret_cast<const u32x4*>(A + (size_t)m * L + l);
    }
    if constexpr (!TRANS) {
      // rows = output columns n; each thread takes W_PER_T consecutive words of one row
      constexpr int TPR = SLOTS / W_PER_T;  // threads per row
      const int row = tid / TPR;
      const int w0 = (tid % TPR) * W_PER_T;
      const int n = min(c0 + row, N - 1);
      const int wc = (l0 >> 3) + w0;
      const int32_t* src = packed + (size_t)n * KW + wc;
      // words past the row (the last step when K % BK != 0) are not read: they multiply
      // activation columns that are zero, and are set to code 0.  KW % 4 == 0 and wc is a
      // multiple of W_PER_T, so a 2- or 4-word load is wholly inside or wholly past the row.
      if constexpr (W_PER_T >= 4) {
#pragma unroll
        for (int h = 0; h < W_PER_T / 4; ++h) {
          const u32x4 v = wc + 4 * h < KW ? __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(src) + h)
                                          : u32x4{0u, 0u, 0u, 0u};
          R.w[4 * h] = v[0]; R.w[4 * h + 1] = v[1]; R.w[4 * h + 2] = v[2]; R.w[4 * h + 3] = v[3];
        }
      } else if constexpr (W_PER_T == 2) {
        const u32x2 v = wc < KW ? __builtin_nontemporal_load(reinterpret_cast<const u32x2*>(src)) : u32x2{0u, 0u};
        R.w[0] = v[0]; R.w[1] = v[1];
      } else {
        R.w[0] = wc < KW ? (uint32_t)__builtin_nontemporal_load(src) : 0u;
      }
#pragma unroll
      for (int i = 0; i < MPT; ++i) {
        const size_t mi = meta_index(n, min(wc + i, KW - 1));
        R.s[i] = scales[mi];
        R.z[i] = zeros[mi];
      }
    } else {
      // rows = contraction n (W_PER_T consecutive rows per thread), one word = 8 output columns
      constexpr int WCOLS = BN / 8;
      const int wc = tid % WCOLS;
      const int rb = tid / WCOLS;
      const int wcol = min((c0 >> 3) + wc, KW - 1);
#pragma unroll
      for (int i = 0; i < W_PER_T; ++i) {
        const int n = min(l0 + rb * W_PER_T + i, N - 1);
        R.w[i] = (uint32_t)__builtin_nontemporal_load(packed + (size_t)n * KW + wcol);
        const size_t mi = meta_index(n, wcol);
        R.s[i] = scales[mi];
        R.z[i] = zeros[mi];
      }
    }
  };

  auto store_stage = [&](int kt, const Regs& R, int buf) {
    uint16_t* as = As + buf * BM * LRA;
    uint16_t* bs = Bs + buf * BN * LR;
    if constexpr (!DMA) {
#pragma unroll
      for (int i = 0; i < A_UNITS; ++i) {
        const int u = tid + i * T;
        const int row = u / SLOTS, slot = u % SLOTS;
        const bool in = (KB + kt) * BK + slot * 8 < L;  // columns past the contraction read as zero
        *reinterpret_cast<u32x4*>(as + row * LR + slot * 8) = in ? R.a[i] : u32x4{0u, 0u, 0u, 0u};
      }
    }
    if constexpr (!TRANS) {
      constexpr int TPR = SLOTS / W_PER_T;
      const int row = tid / TPR;
      const int w0 = (tid % TPR) * W_PER_T;
      DqConst d0;
      if constexpr (MPT == 1) d0 = dq_const_mix(R.s[0], R.z[0]);
#pragma unroll
      for (int i = 0; i < W_PER_T; ++i) {
        uint32_t o[4];
        dq_word_op<F16>(R.w[i], MPT == 1 ? d0 : dq_const_mix(R.s[i], R.z[i]), o);
        *reinterpret_cast<u32x4*>(bs + row * LR + (w0 + i) * 8) = u32x4{o[0], o[1], o[2], o[3]};
      }
    } else {
      // dequantize a column of W_PER_T rows x 8 output columns and write it across the
      // contraction axis: output column k = 8 wc + j gets W_PER_T consecutive n values
      constexpr int WCOLS = BN / 8;
      const int wc = tid % WCOLS;
      const int rb = tid / WCOLS;
      // pk[p][j]: column j of rows 2p, 2p + 1 as one operand pair
      constexpr int NP = (W_PER_T + 1) / 2;
      uint32_t pk[NP][8];
#pragma unroll
      for (int p = 0; p < NP; ++p) {
        const int i1 = 2 * p + 1 < W_PER_T ? 2 * p + 1 : 2 * p;
        dq_rows_op<F16>(R.w[2 * p], dq_const_mix(s_of(R, 2 * p), z_of(R, 2 * p)), R.w[i1],
                        dq_const_mix(s_of(R, i1), z_of(R, i1)), pk[p]);
      }
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        uint16_t* dst = bs + (wc * 8 + j) * LR + bswz(wc * 8 + j, rb * W_PER_T);
        if constexpr (W_PER_T == 8) {
          *reinterpret_cast<u32x4*>(dst) = u32x4{pk[0][j], pk[1][j], pk[2][j], pk[3][j]};
        } else if constexpr (W_PER_T == 4) {
          *reinterpret_cast<u32x2*>(dst) = u32x2{pk[0][j], pk[1][j]};
        } else if constexpr (W_PER_T == 2) {
          *reinterpret_cast<uint32_t*>(dst) = pk[0][j];
        } else {
          *dst = (uint16_t)(pk[0][j] & 0xFFFFu);
        }
      }
    }
  };

  f32x16 acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

  // v_mfma_f32_32x32x16_bf16: lane l supplies row (l % 32) of A and column (l % 32) of B,
  // contraction slots 8 (l / 32) .. +7 of the 16-wide step
  const int lr = lane & 31;
  const int lk = (lane >> 5) * 8;
  // activation fragment: row (wm FM + i) 32 + lr, contraction chunk 2 kk + lane / 32
  auto a_frag = [&](const uint16_t* abuf, int i, int kk) -> u32x4 {
    if constexpr (DMA) {
      const int ch = (2 * kk + (lane >> 5)) ^ ((lr >> ASH) & (SLOTS - 1));
      return *reinterpret_cast<const u32x4*>(abuf + (wm * FM * 32 + i * 32 + lr) * LRA + ch * 8);
    } else {
      return *reinterpret_cast<const u32x4*>(abuf + (wm * FM * 32 + lr) * LR + lk + i * 32 * LR + kk * 16);
    }
  };
  auto compute = [&](int buf) {
    const uint16_t* abuf = As + buf * BM * LRA;
    const uint16_t* bs = Bs + buf * BN * LR + (wn * FN * 32 + lr) * LR;
#pragma unroll
    for (int kk = 0; kk < BK / 16; ++kk) {
      u32x4 af[FM], bfr[FN];
#pragma unroll
      for (int i = 0; i < FM; ++i) af[i] = a_frag(abuf, i, kk);
#pragma unroll
      for (int j = 0; j < FN; ++j)
        bfr[j] = *reinterpret_cast<const u32x4*>(bs + j * 32 * LR + bswz(wn * FN * 32 + j * 32 + lr, kk * 16 + lk));
#pragma unroll
      for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j) acc[i][j] = mfma_op<F16>(af[i], bfr[j], acc[i][j]);
    }
  };

  // STAGES == 4 (transposed only): the MFMAs of one step read LDS buffer `buf` while the
  // next step's staged registers R are dequantized and written to buffer `sbuf`, the work
  // cut into one slice per 16-wide sub-step so that it issues between the MFMAs: activation
  // units, then weight words dequantized two rows at a time and rounded to bf16 pairs; the
  // transposed 16-byte rows are written once all W_PER_T rows of a word column are packed.
  auto compute_store = [&](int buf, const Regs& R, int kt_s, int sbuf) {
    static_assert(STAGES != 4 || (TRANS && W_PER_T >= 2 && W_PER_T % 2 == 0), "interleaved stores: transposed tiles");
    if constexpr (STAGES == 4) {
    constexpr int KK = BK / 16;
    constexpr int AU_PER = (A_UNITS + KK - 1) / KK;
    const uint16_t* abuf = As + buf * BM * LRA;
    const uint16_t* bs = Bs + buf * BN * LR + (wn * FN * 32 + lr) * LR;
    uint16_t* asw = As + sbuf * BM * LRA;
    uint16_t* bsw = Bs + sbuf * BN * LR;
    constexpr int WCOLS = BN / 8;
    const int wc = tid % WCOLS;
    const int rb = tid / WCOLS;
    uint32_t pk[W_PER_T / 2][8];
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) {
      u32x4 af[FM], bfr[FN];
#pragma unroll
      for (int i = 0; i < FM; ++i) af[i] = a_frag(abuf, i, kk);
#pragma unroll
      for (int j = 0; j < FN; ++j)
        bfr[j] = *reinterpret_cast<const u32x4*>(bs + j * 32 * LR + bswz(wn * FN * 32 + j * 32 + lr, kk * 16 + lk));
#pragma unroll
      for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j) acc[i][j] = mfma_op<F16>(af[i], bfr[j], acc[i][j]);
      // slice kk of the next step's stores
#pragma unroll
      for (int q = 0; q < AU_PER; ++q) {
        const int i = kk * AU_PER + q;
        if (!DMA && i < A_UNITS) {
          const int u = tid + i * T;
          const int row = u / SLOTS, slot = u % SLOTS;
          const bool in = (KB + kt_s) * BK + slot * 8 < L;
          *reinterpret_cast<u32x4*>(asw + row * LR + slot * 8) = in ? R.a[i] : u32x4{0u, 0u, 0u, 0u};
        }
      }
#pragma unroll
      for (int pp = 0; pp < W_PER_T / 2; ++pp) {
        const int i = 2 * pp;  // rows i, i + 1 of the word column, in slice pp * KK / pairs
        if (pp * KK / (W_PER_T / 2) == kk)
          dq_rows_op<F16>(R.w[i], dq_const_mix(s_of(R, i), z_of(R, i)), R.w[i + 1],
                          dq_const_mix(s_of(R, i + 1), z_of(R, i + 1)), pk[i / 2]);
      }
    }
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      uint16_t* dst = bsw + (wc * 8 + j) * LR + bswz(wc * 8 + j, rb * W_PER_T);
      if constexpr (W_PER_T == 8) *reinterpret_cast<u32x4*>(dst) = u32x4{pk[0][j], pk[1][j], pk[2][j], pk[3][j]};
      else if constexpr (W_PER_T == 4) *reinterpret_cast<u32x2*>(dst) = u32x2{pk[0][j], pk[1][j]};
      else *reinterpret_cast<uint32_t*>(dst) = pk[0][j];
    }
    }
  };

  if constexpr (DMA) {
    // As STAGES == 4 below, with the dY tile of step k + 1 loaded straight into LDS during
    // step k.  Each step issues the direct tile loads and then the weight loads of step
    // k + 2; vector-memory loads complete in issue order, so waiting until only the NW
    // weight loads of the step are outstanding means the tile has landed, while those
    // weights keep two steps to arrive.  The barrier carries no fence (a workgroup fence
    // would wait for every load in flight), so the wait also covers the LDS stores.
    constexpr int NW = W_PER_T + (META == META_GROUP ? 2 * W_PER_T : META == META_ROW ? 2 : 0);
    typedef __attribute__((address_space(3))) void lds_void;
    auto dma_a = [&](int kt, int buf) {
      const uint32_t l0 = (uint32_t)((KB + kt) * BK);
      char* base = reinterpret_cast<char*>(As + buf * BM * LRA);
#pragma unroll
      for (int i = 0; i < A_UNITS; ++i)
        // the whole offset in the range-checked vector offset (rows past M read zero); an
        // int argument, since with an unsigned one the host pass drops the launch stub
        __builtin_amdgcn_raw_ptr_buffer_load_lds(t_ar, (lds_void*)(base + (i * T + wave * 64) * 16), 16,
                                                 (int)(t_aoff[i] + l0 * 2u), 0, 0, 0);
    };
    // s_waitcnt vmcnt(n) lgkmcnt(0), then a barrier with no fence; the clobbers keep memory
    // accesses, and the scheduling barriers all instructions, on their side of it
    auto sync = [&](auto n_tag) {
      constexpr int n = decltype(n_tag)::value;
      __builtin_amdgcn_sched_barrier(0);
      asm volatile("" ::: "memory");
      __builtin_amdgcn_s_waitcnt((n & 15) | 0x70 | ((n >> 4) << 14));
      __builtin_amdgcn_s_barrier();
      asm volatile("" ::: "memory");
      __builtin_amdgcn_sched_barrier(0);
    };
    Regs R0, R1;
    dma_a(0, 0);
    __builtin_amdgcn_sched_barrier(0);
    load_stage(0, R0);
    load_stage(min(1, KT - 1), R1);
    __builtin_amdgcn_sched_barrier(0);
    store_stage(0, R0, 0);
    sync(std::integral_constant<int, 0>());
    int kt = 0;
    for (; kt + 2 <= KT; kt += 2) {
      dma_a(kt + 1, 1);
      __builtin_amdgcn_sched_barrier(0);
      load_stage(kt + 2, R0);
      compute_store(0, R1, kt + 1, 1);
      sync(std::integral_constant<int, NW>());
      dma_a(kt + 2, 0);
      __builtin_amdgcn_sched_barrier(0);
      load_stage(kt + 3, R1);
      compute_store(1, R0, kt + 2, 0);
      sync(std::integral_constant<int, NW>());
    }
    if (kt < KT) compute(0);
    // no direct LDS load may land after the workgroup's LDS is handed on
    __builtin_amdgcn_s_waitcnt(0x0070);
  } else if constexpr (STAGES == 4) {
    // Two LDS stages and two register stages: the loads of step k + 2 are issued before
    // the MFMAs of step k, and step k + 1 (staged during step k - 1) is dequantized and
    // stored in slices between the MFMAs of step k.  Loads past the contraction read
    // clamped (valid) addresses; what they stage is never computed.
    Regs R0, R1;
    load_stage(0, R0);
    load_stage(min(1, KT - 1), R1);
    store_stage(0, R0, 0);
    __syncthreads();
    int kt = 0;
    for (; kt + 2 <= KT; kt += 2) {
      load_stage(kt + 2, R0);
      compute_store(0, R1, kt + 1, 1);
      __syncthreads();
      load_stage(kt + 3, R1);
      compute_store(1, R0, kt + 2, 0);
      __syncthreads();
    }
    if (kt < KT) compute(0);
  } else if constexpr (STAGES == 2) {
    // Two LDS stages, one register stage: the loads of step k+1 are issued before the
    // MFMAs of step k and dequantized into the other LDS buffer after them.
    Regs R0;
    load_stage(0, R0);
    store_stage(0, R0, 0);
    __syncthreads();
    for (int kt = 0; kt < KT; ++kt) {
      const bool more = kt + 1 < KT;
      if (more) load_stage(kt + 1, R0);
      compute(kt & 1);
      if (more) store_stage(kt + 1, R0, (kt + 1) & 1);
      __syncthreads();
    }
  } else {
    // Three LDS stages and two register stages: the global loads of step k + 2 are issued
    // before the MFMAs of step k and stored (dequantized) to LDS at the end of step k + 1,
    // so each load has two steps of MFMA work to arrive.  Unrolled by two so the register
    // stage in flight is never copied; every load in the loop body is unconditional (the
    // compiler's wait counts then keep the other stage in flight) and the tail is peeled.
    Regs R0, R1;
    load_stage(0, R0);
    load_stage(min(1, KT - 1), R1);
    store_stage(0, R0, 0);
    __syncthreads();
    int kt = 0;
    for (; kt + 4 <= KT; kt += 2) {
      load_stage(kt + 2, R0);
      compute(kt % 3);
      store_stage(kt + 1, R1, (kt + 1) % 3);
      __syncthreads();
      load_stage(kt + 3, R1);
      compute((kt + 1) % 3);
      store_stage(kt + 2, R0, (kt + 2) % 3);
      __syncthreads();
    }
    const int rem = KT - kt;  // 1, 2 or 3 steps left; R1 holds step kt + 1
    if (rem == 3) {
      load_stage(kt + 2, R0);
      compute(kt % 3);
      store_stage(kt + 1, R1, (kt + 1) % 3);
      __syncthreads();
      compute((kt + 1) % 3);
      store_stage(kt + 2, R0, (kt + 2) % 3);
      __syncthreads();
      compute((kt + 2) % 3);
    } else if (rem == 2) {
      compute(kt % 3);
      store_stage(kt + 1, R1, (kt + 1) % 3);
      __syncthreads();
      compute((kt + 1) % 3);
    } else {
      compute(kt % 3);
    }
  }

  // ---- epilogue.  Result register r of a 32x32 block sits at row 8 (r / 4) +
  // 4 (lane / 32) + (r % 4), column lane % 32.  A split-K slice writes its partial sums
  // (fp32, no bias) to its own [M][pw] plane of `part`; an unsplit launch stores
  // through the output epilogue (bias, output dtype, output segments).
  const int rbase = m0 + wm * FM * 32 + (lane >> 5) * 4;
  const int cbase = c0 + wn * FN * 32 + lr;
  if (part == nullptr && epi_wide(ep, OUTC) != 0) {  // plain output: four columns per store
#pragma unroll
    for (int j = 0; j < FN; ++j) {
      const EpiQuad q = epi_quad(ep, cbase - lr + j * 32 + (lr & ~3), OUTC);
#pragma unroll
      for (int i = 0; i < FM; ++i) epi_put_block_wide(q, acc[i][j], rbase + i * 32, M, lane);
    }
    return;
  }
#pragma unroll
  for (int j = 0; j < FN; ++j) {
    const int c = cbase + j * 32;
    if (c >= OUTC) continue;
    if (part != nullptr) {
      float* out = part + (size_t)blockIdx.z * M * pw;
      const int pc = c - ct0 * BN;  // column within the plane
#pragma unroll
      for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int m = rbase + i * 32 + (r >> 2) * 8 + (r & 3);
          if (m < M) out[(size_t)m * pw + pc] = acc[i][j][r];
        }
    } else {
      const EpiCol col = epi_col(ep, c);
#pragma unroll
      for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int m = rbase + i * 32 + (r >> 2) * 8 + (r & 3);
          if (m < M) epi_put(ep, col, m, acc[i][j][r]);
        }
    }
  }
}

// Split-K reduction: output columns [c_lo, c_lo + pw) = epilogue(sum over the S partial
// [M][pw] planes, in a fixed order).  VEC (pw and c_lo multiples of 4): four consecutive
// columns per thread, one 16-byte load per plane, and one store of the four columns for a
// plain one-segment output with aligned rows (16 bytes of fp32, 8 of bf16 / fp16); the
// same values, bit for bit.
template <bool VEC>
__global__ __launch_bounds__(256) void splitk_reduce_kernel(const float* __restrict__ part, int S, int64_t M,
                                                            int64_t c_lo, int64_t pw, const Epi ep) {
  const int64_t total = M * pw;
  if constexpr (!VEC) {
    for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < total; i += (int64_t)gridDim.x * 256) {
      float v = part[i];
      for (int s = 1; s < S; ++s) v += part[(size_t)s * total + i];
      const int64_t m = i / pw, c = i - m * pw;
      epi_put(ep, epi_col(ep, c_lo + c), m, v);
    }
  } else {
    typedef float f32x4v __attribute__((ext_vector_type(4)));
    const bool wide = epi_wide(ep, pw) != 0;  // pw and c_lo are multiples of 4 here
    const f32x4v* p4 = reinterpret_cast<const f32x4v*>(part);
    const int64_t total4 = total >> 2;
    for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < total4; i += (int64_t)gridDim.x * 256) {
      f32x4v v = __builtin_nontemporal_load(p4 + i);
      for (int s = 1; s < S; ++s) v += __builtin_nontemporal_load(p4 + (size_t)s * total4 + i);
      const int64_t m = (i << 2) / pw, c = (i << 2) - m * pw;
      if (wide) {
        const float o[4] = {v[0], v[1], v[2], v[3]};
        epi_store4(epi_quad(ep, c_lo + c, c_lo + pw), m, o);
      } else {
#pragma unroll
        for (int u = 0; u < 4; ++u) epi_put(ep, epi_col(ep, c_lo + c + u), m, v[u]);
      }
    }
  }
}

// ---------------------------------------------------------------- host side

namespace {

// Tile configurations.  kind 0: the LDS-staged kernel above (both directions; the
// non-transposed form only serves contractions too long for the register-operand kernel);
// kind 1-6: the non-transposed register-operand kernel (gemm_nt.hip): 128 x 128, 256 x 128,
// 64 x 128, 32 x 128 with four waves, 256 x 256 and 128 x 256 with eight.  slots: workgroups resident per CU; full: workgroups per CU needed for
// full throughput; eff: throughput of a full tile relative to the best of its direction,
// all measured on MI355X at the fine-tune shapes.
struct Cfg {
  int kind;
  int wm, wn, fm, fn, bk, stages;
  const char* name;
  bool transposed;
  int slots, full;
  float eff;
};
constexpr Cfg kCfgs[] = {
    {0, 2, 2, 4, 4, 64, 4, "gemm_t_256x256", true, 1, 1, 0.98f},
    {0, 4, 2, 2, 2, 64, 4, "gemm_t_256x128", true, 1, 1, 1.0f},
    {0, 2, 2, 2, 2, 32, 4, "gemm_t_128x128", true, 3, 2, 0.65f},
    {1, 1, 4, 4, 1, 64, 2, "gemm_nt_128x128", false, 3, 2, 0.92f},
    {2, 1, 4, 8, 1, 64, 2, "gemm_nt_256x128", false, 2, 2, 1.0f},
    {0, 2, 2, 4, 4, 64, 2, "gemm_nt_lds_256x256", false, 1, 1, 0.7f},
    // short-M tiles (5 <= M < 128): fewer rows per tile waste less of it; the dequantization
    // is then shared by fewer rows, so their full-tile efficiency is lower
    {3, 1, 4, 2, 1, 64, 2, "gemm_nt_64x128", false, 4, 2, 0.85f},
    {4, 1, 4, 1, 1, 64, 2, "gemm_nt_32x128", false, 4, 2, 0.5f},
    {0, 1, 4, 1, 1, 64, 4, "gemm_t_32x128", true, 3, 2, 0.3f},
    // eight waves side by side (256 columns) on one activation tile
    {5, 1, 8, 8, 1, 64, 2, "gemm_nt_256x256", false, 1, 1, 1.02f},
    {6, 1, 8, 4, 1, 64, 2, "gemm_nt_128x256", false, 2, 2, 0.94f},
    // transposed 256 x 256 with eight waves (2 x 4, each 128 x 64): two waves per SIMD where
    // the four-wave form has one, and the same LDS tiles
    {0, 2, 4, 4, 2, 64, 4, "gemm_t_w8_256x256", true, 1, 1, 1.25f},
};
constexpr int kNumCfgs = sizeof(kCfgs) / sizeof(kCfgs[0]);
constexpr int kNtLdsCfg = 5;

// splits > 1: every tile's contraction is split.  tail_cols > 0: the first column tiles
// (a whole number of rounds of workgroups) run unsplit and the last tail_cols column tiles
// run with their contraction split tail_splits ways, so the last, partial round of an
// unsplit launch becomes short slices spread over every CU.
struct Plan {
  int cfg;
  int splits;
  int tail_cols = 0, tail_splits = 1;
};

// Choose the tile configuration and the split-K factor: score = full-tile efficiency x
// utilisation x edge-tile useful fraction / (1 + cost of the split-K partial planes).
// Utilisation: with all workgroups resident at once, min(1, workgroups / (CUs x full));
// over several rounds, the filled fraction of the rounds.
// Small forward problems at prefill sizes (M >= 128, under kSmallFlops: a few tens of
// microseconds; the short-M tiles keep their measured scores) are bound by the
// latency of each contraction step and by launch costs, not by the MFMA rate that the scores
// of pick_plan model, so an estimated time picks their plan.  A round of workgroups takes the
// longer of its contraction steps at the latency of one step and its share of the CU's MFMA
// rate at the tile's efficiency; a split adds the reduction launch and the write and read of
// its fp32 partial planes.  Constants measured on MI355X: a latency-bound step ~0.4 us (32 x
// 128 and 64 x 128 tiles, one round, K = 2048), the best tile ~1.05 PFLOP/s at eff = 1, the
// reduction launch ~3 us, partial planes at ~4 TB/s.  At M = 512, (N, K) = (2048, 2048) an
// unsplit 32 x 128 launch took 12.9 us against 19.0 us for the two-way split the scores chose.
constexpr double kSmallFlops = 2e10;
constexpr double kStepS = 0.4e-6, kPeakFlops = 1.05e15, kReduceLaunchS = 3e-6, kPlaneBps = 4e12;

Plan pick_plan_small(const MmArgs& a, const DeviceCaps& caps, bool allow_split) {
  const bool reg_ok = gemm_nt_reg_supported(a);
  const int64_t cus = caps.cus > 0 ? caps.cus : 256;
  Plan best{reg_ok ? 3 : kNtLdsCfg, 1};
  double best_t = 1e30;
  for (int i = 0; i < kNumCfgs; ++i) {
    const Cfg& c = kCfgs[i];
    if (c.transposed || (c.kind != 0) != reg_ok) continue;
    const int64_t bm = c.wm * c.fm * 32, bn = c.wn * c.fn * 32;
    const int64_t tm = (a.M + bm - 1) / bm, tn = (a.N + bn - 1) / bn;
    const int64_t kt = (a.K + c.bk - 1) / c.bk;
    for (int sp = 1; sp <= (allow_split ? 8 : 1); sp *= 2) {
      // >= 8 contraction steps per slice (measured: 4-way slices of 8 steps beat 2-way ones
      // of 16 by 12% at M = 128, (2048, 2048) and M = 512, (512, 2048))
      if (sp > 1 && kt / sp < 8) break;
      const int64_t wgs = tm * tn * sp, steps = (kt + sp - 1) / sp;
      const int64_t rounds = (wgs + cus * c.slots - 1) / (cus * c.slots);
      const int64_t per_cu = std::min<int64_t>(c.slots, (wgs + cus - 1) / cus);
      const double wg_flops = 2.0 * bm * bn * steps * c.bk;
      const double t_round = std::max(steps * kStepS, per_cu * wg_flops / (c.eff * kPeakFlops / cus));
      const double t = rounds * t_round + (sp > 1 ? kReduceLaunchS + 8.0 * sp * a.M * a.N / kPlaneBps : 0.0);
      // ties (both latency-bound) go to the later, smaller tile: measured 3-4% faster at
      // M = 128, (2048, 2048) and M = 512, (512, 2048)
      if (t <= best_t) {
        best_t = t;
        best = Plan{i, sp};
      }
    }
  }
  return best;
}

// W4A16_GEMM_CFG (an A/B benchmarking override) forces one tile configuration; set to any
// value it also keeps mid-M problems on the tiles instead of the mid-M kernel.
const char* gemm_cfg_env() {
  static const char* e = getenv("W4A16_GEMM_CFG");
  return e;
}

Plan pick_plan(const MmArgs& a, const DeviceCaps& caps, bool allow_split) {
  static const int forced = gemm_cfg_env() != nullptr ? atoi(gemm_cfg_env()) : -1;
  const int64_t outc = a.transposed ? a.K : a.N;
  const int64_t L = a.transposed ? a.N : a.K;
  if (forced < 0 && !a.transposed && a.M >= 128 && 2.0 * a.M * outc * L < kSmallFlops)
    return pick_plan_small(a, caps, allow_split);
  const bool reg_ok = gemm_nt_reg_supported(a);
  const int64_t cus = caps.cus > 0 ? caps.cus : 256;
  Plan best{a.transposed ? 1 : (reg_ok ? 3 : kNtLdsCfg), 1};
  float best_score = -1.0f;
  for (int i = 0; i < kNumCfgs; ++i) {
    const Cfg& c = kCfgs[i];
    if (c.transposed != a.transposed) continue;
    if (!a.transposed && (c.kind != 0) != reg_ok) continue;
    if (forced >= 0 && forced < kNumCfgs && kCfgs[forced].transposed == a.transposed && i != forced) continue;
    const int64_t bm = c.wm * c.fm * 32, bn = c.wn * c.fn * 32;
    const int64_t tm = (a.M + bm - 1) / bm, tn = (outc + bn - 1) / bn;
    const int64_t kt = (L + c.bk - 1) / c.bk;
    const float edge = (float)a.M / (float)(tm * bm) * (float)outc / (float)(tn * bn);
    // >= 16 contraction steps per slice and at most 8 slices; for M < 128 (few output tiles)
    // >= 8 steps and up to 16 slices (measured over the mid-M points at the decode shapes:
    // forward 1.6%, transposed 3.8% less time)
    const int min_steps = a.M < 128 ? 8 : 16, max_splits = a.M < 128 ? 16 : 8;
    for (int sp = 1; sp <= (allow_split ? max_splits : 1); sp *= 2) {
      if (sp > 1 && kt / sp < min_steps) break;
      // a one-workgroup-per-CU tile splits only when, unsplit, it would leave more than half
      // the CUs idle (measured: split at half the CUs it lost 2-4% to an unsplit 128 x 128)
      if (sp > 1 && c.slots == 1 && !a.transposed && 2 * tm * tn >= cus) break;
      const int64_t wgs = tm * tn * sp;
      const int64_t resident = cus * c.slots;
      float util;
      if (wgs <= resident) {
        util = std::min(1.0f, (float)wgs / (float)(cus * c.full));
      } else {
        const int64_t rounds = (wgs + resident - 1) / resident;
        util = (float)wgs / (float)(rounds * resident);
      }
      // partial planes: sp writes + sp reads of M x outc fp32 against 2 M outc L flops
      const float over = sp > 1 ? 480.0f * (float)sp / (float)L : 0.0f;
      const float score = c.eff * util * edge / (1.0f + over);
      if (score > best_score) {
        best_score = score;
        best = Plan{i, sp};
      }
      // split tail: whole tile columns that fill the full rounds run unsplit, the rest split
      // (not for the forward one-workgroup-per-CU tile: measured slower than 128 x 128 unsplit)
      if (sp == 1 && allow_split && (a.transposed || c.slots > 1) && wgs > resident && wgs % resident != 0) {
        const int64_t main_cols = wgs / resident * resident / tm;
        const int64_t tail_cols = tn - main_cols;
        if (main_cols > 0 && tail_cols > 0) {
          const int64_t main_rounds = (main_cols * tm + resident - 1) / resident;
          for (int ts = 2; ts <= 8; ts *= 2) {
            if (kt / ts < 16) break;
            const float tail_rounds = (float)((tail_cols * tm * ts + resident - 1) / resident) / (float)ts;
            const float u = (float)wgs / ((float)resident * ((float)main_rounds + tail_rounds));
            // the tail's partial planes, at twice the whole-split rate: measured, a tail also
            // pays a second launch and its reduction does not overlap the main launch
            const float o = (float)tail_cols / (float)tn * 960.0f * (float)ts / (float)L;
            const float sc = c.eff * u * edge / (1.0f + o);
            if (sc > best_score) {
              best_score = sc;
              best = Plan{i, 1, (int)tail_cols, ts};
            }
          }
        }
      }
    }
  }
  return best;
}

size_t split_bytes(const MmArgs& a, const Plan& p) {
  const int64_t outc = a.transposed ? a.K : a.N;
  if (p.splits > 1) return (size_t)p.splits * a.M * outc * sizeof(float);
  if (p.tail_cols > 0) {
    const Cfg& c = kCfgs[p.cfg];
    const int64_t bn = c.wn * c.fn * 32;
    const int64_t tn = (outc + bn - 1) / bn;
    const int64_t pw = outc - (tn - p.tail_cols) * bn;
    return (size_t)p.tail_splits * a.M * pw * sizeof(float);
  }
  return 0;
}

int meta_kind(int mode) { return mode == W4_MODE_GLOBAL ? META_GLOBAL : mode == W4_MODE_ROWWISE ? META_ROW : META_GROUP; }

size_t lds_bytes(const Cfg& c) {
  if (c.kind != 0) return (size_t)2 * c.wm * c.fm * 32 * (c.bk + 8) * 2;  // two activation buffers
  return (size_t)(c.stages == 4 ? 2 : c.stages) * (c.wm * c.fm * 32 + c.wn * c.fn * 32) * (c.bk + 8) * 2;
}

template <bool TRANS, int WM, int WN, int FM, int FN, int BK, int STAGES, int META, bool F16>
hipError_t run_k(const MmArgs& a, const GemmPart& gp, float* part, hipStream_t st) {
  constexpr int BM = WM * FM * 32, BN = WN * FN * 32;
  constexpr int WPT = BN * (BK / 8) / (WM * WN * 64);  // packed words per thread per stage
  // one scale / zero pair per thread when its WPT words (8 * WPT codes, aligned) share a group
  const bool one = TRANS || META != META_GROUP || a.group >= 8 * WPT;
  // transposed interleaved tiles with N % BK == 0 load the dY tile straight into LDS (no
  // activation columns past N to zero)
  constexpr bool DMA_OK = TRANS && STAGES == 4;
  const bool dma = DMA_OK && a.N % BK == 0;
  auto k = dma   ? gemm_kernel<TRANS, WM, WN, FM, FN, BK, META, 1, STAGES, F16, DMA_OK>
           : one ? gemm_kernel<TRANS, WM, WN, FM, FN, BK, META, 1, STAGES, F16, false>
                 : gemm_kernel<TRANS, WM, WN, FM, FN, BK, META, WPT, STAGES, F16, false>;
  const size_t lds = (size_t)(STAGES == 4 ? 2 : STAGES) * (BM * (dma ? BK : BK + 8) + BN * (BK + 8)) * 2;
  if (lds > 64 * 1024) {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(k), hipFuncAttributeMaxDynamicSharedMemorySize,
                                       (int)lds);
    if (e != hipSuccess) return e;
  }
  const int64_t outc = TRANS ? a.K : a.N;
  const int64_t L = TRANS ? a.N : a.K;
  const int kt_all = (int)((L + BK - 1) / BK);
  int splits = gp.splits;
  const int kts = (kt_all + splits - 1) / splits;
  splits = (kt_all + kts - 1) / kts;  // every slice gets at least one contraction step
  const int tn_all = (int)((outc + BN - 1) / BN);
  const int nct = gp.nct > 0 ? gp.nct : tn_all - gp.ct0;
  const int64_t c_lo = (int64_t)gp.ct0 * BN;
  const int pw = (int)(std::min<int64_t>(outc, c_lo + (int64_t)nct * BN) - c_lo);
  const dim3 grid((unsigned)nct, (unsigned)((a.M + BM - 1) / BM), (unsigned)splits);
  const int log2g = 31 - __builtin_clz((unsigned)a.group);
  k<<<grid, WM * WN * 64, lds, st>>>(a.A, a.packed, a.scales, a.zeros, a.ep, (int)a.M, (int)a.N, (int)a.K,
                                      log2g, kts, gp.ct0, pw, splits > 1 ? part : nullptr);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || splits == 1) return e;
  return launch_splitk_reduce(part, splits, a.M, c_lo, pw, a.ep, st);
}

template <bool TRANS, int WM, int WN, int FM, int FN, int BK, int STAGES, int META>
hipError_t run(const MmArgs& a, const GemmPart& gp, float* part, hipStream_t st) {
  return a.a_f16 ? run_k<TRANS, WM, WN, FM, FN, BK, STAGES, META, true>(a, gp, part, st)
                 : run_k<TRANS, WM, WN, FM, FN, BK, STAGES, META, false>(a, gp, part, st);
}

template <bool TRANS, int WM, int WN, int FM, int FN, int BK, int STAGES>
hipError_t run_meta(const MmArgs& a, const GemmPart& gp, float* part, hipStream_t st) {
  switch (meta_kind(a.mode)) {
    case META_GLOBAL: return run<TRANS, WM, WN, FM, FN, BK, STAGES, META_GLOBAL>(a, gp, part, st);
    case META_ROW: return run<TRANS, WM, WN, FM, FN, BK, STAGES, META_ROW>(a, gp, part, st);
    default: return run<TRANS, WM, WN, FM, FN, BK, STAGES, META_GROUP>(a, gp, part, st);
  }
}

hipError_t run_cfg(const MmArgs& a, int cfg, const GemmPart& gp, float* part, hipStream_t st) {
  if (a.transposed) {
    switch (cfg) {
      case 0: return run_meta<true, 2, 2, 4, 4, 64, 4>(a, gp, part, st);
      case 1: return run_meta<true, 4, 2, 2, 2, 64, 4>(a, gp, part, st);
      case 8: return run_meta<true, 1, 4, 1, 1, 64, 4>(a, gp, part, st);
      case 11: return run_meta<true, 2, 4, 4, 2, 64, 4>(a, gp, part, st);
      default: return run_meta<true, 2, 2, 2, 2, 32, 4>(a, gp, part, st);
    }
  }
  switch (kCfgs[cfg].kind) {
    case 1: return launch_gemm_nt_reg(a, 0, gp, part, st);
    case 2: return launch_gemm_nt_reg(a, 1, gp, part, st);
    case 3: return launch_gemm_nt_reg(a, 2, gp, part, st);
    case 4: return launch_gemm_nt_reg(a, 3, gp, part, st);
    case 5: return launch_gemm_nt_reg(a, 4, gp, part, st);
    case 6: return launch_gemm_nt_reg(a, 5, gp, part, st);
    default: return run_meta<false, 2, 2, 4, 4, 64, 2>(a, gp, part, st);
  }
}

hipError_t run_plan(const MmArgs& a, const Plan& p, float* part, hipStream_t st) {
  if (p.tail_cols == 0) return run_cfg(a, p.cfg, GemmPart{p.splits, 0, 0}, part, st);
  const Cfg& c = kCfgs[p.cfg];
  const int64_t bn = c.wn * c.fn * 32;
  const int tn = (int)(((a.transposed ? a.K : a.N) + bn - 1) / bn);
  const hipError_t e = run_cfg(a, p.cfg, GemmPart{1, 0, tn - p.tail_cols}, nullptr, st);
  if (e != hipSuccess) return e;
  return run_cfg(a, p.cfg, GemmPart{p.tail_splits, tn - p.tail_cols, p.tail_cols}, part, st);
}

// The mid-M kernel's plan for a launch with a workspace of ws_bytes (the split plan when its
// planes fit, else the unsplit one); ok = false when the tiles run instead.
SkinnyPlan launched_skinny(const MmArgs& a, const DeviceCaps& caps, size_t ws_bytes) {
  if (gemm_cfg_env() != nullptr || !skinny_supported(a)) return SkinnyPlan{};
  SkinnyPlan p = skinny_plan(a, caps, ws_bytes > 0);
  if (p.ok && skinny_split_bytes(a, p) > ws_bytes) p = skinny_plan(a, caps, false);
  return p;
}

// The plan a launch with a workspace of ws_bytes runs: the split plan when it fits the
// workspace, else the unsplit one.
Plan launched_plan(const MmArgs& a, const DeviceCaps& caps, size_t ws_bytes) {
  Plan p = pick_plan(a, caps, ws_bytes > 0);
  if ((p.splits > 1 || p.tail_cols > 0) && split_bytes(a, p) > ws_bytes) p = pick_plan(a, caps, false);
  return p;
}

}  // namespace

hipError_t launch_splitk_reduce(const float* part, int splits, int64_t M, int64_t c_lo, int64_t pw, const Epi& ep,
                                hipStream_t st) {
  if (pw % 4 == 0 && c_lo % 4 == 0) {
    const int64_t blocks = (M * pw / 4 + 255) / 256;
    splitk_reduce_kernel<true><<<(unsigned)(blocks < 8192 ? blocks : 8192), 256, 0, st>>>(part, splits, M, c_lo, pw, ep);
  } else {
    const int64_t blocks = (M * pw + 255) / 256;
    splitk_reduce_kernel<false><<<(unsigned)(blocks < 8192 ? blocks : 8192), 256, 0, st>>>(part, splits, M, c_lo, pw, ep);
  }
  return hipGetLastError();
}

const char* gemm_name(const MmArgs& a, const DeviceCaps& caps, size_t ws_bytes) {
  static thread_local char buf[64];
  const SkinnyPlan sp = launched_skinny(a, caps, ws_bytes);
  if (sp.ok) return skinny_name(a, sp);
  const Plan p = launched_plan(a, caps, ws_bytes);
  const Cfg& c = kCfgs[p.cfg];
  if (p.tail_cols > 0) {
    snprintf(buf, sizeof(buf), "%s_tail%d_splitk%d", c.name, p.tail_cols, p.tail_splits);
    return buf;
  }
  if (p.splits == 1) return c.name;
  snprintf(buf, sizeof(buf), "%s_splitk%d", c.name, p.splits);
  return buf;
}

size_t gemm_lds_bytes(const MmArgs& a, const DeviceCaps& caps, size_t ws_bytes) {
  const SkinnyPlan sp = launched_skinny(a, caps, ws_bytes);
  if (sp.ok) return sp.lds;
  return lds_bytes(kCfgs[launched_plan(a, caps, ws_bytes).cfg]);
}

size_t gemm_used_workspace_bytes(const MmArgs& a, const DeviceCaps& caps, size_t ws_bytes) {
  const SkinnyPlan sp = launched_skinny(a, caps, ws_bytes);
  if (sp.ok) return skinny_split_bytes(a, sp);
  return split_bytes(a, launched_plan(a, caps, ws_bytes));
}

size_t gemm_workspace_bytes(const MmArgs& a, const DeviceCaps& caps) {
  if (gemm_cfg_env() == nullptr && skinny_supported(a)) {
    const SkinnyPlan sp = skinny_plan(a, caps, true);
    if (sp.ok) return skinny_split_bytes(a, sp);
  }
  return split_bytes(a, pick_plan(a, caps, true));
}

hipError_t launch_gemm(const MmArgs& a, const DeviceCaps& caps, void* ws, size_t ws_bytes, hipStream_t st) {
  const SkinnyPlan sp = launched_skinny(a, caps, ws != nullptr ? ws_bytes : 0);
  if (sp.ok) return launch_skinny(a, sp, static_cast<float*>(ws), st);
  return run_plan(a, launched_plan(a, caps, ws != nullptr ? ws_bytes : 0), static_cast<float*>(ws), st);
}

}  // namespace w4
