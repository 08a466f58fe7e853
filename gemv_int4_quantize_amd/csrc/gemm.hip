// MFMA W4A16 GEMM for gfx950, both directions on one packed buffer:
//   non-transposed  Y[m][n]  = sum_k X[m][k]  * w[n][k] (+ bias[n])
//   transposed      dX[m][k] = sum_n dY[m][n] * w[n][k] (+ bias[k])
// with w = bf16_rne((q - z) * s), bf16 MFMA operands and fp32 accumulation.
// Sources: Objective 2 of "Quantized LLM Inference with Triton Kernels"
// (Y = X_bf16 @ W_int4^T); "Re-write HQQ Fused Gemm Transpose" (pytorch/ao #185:
// the transposed product reads the same packed weights, scales and zeros);
// "[Kernel] Adding bias epilogue support for cutlass_scaled_mm" (vLLM #5560).
//
// Structure (one workgroup = WM x WN waves, output tile BM x BN, contraction step 32):
//   * the activation tile (X or dY, contraction along its rows) goes global -> LDS;
//   * the packed weight tile is loaded to registers, dequantized in registers with
//     v_fma_mix_f32 + v_cvt_pk_bf16_f32, and written to LDS as a bf16 tile whose
//     rows are output columns and whose 32 columns are the contraction, so each MFMA
//     operand is one 16-byte LDS read in both directions.  Non-transposed, a packed
//     word already runs along the contraction; transposed, each thread dequantizes a
//     column of RPT rows of one word and writes it across the contraction axis;
//   * two LDS stages: the global loads of step k+1 are in flight during the MFMAs of
//     step k, and their dequantization follows them; one barrier per step;
//   * LDS rows are 80 bytes (64 + 16 pad) so the 16 rows read by one MFMA operand load
//     fall in distinct banks;
//   * v_mfma_f32_16x16x32_bf16: lane l holds row (l % 16), contraction slots
//     8 (l / 16) .. +7 of A, column (l % 16) and the same slots of B, and rows
//     4 (l / 16) .. +3 of column (l % 16) of the result.
#include "common.h"
#include "launch.h"

namespace w4 {

constexpr int kBK = 32;       // contraction per stage
constexpr int kLdsRow = 40;   // bf16 per LDS row (32 + 8 pad)

template <bool TRANS, int WM, int WN, int FM, int FN, int META>
__global__ __launch_bounds__(WM * WN * 64) void gemm_kernel(const uint16_t* __restrict__ A,
                                                            const int32_t* __restrict__ packed,
                                                            const uint16_t* __restrict__ scales,
                                                            const uint16_t* __restrict__ zeros,
                                                            const float* __restrict__ bias, float* __restrict__ Y,
                                                            int M, int N, int K, int g) {
  constexpr int T = WM * WN * 64;
  constexpr int BM = WM * FM * 16;
  constexpr int BN = WN * FN * 16;
  constexpr int A_UNITS = BM * 4 / T;  // 16-byte units of the activation tile per thread
  static_assert(A_UNITS >= 1 && BM * 4 % T == 0, "activation tile split");
  constexpr int W_PER_T = BN * 4 / T;  // packed words per thread per stage
  static_assert(W_PER_T >= 1 && W_PER_T <= 4 && BN * 4 % T == 0, "weight tile split");

  __shared__ __attribute__((aligned(16))) uint16_t As[2][BM * kLdsRow];
  __shared__ __attribute__((aligned(16))) uint16_t Bs[2][BN * kLdsRow];

  const int L = TRANS ? N : K;      // contraction length
  const int OUTC = TRANS ? K : N;   // output columns
  const int KW = K >> 3;            // packed words per weight row
  const int gpr = META == META_GROUP ? K / g : 1;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave / WN, wn = wave % WN;
  const int m0 = blockIdx.y * BM;
  const int c0 = blockIdx.x * BN;
  const int KT = (L + kBK - 1) / kBK;

  // ---- staging registers
  u32x4 areg[A_UNITS];
  uint32_t wreg[W_PER_T];
  uint16_t sreg[W_PER_T], zreg[W_PER_T];

  auto meta_index = [&](int n, int wcol) -> size_t {
    if constexpr (META == META_GLOBAL) return 0;
    else if constexpr (META == META_ROW) return (size_t)n;
    else return (size_t)n * gpr + (wcol * 8) / g;
  };

  auto load_stage = [&](int kt) {
    const int l0 = kt * kBK;
#pragma unroll
    for (int i = 0; i < A_UNITS; ++i) {
      const int u = tid + i * T;
      const int row = u >> 2, slot = u & 3;
      const int m = min(m0 + row, M - 1);
      const int l = l0 + slot * 8;
      if (l < L) {
        areg[i] = *reinterpret_cast<const u32x4*>(A + (size_t)m * L + l);
      } else {
        areg[i] = u32x4{0u, 0u, 0u, 0u};
      }
    }
    if constexpr (!TRANS) {
      // rows = output columns n, words along the contraction
      constexpr int TPR = 4 / W_PER_T;  // threads per row
      const int row = tid / TPR;
      const int w0 = (tid % TPR) * W_PER_T;
      const int n = min(c0 + row, N - 1);
      const int wc = (l0 >> 3) + w0;
      const int32_t* src = packed + (size_t)n * KW + wc;
      if constexpr (W_PER_T == 4) {
        const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(src));
        wreg[0] = v[0]; wreg[1] = v[1]; wreg[2] = v[2]; wreg[3] = v[3];
      } else if constexpr (W_PER_T == 2) {
        const u32x2 v = __builtin_nontemporal_load(reinterpret_cast<const u32x2*>(src));
        wreg[0] = v[0]; wreg[1] = v[1];
      } else {
        wreg[0] = (uint32_t)__builtin_nontemporal_load(src);
      }
#pragma unroll
      for (int i = 0; i < W_PER_T; ++i) {
        const size_t mi = meta_index(n, wc + i);
        sreg[i] = scales[mi];
        zreg[i] = zeros[mi];
      }
    } else {
      // rows = contraction n, words = output columns k (8 per word)
      constexpr int WCOLS = BN / 8;
      const int wc = tid % WCOLS;
      const int rb = tid / WCOLS;
      const int wcol = min((c0 >> 3) + wc, KW - 1);
#pragma unroll
      for (int i = 0; i < W_PER_T; ++i) {
        const int n = min(l0 + rb * W_PER_T + i, N - 1);
        wreg[i] = (uint32_t)__builtin_nontemporal_load(packed + (size_t)n * KW + wcol);
        const size_t mi = meta_index(n, wcol);
        sreg[i] = scales[mi];
        zreg[i] = zeros[mi];
      }
    }
  };

  auto store_stage = [&](int buf) {
    uint16_t* as = As[buf];
    uint16_t* bs = Bs[buf];
#pragma unroll
    for (int i = 0; i < A_UNITS; ++i) {
      const int u = tid + i * T;
      const int row = u >> 2, slot = u & 3;
      *reinterpret_cast<u32x4*>(as + row * kLdsRow + slot * 8) = areg[i];
    }
    if constexpr (!TRANS) {
      constexpr int TPR = 4 / W_PER_T;
      const int row = tid / TPR;
      const int w0 = (tid % TPR) * W_PER_T;
#pragma unroll
      for (int i = 0; i < W_PER_T; ++i) {
        const DqConst d = dq_const(sreg[i], zreg[i]);
        uint32_t o[4];
        dq_word_bf16(wreg[i], d, o);
        *reinterpret_cast<u32x4*>(bs + row * kLdsRow + (w0 + i) * 8) = u32x4{o[0], o[1], o[2], o[3]};
      }
    } else {
      constexpr int WCOLS = BN / 8;
      const int wc = tid % WCOLS;
      const int rb = tid / WCOLS;
      float v[W_PER_T][8];
#pragma unroll
      for (int i = 0; i < W_PER_T; ++i) dq_word_f32(wreg[i], dq_const(sreg[i], zreg[i]), v[i]);
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        uint16_t* dst = bs + (wc * 8 + j) * kLdsRow + rb * W_PER_T;
        if constexpr (W_PER_T == 4) {
          *reinterpret_cast<u32x2*>(dst) = u32x2{pack_bf16x2(v[0][j], v[1][j]), pack_bf16x2(v[2][j], v[3][j])};
        } else if constexpr (W_PER_T == 2) {
          *reinterpret_cast<uint32_t*>(dst) = pack_bf16x2(v[0][j], v[1][j]);
        } else {
          *dst = (uint16_t)(pack_bf16x2(v[0][j], 0.0f) & 0xFFFFu);
        }
      }
    }
  };

  f32x4 acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  load_stage(0);
  store_stage(0);
  __syncthreads();

  const int lr = lane & 15;        // operand row (A) / column (B)
  const int lk = (lane >> 4) * 8;  // contraction slot
  for (int kt = 0; kt < KT; ++kt) {
    const int buf = kt & 1;
    const bool more = kt + 1 < KT;
    if (more) load_stage(kt + 1);
    const uint16_t* as = As[buf] + (wm * FM * 16 + lr) * kLdsRow + lk;
    const uint16_t* bs = Bs[buf] + (wn * FN * 16 + lr) * kLdsRow + lk;
    bf16x8 af[FM], bfr[FN];
#pragma unroll
    for (int i = 0; i < FM; ++i) af[i] = *reinterpret_cast<const bf16x8*>(as + i * 16 * kLdsRow);
#pragma unroll
    for (int j = 0; j < FN; ++j) bfr[j] = *reinterpret_cast<const bf16x8*>(bs + j * 16 * kLdsRow);
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int j = 0; j < FN; ++j) acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[i], bfr[j], acc[i][j], 0, 0, 0);
    if (more) store_stage(buf ^ 1);
    __syncthreads();
  }

  // ---- epilogue: bias in fp32, masked fp32 stores
  const int rbase = m0 + wm * FM * 16 + (lane >> 4) * 4;
  const int cbase = c0 + wn * FN * 16 + lr;
#pragma unroll
  for (int j = 0; j < FN; ++j) {
    const int c = cbase + j * 16;
    if (c >= OUTC) continue;
    const float b = bias != nullptr ? bias[c] : 0.0f;
#pragma unroll
    for (int i = 0; i < FM; ++i) {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int m = rbase + i * 16 + r;
        if (m < M) Y[(size_t)m * OUTC + c] = acc[i][j][r] + b;
      }
    }
  }
}

// ---------------------------------------------------------------- host side

namespace {

struct Cfg {
  int wm, wn, fm, fn;
  const char* name_nt;
  const char* name_t;
};

constexpr Cfg kCfgs[] = {
    {2, 2, 8, 4, "gemm_nt_256x128", "gemm_t_256x128"},
    {1, 4, 8, 4, "gemm_nt_128x256", "gemm_t_128x256"},
    {2, 2, 4, 4, "gemm_nt_128x128", "gemm_t_128x128"},
};

int pick(const MmArgs& a) {
  const int64_t outc = a.transposed ? a.K : a.N;
  auto tiles = [&](const Cfg& c) {
    const int64_t bm = c.wm * c.fm * 16, bn = c.wn * c.fn * 16;
    return ((a.M + bm - 1) / bm) * ((outc + bn - 1) / bn);
  };
  if (a.M > 128 && tiles(kCfgs[0]) >= 256) return 0;
  if (tiles(kCfgs[1]) >= 256) return 1;
  return 2;
}

int meta_kind(int mode) { return mode == W4_MODE_GLOBAL ? META_GLOBAL : mode == W4_MODE_ROWWISE ? META_ROW : META_GROUP; }

template <bool TRANS, int WM, int WN, int FM, int FN, int META>
hipError_t run(const MmArgs& a, hipStream_t st) {
  constexpr int BM = WM * FM * 16, BN = WN * FN * 16;
  const int64_t outc = TRANS ? a.K : a.N;
  const dim3 grid((unsigned)((outc + BN - 1) / BN), (unsigned)((a.M + BM - 1) / BM));
  gemm_kernel<TRANS, WM, WN, FM, FN, META><<<grid, WM * WN * 64, 0, st>>>(a.A, a.packed, a.scales, a.zeros, a.bias,
                                                                          a.Y, (int)a.M, (int)a.N, (int)a.K, a.group);
  return hipGetLastError();
}

template <bool TRANS, int WM, int WN, int FM, int FN>
hipError_t run_meta(const MmArgs& a, hipStream_t st) {
  switch (meta_kind(a.mode)) {
    case META_GLOBAL: return run<TRANS, WM, WN, FM, FN, META_GLOBAL>(a, st);
    case META_ROW: return run<TRANS, WM, WN, FM, FN, META_ROW>(a, st);
    default: return run<TRANS, WM, WN, FM, FN, META_GROUP>(a, st);
  }
}

template <bool TRANS>
hipError_t run_cfg(const MmArgs& a, hipStream_t st) {
  switch (pick(a)) {
    case 0: return run_meta<TRANS, 2, 2, 8, 4>(a, st);
    case 1: return run_meta<TRANS, 1, 4, 8, 4>(a, st);
    default: return run_meta<TRANS, 2, 2, 4, 4>(a, st);
  }
}

}  // namespace

const char* gemm_name(const MmArgs& a) {
  const Cfg& c = kCfgs[pick(a)];
  return a.transposed ? c.name_t : c.name_nt;
}

size_t gemm_lds_bytes(const MmArgs& a) {
  const Cfg& c = kCfgs[pick(a)];
  return (size_t)2 * (c.wm * c.fm * 16 + c.wn * c.fn * 16) * kLdsRow * 2;
}

hipError_t launch_gemm(const MmArgs& a, hipStream_t st) {
  return a.transposed ? run_cfg<true>(a, st) : run_cfg<false>(a, st);
}

}  // namespace w4
