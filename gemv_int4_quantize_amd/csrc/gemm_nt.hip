// Non-transposed MFMA W4A16 GEMM for gfx950 with the weight operand dequantized straight
// into MFMA registers:  Y[m][n] = sum_k X[m][k] * w[n][k] (+ bias[n]),
// w = bf16_rne((q - z) * s), bf16 MFMA operands, fp32 accumulation (or, with fp16
// activations, an fp16 weight operand and v_mfma_f32_32x32x16_f16).
// Sources: Objective 2 of "Quantized LLM Inference with Triton Kernels" (Y = X_bf16 @
// W_int4^T); "[Kernel] Adding bias epilogue support for cutlass_scaled_mm" (vLLM #5560).
//
// Why this shape on gfx950: the B operand of v_mfma_f32_32x32x16_bf16 is, per lane, eight
// consecutive contraction values of one output column -- exactly one packed int32 word of
// a weight row.  So each lane loads its own words (one dwordx4 = 32 contraction values of
// one row per 64-wide step) and dequantizes them into operand registers; the weights never
// pass through LDS.  Only the activation tile is staged in LDS (shared by the 4 waves).
//   * workgroup = NW (4 or 8) waves side by side along N; wave w owns output columns
//     [c0 + 32 FN w, +32 FN) and all BM = 32 FM rows of the tile.  Eight waves share one
//     activation tile across 256 columns: half the activation loads (and L2 reads) per
//     MFMA of four;
//   * within a 64-wide contraction step the contraction order is permuted: MFMA step kk,
//     operand slot 8 h + t (h = lane / 32) is contraction index k0 + 32 h + 8 kk + t, so a
//     lane's four words for the step are contiguous; the activation fragment is read from
//     LDS with the same mapping;
//   * activation tiles: global -> LDS with direct loads (buffer_load ... lds: no staging
//     registers, no LDS store instructions), two buffers, the next step's tile in flight
//     while a step computes; the 16-byte chunks of a 128-byte row are XOR-swizzled so the
//     32 rows a fragment read touches fall in distinct banks.  When K % 64 != 0 the tile
//     goes global -> VGPR -> LDS instead (rows padded by 16 bytes, loaded two steps
//     ahead), so the columns past K can be zeroed.  Weight words one step ahead; one
//     barrier per step;
//   * inside a step, the LDS fragments and the dequantized words of sub-step kk+1 are
//     produced while the MFMAs of kk issue;
//   * scale / zero: rowwise and global modes load them once; groupwise loads, once per
//     two steps, the 128 / g groups those steps cover with one wide load per array (when
//     K % 128 == 0, else one pair per step);
//   * dequantization: v_fma_mix_f32 on nibbles masked into fp16 halves, then
//     v_cvt_pk_bf16_f32 (17 VALU per word); with FM = 4 row blocks per wave that is about
//     4 VALU per MFMA, which the matrix core mostly overlaps;
//   * split-K: blockIdx.z takes a contiguous range of steps and writes fp32 partial sums
//     to its own plane; a separate kernel sums the planes in a fixed order.
#include <algorithm>

#include "common.h"
#include "epilogue.h"
#include "launch.h"

namespace w4 {

namespace {

typedef __amdgpu_buffer_rsrc_t rsrc_t;
typedef uint32_t u32x2v __attribute__((ext_vector_type(2)));
constexpr int kRsrcDword3 = 0x00020000;  // raw buffer, 32-bit data format (gfx9 class)

__device__ __forceinline__ rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, (int)bytes, kRsrcDword3);
}

constexpr int kBK = 64;   // contraction per step
constexpr int kLR = 72;   // LDS row: 64 bf16 + 8 padding

// META: 0 one (scale, zero) per row (rowwise / global), 1 groupwise with one wide load per
// two steps, 2 groupwise with one pair per step.  GPW: groups per 32-value lane chunk
// (2 when g = 16).  KTAIL: K % 64 != 0 (activation columns past K are zeroed in LDS).
// WB (META 1): bytes of one wide load, a compile-time width so that the loop holds exactly
// one load form; SPL (META 1): the contraction steps one wide load covers (2, or 4 / 8 when
// K allows: four or eight times fewer scale / zero loads).  One load holds the pairs of
// SPL * 64 / g consecutive groups, so g = 128 SPL / WB when a group is at most 64 SPL wide.
template <int FM, int FN, int GPW, int META, bool KTAIL, int WB, bool F16, bool DMA, int SPL, int NW>
__global__ __launch_bounds__(NW * 64, NW == 4 || FM < 8 ? 2 : 1) void gemm_nt_kernel(const uint16_t* __restrict__ A,
                                                         const int32_t* __restrict__ packed,
                                                         const uint16_t* __restrict__ scales,
                                                         const uint16_t* __restrict__ zeros,
                                                         const Epi ep,
                                                         int M, int N, int K, int meta_row, int log2g,
                                                         int kt_per_slice, int ct0, int pw,
                                                         float* __restrict__ part) {
  constexpr int BM = FM * 32, BN = NW * FN * 32;
  constexpr int NT = NW * 64;       // threads
  constexpr int AU = BM * 8 / NT;   // 16-byte activation units per thread per step
  static_assert(AU * NT == BM * 8, "whole activation units per thread");
  static_assert(!(DMA && KTAIL), "direct LDS loads cannot zero the columns past K");
  static_assert(SPL == 2 || (DMA && META == 1), "wide scale / zero loads over more than two steps: direct path");
  extern __shared__ __attribute__((aligned(16))) uint16_t smem[];
  uint16_t* As0 = smem;
  uint16_t* As1 = smem + BM * kLR;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int m0 = blockIdx.y * BM, c0 = (blockIdx.x + ct0) * BN;
  const int KT_ALL = (K + kBK - 1) / kBK;
  const int KB = blockIdx.z * kt_per_slice;  // first step of this slice (even)
  const int KT = min(KT_ALL - KB, kt_per_slice);
  const int KW = K >> 3;

  // Every load goes through a resource rebased at its contraction step (scalar arithmetic)
  // that holds what is left of its range, so a lane's offset stays fixed and no VALU goes
  // to addressing; the bounds are those of one resource over the whole range.
  // (sizes stay below 2^31; a signed max keeps the clamp on the scalar unit, where the
  // unsigned saturating form would move the descriptor into vector registers)
  auto at = [](const void* base, uint32_t bytes, uint32_t o) {
    return make_rsrc(static_cast<const char*>(base) + o, (uint32_t)max((int)bytes - (int)o, 0));
  };
  // activations: the tile's rows (rows past M read as zero)
  const void* a_base = A + (size_t)m0 * K;
  const uint32_t a_bytes = (uint32_t)(min(BM, M - m0) * K * 2);
  // DMA: LDS slot u (16 bytes) of a buffer holds row u / 8, chunk (u % 8) ^ ((u / 32) % 8)
  // of the tile: the XOR keeps the 32 rows of a fragment read in distinct 16-byte banks
  uint32_t a_off[AU];
#pragma unroll
  for (int i = 0; i < AU; ++i) {
    const int u = tid + i * NT;
    const int ch = DMA ? ((u & 7) ^ ((u >> 5) & 7)) : (u & 7);
    a_off[i] = (uint32_t)((u >> 3) * K * 2 + ch * 16);
  }
  // weights: this wave's 32 FN rows (rows past N read as zero)
  const int n0w = c0 + wave * FN * 32;
  const int rows_w = max(0, min(FN * 32, N - n0w));
  const int nb = min(n0w, N - 1);
  const void* b_base = packed + (size_t)nb * KW;
  const uint32_t b_bytes = (uint32_t)(rows_w * KW * 4);
  const uint32_t mbytes = meta_row > 0 ? (uint32_t)(rows_w * meta_row * 2) : (rows_w > 0 ? 2u : 0u);
  const void* s_base = scales + (size_t)nb * meta_row;
  const void* z_base = zeros + (size_t)nb * meta_row;
  const int h = lane >> 5, lr = lane & 31;
  uint32_t b_off[FN], mrow_off[FN], m_off[FN][GPW];
#pragma unroll
  for (int j = 0; j < FN; ++j) {
    b_off[j] = (uint32_t)((lr + j * 32) * KW * 4 + h * 16);
    mrow_off[j] = (uint32_t)((lr + j * 32) * meta_row * 2);
#pragma unroll
    for (int q = 0; q < GPW; ++q) m_off[j][q] = mrow_off[j] + (((uint32_t)(h * 32 + q * 16) >> log2g) * 2);
  }

  struct ARegs {
    u32x4 a[AU];
  };
  struct BRegs {
    u32x4 w[FN];
    uint32_t s[FN][GPW], z[FN][GPW];
  };
  struct MRegs {
    u32x4 s[FN], z[FN];
  };

  auto load_a = [&](int kt, ARegs& R) {
#pragma unroll
    for (int i = 0; i < AU; ++i)
      R.a[i] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(at(a_base, a_bytes, kt * kBK * 2),
                                                                               a_off[i], 0, 0));
  };
  auto load_b = [&](int kt, BRegs& R) {
    const uint32_t mk = ((uint32_t)(kt * kBK) >> log2g) * 2;
    const rsrc_t br = at(b_base, b_bytes, kt * 32);
#pragma unroll
    for (int j = 0; j < FN; ++j) {
      R.w[j] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(br, b_off[j], 0, 0));
      if constexpr (META == 2) {
        const rsrc_t sr = at(s_base, mbytes, mk), zr = at(z_base, mbytes, mk);
#pragma unroll
        for (int q = 0; q < GPW; ++q) {
          R.s[j][q] = __builtin_amdgcn_raw_buffer_load_b16(sr, m_off[j][q], 0, 0);
          R.z[j][q] = __builtin_amdgcn_raw_buffer_load_b16(zr, m_off[j][q], 0, 0);
        }
      }
    }
  };
  // groups of steps kt, kt + 1 (kt even): 128 / g consecutive pairs, aligned because
  // K % 128 == 0 makes every row's group count a multiple of 128 / g
  auto load_m = [&](int kt, MRegs& R) {
    const uint32_t mk = ((uint32_t)(kt * kBK) >> log2g) * 2;
    const rsrc_t sr = at(s_base, mbytes, mk), zr = at(z_base, mbytes, mk);
#pragma unroll
    for (int j = 0; j < FN; ++j) {
      const uint32_t o = mrow_off[j];
      if constexpr (WB == 16) {
        R.s[j] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(sr, o, 0, 0));
        R.z[j] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(zr, o, 0, 0));
      } else if constexpr (WB == 8) {
        const u32x2v a = __builtin_bit_cast(u32x2v, __builtin_amdgcn_raw_buffer_load_b64(sr, o, 0, 0));
        const u32x2v b = __builtin_bit_cast(u32x2v, __builtin_amdgcn_raw_buffer_load_b64(zr, o, 0, 0));
        R.s[j] = u32x4{a[0], a[1], 0u, 0u};
        R.z[j] = u32x4{b[0], b[1], 0u, 0u};
      } else if constexpr (WB == 4) {
        R.s[j] = u32x4{__builtin_amdgcn_raw_buffer_load_b32(sr, o, 0, 0), 0u, 0u, 0u};
        R.z[j] = u32x4{__builtin_amdgcn_raw_buffer_load_b32(zr, o, 0, 0), 0u, 0u, 0u};
      } else {
        R.s[j] = u32x4{(uint32_t)__builtin_amdgcn_raw_buffer_load_b16(sr, o, 0, 0), 0u, 0u, 0u};
        R.z[j] = u32x4{(uint32_t)__builtin_amdgcn_raw_buffer_load_b16(zr, o, 0, 0), 0u, 0u, 0u};
      }
    }
  };
  auto half_of = [&](const u32x4& v, int e) -> uint16_t { return (uint16_t)(v[e >> 1] >> ((e & 1) * 16)); };
  auto store_a = [&](int kt, const ARegs& R, uint16_t* buf) {
#pragma unroll
    for (int i = 0; i < AU; ++i) {
      const int u = tid + i * NT;
      u32x4 v = R.a[i];
      // past K the weight words are another row's (finite) codes: the activations must be 0
      if constexpr (KTAIL) {
        if (kt * kBK + (u & 7) * 8 >= K) v = u32x4{0u, 0u, 0u, 0u};
      }
      *reinterpret_cast<u32x4*>(buf + (u >> 3) * kLR + (u & 7) * 8) = v;
    }
  };

  f32x16 acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

  auto dequant = [&](const BRegs& B, const DqConst (&dc)[FN][GPW], int kk, u32x4 (&bfr)[FN]) {
#pragma unroll
    for (int j = 0; j < FN; ++j) {
      uint32_t o[4];
      dq_word_op<F16>(B.w[j][kk], dc[j][GPW == 2 ? kk / 2 : 0], o);
      bfr[j] = u32x4{o[0], o[1], o[2], o[3]};
    }
  };
  auto read_a = [&](const uint16_t* buf, int kk, u32x4 (&af)[FM]) {
    if constexpr (DMA) {
      // row i 32 + lr, chunk (4 h + kk) ^ ((lr / 4) % 8) of a 128-byte row
      const char* as = reinterpret_cast<const char*>(buf) + lr * 128 + (((4 * h + kk) ^ ((lr >> 2) & 7)) << 4);
#pragma unroll
      for (int i = 0; i < FM; ++i) af[i] = *reinterpret_cast<const u32x4*>(as + i * 32 * 128);
    } else {
      const uint16_t* as = buf + lr * kLR + h * 32 + kk * 8;
#pragma unroll
      for (int i = 0; i < FM; ++i) af[i] = *reinterpret_cast<const u32x4*>(as + i * 32 * kLR);
    }
  };
  auto compute = [&](const BRegs& B, const DqConst (&dc)[FN][GPW], const uint16_t* buf) {
    u32x4 af[2][FM], bfr[2][FN];
    read_a(buf, 0, af[0]);
    dequant(B, dc, 0, bfr[0]);
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      const int c = kk & 1;
      if (kk < 3) {
        read_a(buf, kk + 1, af[c ^ 1]);
        dequant(B, dc, kk + 1, bfr[c ^ 1]);
      }
#pragma unroll
      for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j)
          acc[i][j] = mfma_op<F16>(af[c][i], bfr[c][j], acc[i][j]);
    }
  };
  // dequantization constants of step p of a wide load's SPL steps: this lane's 16 values
  // (q-th group of them when g = 16) start at column 64 p + 32 h + 16 q of the block, in
  // group (64 p + 32 h + 16 q) / GW with GW = 128 SPL / WB (g, or 128 for any g >= 128
  // at SPL = 2, where one pair covers both steps)
  auto dc_wide = [&](const MRegs& R, int p, DqConst (&dc)[FN][GPW]) {
    constexpr int GW = WB > 0 ? 128 * SPL / WB : 1;
#pragma unroll
    for (int j = 0; j < FN; ++j)
#pragma unroll
      for (int q = 0; q < GPW; ++q) {
        const int e = (64 * p + 32 * h + 16 * q) / GW;
        dc[j][q] = dq_const_mix(half_of(R.s[j], e), half_of(R.z[j], e));
      }
  };
  auto dc_step = [&](const BRegs& B, DqConst (&dc)[FN][GPW]) {
#pragma unroll
    for (int j = 0; j < FN; ++j)
#pragma unroll
      for (int q = 0; q < GPW; ++q) dc[j][q] = dq_const_mix((uint16_t)B.s[j][q], (uint16_t)B.z[j][q]);
  };

  ARegs A0, A1;
  BRegs B0, B1;
  MRegs MM;
  DqConst dcA[FN][GPW], dcB[FN][GPW];
  if constexpr (META == 0) {
#pragma unroll
    for (int j = 0; j < FN; ++j) {
      const uint16_t sv = __builtin_amdgcn_raw_buffer_load_b16(at(s_base, mbytes, 0), mrow_off[j], 0, 0);
      const uint16_t zv = __builtin_amdgcn_raw_buffer_load_b16(at(z_base, mbytes, 0), mrow_off[j], 0, 0);
      dcA[j][0] = dq_const_mix(sv, zv);
      dcB[j][0] = dcA[j][0];
    }
  }
  // steps KB + t; loads past the slice read other (finite) data or zeros and are never used
  if constexpr (DMA) {
    // Activation tiles go global -> LDS directly (buffer_load ... lds, no registers, no LDS
    // store instructions) into two buffers: the tile of step t + 1 is loaded while step t
    // computes.  Each step issues its weight (and scale / zero) loads, then the tile loads.
    constexpr int BUFB = BM * 128;  // bytes per buffer
    typedef __attribute__((address_space(3))) void lds_void;
    char* lds = reinterpret_cast<char*>(smem);
    auto dma = [&](int kt, int buf) {
      const rsrc_t ar = at(a_base, a_bytes, kt * kBK * 2);
#pragma unroll
      for (int i = 0; i < AU; ++i)
        // the lane's offset in the range-checked vector offset (the step's start is in the
        // resource base): reads past the tile's rows (steps past the slice, rows past M)
        // return zeros.  The explicit int matters: with an unsigned argument the host pass
        // silently drops the kernel's launch stub.
        __builtin_amdgcn_raw_ptr_buffer_load_lds(ar, (lds_void*)(lds + buf * BUFB + (i * NT + wave * 64) * 16), 16,
                                                 (int)a_off[i], 0, 0, 0);
    };
    // Barrier once every load of this wave has landed (s_waitcnt vmcnt(0) lgkmcnt(0)).  The compiler
    // does not track which LDS bytes a direct load writes, so this wait is explicit, and
    // the barrier carries no fence.  Every LDS read of the step has fed its MFMA by then;
    // the clobbers keep memory accesses, and the scheduling barriers keep all instructions,
    // on their side of the barrier.
    auto sync = [&]() {
      __builtin_amdgcn_sched_barrier(0);
      asm volatile("" ::: "memory");
      __builtin_amdgcn_s_waitcnt(0x0070);  // vmcnt(0) lgkmcnt(0)
      __builtin_amdgcn_s_barrier();
      asm volatile("" ::: "memory");
      __builtin_amdgcn_sched_barrier(0);
    };
    load_b(KB, B0);
    if constexpr (META == 1) load_m(KB, MM);
    __builtin_amdgcn_sched_barrier(0);
    dma(KB, 0);
    sync();
    // step kt = KB + t + p (p-th of a block of SPL steps): loads of step kt + 1, then the
    // products of step kt from LDS buffer p % 2 and weight registers Bc.  A wave raises its
    // priority for its dequantization and MFMAs so the matrix pipe of a SIMD shared by two
    // waves stays fed (measured: forward QLoRA pair +0.8%)
    auto step = [&](BRegs& Bc, BRegs& Bn, int p, int kt) {
      load_b(kt + 1, Bn);
      __builtin_amdgcn_sched_barrier(0);
      dma(kt + 1, (p + 1) & 1);
      __builtin_amdgcn_sched_barrier(0);
      const uint16_t* buf = reinterpret_cast<const uint16_t*>(lds + (p & 1) * BUFB);
      if constexpr (META == 0) {
        __builtin_amdgcn_s_setprio(1);
        compute(Bc, dcA, buf);
        __builtin_amdgcn_s_setprio(0);
      } else {
        DqConst dc[FN][GPW];
        if constexpr (META == 1) {
          dc_wide(MM, p, dc);
          if (p == SPL - 1) load_m(kt + 1, MM);  // the next block's pairs, once these are read
        } else {
          dc_step(Bc, dc);
        }
        __builtin_amdgcn_s_setprio(1);
        compute(Bc, dc, buf);
        __builtin_amdgcn_s_setprio(0);
      }
      sync();
    };
    if constexpr (SPL > 2) {
      // blocks of SPL steps start on multiples of SPL (slices too, and K is a multiple of
      // SPL steps), so step parity picks the buffers
      for (int t = 0; t < KT; t += SPL) {
#pragma unroll
        for (int p = 0; p < SPL; ++p) {
          if (p & 1) step(B1, B0, p, KB + t + p);
          else step(B0, B1, p, KB + t + p);
        }
      }
    } else {
      // two steps per iteration and a peeled last step (measured faster than the block form
      // for rowwise and g = 16)
      int t = 0;
      for (; t + 2 <= KT; t += 2) {
        const int kt = KB + t;
        load_b(kt + 1, B1);
        __builtin_amdgcn_sched_barrier(0);
        dma(kt + 1, 1);
        __builtin_amdgcn_sched_barrier(0);
        if constexpr (META == 1) {
          dc_wide(MM, 0, dcA);
          dc_wide(MM, 1, dcB);
        } else if constexpr (META == 2) {
          dc_step(B0, dcA);
        }
        __builtin_amdgcn_s_setprio(1);
        compute(B0, dcA, reinterpret_cast<const uint16_t*>(lds));
        __builtin_amdgcn_s_setprio(0);
        sync();
        load_b(kt + 2, B0);
        if constexpr (META == 1) load_m(kt + 2, MM);
        __builtin_amdgcn_sched_barrier(0);
        dma(kt + 2, 0);
        __builtin_amdgcn_sched_barrier(0);
        if constexpr (META == 2) dc_step(B1, dcB);
        __builtin_amdgcn_s_setprio(1);
        compute(B1, dcB, reinterpret_cast<const uint16_t*>(lds + BUFB));
        __builtin_amdgcn_s_setprio(0);
        sync();
      }
      if (t < KT) {
        if constexpr (META == 1) dc_wide(MM, 0, dcA);
        else if constexpr (META == 2) dc_step(B0, dcA);
        compute(B0, dcA, reinterpret_cast<const uint16_t*>(lds));
      }
    }
  } else {
  load_b(KB, B0);
  if constexpr (META == 1) load_m(KB, MM);
  load_a(KB, A0);
  load_a(KB + min(1, KT - 1), A1);
  store_a(KB, A0, As0);
  __syncthreads();
  int t = 0;
  for (; t + 2 <= KT; t += 2) {
    const int kt = KB + t;
    load_b(kt + 1, B1);
    load_a(kt + 2, A0);
    store_a(kt + 1, A1, As1);
    if constexpr (META == 1) {
      dc_wide(MM, 0, dcA);
      dc_wide(MM, 1, dcB);
    } else if constexpr (META == 2) {
      dc_step(B0, dcA);
    }
    compute(B0, dcA, As0);
    __syncthreads();
    load_b(kt + 2, B0);
    if constexpr (META == 1) load_m(kt + 2, MM);
    load_a(kt + 3, A1);
    store_a(kt + 2, A0, As0);
    if constexpr (META == 2) dc_step(B1, dcB);
    compute(B1, dcB, As1);
    __syncthreads();
  }
  if (t < KT) {
    if constexpr (META == 1) dc_wide(MM, 0, dcA);
    else if constexpr (META == 2) dc_step(B0, dcA);
    compute(B0, dcA, As0);
  }
  }

  // epilogue: result register r of a 32x32 block is row 8 (r / 4) + 4 h + (r % 4), column
  // lr; a split-K slice writes its partial sums (no bias, fp32) to its own [M][pw] plane,
  // an unsplit launch stores through the output epilogue (four columns per store for a
  // plain one-segment output)
  const int rbase = m0 + h * 4;
  if (part == nullptr && epi_wide(ep, N) != 0) {
#pragma unroll
    for (int j = 0; j < FN; ++j) {
      const EpiQuad q = epi_quad(ep, n0w + j * 32 + (lr & ~3), N);
#pragma unroll
      for (int i = 0; i < FM; ++i) epi_put_block_wide(q, acc[i][j], rbase + i * 32, M, lane);
    }
    return;
  }
#pragma unroll
  for (int j = 0; j < FN; ++j) {
    const int c = n0w + j * 32 + lr;
    if (c >= N) continue;
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

template <int FM, int FN, int NW, int GPW, int META, bool KTAIL, int WB, bool F16, bool DMA, int SPL = 2>
hipError_t launch_cfg(const MmArgs& a, const GemmPart& gp, float* part, hipStream_t st) {
  auto k = gemm_nt_kernel<FM, FN, GPW, META, KTAIL, WB, F16, DMA, SPL, NW>;
  constexpr int BM = FM * 32, BN = NW * FN * 32;
  const int lds = DMA ? 2 * BM * 128 : 2 * BM * kLR * 2;
  if (lds > 64 * 1024) {
    const hipError_t e = hipFuncSetAttribute((const void*)k, hipFuncAttributeMaxDynamicSharedMemorySize, lds);
    if (e != hipSuccess) return e;
  }
  const int kt_all = (int)((a.K + kBK - 1) / kBK);
  int splits = gp.splits;
  int kts = (kt_all + splits - 1) / splits;
  kts = (kts + SPL - 1) / SPL * SPL;  // slices start on whole wide scale / zero loads
  splits = (kt_all + kts - 1) / kts;  // every slice gets at least one step
  const int meta_row = a.mode == W4_MODE_GLOBAL ? 0 : a.mode == W4_MODE_ROWWISE ? 1 : (int)(a.K / a.group);
  const int log2g = a.mode == W4_MODE_GROUPWISE ? 31 - __builtin_clz((unsigned)a.group) : 31;
  const int tn_all = (int)((a.N + BN - 1) / BN);
  const int nct = gp.nct > 0 ? gp.nct : tn_all - gp.ct0;
  const int64_t c_lo = (int64_t)gp.ct0 * BN;
  const int pw = (int)(std::min<int64_t>(a.N, c_lo + (int64_t)nct * BN) - c_lo);
  const dim3 grid((unsigned)nct, (unsigned)((a.M + BM - 1) / BM), (unsigned)splits);
  k<<<grid, NW * 64, lds, st>>>(a.A, a.packed, a.scales, a.zeros, a.ep, (int)a.M, (int)a.N, (int)a.K, meta_row,
                            log2g, kts, gp.ct0, pw, splits > 1 ? part : nullptr);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess || splits == 1) return e;
  return launch_splitk_reduce(part, splits, a.M, c_lo, pw, a.ep, st);
}

template <int FM, int FN, int NW, bool KTAIL, bool F16, bool DMA>
hipError_t launch_meta(const MmArgs& a, const GemmPart& gp, float* part, hipStream_t st) {
  if (a.mode != W4_MODE_GROUPWISE) return launch_cfg<FM, FN, NW, 1, 0, KTAIL, 0, F16, DMA>(a, gp, part, st);
  const bool g16 = a.group == 16;
  if (a.K % 128 == 0) {
    // direct path: one 16- or 8-byte load covering 4 or 8 steps where K allows
    switch (a.group) {
      case 16: return launch_cfg<FM, FN, NW, 2, 1, KTAIL, 16, F16, DMA>(a, gp, part, st);
      case 32:
        if constexpr (DMA)
          if (a.K % 256 == 0) return launch_cfg<FM, FN, NW, 1, 1, KTAIL, 16, F16, DMA, 4>(a, gp, part, st);
        return launch_cfg<FM, FN, NW, 1, 1, KTAIL, 8, F16, DMA>(a, gp, part, st);
      case 64:
        if constexpr (DMA) {
          if (a.K % 512 == 0) return launch_cfg<FM, FN, NW, 1, 1, KTAIL, 16, F16, DMA, 8>(a, gp, part, st);
          if (a.K % 256 == 0) return launch_cfg<FM, FN, NW, 1, 1, KTAIL, 8, F16, DMA, 4>(a, gp, part, st);
        }
        return launch_cfg<FM, FN, NW, 1, 1, KTAIL, 4, F16, DMA>(a, gp, part, st);
      case 128:
        if constexpr (DMA)
          if (a.K % 512 == 0) return launch_cfg<FM, FN, NW, 1, 1, KTAIL, 8, F16, DMA, 8>(a, gp, part, st);
        return launch_cfg<FM, FN, NW, 1, 1, KTAIL, 2, F16, DMA>(a, gp, part, st);
      default: return launch_cfg<FM, FN, NW, 1, 1, KTAIL, 2, F16, DMA>(a, gp, part, st);
    }
  }
  return g16 ? launch_cfg<FM, FN, NW, 2, 2, KTAIL, 0, F16, DMA>(a, gp, part, st)
             : launch_cfg<FM, FN, NW, 1, 2, KTAIL, 0, F16, DMA>(a, gp, part, st);
}

template <int FM, int FN, int NW>
hipError_t launch_tile(const MmArgs& a, const GemmPart& gp, float* part, hipStream_t st) {
  // K % 64 == 0: direct LDS loads of the activation tile; otherwise the register path,
  // which zeroes the activation columns past K
  if (a.K % kBK != 0)
    return a.a_f16 ? launch_meta<FM, FN, NW, true, true, false>(a, gp, part, st)
                   : launch_meta<FM, FN, NW, true, false, false>(a, gp, part, st);
  return a.a_f16 ? launch_meta<FM, FN, NW, false, true, true>(a, gp, part, st)
                 : launch_meta<FM, FN, NW, false, false, true>(a, gp, part, st);
}

}  // namespace

bool gemm_nt_reg_supported(const MmArgs& a) {
  // 32-bit buffer offsets: a 256-row activation tile must stay below 2 GiB
  return !a.transposed && a.K <= ((int64_t)1 << 21);
}

hipError_t launch_gemm_nt_reg(const MmArgs& a, int tile, const GemmPart& gp, float* part, hipStream_t st) {
  switch (tile) {
    case 0: return launch_tile<4, 1, 4>(a, gp, part, st);  // 128 x 128
    case 1: return launch_tile<8, 1, 4>(a, gp, part, st);  // 256 x 128
    case 2: return launch_tile<2, 1, 4>(a, gp, part, st);  // 64 x 128
    case 4: return launch_tile<8, 1, 8>(a, gp, part, st);  // 256 x 256, eight waves
    case 5: return launch_tile<4, 1, 8>(a, gp, part, st);  // 128 x 256, eight waves
    default: return launch_tile<1, 1, 4>(a, gp, part, st);  // 32 x 128
  }
}

}  // namespace w4
