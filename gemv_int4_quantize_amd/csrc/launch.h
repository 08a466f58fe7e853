// Internal launchers of the W4A16 library (host side).  Arguments are validated
// by the C ABI layer before any of these is called.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "../../include/w4a16.h"

namespace w4 {

// intz: integer zero points (z = clamp(rint(-min / s), 0, 15), q = clamp(rint(w / s) + z, 0, 15))
hipError_t launch_quantize(const void* W, int dt, int64_t N, int64_t K, int mode, int g, int intz, int32_t* packed,
                           uint16_t* scales, uint16_t* zeros, void* ws, hipStream_t st);
size_t quantize_workspace_bytes(int mode);

hipError_t launch_dequantize(const int32_t* packed, const uint16_t* scales, const uint16_t* zeros, int64_t N,
                             int64_t K, int mode, int g, void* out, int out_dt, hipStream_t st);

// Output epilogue of a matmul (passed to the kernels by value): output column c of
// row m gets out_rne(acc + bias[c]) in dtype dt, stored in the segment s holding c at
// y[s] + m * ld[s] + (c - c0[s]).  The bias, when present, has the output dtype.
constexpr int kMaxSegs = 4;
struct Epi {
  const void* bias;             // nullptr or [outc] elements of dt
  int dt;                       // W4_DT_F32, W4_DT_F16 or W4_DT_BF16
  int nseg;                     // 1 .. kMaxSegs
  int64_t c0[kMaxSegs];         // first column of each segment (INT64_MAX past nseg)
  void* y[kMaxSegs];
  int64_t ld[kMaxSegs];         // row stride of each segment, in elements
};

// Matmul problem after validation: A [M][L] bf16 (L = contraction), packed [N][K/8].
struct MmArgs {
  const uint16_t* A;
  const int32_t* packed;
  const uint16_t* scales;
  const uint16_t* zeros;
  Epi ep;
  int64_t M, N, K;
  int mode;   // w4_mode
  int group;  // GROUPWISE g, else K
  bool transposed;
  bool a_f16;  // activations (and the weight operand) fp16 instead of bf16
};

// Properties of the current device that kernel plans depend on.
struct DeviceCaps {
  size_t lds;  // dynamic LDS bytes one workgroup may use
  int cus;     // compute units
};

// GEMV (M <= 4, non-transposed).  Returns false if this shape cannot run on it
// (LDS footprint), so the caller can fall back to the GEMM.
bool gemv_supported(const MmArgs& a, const DeviceCaps& caps);
const char* gemv_name(const MmArgs& a);
size_t gemv_lds_bytes(const MmArgs& a, const DeviceCaps& caps);
hipError_t launch_gemv(const MmArgs& a, const DeviceCaps& caps, hipStream_t st);

// GEMM: the workspace the split-K plan wants (0 if none), and for a launch given a
// workspace of ws_bytes (0: none) the plan it runs -- split only when ws_bytes holds the
// split plan's bytes: its kernel name (with a split-K or split-tail suffix), the LDS bytes
// of its tile and the workspace bytes it uses.  launch_gemm runs that same plan.
size_t gemm_workspace_bytes(const MmArgs& a, const DeviceCaps& caps);
const char* gemm_name(const MmArgs& a, const DeviceCaps& caps, size_t ws_bytes);
size_t gemm_lds_bytes(const MmArgs& a, const DeviceCaps& caps, size_t ws_bytes);
size_t gemm_used_workspace_bytes(const MmArgs& a, const DeviceCaps& caps, size_t ws_bytes);
hipError_t launch_gemm(const MmArgs& a, const DeviceCaps& caps, void* ws, size_t ws_bytes, hipStream_t st);

// The part of a GEMM one launch covers: output column tiles [ct0, ct0 + nct) (nct = 0:
// all of them from ct0 on), with the contraction cut into `splits` slices.  With
// splits > 1 each slice writes its fp32 partial sums to its own plane of the workspace,
// [M][pw] where pw is the number of covered columns (column ct0 * BN first), and a
// reduction finishes them through the output epilogue.
struct GemmPart {
  int splits = 1;
  int ct0 = 0, nct = 0;
};

// Non-transposed GEMM with the weight operand dequantized into MFMA registers
// (tile 0: 128 x 128, 1: 256 x 128, 2: 64 x 128, 3: 32 x 128).
bool gemm_nt_reg_supported(const MmArgs& a);
hipError_t launch_gemm_nt_reg(const MmArgs& a, int tile, const GemmPart& gp, float* part, hipStream_t st);

// Mid-M forward matmul (kSkinnyMinM <= M <= kSkinnyMaxM) on 16x16x32 MFMAs with the
// activations held in registers (skinny.hip).  A plan covers the rows in `blocks` blocks of
// `rpb` rows and the contraction in `splits` ranges of `units_per_split` 128-column units;
// with splits > 1 the sums go to [splits][M][N] fp32 planes and the split-K reduction
// finishes them.  ok = false: this problem does not fit the kernel (the GEMM tiles run).
constexpr int kSkinnyMinM = 5, kSkinnyMaxM = 32;
struct SkinnyPlan {
  bool ok = false;
  int MB = 1, UP = 1;  // 16-row blocks of X; 128-column units per wave
  int splits = 1, units_per_split = 0;
  int rpb = 0, blocks = 0;
  int log2gr = 0;  // the partial sums are reduced in rounds of 2^log2gr 16-row groups
  size_t lds = 0;
};
bool skinny_supported(const MmArgs& a);
SkinnyPlan skinny_plan(const MmArgs& a, const DeviceCaps& caps, bool allow_split);
size_t skinny_split_bytes(const MmArgs& a, const SkinnyPlan& p);
const char* skinny_name(const MmArgs& a, const SkinnyPlan& p);
hipError_t launch_skinny(const MmArgs& a, const SkinnyPlan& p, float* part, hipStream_t st);

// Output columns [c_lo, c_lo + pw) = epilogue(sum of `splits` fp32 [M][pw] planes, in a
// fixed order).
hipError_t launch_splitk_reduce(const float* part, int splits, int64_t M, int64_t c_lo, int64_t pw, const Epi& ep,
                                hipStream_t st);

}  // namespace w4
