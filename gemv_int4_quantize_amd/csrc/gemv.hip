// Batched decode GEMV, M <= 4, non-transposed:  Y[m][n] = sum_k X[m][k] * w[n][k] (+ bias[n]),
// w = bf16_rne((q - z) * s), fp32 accumulation.
//
// Design ("Modify small-batched weight only quantization", TensorRT-LLM #2213, names
// load stalls and duplicate scale / zero requests as the costs of this kernel; here
// on gfx950 with no matrix cores):
//   * each wave owns R rows over the full K (split-K inside the wave, no partial
//     results leave the wave); lane l streams 16-byte chunks c = l, l+64, ... of
//     every row (32 codes each), so one wave-wide load is 1 KB contiguous;
//   * X streams through two LDS windows of 2048 columns ([m][word][chunk], so that
//     consecutive lanes read consecutive 16-byte slots, free of bank conflicts); the
//     block refills one window while it computes on the other, so the LDS footprint
//     (8 KB per activation row) does not grow with K;
//   * the scale / zero bits of a chunk's group are loaded with the chunk, one
//     iteration ahead (the lanes that share a group issue the same address inside one
//     wave-wide load, which the memory pipeline merges into one request);
//   * dequantization is v_fma_mix_f32 on nibbles masked into fp16 halves, bf16
//     rounding by v_cvt_pk_bf16_f32, products by v_dot2_f32_bf16;
//   * the R*M partial sums of a wave are reduced with a transposing butterfly, so
//     every shuffle step halves the number of live values.
#include "common.h"
#include "launch.h"


namespace w4 {

// Lane l ends up holding the wave-wide sum of value (l >> (6 - log2 V)).
template <int V>
__device__ __forceinline__ float transpose_reduce(float (&v)[V], int lane) {
  int n = V;
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) {
    if (n > 1) {
      const int half = n / 2;
      const bool upper = (lane & o) != 0;
#pragma unroll
      for (int i = 0; i < V / 2; ++i) {
        if (i < half) {
          const float send = upper ? v[i] : v[i + half];
          const float keep = upper ? v[i + half] : v[i];
          v[i] = keep + __shfl_xor(send, o);
        }
      }
      n = half;
    } else {
      v[0] += __shfl_xor(v[0], o);
    }
  }
  return v[0];
}

// Per-lane state of one pipeline stage: the 16-byte chunk of every row and the
// raw fp16 scale / zero bits of the group(s) it belongs to (GPC groups per chunk).
template <int R, int GPC>
struct Stage {
  u32x4 w[R];
  uint16_t s[R][GPC], z[R][GPC];  // kept 16-bit: v_fma_mix_f32 reads the low half as fp16
};

template <int M, int R, int META, int WAVES, int GPC>
__global__ __launch_bounds__(WAVES * 64) void gemv_kernel(const uint16_t* __restrict__ X,
                                                          const int32_t* __restrict__ packed,
                                                          const uint16_t* __restrict__ scales,
                                                          const uint16_t* __restrict__ zeros,
                                                          const float* __restrict__ bias, float* __restrict__ Y,
                                                          int N, int K, int log2g) {
  // Two LDS windows of X, each [m][word][chunk] over the 2048 columns of one iteration:
  // the block refills one window while it computes on the other.
  __shared__ u32x4 xwin[2][M * 4 * 64];
  constexpr int T = WAVES * 64;
  constexpr int XUNITS = M * 4 * 64;  // 16-byte units per window
  const int KS = K >> 5;              // 16-byte chunks (32 codes) per row
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  // the wave index is uniform: keep every row-dependent value in scalar registers
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int row0 = (blockIdx.x * WAVES + wave) * R;
  const int iters = (KS + 63) >> 6;
  const int gpr = META == META_GROUP ? K >> log2g : 1;
  const int KW = K >> 3;

  const u32x4* prow[R];
  const uint16_t* srow[R];
  const uint16_t* zrow[R];
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const int n = min(row0 + r, N - 1);
    prow[r] = reinterpret_cast<const u32x4*>(packed + (size_t)n * KW);
    srow[r] = scales + (size_t)n * gpr;
    zrow[r] = zeros + (size_t)n * gpr;
  }

  // X units this thread moves into a window: unit u = (m * 64 + chunk) * 4 + word
  constexpr int XPT = (XUNITS + T - 1) / T;
  u32x4 xr[XPT];
  auto xload = [&](int it) {
#pragma unroll
    for (int i = 0; i < XPT; ++i) {
      const int u = tid + i * T;
      if (u < XUNITS) {
        const int m = u >> 8, c = ((u >> 2) & 63) + it * 64, w = u & 3;
        xr[i] = c < KS ? *reinterpret_cast<const u32x4*>(X + (size_t)m * K + c * 32 + w * 8) : u32x4{0, 0, 0, 0};
      }
    }
  };
  auto xstore = [&](int buf) {
#pragma unroll
    for (int i = 0; i < XPT; ++i) {
      const int u = tid + i * T;
      if (u < XUNITS) {
        const int m = u >> 8, c = (u >> 2) & 63, w = u & 3;
        xwin[buf][(m * 4 + w) * 64 + c] = xr[i];
      }
    }
  };

  // weight stage of iteration `it`: one chunk per row and its scale / zero bits
  auto load = [&](int it, Stage<R, GPC>& st) {
    const int c = min(it * 64 + lane, KS - 1);
#pragma unroll
    for (int r = 0; r < R; ++r) st.w[r] = __builtin_nontemporal_load(prow[r] + c);
    if constexpr (META == META_GROUP) {
#pragma unroll
      for (int q = 0; q < GPC; ++q) {
        const int G = (c * 32 + q * 16) >> log2g;
#pragma unroll
        for (int r = 0; r < R; ++r) {
          st.s[r][q] = srow[r][G];
          st.z[r][q] = zrow[r][G];
        }
      }
    }
  };

  float acc[R][M];
#pragma unroll
  for (int r = 0; r < R; ++r)
#pragma unroll
    for (int m = 0; m < M; ++m) acc[r][m] = 0.0f;

  DqConst rc[R];
  auto compute = [&](int it, const Stage<R, GPC>& st, int buf) {
    if (it * 64 + lane >= KS) return;
    DqConst dc[R][GPC];
    if constexpr (META == META_GROUP) {
#pragma unroll
      for (int r = 0; r < R; ++r)
#pragma unroll
        for (int q = 0; q < GPC; ++q) dc[r][q] = dq_const_mix(st.s[r][q], st.z[r][q]);
    }
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      u32x4 xv[M];
#pragma unroll
      for (int m = 0; m < M; ++m) xv[m] = xwin[buf][(m * 4 + w) * 64 + lane];
#pragma unroll
      for (int r = 0; r < R; ++r) {
        uint32_t bw[4];
        if constexpr (META == META_GROUP)
          dq_word_bf16(st.w[r][w], dc[r][GPC == 2 ? w / 2 : 0], bw);
        else
          dq_word_bf16(st.w[r][w], rc[r], bw);
#pragma unroll
        for (int m = 0; m < M; ++m)
#pragma unroll
          for (int i = 0; i < 4; ++i) acc[r][m] = dot2_bf16(bw[i], xv[m][i], acc[r][m]);
      }
    }
  };

  Stage<R, GPC> A, B;
  xload(0);
  load(0, A);
  if constexpr (META != META_GROUP) {
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const int mi = META == META_GLOBAL ? 0 : min(row0 + r, N - 1);
      rc[r] = dq_const_mix(scales[mi], zeros[mi]);
    }
  }
  xstore(0);
  __syncthreads();

  // Two register stages, unrolled by two so the in-flight stage is never copied.  The
  // next X window is requested before the next weight stage, so storing it to LDS never
  // waits for the weights; the loop body issues exactly one weight stage while consuming
  // the other (no conditional loads), and the tail is peeled.
  int it = 0;
  for (; it + 2 < iters; it += 2) {
    xload(it + 1);
    load(it + 1, B);
    compute(it, A, 0);
    xstore(1);
    __syncthreads();
    xload(it + 2);
    load(it + 2, A);
    compute(it + 1, B, 1);
    xstore(0);
    __syncthreads();
  }
  if (it + 1 < iters) {
    xload(it + 1);
    load(it + 1, B);
    compute(it, A, 0);
    xstore(1);
    __syncthreads();
    compute(it + 1, B, 1);
  } else {
    compute(it, A, 0);
  }

  // reduce R x MP partial sums across the wave (MP = M padded to a power of two)
  constexpr int MP = M == 3 ? 4 : M;
  constexpr int V = R * MP;
  float v[V];
#pragma unroll
  for (int r = 0; r < R; ++r)
#pragma unroll
    for (int m = 0; m < MP; ++m) v[r * MP + m] = m < M ? acc[r][m] : 0.0f;
  constexpr int LOGV = V == 1 ? 0 : V == 2 ? 1 : V == 4 ? 2 : V == 8 ? 3 : V == 16 ? 4 : 5;
  const float sum = transpose_reduce<V>(v, lane);
  constexpr int SPAN = 64 / V;
  if ((lane & (SPAN - 1)) == 0) {
    const int idx = lane >> (6 - LOGV);
    const int r = idx / MP, m = idx - (idx / MP) * MP;
    const int n = row0 + r;
    if (m < M && n < N) Y[(size_t)m * N + n] = sum + (bias != nullptr ? bias[n] : 0.0f);
  }
}

// ---------------------------------------------------------------- host side

namespace {

struct GemvPlan {
  int R, waves;
  size_t lds;
};

int meta_kind(int mode) { return mode == W4_MODE_GLOBAL ? META_GLOBAL : mode == W4_MODE_ROWWISE ? META_ROW : META_GROUP; }

GemvPlan plan(const MmArgs& a) {
  // rows per wave and waves per block: keep >= 256 blocks (one per CU) in flight
  GemvPlan p;
  p.waves = 8;
  p.R = a.N >= 16 * 512 ? 2 : 1;
  if (a.N < 8 * 256) p.waves = 4;
  p.lds = (size_t)2 * a.M * 4 * 64 * 16;
  return p;
}

template <int M, int R, int META, int WAVES>
hipError_t run(const MmArgs& a, const GemvPlan& p, hipStream_t st) {
  auto k = (META == META_GROUP && a.group == 16) ? gemv_kernel<M, R, META, WAVES, 2> : gemv_kernel<M, R, META, WAVES, 1>;
  const int rows_per_block = R * WAVES;
  const dim3 grid((unsigned)((a.N + rows_per_block - 1) / rows_per_block));
  const int log2g = 31 - __builtin_clz((unsigned)a.group);  // GROUPWISE g is a power of two
  k<<<grid, WAVES * 64, 0, st>>>(a.A, a.packed, a.scales, a.zeros, a.bias, a.Y, (int)a.N, (int)a.K, log2g);
  return hipGetLastError();
}

template <int M, int R, int META>
hipError_t run_w(const MmArgs& a, const GemvPlan& p, hipStream_t st) {
  return p.waves == 4 ? run<M, R, META, 4>(a, p, st) : run<M, R, META, 8>(a, p, st);
}

template <int M, int META>
hipError_t run_r(const MmArgs& a, const GemvPlan& p, hipStream_t st) {
  return p.R == 2 ? run_w<M, 2, META>(a, p, st) : run_w<M, 1, META>(a, p, st);
}

template <int M>
hipError_t run_meta(const MmArgs& a, const GemvPlan& p, hipStream_t st) {
  switch (meta_kind(a.mode)) {
    case META_GLOBAL: return run_r<M, META_GLOBAL>(a, p, st);
    case META_ROW: return run_r<M, META_ROW>(a, p, st);
    default: return run_r<M, META_GROUP>(a, p, st);
  }
}

}  // namespace

bool gemv_supported(const MmArgs& a, size_t lds_limit) {
  if (a.transposed || a.M < 1 || a.M > 4) return false;
  if (a.N > (int64_t)1 << 30 || a.K > (int64_t)1 << 30) return false;
  return plan(a).lds <= lds_limit;
}

const char* gemv_name(const MmArgs& a) {
  static const char* names[] = {"gemv_m1", "gemv_m2", "gemv_m3", "gemv_m4"};
  return names[a.M - 1];
}

hipError_t launch_gemv(const MmArgs& a, hipStream_t st) {
  const GemvPlan p = plan(a);
  switch (a.M) {
    case 1: return run_meta<1>(a, p, st);
    case 2: return run_meta<2>(a, p, st);
    case 3: return run_meta<3>(a, p, st);
    default: return run_meta<4>(a, p, st);
  }
}

}  // namespace w4
