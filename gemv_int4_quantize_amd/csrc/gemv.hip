// Batched decode GEMV, M <= 4, non-transposed:  Y[m][n] = sum_k X[m][k] * w[n][k] (+ bias[n]),
// w = bf16_rne((q - z) * s), fp32 accumulation.
//
// Design ("Modify small-batched weight only quantization", TensorRT-LLM #2213, names
// load stalls and duplicate scale / zero requests as the costs of this kernel; here
// on gfx950 with no matrix cores):
//   * each wave owns R rows over the full K (split-K inside the wave, no partial
//     results leave the wave); lane l streams 16-byte chunks c = l, l+64, ... of
//     every row (32 codes each), so one wave-wide load is 1 KB contiguous;
//   * X is staged once per workgroup in LDS as 4 planes ([m][word][chunk]) so that
//     consecutive lanes read consecutive 16-byte slots (no bank conflicts);
//   * GROUPWISE scale / zero pairs of the 2048 columns one iteration covers are
//     loaded once per group by the wave and staged in LDS as the fp32 constants of
//     the in-register dequantization (s*2^24, s*2^20, -z*s);
//   * dequantization is v_fma_mix_f32 on nibbles masked into fp16 halves, bf16
//     rounding by v_cvt_pk_bf16_f32, products by v_dot2_f32_bf16;
//   * the R*M partial sums of a wave are reduced with a transposing butterfly, so
//     every shuffle step halves the number of live values.
#include "common.h"
#include "launch.h"

#include <atomic>

namespace w4 {

struct alignas(16) DqEntry {
  float s24, s20, nzs, pad;
};

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

template <int M, int R, int META, int WAVES>
__global__ __launch_bounds__(WAVES * 64) void gemv_kernel(const uint16_t* __restrict__ X,
                                                          const int32_t* __restrict__ packed,
                                                          const uint16_t* __restrict__ scales,
                                                          const uint16_t* __restrict__ zeros,
                                                          const float* __restrict__ bias, float* __restrict__ Y,
                                                          int N, int K, int g) {
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  const int KS = K >> 5;  // 16-byte chunks (32 codes) per row
  u32x4* xs = reinterpret_cast<u32x4*>(smem);
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int row0 = (blockIdx.x * WAVES + wave) * R;
  const int iters = (KS + 63) >> 6;

  // groups covered by one iteration (2048 columns) and the per-wave table
  const int gpi = META == META_GROUP ? (g >= 2048 ? 1 : 2048 / g) : 1;
  DqEntry* tbl = reinterpret_cast<DqEntry*>(smem + (size_t)M * K * 2) + (size_t)wave * R * gpi;
  const int gpr = META == META_GROUP ? K / g : 1;

  int rows[R];
#pragma unroll
  for (int r = 0; r < R; ++r) rows[r] = min(row0 + r, N - 1);

  // first packed chunk of every row: in flight while X is staged
  u32x4 wv[R];
  {
    const int c = min(lane, KS - 1);
#pragma unroll
    for (int r = 0; r < R; ++r)
      wv[r] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(packed + (size_t)rows[r] * (K >> 3)) + c);
  }

  // stage X in the plane layout
  for (int u = threadIdx.x; u < M * KS * 4; u += WAVES * 64) {
    const int m = u / (KS * 4);
    const int rem = u - m * KS * 4;
    const int c = rem >> 2, w = rem & 3;
    xs[(m * 4 + w) * KS + c] = *reinterpret_cast<const u32x4*>(X + (size_t)m * K + c * 32 + w * 8);
  }

  DqConst rc[R];
  if constexpr (META != META_GROUP) {
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const int mi = META == META_GLOBAL ? 0 : rows[r];
      rc[r] = dq_const(scales[mi], zeros[mi]);
    }
  }
  __syncthreads();

  float acc[R][M];
#pragma unroll
  for (int r = 0; r < R; ++r)
#pragma unroll
    for (int m = 0; m < M; ++m) acc[r][m] = 0.0f;

  for (int it = 0; it < iters; ++it) {
    const int c = it * 64 + lane;
    const bool valid = c < KS;
    const int cc = valid ? c : KS - 1;

    int g0 = 0;
    if constexpr (META == META_GROUP) {
      g0 = (it * 2048) / g;
      for (int e = lane; e < R * gpi; e += 64) {
        const int r = e / gpi;
        const int G = min(g0 + (e - r * gpi), gpr - 1);
        const size_t mi = (size_t)rows[r] * gpr + G;
        const DqConst d = dq_const(scales[mi], zeros[mi]);
        DqEntry t;
        t.s24 = d.s24;
        t.s20 = d.s20;
        t.nzs = d.nzs;
        t.pad = 0.0f;
        tbl[e] = t;
      }
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    }

    // prefetch the next iteration's chunks
    u32x4 nv[R];
    const bool more = it + 1 < iters;
    if (more) {
      const int cn = min(c + 64, KS - 1);
#pragma unroll
      for (int r = 0; r < R; ++r)
        nv[r] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(packed + (size_t)rows[r] * (K >> 3)) + cn);
    }

    if (valid) {
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        u32x4 xv[M];
#pragma unroll
        for (int m = 0; m < M; ++m) xv[m] = xs[(m * 4 + w) * KS + cc];
#pragma unroll
        for (int r = 0; r < R; ++r) {
          DqConst d;
          if constexpr (META == META_GROUP) {
            const DqEntry t = tbl[r * gpi + ((cc * 32 + w * 8) / g - g0)];
            d.s24 = t.s24;
            d.s20 = t.s20;
            d.nzs = t.nzs;
          } else {
            d = rc[r];
          }
          uint32_t bw[4];
          dq_word_bf16(wv[r][w], d, bw);
#pragma unroll
          for (int m = 0; m < M; ++m)
#pragma unroll
            for (int i = 0; i < 4; ++i) acc[r][m] = dot2_bf16(bw[i], xv[m][i], acc[r][m]);
        }
      }
    }
    if (more) {
#pragma unroll
      for (int r = 0; r < R; ++r) wv[r] = nv[r];
    }
    if constexpr (META == META_GROUP) {
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    }
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
  GemvPlan p;
  const size_t xbytes = (size_t)a.M * a.K * 2;
  // rows per wave: keep at least ~512 waves in flight
  p.R = a.N >= 512 * 4 ? 4 : (a.N >= 512 * 2 ? 2 : 1);
  // waves per block: enough waves per CU despite the X copy each block holds
  p.waves = xbytes <= 40 * 1024 ? 4 : (xbytes <= 72 * 1024 ? 8 : 16);
  const int gpi = a.mode == W4_MODE_GROUPWISE ? (a.group >= 2048 ? 1 : 2048 / a.group) : 0;
  p.lds = xbytes + (size_t)p.waves * p.R * gpi * sizeof(DqEntry);
  return p;
}

template <int M, int R, int META, int WAVES>
hipError_t run(const MmArgs& a, const GemvPlan& p, hipStream_t st) {
  auto k = gemv_kernel<M, R, META, WAVES>;
  if (p.lds > 64 * 1024) {
    // opt in to the large LDS footprint (once per kernel instantiation)
    static std::atomic<size_t> granted{0};
    if (granted.load() < p.lds) {
      hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(k),
                                         hipFuncAttributeMaxDynamicSharedMemorySize, (int)p.lds);
      if (e != hipSuccess) return e;
      granted.store(p.lds);
    }
  }
  const int rows_per_block = R * WAVES;
  const dim3 grid((unsigned)((a.N + rows_per_block - 1) / rows_per_block));
  k<<<grid, WAVES * 64, p.lds, st>>>(a.A, a.packed, a.scales, a.zeros, a.bias, a.Y, (int)a.N, (int)a.K, a.group);
  return hipGetLastError();
}

template <int M, int R, int META>
hipError_t run_w(const MmArgs& a, const GemvPlan& p, hipStream_t st) {
  switch (p.waves) {
    case 4: return run<M, R, META, 4>(a, p, st);
    case 8: return run<M, R, META, 8>(a, p, st);
    default: return run<M, R, META, 16>(a, p, st);
  }
}

template <int M, int META>
hipError_t run_r(const MmArgs& a, const GemvPlan& p, hipStream_t st) {
  switch (p.R) {
    case 4: return run_w<M, 4, META>(a, p, st);
    case 2: return run_w<M, 2, META>(a, p, st);
    default: return run_w<M, 1, META>(a, p, st);
  }
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
