// Batched decode GEMV, M <= 4, non-transposed:  Y[m][n] = sum_k X[m][k] * w[n][k] (+ bias[n]),
// w = bf16_rne((q - z) * s), fp32 accumulation.
//
// Design ("Modify small-batched weight only quantization", TensorRT-LLM #2213, names
// load stalls and duplicate scale / zero requests as the costs of this kernel; here
// on gfx950 with no matrix cores):
//   * one workgroup (16 waves) per contiguous block of rows, about one block per CU:
//     X is staged into LDS once per workgroup (in phases of up to PW x 2048 columns
//     when M*K does not fit), so activation traffic does not grow with N; the staging
//     uses direct global -> LDS loads issued ahead of the first weight loads, so the
//     first product waits for X and not for the weights behind it;
//   * each wave streams row groups of R rows over K; lane l owns the 16-byte chunk
//     c = it*64 + l of a row (32 codes), so one wave-wide load is 1 KB contiguous;
//   * weights, scales and zeros come in through buffer loads whose per-lane offset
//     is fixed and whose row base is a scalar resource: no per-chunk address
//     arithmetic, and rows / groups past the end read as zero (no bounds branches);
//   * a two-slot register pipeline runs over the flattened (row group, iteration)
//     steps of a wave, so the next row's loads are in flight while a row finishes;
//   * dequantization is v_fma_mix_f32 on nibbles masked into fp16 halves, bf16
//     rounding by v_cvt_pk_bf16_f32, products by v_dot2_f32_bf16 (fp16 activations:
//     v_cvt_pk_f16_f32 rounding, products by v_dot2_f32_f16);
//   * the R*M partial sums of a row group are reduced across the wave with a
//     transposing butterfly on v_permlane32_swap / v_permlane16_swap and DPP row
//     moves (no LDS round trips), parked in LDS, and written out at the end through
//     the output epilogue (bias, output dtype, output segments).
#include <algorithm>
#include <atomic>

#include "common.h"
#include "epilogue.h"
#include "launch.h"

namespace w4 {

namespace {

typedef __amdgpu_buffer_rsrc_t rsrc_t;
// dword 3 of a raw buffer resource on gfx9-class devices (32-bit data format)
constexpr int kRsrcDword3 = 0x00020000;
// cache-policy operand of a buffer load: the non-temporal hint (nt on gfx950)
constexpr int kNonTemporal = 2;

__device__ __forceinline__ rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, (int)bytes, kRsrcDword3);
}

template <int CTRL>
__device__ __forceinline__ float dpp_move(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xF, 0xF, false));
}

// One butterfly stage on partners lane ^ o: while more than one value is live, the lanes
// with the partner bit set keep the upper half of the values and the others the lower
// half (transposing); with one value left it is a plain sum.
template <int V>
__device__ __forceinline__ void swap_stage32(float (&v)[V], int& n) {
  if (n > 1) {
#pragma unroll
    for (int i = 0; i < V / 2; ++i)
      if (i < n / 2) {
        // lanes 0..31 receive lane+32's first operand, lanes 32..63 lane-32's second
        auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v[i]), __float_as_uint(v[i + n / 2]), false, false);
        v[i] = __uint_as_float(r[0]) + __uint_as_float(r[1]);
      }
    n /= 2;
  } else {
    auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v[0]), __float_as_uint(v[0]), false, false);
    v[0] = __uint_as_float(r[0]) + __uint_as_float(r[1]);
  }
}

template <int V>
__device__ __forceinline__ void swap_stage16(float (&v)[V], int& n) {
  if (n > 1) {
#pragma unroll
    for (int i = 0; i < V / 2; ++i)
      if (i < n / 2) {
        auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v[i]), __float_as_uint(v[i + n / 2]), false, false);
        v[i] = __uint_as_float(r[0]) + __uint_as_float(r[1]);
      }
    n /= 2;
  } else {
    auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v[0]), __float_as_uint(v[0]), false, false);
    v[0] = __uint_as_float(r[0]) + __uint_as_float(r[1]);
  }
}

template <int CTRL, int BIT, int V>
__device__ __forceinline__ void dpp_stage(float (&v)[V], int& n, int lane) {
  if (n > 1) {
    const bool up = (lane & BIT) != 0;
#pragma unroll
    for (int i = 0; i < V / 2; ++i)
      if (i < n / 2) {
        const float send = up ? v[i] : v[i + n / 2];
        const float keep = up ? v[i + n / 2] : v[i];
        v[i] = keep + dpp_move<CTRL>(send);
      }
    n /= 2;
  } else {
    v[0] += dpp_move<CTRL>(v[0]);
  }
}

// Wave-wide reduction of V partial sums (V <= 16): lane l ends up holding the total of
// value l >> (6 - log2 V).  Partners: lane ^ 32, lane ^ 16 (permlane swaps), lane ^ 15
// (DPP row_mirror), lane ^ 7 (row_half_mirror), lane ^ 2 and lane ^ 1 (quad_perm).
template <int V>
__device__ __forceinline__ float wave_reduce(float (&v)[V], int lane) {
  static_assert(V >= 1 && V <= 16 && (V & (V - 1)) == 0, "V is a power of two <= 16");
  int n = V;
  swap_stage32(v, n);
  swap_stage16(v, n);
  dpp_stage<0x140, 8>(v, n, lane);  // row_mirror
  dpp_stage<0x141, 4>(v, n, lane);  // row_half_mirror
  v[0] += dpp_move<0x4E>(v[0]);     // quad_perm [2,3,0,1]
  v[0] += dpp_move<0xB1>(v[0]);     // quad_perm [1,0,3,2]
  return v[0];
}

// Per-lane state of one pipeline step: the 16-byte chunk of each of R rows and the
// fp16 scale / zero bits of the group(s) it belongs to (GPC groups per chunk).
template <int R, int GPC>
struct Stage {
  u32x4 w[R];
  uint16_t s[R][GPC], z[R][GPC];  // fp16 bits; v_fma_mix_f32 reads the low half of the register
};

constexpr int kWaves = 16;

// meta_row: (scale, zero) pairs per row (K / g, 1 for ROWWISE, 0 for GLOBAL);
// log2g: group shift (31 for ROWWISE / GLOBAL, so every column maps to pair 0 of its row).
// Output argument: the general epilogue (output dtype, bias dtype, segments) when GEN, else
// just the fp32 bias and Y [M][N] pointers -- a 64-byte argument block instead of 160,
// which measurably shortens these few-microsecond launches.
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

// F16: fp16 activations and an fp16 weight operand (else bf16).
template <int M, int R, int GPC, bool GEN, bool F16>
__global__ __launch_bounds__(kWaves * 64) void gemv_kernel(const uint16_t* __restrict__ X,
                                                           const int32_t* __restrict__ packed,
                                                           const uint16_t* __restrict__ scales,
                                                           const uint16_t* __restrict__ zeros,
                                                           int N, int K, int meta_row, int geo,
                                                           const typename OutArg<GEN>::type ep) {
  // geo packs log2g (bits 0-4), rows_per_block (5-15) and phase_iters (16-30): with the
  // plain output the whole argument block is one 64-byte line.  The output argument comes
  // last: the twelve dwords before it are what the build preloads into SGPRs at dispatch,
  // and the output is needed only at the end.
  const int log2g = geo & 31, rows_per_block = (geo >> 5) & 2047, phase_iters = geo >> 16;
  extern __shared__ u32x4 smem[];
  constexpr int T = kWaves * 64;
  const int KS = K >> 5;               // 16-byte chunks per row
  const int iters = (KS + 63) >> 6;    // 2048-column iterations per row
  const int PW = phase_iters;          // iterations whose X is resident at a time
  u32x4* xs = smem;                                             // [PW][M][4 words][64 chunks]
  float* outs = reinterpret_cast<float*>(smem + PW * M * 256);  // [rows_per_block][M]
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int r0 = blockIdx.x * rows_per_block;
  const int r1 = min(r0 + rows_per_block, N);
  const int KW = K >> 3;
  const uint32_t meta_bytes = meta_row > 0 ? (uint32_t)meta_row * 2 : 2u;
  // row groups rg = wave, wave + 16, ... of R rows each
  const int nrg = (r1 - r0 + R - 1) / R;
  const int my_rg = nrg > wave ? (nrg - wave + kWaves - 1) / kWaves : 0;

  const uint32_t vo = lane * 16;
  uint32_t vs[GPC];
#pragma unroll
  for (int q = 0; q < GPC; ++q) vs[q] = ((uint32_t)(lane * 32 + q * 16) >> log2g) * 2;

  // Loads of step (row group k, iteration it); a row group past this wave's last one, or
  // a row past the block, gets a zero-sized resource and reads zeros without a request.
  // The resources start at the iteration's first chunk / pair and hold what is left of
  // the row (scalar arithmetic), so the per-lane offsets vo and vs[q] never change.
  auto load = [&](int k, int it, Stage<R, GPC>& st) {
    const int rg = wave + k * kWaves;
    const uint32_t so = ((uint32_t)(it * 2048) >> log2g) * 2;  // < meta_bytes for it < iters
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const int row = r0 + rg * R + r;
      const bool ok = k < my_rg && row < r1;
      const int n = min(row, r1 - 1);
      const rsrc_t pr = make_rsrc(packed + (size_t)n * KW + it * 256, ok ? (uint32_t)(KW - it * 256) * 4 : 0u);
      const rsrc_t sr = make_rsrc(reinterpret_cast<const char*>(scales + (size_t)n * meta_row) + so,
                                  ok ? meta_bytes - so : 0u);
      const rsrc_t zr = make_rsrc(reinterpret_cast<const char*>(zeros + (size_t)n * meta_row) + so,
                                  ok ? meta_bytes - so : 0u);
      // non-temporal (nt): the weights are streamed once; measured 2-4% on the decode sweep,
      // where the scale / zero loads marked the same way gained less
      st.w[r] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(pr, vo, 0, kNonTemporal));
#pragma unroll
      for (int q = 0; q < GPC; ++q) {
        st.s[r][q] = __builtin_amdgcn_raw_buffer_load_b16(sr, vs[q], 0, 0);
        st.z[r][q] = __builtin_amdgcn_raw_buffer_load_b16(zr, vs[q], 0, 0);
      }
    }
  };

  float acc[R][M];
#pragma unroll
  for (int r = 0; r < R; ++r)
#pragma unroll
    for (int m = 0; m < M; ++m) acc[r][m] = 0.0f;

  typedef __attribute__((address_space(3))) void lds_void;
  constexpr int kLoadsPerStep = R * (1 + 2 * GPC);  // vector-memory instructions of one load()
  static_assert(kLoadsPerStep < 64, "vmcnt holds 6 bits");
  Stage<R, GPC> A, B;
  for (int p0 = 0; p0 < iters; p0 += PW) {
    const int pw = min(PW, iters - p0);
    const int steps = my_rg * pw;
    // step t of this phase -> (row group k = t / pw, iteration p0 + t % pw)
    int lk = 0, lit = 0, ck = 0, cit = 0;
    auto advance = [&](int& k, int& it) {
      if (++it == pw) {
        it = 0;
        ++k;
      }
    };
    // X columns of this phase -> LDS by direct loads (no staging registers, no LDS store
    // instructions), issued ahead of the phase's first weight loads so that the barrier
    // below waits for X alone.  Row j of the tile (iteration il, row m, word w) is one
    // wave-wide load: lane c fills slot 64 j + c.  Chunks past K are zeroed by stores.
    if (p0 > 0) __syncthreads();  // every wave is done with the previous phase's X
    const int nj = pw * M * 4;
    for (int j = wave; j < nj; j += kWaves) {
      const int il = j / (M * 4), rj = j - il * (M * 4), m = rj >> 2, w = rj & 3;
      const int col = ((p0 + il) * 64 + lane) * 32 + w * 8;
      if (col < K)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(make_rsrc(X + (size_t)m * K, (uint32_t)K * 2),
                                                 (lds_void*)(xs + j * 64), 16, col * 2, 0, 0, 0);
      else
        xs[j * 64 + lane] = u32x4{0u, 0u, 0u, 0u};
    }
    __builtin_amdgcn_sched_barrier(0);
    load(lk, p0 + lit, A);
    advance(lk, lit);
    // Loads complete in issue order: X has landed once at most the one step of weight loads
    // issued after it is outstanding; the zero stores by lgkmcnt(0).  The barrier carries no
    // fence, which would also wait for those weight loads; the clobbers keep memory
    // accesses, and the scheduling barriers keep all instructions, on their side of it.
    __builtin_amdgcn_sched_barrier(0);
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_waitcnt((kLoadsPerStep & 15) | 0x70 | ((kLoadsPerStep >> 4) << 14));  // vmcnt(n) lgkmcnt(0)
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    __builtin_amdgcn_sched_barrier(0);

    auto compute = [&](const Stage<R, GPC>& st) {
      DqConst dc[R][GPC];
#pragma unroll
      for (int r = 0; r < R; ++r)
#pragma unroll
        for (int q = 0; q < GPC; ++q) dc[r][q] = dq_const_mix(st.s[r][q], st.z[r][q]);
      const u32x4* xb = xs + cit * M * 256 + lane;
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        u32x4 xv[M];
#pragma unroll
        for (int m = 0; m < M; ++m) xv[m] = xb[(m * 4 + w) * 64];
#pragma unroll
        for (int r = 0; r < R; ++r) {
          uint32_t bw[4];
          dq_word_op<F16>(st.w[r][w], dc[r][GPC == 2 ? w / 2 : 0], bw);
#pragma unroll
          for (int m = 0; m < M; ++m)
#pragma unroll
            for (int i = 0; i < 4; ++i) acc[r][m] = dot2_op<F16>(bw[i], xv[m][i], acc[r][m]);
        }
      }
      if (cit == pw - 1) {
        // this phase of the row group is done: reduce across the wave, accumulate in LDS
        constexpr int MP = M == 3 ? 4 : M;
        constexpr int V = R * MP;
        constexpr int LOGV = V == 1 ? 0 : V == 2 ? 1 : V == 4 ? 2 : V == 8 ? 3 : 4;
        float v[V];
#pragma unroll
        for (int r = 0; r < R; ++r)
#pragma unroll
          for (int m = 0; m < MP; ++m) v[r * MP + m] = m < M ? acc[r][m] : 0.0f;
        const float sum = wave_reduce<V>(v, lane);
        constexpr int SPAN = 64 / V;
        const int idx = lane >> (6 - LOGV);
        const int r = idx / MP, m = idx - (idx / MP) * MP;
        const int lr = (wave + ck * kWaves) * R + r;  // row within the block
        if ((lane & (SPAN - 1)) == 0 && m < M && r0 + lr < r1) {
          float* o = outs + lr * M + m;  // each (row, m) belongs to one wave: no race
          *o = p0 == 0 ? sum : *o + sum;
        }
#pragma unroll
        for (int rr = 0; rr < R; ++rr)
#pragma unroll
          for (int mm = 0; mm < M; ++mm) acc[rr][mm] = 0.0f;
      }
      advance(ck, cit);
    };

    // two slots, unrolled by two: the slot being filled is never the one being read,
    // and every iteration issues exactly one step of loads (exact wait counts).  A wave
    // raises its priority while it issues a step's loads, so the sequencer lets loads out
    // ahead of other waves' dequantization (measured: decode sweep +1.5%)
    int t = 0;
    for (; t + 2 <= steps; t += 2) {
      __builtin_amdgcn_s_setprio(2);
      load(lk, p0 + lit, B);
      advance(lk, lit);
      __builtin_amdgcn_s_setprio(0);
      compute(A);
      __builtin_amdgcn_s_setprio(2);
      load(lk, p0 + lit, A);
      advance(lk, lit);
      __builtin_amdgcn_s_setprio(0);
      compute(B);
    }
    if (t < steps) compute(A);
  }

  __syncthreads();
  if constexpr (!GEN) {
    float* Y = ep.Y;
    const float* bias = ep.bias;
    for (int u = tid; u < (r1 - r0) * M; u += T) {
      const int m = u / (r1 - r0), lr = u - m * (r1 - r0);
      const int n = r0 + lr;
      Y[(size_t)m * N + n] = outs[lr * M + m] + (bias != nullptr ? bias[n] : 0.0f);
    }
  } else {
    for (int u = tid; u < (r1 - r0) * M; u += T) {
      const int m = u / (r1 - r0), lr = u - m * (r1 - r0);
      const int n = r0 + lr;
      epi_put(ep, epi_col(ep, n), m, outs[lr * M + m]);
    }
  }
}

struct GemvPlan {
  int R;
  int blocks, rows_per_block;
  int phase_iters;
  size_t lds;
};

GemvPlan plan(const MmArgs& a, const DeviceCaps& caps) {
  GemvPlan p;
  const int iters = (int)((a.K / 32 + 63) / 64);
  const size_t x_iter = (size_t)a.M * 4096;  // LDS bytes of X per 2048-column iteration
  // Tall weights: two rows per wave halve the X reads from LDS; one block per CU.
  // Otherwise one row per wave, and two blocks per CU (twice the waves to hide latency)
  // only for short rows (at most two 2048-column iterations) when each block still gets a
  // row per wave (N >= 8192).  Otherwise one block per CU measured faster, X being staged
  // half as often: 2048 x 2048 8 % at every M, 4096 x 11008 up to 7 %, 8192 x 8192 5-6 %
  // at M = 2..4.
  p.R = a.N >= 16384 ? 2 : 1;
  const int per_cu = p.R == 1 && iters <= 2 && (size_t)iters * x_iter <= 72 * 1024 &&
                             a.N >= (int64_t)2 * caps.cus * kWaves
                         ? 2
                         : 1;
  p.blocks = caps.cus * per_cu;
  p.rows_per_block = (int)((a.N + p.blocks - 1) / p.blocks);
  if (p.rows_per_block > 1024) p.rows_per_block = 1024;
  p.blocks = (int)((a.N + p.rows_per_block - 1) / p.rows_per_block);
  const size_t outs = (size_t)p.rows_per_block * a.M * 4;
  const size_t budget = caps.lds > outs ? caps.lds - outs : 0;
  p.phase_iters = (int)std::min<size_t>((size_t)iters, budget / x_iter);
  p.lds = (size_t)p.phase_iters * x_iter + outs;
  return p;
}

int meta_row(const MmArgs& a) {
  if (a.mode == W4_MODE_GLOBAL) return 0;
  if (a.mode == W4_MODE_ROWWISE) return 1;
  return (int)(a.K / a.group);
}

template <int M, int R, int GPC, bool GEN, bool F16>
hipError_t run(const MmArgs& a, const GemvPlan& p, hipStream_t st) {
  auto k = gemv_kernel<M, R, GPC, GEN, F16>;
  static std::atomic<int> lds_set{64 * 1024};  // largest dynamic LDS size enabled so far
  if ((int)p.lds > lds_set.load()) {
    const hipError_t e = hipFuncSetAttribute((const void*)k, hipFuncAttributeMaxDynamicSharedMemorySize, (int)p.lds);
    if (e != hipSuccess) return e;
    lds_set.store((int)p.lds);
  }
  const int log2g = a.mode == W4_MODE_GROUPWISE ? 31 - __builtin_clz((unsigned)a.group) : 31;
  typename OutArg<GEN>::type out;
  if constexpr (GEN) out = a.ep;
  else out = PlainOut{static_cast<const float*>(a.ep.bias), static_cast<float*>(a.ep.y[0])};
  k<<<p.blocks, kWaves * 64, p.lds, st>>>(a.A, a.packed, a.scales, a.zeros, (int)a.N, (int)a.K, meta_row(a),
                                           log2g | (p.rows_per_block << 5) | (p.phase_iters << 16), out);
  return hipGetLastError();
}

template <int M, bool GEN, bool F16>
hipError_t run_g(const MmArgs& a, const GemvPlan& p, hipStream_t st) {
  const bool g16 = a.mode == W4_MODE_GROUPWISE && a.group == 16;  // two groups per 32-code chunk
  if (p.R == 2) return g16 ? run<M, 2, 2, GEN, F16>(a, p, st) : run<M, 2, 1, GEN, F16>(a, p, st);
  return g16 ? run<M, 1, 2, GEN, F16>(a, p, st) : run<M, 1, 1, GEN, F16>(a, p, st);
}

template <int M>
hipError_t run_m(const MmArgs& a, const GemvPlan& p, hipStream_t st) {
  const Epi& e = a.ep;
  const bool plain = e.nseg == 1 && e.dt == W4_DT_F32 && e.ld[0] == a.N;
  if (a.a_f16) return plain ? run_g<M, false, true>(a, p, st) : run_g<M, true, true>(a, p, st);
  return plain ? run_g<M, false, false>(a, p, st) : run_g<M, true, false>(a, p, st);
}

}  // namespace

bool gemv_supported(const MmArgs& a, const DeviceCaps& caps) {
  if (a.transposed || a.M < 1 || a.M > 4) return false;
  if (a.N > (int64_t)1 << 30 || a.K > (int64_t)1 << 30) return false;
  return plan(a, caps).phase_iters >= 1;
}

size_t gemv_lds_bytes(const MmArgs& a, const DeviceCaps& caps) { return plan(a, caps).lds; }

const char* gemv_name(const MmArgs& a) {
  static const char* names[] = {"gemv_m1", "gemv_m2", "gemv_m3", "gemv_m4"};
  return names[a.M - 1];
}

hipError_t launch_gemv(const MmArgs& a, const DeviceCaps& caps, hipStream_t st) {
  const GemvPlan p = plan(a, caps);
  switch (a.M) {
    case 1: return run_m<1>(a, p, st);
    case 2: return run_m<2>(a, p, st);
    case 3: return run_m<3>(a, p, st);
    default: return run_m<4>(a, p, st);
  }
}

}  // namespace w4
