// C ABI of the W4A16 library: argument validation, dispatch, error reporting.
// The declarations and the contract of every entry point are in include/w4a16.h.
#include <hip/hip_runtime.h>

#include <atomic>
#include <cstdarg>
#include <mutex>
#include <cstdio>
#include <cstring>
#include <string>

#include "launch.h"

namespace {

thread_local std::string g_last_error;

int fail(int status, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
int fail(int status, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return status;
}

int ok() {
  g_last_error.clear();
  return W4_OK;
}

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

bool is_pow2(int64_t v) { return v > 0 && (v & (v - 1)) == 0; }

int check_desc(const w4_desc* d) {
  if (d == nullptr) return fail(W4_ERR_INVALID, "desc is NULL");
  if (d->N < 1) return fail(W4_ERR_INVALID, "N = %lld must be >= 1", (long long)d->N);
  if (d->K < 8 || d->K % 8 != 0) return fail(W4_ERR_INVALID, "K = %lld must be a positive multiple of 8", (long long)d->K);
  if (d->N > ((int64_t)1 << 31) - 1 || d->K > ((int64_t)1 << 31) - 1)
    return fail(W4_ERR_UNSUPPORTED, "N and K must fit in int32");
  if (d->N * (d->K / 8) > ((int64_t)1 << 40)) return fail(W4_ERR_UNSUPPORTED, "matrix too large");
  switch (d->mode) {
    case W4_MODE_GLOBAL:
    case W4_MODE_ROWWISE:
      break;
    case W4_MODE_GROUPWISE:
      if (!is_pow2(d->group) || d->group < 16 || d->group > 4096)
        return fail(W4_ERR_INVALID, "group = %d must be a power of two in [16, 4096]", d->group);
      if (d->group > d->K || d->K % d->group != 0)
        return fail(W4_ERR_INVALID, "group = %d must divide K = %lld", d->group, (long long)d->K);
      break;
    default:
      return fail(W4_ERR_INVALID, "mode = %d is not GLOBAL, ROWWISE or GROUPWISE", d->mode);
  }
  return W4_OK;
}

int64_t pairs_of(const w4_desc* d) {
  if (d->mode == W4_MODE_GLOBAL) return 1;
  if (d->mode == W4_MODE_ROWWISE) return d->N;
  return d->N * (d->K / d->group);
}

w4::DeviceCaps device_caps() {
  // queried once per process (one device type); without a device (host-only queries on a
  // machine with no GPU) the figures are MI355X's: 160 KB of LDS per workgroup, 256 CUs
  static std::atomic<long long> lds{-1}, cus{-1};
  if (lds.load() < 0) {
    int dev = 0, bytes = 0, n = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&bytes, hipDeviceAttributeMaxSharedMemoryPerBlock, dev) != hipSuccess || bytes <= 0)
      bytes = 160 * 1024;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
    cus.store(n);
    lds.store(bytes);
  }
  return w4::DeviceCaps{(size_t)lds.load(), (int)cus.load()};
}

int launched(hipError_t e, const char* what) {
  if (e != hipSuccess) return fail(W4_ERR_LAUNCH, "%s: %s", what, hipGetErrorString(e));
  return ok();
}

int check_mm(const uint16_t* A, int64_t M, const int32_t* packed, const uint16_t* scales, const uint16_t* zeros,
             const w4_desc* desc, int transposed) {
  int s = check_desc(desc);
  if (s != W4_OK) return s;
  if (M < 0) return fail(W4_ERR_INVALID, "M = %lld must be >= 0", (long long)M);
  if (M > ((int64_t)1 << 31) - 1) return fail(W4_ERR_UNSUPPORTED, "M must fit in int32");
  if (desc->K % 32 != 0) return fail(W4_ERR_UNSUPPORTED, "matmul needs K %% 32 == 0 (K = %lld)", (long long)desc->K);
  if (transposed && desc->N % 8 != 0)
    return fail(W4_ERR_UNSUPPORTED, "transposed matmul needs N %% 8 == 0 (N = %lld)", (long long)desc->N);
  // the transposed GEMM addresses a 256-row activation tile and 64 weight rows per step
  // with 32-bit buffer offsets
  if (transposed && (desc->N >= ((int64_t)1 << 22) || desc->K > ((int64_t)1 << 21)))
    return fail(W4_ERR_UNSUPPORTED, "transposed matmul needs N < 2^22 and K <= 2^21 (N = %lld, K = %lld)",
                (long long)desc->N, (long long)desc->K);
  if (M == 0) return W4_OK;
  if (!A || !packed || !scales || !zeros) return fail(W4_ERR_INVALID, "a required pointer is NULL");
  if (!aligned(A, 16) || !aligned(packed, 16)) return fail(W4_ERR_ALIGN, "A and packed must be 16-byte aligned");
  if (!aligned(scales, 2) || !aligned(zeros, 2)) return fail(W4_ERR_ALIGN, "scales / zeros must be 2-byte aligned");
  return W4_OK;
}

// Output epilogue from the caller's bias, dtype and segments (validated).
int make_epi(const w4_desc* desc, int transposed, int64_t M, const void* bias, int out_dtype, const w4_out_seg* segs,
             int nsegs, w4::Epi* ep) {
  if (out_dtype != W4_DT_F32 && out_dtype != W4_DT_F16 && out_dtype != W4_DT_BF16)
    return fail(W4_ERR_INVALID, "out_dtype = %d must be F32, F16 or BF16", out_dtype);
  if (segs == nullptr || nsegs < 1 || nsegs > w4::kMaxSegs)
    return fail(W4_ERR_INVALID, "nsegs = %d must be in [1, %d] with a segment array", nsegs, w4::kMaxSegs);
  const int64_t outc = transposed ? desc->K : desc->N;
  const size_t esz = out_dtype == W4_DT_F32 ? 4 : 2;
  int64_t c = 0;
  for (int i = 0; i < w4::kMaxSegs; ++i) {
    if (i < nsegs) {
      const w4_out_seg& g = segs[i];
      if (g.cols < 1 || g.ld < g.cols)
        return fail(W4_ERR_INVALID, "segment %d: cols = %lld must be >= 1 and ld = %lld >= cols", i,
                    (long long)g.cols, (long long)g.ld);
      if (M > 0 && g.Y == nullptr) return fail(W4_ERR_INVALID, "segment %d: Y is NULL", i);
      if (M > 0 && !aligned(g.Y, esz)) return fail(W4_ERR_ALIGN, "segment %d: Y must be %zu-byte aligned", i, esz);
      ep->c0[i] = c;
      ep->y[i] = g.Y;
      ep->ld[i] = g.ld;
      c += g.cols;
    } else {
      ep->c0[i] = INT64_MAX;
      ep->y[i] = nullptr;
      ep->ld[i] = 0;
    }
  }
  if (c != outc)
    return fail(W4_ERR_INVALID, "segment columns sum to %lld, the output has %lld", (long long)c, (long long)outc);
  if (bias != nullptr && !aligned(bias, esz)) return fail(W4_ERR_ALIGN, "bias must be %zu-byte aligned", esz);
  ep->bias = bias;
  ep->dt = out_dtype;
  ep->nseg = nsegs;
  return W4_OK;
}

w4::MmArgs make_args(const uint16_t* A, int64_t M, const int32_t* packed, const uint16_t* scales,
                     const uint16_t* zeros, const w4_desc* desc, int transposed, const w4::Epi& ep,
                     bool a_f16 = false) {
  w4::MmArgs a;
  a.a_f16 = a_f16;
  a.A = A;
  a.packed = packed;
  a.scales = scales;
  a.zeros = zeros;
  a.ep = ep;
  a.M = M;
  a.N = desc->N;
  a.K = desc->K;
  a.mode = desc->mode;
  a.group = desc->mode == W4_MODE_GROUPWISE ? desc->group : (int)desc->K;
  a.transposed = transposed != 0;
  return a;
}

int run_mm(const w4::MmArgs& a, void* ws, size_t ws_bytes, void* stream) {
  const hipStream_t st = static_cast<hipStream_t>(stream);
  const w4::DeviceCaps caps = device_caps();
  if (w4::gemv_supported(a, caps)) return launched(w4::launch_gemv(a, caps, st), "gemv");
  const size_t wsb = ws != nullptr ? ws_bytes : 0;
  // the footprint of the plan this call launches (split or not, given its workspace)
  const size_t lds = w4::gemm_lds_bytes(a, caps, wsb);
  if (lds > caps.lds)
    return fail(W4_ERR_RESOURCE, "GEMM tile needs %zu bytes of LDS, the device allows %zu", lds, caps.lds);
  if (ws != nullptr && !aligned(ws, 16)) return fail(W4_ERR_ALIGN, "workspace must be 16-byte aligned");
  return launched(w4::launch_gemm(a, caps, ws, wsb, st), "gemm");
}

// Split-K scratch of w4a16_mm_noalloc, for callers that cannot allocate: a file-scope
// device array, one copy per GPU, held until the process ends.  Host code uses the
// address hipGetSymbolAddress returns for the current device, never the array's name.
constexpr size_t kScratchBytes = (size_t)64 << 20;
__device__ __attribute__((aligned(256))) float scratch[kScratchBytes / sizeof(float)];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// The device address of `scratch` on the current device (looked up once per device).
int scratch_of_current_device(void** ptr) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(W4_ERR_LAUNCH, "hipGetDevice: %s", hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxDevices) return fail(W4_ERR_UNSUPPORTED, "device %d is past the %d the library tracks", dev, kMaxDevices);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || p == nullptr)
      return fail(W4_ERR_LAUNCH, "hipGetSymbolAddress(scratch): %s", hipGetErrorString(e));
    g_scratch_ptr[dev] = p;
  }
  *ptr = g_scratch_ptr[dev];
  return W4_OK;
}

}  // namespace

extern "C" {

int w4_meta_pairs(const w4_desc* desc, int64_t* pairs) {
  int s = check_desc(desc);
  if (s != W4_OK) return s;
  if (!pairs) return fail(W4_ERR_INVALID, "pairs is NULL");
  *pairs = pairs_of(desc);
  return ok();
}

int w4_workspace_bytes(const w4_desc* desc, int op, int64_t M, size_t* bytes) {
  int s = check_desc(desc);
  if (s != W4_OK) return s;
  if (!bytes) return fail(W4_ERR_INVALID, "bytes is NULL");
  switch (op) {
    case W4_OP_QUANTIZE: *bytes = w4::quantize_workspace_bytes(desc->mode); break;
    case W4_OP_DEQUANTIZE: *bytes = 0; break;
    case W4_OP_MM:
    case W4_OP_MM_T: {
      *bytes = 0;
      if (M < 1 || M > ((int64_t)1 << 31) - 1 || desc->K % 32 != 0) break;
      static const uint16_t dummy[8] __attribute__((aligned(16))) = {0};
      const w4::Epi ep = {};
      const w4::MmArgs a = make_args(dummy, M, reinterpret_cast<const int32_t*>(dummy), dummy, dummy, desc,
                                     op == W4_OP_MM_T, ep);
      if (!w4::gemv_supported(a, device_caps())) *bytes = w4::gemm_workspace_bytes(a, device_caps());
      break;
    }
    default: return fail(W4_ERR_INVALID, "op = %d is unknown", op);
  }
  return ok();
}

int w4_quantize_pack_zp(const void* W, int w_dtype, const w4_desc* desc, int zero_kind, int32_t* packed,
                        uint16_t* scales, uint16_t* zeros, void* ws, size_t ws_bytes, void* stream) {
  int s = check_desc(desc);
  if (s != W4_OK) return s;
  if (w_dtype != W4_DT_F32 && w_dtype != W4_DT_F16 && w_dtype != W4_DT_BF16)
    return fail(W4_ERR_INVALID, "w_dtype = %d is not F32, F16 or BF16", w_dtype);
  if (zero_kind != W4_ZERO_FP16 && zero_kind != W4_ZERO_INT)
    return fail(W4_ERR_INVALID, "zero_kind = %d is not W4_ZERO_FP16 or W4_ZERO_INT", zero_kind);
  if (!W || !packed || !scales || !zeros) return fail(W4_ERR_INVALID, "a required pointer is NULL");
  if (!aligned(W, 16)) return fail(W4_ERR_ALIGN, "W must be 16-byte aligned");
  if (!aligned(packed, 4) || !aligned(scales, 2) || !aligned(zeros, 2))
    return fail(W4_ERR_ALIGN, "packed must be 4-byte, scales / zeros 2-byte aligned");
  const size_t need = w4::quantize_workspace_bytes(desc->mode);
  if (need > 0) {
    if (!ws || ws_bytes < need)
      return fail(W4_ERR_RESOURCE, "GLOBAL mode needs a workspace of %zu bytes (got %zu)", need, ws_bytes);
    if (!aligned(ws, 8)) return fail(W4_ERR_ALIGN, "workspace must be 8-byte aligned");
  }
  const int g = desc->mode == W4_MODE_GROUPWISE ? desc->group : (int)desc->K;
  return launched(w4::launch_quantize(W, w_dtype, desc->N, desc->K, desc->mode, g, zero_kind == W4_ZERO_INT, packed,
                                      scales, zeros, ws, static_cast<hipStream_t>(stream)),
                  "quantize_pack");
}

int w4_quantize_pack(const void* W, int w_dtype, const w4_desc* desc, int32_t* packed, uint16_t* scales,
                     uint16_t* zeros, void* ws, size_t ws_bytes, void* stream) {
  return w4_quantize_pack_zp(W, w_dtype, desc, W4_ZERO_FP16, packed, scales, zeros, ws, ws_bytes, stream);
}

int w4_dequantize(const int32_t* packed, const uint16_t* scales, const uint16_t* zeros, const w4_desc* desc,
                  void* out, int out_dtype, void* stream) {
  int s = check_desc(desc);
  if (s != W4_OK) return s;
  if (out_dtype != W4_DT_BF16 && out_dtype != W4_DT_F32 && out_dtype != W4_DT_F16)
    return fail(W4_ERR_INVALID, "out_dtype = %d must be BF16, F16 or F32", out_dtype);
  if (!packed || !scales || !zeros || !out) return fail(W4_ERR_INVALID, "a required pointer is NULL");
  if (!aligned(out, 16) || !aligned(packed, 4) || !aligned(scales, 2) || !aligned(zeros, 2))
    return fail(W4_ERR_ALIGN, "out must be 16-byte, packed 4-byte, scales / zeros 2-byte aligned");
  const int g = desc->mode == W4_MODE_GROUPWISE ? desc->group : (int)desc->K;
  return launched(w4::launch_dequantize(packed, scales, zeros, desc->N, desc->K, desc->mode, g, out, out_dtype,
                                        static_cast<hipStream_t>(stream)),
                  "dequantize");
}

int w4a16_mm(const uint16_t* A, int64_t M, const int32_t* packed, const uint16_t* scales, const uint16_t* zeros,
             const w4_desc* desc, int transposed, const float* bias, float* Y, void* ws, size_t ws_bytes,
             void* stream) {
  int s = check_mm(A, M, packed, scales, zeros, desc, transposed);
  if (s != W4_OK) return s;
  if (M == 0) return ok();
  if (Y == nullptr) return fail(W4_ERR_INVALID, "a required pointer is NULL");
  const int64_t outc = transposed ? desc->K : desc->N;
  const w4_out_seg seg = {Y, outc, outc};
  w4::Epi ep;
  s = make_epi(desc, transposed, M, bias, W4_DT_F32, &seg, 1, &ep);
  if (s != W4_OK) return s;
  return run_mm(make_args(A, M, packed, scales, zeros, desc, transposed, ep), ws, ws_bytes, stream);
}

int w4a16_mm_out(const void* A, int a_dtype, int64_t M, const int32_t* packed, const uint16_t* scales,
                 const uint16_t* zeros, const w4_desc* desc, int transposed, const void* bias, int out_dtype,
                 const w4_out_seg* segs, int nsegs, void* ws, size_t ws_bytes, void* stream) {
  if (a_dtype != W4_DT_BF16 && a_dtype != W4_DT_F16)
    return fail(W4_ERR_INVALID, "a_dtype = %d must be BF16 or F16", a_dtype);
  const uint16_t* A16 = static_cast<const uint16_t*>(A);
  int s = check_mm(A16, M, packed, scales, zeros, desc, transposed);
  if (s != W4_OK) return s;
  w4::Epi ep;
  s = make_epi(desc, transposed, M, bias, out_dtype, segs, nsegs, &ep);
  if (s != W4_OK) return s;
  if (M == 0) return ok();
  return run_mm(make_args(A16, M, packed, scales, zeros, desc, transposed, ep, a_dtype == W4_DT_F16), ws, ws_bytes,
                stream);
}

int w4a16_mm_noalloc(const uint16_t* A, int64_t M, const int32_t* packed, const uint16_t* scales,
                     const uint16_t* zeros, const w4_desc* desc, int transposed, const float* bias, float* Y,
                     void* stream) {
  int s = check_mm(A, M, packed, scales, zeros, desc, transposed);
  if (s != W4_OK) return s;
  if (M == 0) return ok();
  if (Y == nullptr) return fail(W4_ERR_INVALID, "a required pointer is NULL");
  const int64_t outc = transposed ? desc->K : desc->N;
  const w4_out_seg seg = {Y, outc, outc};
  w4::Epi ep;
  s = make_epi(desc, transposed, M, bias, W4_DT_F32, &seg, 1, &ep);
  if (s != W4_OK) return s;
  const w4::MmArgs a = make_args(A, M, packed, scales, zeros, desc, transposed, ep);
  const w4::DeviceCaps caps = device_caps();
  // the plan w4a16_mm runs with the workspace w4_workspace_bytes reports
  const size_t need = w4::gemv_supported(a, caps) ? 0 : w4::gemm_workspace_bytes(a, caps);
  if (need > kScratchBytes)
    return fail(W4_ERR_RESOURCE,
                "the split-K planes need %zu bytes, the static scratch holds %zu: use w4a16_mm with a workspace",
                need, kScratchBytes);
  void* ws = nullptr;
  if (need > 0) {
    s = scratch_of_current_device(&ws);
    if (s != W4_OK) return s;
  }
  return run_mm(a, ws, need, stream);
}

const char* w4a16_mm_kernel(int64_t M, const w4_desc* desc, int transposed) {
  // validation without pointers: use a dummy aligned address
  static const uint16_t dummy[8] __attribute__((aligned(16))) = {0};
  const void* p = dummy;
  int s = check_mm(static_cast<const uint16_t*>(p), M, static_cast<const int32_t*>(p), dummy, dummy, desc,
                   transposed);
  if (s != W4_OK || M == 0) return nullptr;
  const w4::Epi ep = {};
  const w4::MmArgs a = make_args(dummy, M, static_cast<const int32_t*>(p), dummy, dummy, desc, transposed, ep);
  if (w4::gemv_supported(a, device_caps())) return w4::gemv_name(a);
  return w4::gemm_name(a, device_caps(), SIZE_MAX);
}

int w4a16_mm_plan(int64_t M, const w4_desc* desc, int transposed, size_t ws_bytes, w4_mm_plan* plan) {
  if (plan == nullptr) return fail(W4_ERR_INVALID, "plan is NULL");
  static const uint16_t dummy[8] __attribute__((aligned(16))) = {0};
  const void* p = dummy;
  int s = check_mm(static_cast<const uint16_t*>(p), M, static_cast<const int32_t*>(p), dummy, dummy, desc,
                   transposed);
  if (s != W4_OK) return s;
  *plan = w4_mm_plan{"none", 0, 0};
  if (M == 0) return ok();
  const w4::Epi ep = {};
  const w4::MmArgs a = make_args(dummy, M, static_cast<const int32_t*>(p), dummy, dummy, desc, transposed, ep);
  const w4::DeviceCaps caps = device_caps();
  if (w4::gemv_supported(a, caps)) {
    *plan = w4_mm_plan{w4::gemv_name(a), w4::gemv_lds_bytes(a, caps), 0};
    return ok();
  }
  *plan = w4_mm_plan{w4::gemm_name(a, caps, ws_bytes), w4::gemm_lds_bytes(a, caps, ws_bytes),
                     w4::gemm_used_workspace_bytes(a, caps, ws_bytes)};
  if (plan->lds_bytes > caps.lds)
    return fail(W4_ERR_RESOURCE, "GEMM tile needs %zu bytes of LDS, the device allows %zu", plan->lds_bytes,
                caps.lds);
  return ok();
}

static_assert(sizeof(w4_serial_header) == 128, "the serialized header is 128 bytes");

int w4_serial_layout(const w4_desc* desc, int zero_kind, w4_serial_header* hdr) {
  if (hdr == nullptr) return fail(W4_ERR_INVALID, "hdr is NULL");
  int s = check_desc(desc);
  if (s != W4_OK) return s;
  if (zero_kind != W4_ZERO_FP16 && zero_kind != W4_ZERO_INT)
    return fail(W4_ERR_INVALID, "zero_kind = %d is not W4_ZERO_FP16 or W4_ZERO_INT", zero_kind);
  int64_t pairs = 0;
  s = w4_meta_pairs(desc, &pairs);
  if (s != W4_OK) return s;
  auto up64 = [](uint64_t x) { return (x + 63) & ~(uint64_t)63; };
  w4_serial_header h;
  memset(&h, 0, sizeof(h));
  memcpy(h.magic, W4_SERIAL_MAGIC, sizeof(W4_SERIAL_MAGIC));
  h.version = W4_SERIAL_VERSION;
  h.header_bytes = sizeof(w4_serial_header);
  h.N = desc->N;
  h.K = desc->K;
  h.mode = desc->mode;
  h.group = desc->mode == W4_MODE_GROUPWISE ? desc->group : 0;
  h.zero_kind = zero_kind;
  h.packed_offset = up64(sizeof(w4_serial_header));
  h.packed_bytes = (uint64_t)desc->N * (uint64_t)(desc->K / 8) * 4;
  h.meta_bytes = (uint64_t)pairs * 2;
  h.scales_offset = up64(h.packed_offset + h.packed_bytes);
  h.zeros_offset = up64(h.scales_offset + h.meta_bytes);
  h.total_bytes = up64(h.zeros_offset + h.meta_bytes);
  *hdr = h;
  return ok();
}

int w4_serial_parse(const void* bytes, size_t len, w4_desc* desc, int* zero_kind) {
  if (bytes == nullptr || desc == nullptr || zero_kind == nullptr)
    return fail(W4_ERR_INVALID, "a required pointer is NULL");
  if (len < sizeof(w4_serial_header))
    return fail(W4_ERR_INVALID, "%zu bytes cannot hold the %zu-byte header", len, sizeof(w4_serial_header));
  w4_serial_header h;
  memcpy(&h, bytes, sizeof(h));
  if (memcmp(h.magic, W4_SERIAL_MAGIC, sizeof(W4_SERIAL_MAGIC)) != 0) return fail(W4_ERR_INVALID, "bad magic");
  if (h.version != W4_SERIAL_VERSION) return fail(W4_ERR_INVALID, "version %u is not %d", h.version, W4_SERIAL_VERSION);
  const w4_desc d = {h.N, h.K, h.mode, h.group};
  w4_serial_header want;
  int s = w4_serial_layout(&d, h.zero_kind, &want);
  if (s != W4_OK) return s;
  if (memcmp(&h, &want, sizeof(h)) != 0) return fail(W4_ERR_INVALID, "header sizes or offsets do not match the layout");
  if (h.total_bytes > len)
    return fail(W4_ERR_INVALID, "the weight needs %llu bytes, %zu are available", (unsigned long long)h.total_bytes,
                len);
  *desc = d;
  *zero_kind = h.zero_kind;
  return ok();
}

const char* w4_status_string(int status) {
  switch (status) {
    case W4_OK: return "W4_OK";
    case W4_ERR_INVALID: return "W4_ERR_INVALID";
    case W4_ERR_UNSUPPORTED: return "W4_ERR_UNSUPPORTED";
    case W4_ERR_ALIGN: return "W4_ERR_ALIGN";
    case W4_ERR_RESOURCE: return "W4_ERR_RESOURCE";
    case W4_ERR_LAUNCH: return "W4_ERR_LAUNCH";
  }
  return "W4_ERR_UNKNOWN";
}

const char* w4_last_error(void) { return g_last_error.c_str(); }

const char* w4_version(void) { return "w4a16-gfx950 0.1.0"; }

}  // extern "C"
