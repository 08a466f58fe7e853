/*
 * w4a16.h -- C ABI of the MI355X (gfx950) weight-only int4 library.
 *
 * Two operations, following these pages:
 *   - "Quantized LLM Inference with Triton Kernels" (anaaaiva/llm-quantization),
 *     Objectives 1-2: FP16 -> INT4 quantization with global / rowwise /
 *     groupwise scale and zero, packed into INT32 words; Y = X_bf16 @ W_int4^T.
 *   - "Re-write HQQ Fused Gemm Transpose" (pytorch/ao #185): the transposed
 *     product reads the same packed weights, scales and zeros, with no repacking.
 *   - "[Kernel] Adding bias epilogue support for cutlass_scaled_mm" (vLLM #5560):
 *     an optional fp32 bias added in the epilogue.
 *   - "Modify small-batched weight only quantization" (TensorRT-LLM #2213): the
 *     batched decode GEMV (M <= 4) at 4 bits with group size 128.
 *
 * Data layout (every buffer row-major and contiguous):
 *   W       [N][K]    fp32, fp16 or bf16 weights to quantize.
 *   packed  [N][K/8]  int32; code k = 8c + j of row n is bits 4j..4j+3 of word c.
 *   scales  fp16 bits: GLOBAL [1], ROWWISE [N], GROUPWISE [N][K/g] (group fastest).
 *   zeros   fp16 bits, same shape as scales.
 *   A       bf16 bits: X [M][K] (non-transposed) or dY [M][N] (transposed).
 *   Y       fp32: [M][N] (non-transposed) or [M][K] (transposed); w4a16_mm_out
 *           also writes bf16 / fp16 and splits the columns over up to 4 outputs.
 *   bias    optional, in the output dtype: length N (non-transposed) or K (transposed).
 *
 * Arithmetic:
 *   s = fp16_rne((max - min) / 15) per group, replaced by 1 when it is 0 or not
 *   finite; z = fp16_rne((0 - min) / s); q = clamp(rint(w / s + z), 0, 15), all
 *   in IEEE fp32.  When that z is not finite (a group whose range is below
 *   15 |min| / 65504, which only fp32 weights reach), the group is quantized as
 *   a constant one: s = 1 and z = fp16_rne(0 - min).  The matmul weight
 *   operand is bf16_rne((q - z) * s) and products accumulate in fp32.
 *
 * Ownership and execution: every pointer is a device pointer owned by the caller
 * (except the descriptor and the host out-parameters).  The library never
 * allocates, frees or synchronizes; work is enqueued on `stream` (a hipStream_t,
 * 0 = the null stream) and device faults surface at the caller's next
 * synchronization.  Entry points are thread-safe; the error detail is per thread.
 *
 * Errors: arguments are validated on the host before any launch.  On failure an
 * entry point returns a negative status, enqueues nothing and records a message
 * readable with w4_last_error().
 */
#ifndef W4A16_H
#define W4A16_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  W4_OK = 0,
  W4_ERR_INVALID = -1,     /* bad size, mode, group, null pointer, bias length */
  W4_ERR_UNSUPPORTED = -2, /* valid but not provided (e.g. matmul with K % 32 != 0) */
  W4_ERR_ALIGN = -3,       /* a pointer is not aligned as required */
  W4_ERR_RESOURCE = -4,    /* workspace too small or LDS footprint over the device limit */
  W4_ERR_LAUNCH = -5       /* the HIP runtime rejected a launch */
} w4_status;

typedef enum { W4_MODE_GLOBAL = 0, W4_MODE_ROWWISE = 1, W4_MODE_GROUPWISE = 2 } w4_mode;

typedef enum { W4_DT_F32 = 0, W4_DT_F16 = 1, W4_DT_BF16 = 2 } w4_dtype;

typedef enum { W4_OP_QUANTIZE = 0, W4_OP_MM = 1, W4_OP_MM_T = 2, W4_OP_DEQUANTIZE = 3 } w4_op;

/* Zero-point kind of a quantization: a real fp16 zero (the default), or an
 * integer zero point in [0, 15] (AWQ style), also stored in the fp16 zeros. */
typedef enum { W4_ZERO_FP16 = 0, W4_ZERO_INT = 1 } w4_zero_kind;

/* Shape and grouping of one quantized weight.  N >= 1 rows, K >= 8 columns,
 * K % 8 == 0.  `group` is the GROUPWISE group size g along K (a power of two in
 * [16, 4096] with K % g == 0); it is ignored for GLOBAL and ROWWISE. */
typedef struct {
  int64_t N;
  int64_t K;
  int32_t mode;  /* w4_mode */
  int32_t group;
} w4_desc;

/* Number of (scale, zero) pairs: 1 (GLOBAL), N (ROWWISE), N*K/g (GROUPWISE).
 * Host only. */
int w4_meta_pairs(const w4_desc* desc, int64_t* pairs);

/* Device workspace, in bytes, that `op` needs for this descriptor (0 if none);
 * M is the activation row count for the matmul ops.  For W4_OP_MM / W4_OP_MM_T
 * a nonzero size is optional: it is the fp32 scratch of a split-K GEMM
 * (S partial [M][out] planes, summed in a fixed order, so results stay
 * deterministic), which the library plans when the output has too few tiles to
 * fill the device.  Host only. */
int w4_workspace_bytes(const w4_desc* desc, int op, int64_t M, size_t* bytes);

/* Quantize and pack W [N][K] (dtype w_dtype) into packed [N][K/8] int32 and the
 * fp16 scales / zeros.  W must be 16-byte aligned; packed, scales and zeros
 * 4/2/2-byte aligned.  GLOBAL mode needs the workspace reported by
 * w4_workspace_bytes (two kernels: a min/max pass, then the quantize pass);
 * other modes take ws = NULL.  Source: Objective 1 of "Quantized LLM
 * Inference with Triton Kernels". */
int w4_quantize_pack(const void* W, int w_dtype, const w4_desc* desc,
                     int32_t* packed, uint16_t* scales, uint16_t* zeros,
                     void* ws, size_t ws_bytes, void* stream);

/* w4_quantize_pack with a choice of zero point.  W4_ZERO_FP16 is
 * w4_quantize_pack.  W4_ZERO_INT rounds the zero point to an integer, the AWQ
 * style of the W4A16 AWQ g = 128 workload of "Modify small-batched weight only
 * quantization":  z = clamp(rint((0 - min) / s), 0, 15),
 * q = clamp(rint(w / s) + z, 0, 15)  (s as above), so q - z is an integer and
 * the weight operand is bf16_rne((q - z) * s).  The zero is stored in the same
 * fp16 zeros array (exactly), so every other entry point reads either kind.
 * zero_kind outside these two is W4_ERR_INVALID; the rest is as for
 * w4_quantize_pack. */
int w4_quantize_pack_zp(const void* W, int w_dtype, const w4_desc* desc, int zero_kind,
                        int32_t* packed, uint16_t* scales, uint16_t* zeros,
                        void* ws, size_t ws_bytes, void* stream);

/* Dequantize packed weights to out [N][K]: out_dtype W4_DT_BF16 writes the
 * matmul operand bf16_rne(fp32(q - z) * s), W4_DT_F16 writes the fp16-activation
 * operand fp16_rne(fp32(q - z) * s), W4_DT_F32 writes fp32(q - z) * s.
 * Bit-exact with the definition above.  out must be 16-byte aligned.  Source:
 * the dequantize() reference path of "Re-write HQQ Fused Gemm Transpose". */
int w4_dequantize(const int32_t* packed, const uint16_t* scales, const uint16_t* zeros,
                  const w4_desc* desc, void* out, int out_dtype, void* stream);

/* W4A16 matmul on the packed weight of `desc`, fp32 accumulation, fp32 output.
 *   transposed == 0: Y[m][n] = sum_k A[m][k] * w[n][k] (+ bias[n]),  A = X  [M][K]
 *   transposed != 0: Y[m][k] = sum_n A[m][n] * w[n][k] (+ bias[k]),  A = dY [M][N]
 * where w[n][k] = bf16_rne((q - z) * s).  The transposed mode reads the same
 * packed, scales and zeros buffers.  M == 0 is a no-op.  K % 32 == 0 is
 * required, and the transposed mode also needs N % 8 == 0, N < 2^22 and
 * K <= 2^21 (W4_ERR_UNSUPPORTED otherwise).  A and packed must be 16-byte
 * aligned, Y and bias 4-byte aligned.  M <= 4 non-transposed runs the
 * memory-bound GEMV (no matrix cores); other shapes run the MFMA GEMM.  ws may
 * always be NULL: the GEMM then runs unsplit.  A workspace of at least the
 * bytes w4_workspace_bytes reports (16-byte aligned, owned by the caller, free
 * to reuse once the stream has run the call) lets a GEMM with few output tiles
 * split its contraction; a smaller one is ignored.  Sources: Objective 2 of
 * "Quantized LLM Inference with Triton Kernels"; "Re-write HQQ Fused Gemm
 * Transpose"; "[Kernel] Adding bias epilogue support for cutlass_scaled_mm";
 * "Modify small-batched weight only quantization". */
int w4a16_mm(const uint16_t* A, int64_t M, const int32_t* packed, const uint16_t* scales,
             const uint16_t* zeros, const w4_desc* desc, int transposed, const float* bias,
             float* Y, void* ws, size_t ws_bytes, void* stream);

/* w4a16_mm for callers that cannot allocate (code under HIP graph capture, tight
 * serving loops, harnesses that forbid it): the same operands, plan and results
 * as w4a16_mm given the workspace w4_workspace_bytes reports, with the split-K
 * partial planes in a static device scratch of the library (64 MiB per GPU,
 * held until the process ends) instead of a caller workspace.  A plan whose
 * planes need more returns W4_ERR_RESOURCE before anything is enqueued (call
 * w4a16_mm with a workspace then).  Every call on one GPU shares that GPU's
 * scratch: calls that overlap on one GPU (concurrent streams, or threads) race,
 * so serialize them.  Each plane is written whole before it is read, so nothing
 * carries over from the previous call.  The library does not allocate, free or
 * synchronize here either. */
int w4a16_mm_noalloc(const uint16_t* A, int64_t M, const int32_t* packed, const uint16_t* scales,
                     const uint16_t* zeros, const w4_desc* desc, int transposed, const float* bias,
                     float* Y, void* stream);

/* One output segment of w4a16_mm_out: it receives the next `cols` output columns
 * (segments cover the output columns in order), column j of the segment at row m
 * being Y[m * ld + j] in the call's out_dtype.  Y device pointer, ld >= cols. */
typedef struct {
  void* Y;
  int64_t cols;
  int64_t ld;
} w4_out_seg;

/* w4a16_mm with the activation dtype and the output epilogue spelled out:
 *   a_dtype W4_DT_BF16 (as w4a16_mm) or W4_DT_F16: fp16 activations multiply the
 *   fp16 weight operand fp16_rne(fp32(q - z) * s), fp32 accumulation;
 *   out = out_rne(acc + bias[c]) for output column c, acc the fp32 sum;
 *   out_dtype W4_DT_F32, W4_DT_BF16 or W4_DT_F16 (round to nearest even);
 *   bias NULL or outc values (N non-transposed, K transposed) in out_dtype,
 *   converted exactly to fp32 and added before the one rounding;
 *   segs[0 .. nsegs-1], 1 <= nsegs <= 4, split the outc output columns, so a
 *   fused Q/K/V weight writes Q, K and V to separate tensors in one launch.
 * The segment columns must sum to outc; each Y and the bias must be aligned to
 * the element size.  Everything else (operands, workspace, stream, errors) is
 * as for w4a16_mm, which equals this call with W4_DT_F32 and one segment of
 * ld = outc.  Sources: "[Kernel] Adding bias epilogue support for
 * cutlass_scaled_mm" (vLLM #5560: the bias in the output dtype); "Add fused QKV
 * HQQ triton_mm test" (pytorch/ao #306: one fused Q/K/V product). */
int w4a16_mm_out(const void* A, int a_dtype, int64_t M, const int32_t* packed,
                 const uint16_t* scales, const uint16_t* zeros, const w4_desc* desc,
                 int transposed, const void* bias, int out_dtype, const w4_out_seg* segs,
                 int nsegs, void* ws, size_t ws_bytes, void* stream);

/* Name of the kernel w4a16_mm would launch for these arguments ("gemv_m4",
 * "gemm_nt_256x128", "gemm_t_256x256_splitk4", ...) given the workspace
 * w4_workspace_bytes reports, or NULL when they are invalid.  Host only. */
const char* w4a16_mm_kernel(int64_t M, const w4_desc* desc, int transposed);

/* The launch w4a16_mm / w4a16_mm_out makes for these arguments when given a
 * workspace of ws_bytes (0: none): `kernel` is its kernel name, as
 * w4a16_mm_kernel reports it for the full workspace ("none" for M == 0; the
 * string lives in storage of the calling thread until its next call),
 * `lds_bytes` the LDS one workgroup of that kernel uses, and `workspace_bytes`
 * the part of the workspace it writes (0 when the contraction is not split;
 * a workspace smaller than the split plan needs is not used).  Returns
 * W4_ERR_RESOURCE when lds_bytes is above the device's limit (the matmul
 * would fail the same way), else the argument checks of w4a16_mm without its
 * pointers.  Host only. */
typedef struct {
  const char* kernel;
  size_t lds_bytes;
  size_t workspace_bytes;
} w4_mm_plan;
int w4a16_mm_plan(int64_t M, const w4_desc* desc, int transposed, size_t ws_bytes, w4_mm_plan* plan);

/* Serialized packed weight: this 128-byte little-endian header, then the packed
 * words [N][K/8] int32, the scales and the zeros (fp16 bits, w4_meta_pairs each),
 * every section starting at a 64-byte aligned offset from the start of the
 * header.  The packed words are also the INT8 packing of Objective 1 of
 * "Quantized LLM Inference with Triton Kernels" read as bytes. */
#define W4_SERIAL_MAGIC "W4A16PK"
#define W4_SERIAL_VERSION 1
typedef struct {
  char magic[8];          /* W4_SERIAL_MAGIC, NUL-terminated */
  uint32_t version;       /* W4_SERIAL_VERSION */
  uint32_t header_bytes;  /* 128 */
  int64_t N, K;
  int32_t mode, group;    /* as in w4_desc */
  int32_t zero_kind;      /* w4_zero_kind the zeros were made with */
  int32_t reserved0;
  uint64_t packed_offset, packed_bytes;
  uint64_t scales_offset, zeros_offset, meta_bytes;
  uint64_t total_bytes;   /* header + sections, a multiple of 64 */
  uint8_t reserved[32];
} w4_serial_header;

/* Fill *hdr for a weight of this descriptor and zero kind (sizes and offsets
 * included; reserved bytes zero).  Host only; W4_ERR_INVALID on a bad
 * descriptor, zero kind or NULL. */
int w4_serial_layout(const w4_desc* desc, int zero_kind, w4_serial_header* hdr);

/* Check a serialized header read from `bytes` (at least `len` bytes available)
 * and return its descriptor and zero kind: the magic, version, descriptor,
 * section sizes, 64-byte alignment, ordering and total size must all match what
 * w4_serial_layout gives, and total_bytes must not exceed len.  Host only;
 * W4_ERR_INVALID on any mismatch or NULL. */
int w4_serial_parse(const void* bytes, size_t len, w4_desc* desc, int* zero_kind);

/* Human-readable name of a status code. */
const char* w4_status_string(int status);

/* Detail of the last failure on the calling thread ("" if none). */
const char* w4_last_error(void);

/* Library version string. */
const char* w4_version(void);

#ifdef __cplusplus
}
#endif

#endif /* W4A16_H */
