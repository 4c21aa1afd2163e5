/*
 * ddg.h -- C ABI of libddg.so: low-bit (3..7 bit) per-group weight
 * quantization and the dequantize-on-the-fly GEMM of a diffusion-transformer
 * linear layer, for AMD Instinct MI355X (gfx950).
 *
 * Sources (cited by title and section):
 *   [WDQ]  The Wan-Dancer-14B mixed-precision quantization report (mtrt.cn):
 *          §3.1 per-group(128) symmetric quantization, §3.3 multi-bit packed
 *          storage and the stored record (packed / scales / bit width / padded
 *          input dimension), §3.4 GPU-native dequantize, §5.4 dequantize then
 *          bf16 matmul.
 *   [SVDQ] "SVDQuant：4-bit量化让扩散模型在消费级GPU上高效运行" (kongchang.com):
 *          section "技术原理详解" (16-bit low-rank branch plus quantized residual).
 *
 * Conventions shared by every entry point:
 *   - W is out x in = N x K, row-major; groups are 128 consecutive inputs of a
 *     row ([WDQ] §3.1).  K must be a positive multiple of 128; a caller with
 *     another input size zero-pads W and X to the next multiple of 128 (the
 *     record's padded input dimension, [WDQ] §3.3).
 *   - Quantizer ([WDQ] §3.1), all in IEEE float32:
 *       a = max |w| over the group;  step = (2 * fl(a * 1.01f)) / (2^bits - 1);
 *       q = clamp(round_half_even(fl(w / step)), -n_half, n_half),
 *       n_half = 2^(bits-1) - 1;  code q_u = q + n_half in [0, 2^bits - 2];
 *       scale = step.  An all-zero group gets q = 0 and scale 0.  The
 *       products rely on that code range: a record holding the all-ones code
 *       2^bits - 1 (which the quantizer never writes) gives undefined outputs.
 *   - Packed layout ([WDQ] §3.3): the row-major codes form one continuous
 *     bitstream, each code written with `bits` bits, most significant bit
 *     first; stream bit 0 is the MSB of byte 0.  A row takes K*bits/8 bytes,
 *     a group 16*bits bytes.  For bits = 4 the even-index code is the high
 *     nibble.  Total N*K*bits/8 bytes.
 *   - Scales: float32, N x (K/128), row-major.
 *   - Dequantized weight fed to the matmul ([WDQ] §3.4, §5.4):
 *       w_hat = bf16_round_nearest_even(fl32((q_u - n_half) * scale)).
 *   - X is M x K bf16 row-major; Y is M x N row-major, bf16 or float32;
 *     products accumulate in float32.  Y is overwritten, never accumulated.
 *
 * Memory, streams, errors:
 *   - Every buffer pointer is a DEVICE pointer owned by the caller; the
 *     library never allocates, frees or synchronizes.  Buffers must not
 *     overlap, except as stated.
 *   - Every launch is asynchronous on `stream` (0 = the default stream).
 *     Calls keep no mutable state between calls and may come from any thread.
 *   - Return value: DDG_OK (0) or a negative ddg_status.  Arguments are
 *     validated on the host before anything is launched; on error nothing is
 *     launched and no memory is touched.  DDG_ERR_HIP means a launch failed
 *     (the HIP error is left for hipGetLastError).
 *   - Alignment: x, w, packed, y, lora_* and workspace must be 16-byte
 *     aligned; scales 4-byte aligned.
 */
#ifndef DDG_H
#define DDG_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define DDG_GROUP 128      /* weights per scale ([WDQ] §3.1) */
/* Most weights (n * k; for the FP4/FP6 quantizers with n padded to a
 * multiple of 32) that a weight quantizer or ddg_dequantize takes in one
 * call: one lane per 32 weights keeps the launch below 2^32 work-items. */
#define DDG_CHUNK_WEIGHTS_MAX ((INT64_C(1) << 37) - 8192)
#define DDG_VERSION 1

typedef enum ddg_dtype {
  DDG_BF16 = 0,
  DDG_F32 = 1
} ddg_dtype;

typedef enum ddg_status {
  DDG_OK = 0,
  DDG_ERR_ARG = -1,          /* null pointer, bad enum, bits outside 3..7   */
  DDG_ERR_SHAPE = -2,        /* sizes not allowed (see each call)           */
  DDG_ERR_ALIGN = -3,        /* pointer misaligned                          */
  DDG_ERR_WORKSPACE = -4,    /* workspace smaller than required             */
  DDG_ERR_HIP = -5,          /* a HIP launch or query failed                */
  DDG_ERR_UNSUPPORTED = -6   /* no gfx950 device current                    */
} ddg_status;

/* Library version (DDG_VERSION). */
int ddg_version(void);

/* Text for a status code (static string, never NULL). */
const char* ddg_status_string(int status);

/*
 * Sizes of the packed record for an N x K weight at `bits` ([WDQ] §3.3 table:
 * 3 bit 8 weights -> 3 bytes, 4 bit 2 -> 1, 5 bit 8 -> 5, 6 bit 4 -> 3,
 * 7 bit 8 -> 7).  Host-only, no device access.
 *   packed_bytes <- N*K*bits/8,  n_scales <- N*K/128.
 * Errors: DDG_ERR_ARG (null output, bits), DDG_ERR_SHAPE (n < 0, k not a
 * positive multiple of 128, overflow).
 */
int ddg_packed_bytes(int64_t n, int64_t k, int bits, int64_t* packed_bytes,
                     int64_t* n_scales);

/*
 * Quantize and pack ([WDQ] §3.1 quantizer, §3.3 packing).
 *   w       N x K weights, bf16 or float32 (w_dtype), finite values.
 *   packed  out: N*K*bits/8 bytes (layout above), fully written.
 *   scales  out: N*(K/128) float32, fully written.
 * Results are bit-exact: the arithmetic is the IEEE float32 sequence above
 * (correctly rounded multiply and divide, no fused operations, subnormals
 * kept).  n == 0 is a no-op.
 * Errors: DDG_ERR_ARG, DDG_ERR_SHAPE (n < 0; k not a positive multiple of
 * 128; n * k above DDG_CHUNK_WEIGHTS_MAX), DDG_ERR_ALIGN, DDG_ERR_HIP.
 */
int ddg_quantize_pack(const void* w, int w_dtype, int64_t n, int64_t k, int bits,
                      uint8_t* packed, float* scales, hipStream_t stream);

/*
 * Dense dequantization ([WDQ] §3.4): w_out (N x K bf16) = w_hat for every
 * weight.  For checking and for callers that want a dense copy; the GEMM
 * below never materializes it.  n == 0 is a no-op.
 * Errors: as ddg_quantize_pack.
 */
int ddg_dequantize(const uint8_t* packed, const float* scales, int bits, int64_t n,
                   int64_t k, void* w_out, hipStream_t stream);

/*
 * Y = X * w_hat^T ([WDQ] §3.4 + §5.4, dequantizing inside the GEMM).
 *   x       M x K bf16.       packed/scales: the record of an N x K weight.
 *   y       M x N, y_dtype (DDG_BF16 or DDG_F32), fully overwritten.
 *   workspace, workspace_bytes
 *           optional device scratch (NULL, 0: none; 16-byte aligned).  With
 *           at least ddg_workspace_bytes(M, N, K, 0) bytes, K may be split
 *           across workgroups, partial sums exchanged through the workspace:
 *           products with M > 64 whose output tiles would fill the compute
 *           units unevenly (split-K, stream-K), and products with M <= 16 and
 *           K >= 8192 whose outputs are narrow (fewer than 12800 columns).
 *           Its contents need no initialisation and are scratch afterwards;
 *           calls that share a workspace must be ordered (one stream).
 *           Results then differ from the call without workspace only in
 *           float32 summation order (the same on every call).
 *           Graph capture: the exchange is tagged with an epoch that the
 *           host draws per call, so a captured call that splits K would
 *           repeat its epoch on every replay and could read an earlier
 *           replay's partial sums.  Under capture, pass no workspace.
 * Requirements: M >= 0 (M == 0 is a no-op), N a positive multiple of 16,
 * K a positive multiple of 128 and at most 2^20, M, N <= 2^31 - 1.
 * Errors: DDG_ERR_ARG, DDG_ERR_SHAPE, DDG_ERR_ALIGN, DDG_ERR_HIP.
 */
int ddg_dequant_gemm(const void* x, int64_t m, int64_t k, const uint8_t* packed,
                     const float* scales, int bits, int64_t n, void* y, int y_dtype,
                     void* workspace, size_t workspace_bytes, hipStream_t stream);

/* One product of a grouped call: y = x * w_hat^T, arguments as in
 * ddg_dequant_gemm. */
typedef struct ddg_gemm_desc {
  const void* x;            /* M x K bf16                                   */
  const uint8_t* packed;    /* record of an N x K weight at `bits`          */
  const float* scales;
  void* y;                  /* M x N, y_dtype                               */
  int64_t m, k, n;
  int bits;
  int y_dtype;
} ddg_gemm_desc;

#define DDG_MAX_GROUPED 256   /* products per ddg_dequant_gemm_grouped call */

/*
 * Several independent products in as few launches as possible ([WDQ] §1.3
 * and §3.4: packed weights stay resident and are dequantized per block on
 * the fly; §3.2: each tensor gets its own bit width, so e.g. the q, k and v
 * projections of a block cannot share one packed tensor).  Equivalent to
 * ddg_dequant_gemm on every descriptor, with every requirement of that call.
 * Products go into one launch per 16 products (mixed bit widths and shapes)
 * of the same class: M <= 16; 16 < M <= 32; 32 < M <= 64; M > 64 (the
 * large-M kernel's 256 x 256 tiles, deepest K first; these results equal
 * bit for bit those of a separate call that takes the same whole tiles, i.e.
 * one without K split and without 256 x 192 tiles).  All launches are on
 * `stream`.
 *   descs   host array of `count` descriptors, read during the call only.
 *   count   0 .. DDG_MAX_GROUPED (0 is a no-op).
 * No y may overlap another product's inputs or output.  Results equal those
 * of separate calls up to floating-point summation order.
 * Errors: as ddg_dequant_gemm, for the first failing descriptor (nothing is
 * launched then), DDG_ERR_ARG for a null descs with count > 0, DDG_ERR_SHAPE
 * for count outside 0..DDG_MAX_GROUPED.
 */
int ddg_dequant_gemm_grouped(const ddg_gemm_desc* descs, int count, hipStream_t stream);

/*
 * Workspace bytes for an M x K input and an N x K weight: with r = 0, what
 * ddg_dequant_gemm can use for split K (M > 64: 64 MiB of partial sums and
 * a flag per workgroup where the output has fewer than 1024 tiles of
 * 256 x 256; M <= 16, K >= 8192, N < 12800: 8 KiB of partial sums and 64
 * bytes of flags per 16 output columns, padded to 64 columns; else 0); with
 * rank r, what ddg_lowrank_fused_gemm needs: the M x r bf16 intermediate T,
 * rounded up to 256 bytes, followed by that split-K area and, for M <= 64
 * and K >= 1024, the float32 partials of the T pre-pass split over K
 * (ceil(G / c) chunks of c = ceil(G / 32) groups, G = K / 128, times M x r
 * floats, rounded up to 256).
 * Host-only.
 * Errors: DDG_ERR_ARG (null), DDG_ERR_SHAPE (m, n or k negative or m, n above
 * 2^31 - 1, r not 0 and outside 8..128 or not a multiple of 8).
 */
int ddg_workspace_bytes(int64_t m, int64_t n, int64_t k, int r, size_t* bytes);

/*
 * T = bf16(X * L1) on its own: the down projection of the 16-bit low-rank
 * branch ([SVDQ] 技术原理详解: the branch is a product with the two factors
 * of the SVD, kept in 16 bits).  ddg_lowrank_fused_gemm runs this pre-pass
 * into its workspace before its product (for M <= 64, given room for its
 * partials, the same sums split over K, which may differ in the last bf16
 * place).  This call is for callers that keep T, for example to check or
 * time it.
 *   x          device, M x K bf16, row-major
 *   lora_down  device, r x K bf16 = L1^T (row j: the j-th input projection)
 *   t          device, M x r bf16, row-major (output, fully overwritten; the
 *              caller owns it)
 * Each element is summed in float32 and rounded to bf16 once.
 * Requirements: K a positive multiple of 128, at most 2^20; 8 <= r <= 128,
 * r % 8 == 0; M at most 2^28 - 16 (16 rows per workgroup of 256 lanes keeps
 * the launch below 2^32 work-items); x, lora_down and t 16-byte aligned.
 * M == 0 is a no-op.
 * Errors: DDG_ERR_SHAPE (M negative or above 2^28 - 16, K or r out of range),
 * DDG_ERR_ARG (null pointer), DDG_ERR_ALIGN, DDG_ERR_HIP.
 */
int ddg_lowrank_down(const void* x, int64_t m, int64_t k, const void* lora_down, int r, void* t,
                     hipStream_t stream);

/*
 * Y = X * w_hat^T + T * L2 with T = bf16(X * L1)  ([SVDQ] 技术原理详解: a
 * 16-bit low-rank branch beside the quantized residual; the residual's record
 * is packed/scales).  The low-rank factors are passed in the layout of linear
 * weights (out x in):
 *   lora_down  r x K bf16  = L1^T   (row j: the j-th input projection)
 *   lora_up    N x r bf16  = L2^T   (row n: output n's branch weights)
 * T is computed in float32 and rounded to bf16 once (the branch is a bf16
 * product); the branch term T * L2 is summed into the same float32
 * accumulator as the main product before y is written.
 *   workspace  device scratch: T first (M * r * 2 bytes rounded up to 256,
 *              required), then optionally the split-K area of
 *              ddg_dequant_gemm and, for M <= 64 and K >= 1024, the T
 *              pre-pass's partials; ddg_workspace_bytes(M, N, K, r) bytes
 *              hold all three.  With room for the partials, the pre-pass
 *              splits K over workgroups and adds the partials in a fixed
 *              order (T may then differ from the unsplit pre-pass's in the
 *              last bf16 place; either way it repeats bit for bit).  Its
 *              contents are scratch (no initial state needed).  Under graph
 *              capture, pass a workspace of T's bytes alone (whole tiles and
 *              the unsplit pre-pass; see ddg_dequant_gemm), or call
 *              ddg_lowrank_fused_gemm_noalloc.
 * Requirements: as ddg_dequant_gemm, plus 8 <= r <= 128, r % 8 == 0, and
 * M at most 2^28 - 16 (the T pre-pass gives 16 rows to each workgroup of
 * 256 lanes, and a launch stays below 2^32 work-items).
 * Errors: DDG_ERR_ARG, DDG_ERR_SHAPE, DDG_ERR_ALIGN, DDG_ERR_WORKSPACE,
 * DDG_ERR_HIP.
 */
int ddg_lowrank_fused_gemm(const void* x, int64_t m, int64_t k, const uint8_t* packed,
                           const float* scales, int bits, int64_t n,
                           const void* lora_down, const void* lora_up, int r,
                           void* y, int y_dtype, void* workspace,
                           size_t workspace_bytes, hipStream_t stream);

/*
 * ddg_lowrank_fused_gemm for callers that cannot allocate device memory
 * (code under HIP graph capture, tight serving loops, harnesses that forbid
 * allocation): the same arguments without `workspace`, and the results of
 * ddg_lowrank_fused_gemm given a workspace of T's bytes alone (whole output
 * tiles, K never split across workgroups; with a larger workspace that call
 * may split K, which sums in another order).  T goes to
 * a device array of DDG_NOALLOC_SCRATCH_BYTES bytes inside the library, one
 * per GPU, held from the first call on that GPU until the process ends (the
 * first call on a GPU looks up its address; no call allocates).  Every call on
 * a GPU shares that GPU's array: calls that overlap on one GPU (other streams,
 * other threads) race and give undefined results; calls on one stream are
 * ordered and safe.  Requirements and errors as ddg_lowrank_fused_gemm, plus
 * DDG_ERR_WORKSPACE when T needs more than the array (M * r * 2 bytes, rounded
 * up to 256, above DDG_NOALLOC_SCRATCH_BYTES: M * r up to 4,194,304, e.g.
 * 32768 tokens at rank 128).
 */
#define DDG_NOALLOC_SCRATCH_BYTES (8 * 1024 * 1024)
int ddg_lowrank_fused_gemm_noalloc(const void* x, int64_t m, int64_t k, const uint8_t* packed,
                                   const float* scales, int bits, int64_t n,
                                   const void* lora_down, const void* lora_up, int r,
                                   void* y, int y_dtype, hipStream_t stream);

/*
 * Quantization error of an N x K weight at every width 3..7 ([WDQ] §3.2:
 * the per-tensor error tables the bit allocation searches over; §3.1: the
 * quantizer of ddg_quantize_pack, float32 arithmetic bit for bit):
 *   row_sse[5 i + (b - 3)] = sum over row i of (w - w_hat32)^2,
 *   w_hat32 = fl32((q_u - n_half) * scale), summed in float64;
 *   total_sse[b - 3] = the rows' sum in a fixed order (deterministic).
 *   w          N x K bf16 or float32 (w_dtype), finite.
 *   row_sse    device, N x 5 doubles (also the scratch of the total).
 *   total_sse  device, 5 doubles.
 * n == 0 writes zero totals.  Errors: DDG_ERR_ARG, DDG_ERR_SHAPE (n < 0 or
 * above DDG_SSE_ROWS_MAX (one workgroup of up to 256 lanes per row: the launch
 * stays below 2^32 work-items), k not a positive multiple of 128 or above
 * 2^31), DDG_ERR_ALIGN (w 16-byte, the outputs 8-byte), DDG_ERR_HIP,
 * DDG_ERR_UNSUPPORTED.
 */
#define DDG_SSE_ROWS_MAX ((INT64_C(1) << 24) - 1)
int ddg_quant_sse(const void* w, int w_dtype, int64_t n, int64_t k, double* row_sse,
                  double* total_sse, hipStream_t stream);

/*
 * PD-guided mixed-precision bit allocation ([WDQ] §3.2).  Host only: every
 * pointer is a host pointer and nothing runs on the GPU.  With the per-weight
 * errors mse_i(c) = sse_i(c) / n_i (float64 division), minimises the
 * parameter-weighted error sum_i n_i mse_i(b_i) / sum_i n_i (the section's
 * sum of squared errors over the weight count) subject to
 * sum_i n_i b_i / sum_i n_i <= target_bpw by the section's relaxation: one
 * parameter per tensor, b = bmin + sigmoid(t) (bmax - bmin); a softmax over
 * the candidates of -|b - c| / temp, temp = max(2 (1 - it/iters), 0.05),
 * blends the tensor's error row (in percent of the error of the uniform
 * allocation at the candidate nearest the target); loss = error
 * + lambda (bpw - target) + 1e4 (bpw - target)^2.  Plain gradient descent on
 * the parameters and ascent on lambda (from 0.5), both with the step 1/L,
 * L = 2e4 ((bmax - bmin)/4)^2 sum_i (n_i / sum n)^2 the Lipschitz bound of the
 * penalty's gradient.  Each restart's widths come from largest-remainder
 * rounding within the budget: every tensor starts at the candidate at or below
 * its width, then moves up one candidate, by decreasing fraction of the way
 * there (lower index first on ties), while the added bits fit in
 * target * sum n.  The kept restart has the lowest exact error within the
 * budget, else the lowest bpw; ties go to the earlier restart.  Restarts run
 * on up to 16 host threads started and joined inside the call (the inputs are
 * only read meanwhile); the result does not depend on their number.
 *   sse        n x ncand squared-error sums (row i: tensor i, column c: width
 *              candidates[c]; the totals of ddg_quant_sse); finite, >= 0.
 *   nparams    n weight counts, > 0.
 *   candidates ncand (2..8) increasing widths; target_bpw within their range.
 *   t_init     restarts x n starting parameters (the random draws).
 *   bits_out   n chosen widths.
 *   info       NULL or 3 doubles: error, bpw, kept restart.
 * Errors: DDG_ERR_ARG (null pointer, bad table entry, candidates not
 * increasing, target out of range), DDG_ERR_SHAPE (n < 1, ncand outside
 * 2..8, restarts or iters < 1).
 */
int ddg_pd_allocate(const double* sse, const int64_t* nparams, int n, const int* candidates,
                    int ncand, double target_bpw, const double* t_init, int restarts,
                    int iters, int* bits_out, double* info);

/*
 * Random-permuted block-Hadamard (RPBH) rotation of rows (the OrbitQuant
 * article, §2.1 "rotation quantization", §2.2 "offline-online"): for each of the
 * n rows of x (n x d, row-major),
 *   out[r, b h + j] = sum_t H[j, t] / sqrt(h) * s[b h + t] * x[r, perm[b h + t]],
 * H the Sylvester Walsh-Hadamard matrix of order h (H_2k = [[H_k, H_k],
 * [H_k, -H_k]]), s = -1 where signs[i] < 0, else +1.  With perm a permutation
 * of 0..d-1 the map is orthogonal: rotating the weight rows offline (then
 * quantizing them) and the activation rows online leaves X W^T unchanged.
 * Arithmetic in float32 (butterfly order fixed); bf16 outputs are rounded to
 * nearest even.
 *   x, out     device, n x d, x_dtype / out_dtype (DDG_BF16 or DDG_F32),
 *              16-byte aligned.  out may be x itself when the dtypes match;
 *              otherwise the buffers must not overlap.
 *   perm       device, d int32 (4-byte aligned); entries outside [0, d) read as 0.
 *   signs      device, d int8.
 *   h          block size: a power of two, 2..DDG_ROTATE_MAX_H, dividing d.
 *   d          a multiple of 64, at most DDG_ROTATE_MAX_D.
 * n == 0 is a no-op.  Errors: DDG_ERR_ARG (dtype, null pointer, overlapping
 * buffers), DDG_ERR_SHAPE, DDG_ERR_ALIGN, DDG_ERR_HIP, DDG_ERR_UNSUPPORTED.
 */
#define DDG_ROTATE_MAX_D 16384
#define DDG_ROTATE_MAX_H 1024
int ddg_rpbh_rotate(const void* x, int x_dtype, int64_t n, int64_t d, const int32_t* perm,
                    const int8_t* signs, int h, void* out, int out_dtype, hipStream_t stream);

/*
 * FP4 weights and FP8 activations (W4A8), the FP4DiT article: 4-bit
 * floating-point weight formats in groups of 128 (§3.2.1, §4.1) and 8-bit
 * per-token activations (§3.2.3), multiplied on the gfx950 scaled matrix
 * instructions.
 *
 * Formats (sign + magnitude, subnormal when the exponent field is 0):
 *   DDG_FP4_E2M1  bias 1: 0 .5 1 1.5 2 3 4 6
 *   DDG_FP4_E3M0  bias 3: 0 .25 .5 1 2 4 8 16
 *   DDG_FP4_E1M2  bias 1: 0 .25 .5 .75 1 1.25 1.5 1.75
 * code = sign << 3 | magnitude index (a zero magnitude is always code 0).
 */
#define DDG_FP4_E2M1 0
#define DDG_FP4_E3M0 1
#define DDG_FP4_E1M2 2
/*
 * OR-ed into fmt: power-of-two group scales, the block-scale form (E8M0) the
 * gfx950 matrix instructions apply themselves.  The quantizer rounds each
 * group's s up to the next power of two (at least 2^-126; s = 0 stays 0) and
 * quantizes with it; the product then passes each scale's exponent field to
 * the instruction instead of rescaling partial sums.  Scales stay float32 in
 * memory.  The product reads only the exponent field of each scale in this
 * mode, so its wscales must come from the quantizer in the same mode.
 * Weights beyond 2^127 times the format's largest value are not supported.
 */
#define DDG_FP4_POW2 0x100
/*
 * OR-ed into fmt: tiled storage, the same codes and scales reordered for the
 * matrix instructions so that each operand load reads one contiguous 1 KB
 * piece.  Columns go in blocks of 32, the last padded with zero codes and
 * zero scales; blocks are stored in (block, group) order, 2048 bytes each:
 * byte 1024 s + 512 h + 16 j + t of record (b, g) is byte 32 s + 16 h + t
 * of column 32 b + j's 64-byte slice of group g in the row storage.  Scales:
 * 32 floats per record, column 32 b + j at position j.  Sizes:
 * ceil(n/32) * (k/128) * 2048 bytes and ceil(n/32) * (k/128) * 32 floats.
 * The product must be told the storage its weights were written in.
 */
#define DDG_FP4_TILED 0x200

/*
 * Per group of 128 weights along K: s = fl32(amax / vmax), r = fl32(w / s)
 * (correctly rounded), code = the level nearest |r| (ties to the even code);
 * an all-zero group gets s = 0 and codes 0.  packed: n x k/2 bytes, code 2i
 * in the low nibble of byte i of its row; scales: n x k/128 floats (or the
 * tiled storage with DDG_FP4_TILED).
 *   w       device, n x k bf16 or float32 (w_dtype), finite, 16-byte aligned.
 *   packed  device, 16-byte aligned.   scales  device, 4-byte aligned.
 * n == 0 is a no-op.  Errors: DDG_ERR_ARG (fmt, dtype, null), DDG_ERR_SHAPE
 * (k not a positive multiple of 128; ceil(n/32) * 32 * k above
 * DDG_CHUNK_WEIGHTS_MAX), DDG_ERR_ALIGN, DDG_ERR_HIP, DDG_ERR_UNSUPPORTED.
 */
int ddg_fp4_quantize_pack(const void* w, int w_dtype, int64_t n, int64_t k, int fmt,
                          uint8_t* packed, float* scales, hipStream_t stream);

/*
 * Per token (row) of x (m x k bf16): s_x = fl32(amax / 448), r = fl32(x / s_x),
 * xq = the E4M3 code of r (|r| clamped to 448, round to nearest even; E4M3:
 * bias 7, subnormals, largest 448); an all-zero row gets s_x = 0 and zeros.
 *   x   device, 16-byte aligned.  xq  device m x k bytes, 8-byte aligned.
 *   xscales  device, m floats.
 * Errors: DDG_ERR_ARG, DDG_ERR_SHAPE (m above DDG_FP8_ROWS_MAX: one workgroup
 * of 256 lanes per row keeps the launch below 2^32 work-items; k not a
 * positive multiple of 128), DDG_ERR_ALIGN, DDG_ERR_HIP, DDG_ERR_UNSUPPORTED.
 */
#define DDG_FP8_ROWS_MAX ((INT64_C(1) << 24) - 1)
int ddg_fp8_quantize_rows(const void* x, int64_t m, int64_t k, uint8_t* xq, float* xscales,
                          hipStream_t stream);

/*
 * Y[m, n] = s_x[m] * sum_g s_w[n, g] * sum_{k in g} q_x[m, k] v_w[n, k]
 * (q_x, v_w the E4M3 and FP4 values), accumulated in float32 on the matrix
 * cores; y (m x n) in bf16 (rounded once) or float32.  Inputs as written by
 * the two calls above.  DDG_FP4_E2M1 weights enter the matrix instructions as
 * FP4 operands; E3M0 and E1M2 (not matrix formats, every value exact in E4M3)
 * as FP8 operands converted in registers.
 * m == 0 is a no-op.  Errors: DDG_ERR_ARG, DDG_ERR_SHAPE (k a positive
 * multiple of 128 up to 2^20, n >= 1), DDG_ERR_ALIGN (xq, packed 16 bytes),
 * DDG_ERR_HIP, DDG_ERR_UNSUPPORTED.
 */
int ddg_w4a8_gemm(const uint8_t* xq, const float* xscales, int64_t m, int64_t k,
                  const uint8_t* packed, const float* wscales, int fmt, int64_t n, void* y,
                  int y_dtype, hipStream_t stream);

/*
 * 6-bit activations (W4A6), the FP4DiT article §3.2.3 / §4.1 (W4A6) and §3.3
 * (FP6 saves memory over FP8).  Formats (sign + magnitude, subnormal when the
 * exponent field is 0, no infinities):
 *   DDG_FP6_E2M3  bias 1, largest 7.5
 *   DDG_FP6_E3M2  bias 3, largest 28
 */
#define DDG_FP6_E2M3 0
#define DDG_FP6_E3M2 1

/*
 * Per token (row) of x (m x k bf16): s_x = fl32(amax / vmax), r = fl32(x / s_x),
 * code = the nearest FP6 value to |r| (|r| clamped to vmax, ties to the even
 * code), sign in bit 5; an all-zero row gets s_x = 0 and zeros.  xq is the
 * tiled 6-bit storage the product reads: rows padded to a multiple of 32 with
 * zero codes; the 32 codes of (row, group g, 64-wide step s, half h), k =
 * 128 g + 64 s + 32 h + j, form a 192-bit little-endian string (code j at bits
 * 6 j) cut into three 8-byte pieces u; piece u of row 32 b + r is at byte
 * ((2 s + h) * 3 + u) * 256 + 8 r of record (b, g), 3072 bytes, records in
 * (b, g) order.  Size: ceil(m/32) * (k/128) * 3072 bytes.
 *   x   device, 16-byte aligned.  xq  device, 16-byte aligned.
 *   xscales  device, m floats.
 * m == 0 is a no-op.  Errors: DDG_ERR_ARG, DDG_ERR_SHAPE (m above
 * DDG_FP6_ROWS_MAX: 1024 lanes per 16 rows keep the launch below 2^32
 * work-items; k not a positive multiple of 128), DDG_ERR_ALIGN, DDG_ERR_HIP,
 * DDG_ERR_UNSUPPORTED.
 */
#define DDG_FP6_ROWS_MAX ((INT64_C(1) << 26) - 32)
int ddg_fp6_quantize_rows(const void* x, int64_t m, int64_t k, int fmt6, uint8_t* xq, float* xscales,
                          hipStream_t stream);

/*
 * Y[m, n] = s_x[m] * sum_g s_w[n, g] * sum_{k in g} q_x[m, k] v_w[n, k] with q_x
 * the FP6 values of ddg_fp6_quantize_rows (format fmt6) and v_w FP4 weights
 * in tiled storage (fmt = a format | DDG_FP4_TILED, optionally
 * | DDG_FP4_POW2): E2M1 on the FP6 x FP4 matrix instructions, E3M0 and E1M2
 * as FP8 operands (FP6 x FP8); float32 accumulation.  Row storage:
 * DDG_ERR_ARG.  Other arguments and errors as ddg_w4a8_gemm.
 */
int ddg_w4a6_gemm(const uint8_t* xq, const float* xscales, int64_t m, int64_t k, int fmt6,
                  const uint8_t* packed, const float* wscales, int fmt, int64_t n, void* y,
                  int y_dtype, hipStream_t stream);

/*
 * FP6 weights (W6A8).  The FP4DiT article quantizes weights to 4 bits and
 * names FP6 for activations (§3.2.3, §4.1 W4A6), arguing that FP6 saves
 * memory over FP8 (§3.3); this library also offers the two FP6 formats for
 * weights, multiplied with the E4M3 activations of ddg_fp8_quantize_rows on
 * the FP8 x FP6 matrix instructions.
 *
 * Quantizer: per group of 128 weights along K, as ddg_fp4_quantize_pack
 * with the FP6 levels: s = fl32(amax / vmax) (vmax 7.5 or 28; with
 * DDG_FP4_POW2 OR-ed into fmt6 the smallest power of two at least that, and
 * at least 2^-126), r = fl32(w / s) correctly rounded, code = the level
 * nearest |r| (ties to the even code), sign in bit 5; an all-zero group gets
 * s = 0 and codes 0.  packed: the tiled 6-bit storage of
 * ddg_fp6_quantize_rows with the weight's rows (output channels) in place of
 * tokens, ceil(n/32) * (k/128) * 3072 bytes; scales: the tiled order of
 * DDG_FP4_TILED, ceil(n/32) * (k/128) * 32 floats (padding rows: zero codes
 * and scales).
 *   w       device, n x k bf16 or float32 (w_dtype), finite, 16-byte aligned.
 *   packed  device, 16-byte aligned.   scales  device, 4-byte aligned.
 * n == 0 is a no-op.  Errors: DDG_ERR_ARG (fmt6, dtype, null), DDG_ERR_SHAPE
 * (k not a positive multiple of 128, n above 2^31 - 1, ceil(n/32) * 32 * k
 * above DDG_CHUNK_WEIGHTS_MAX), DDG_ERR_ALIGN, DDG_ERR_HIP, DDG_ERR_UNSUPPORTED.
 */
int ddg_fp6_quantize_pack(const void* w, int w_dtype, int64_t n, int64_t k, int fmt6,
                          uint8_t* packed, float* scales, hipStream_t stream);

/*
 * Y[m, n] = s_x[m] * sum_g s_w[n, g] * sum_{k in g} q_x[m, k] v_w[n, k] with q_x
 * the E4M3 values of ddg_fp8_quantize_rows and v_w the FP6 weights of
 * ddg_fp6_quantize_pack (fmt6, with DDG_FP4_POW2 exactly when the weights
 * were quantized with it: the product then applies each scale's exponent
 * field as the instruction's block scale); float32 accumulation, y (m x n)
 * in bf16 (rounded once) or float32.  Other arguments and errors as
 * ddg_w4a8_gemm.
 */
int ddg_w6a8_gemm(const uint8_t* xq, const float* xscales, int64_t m, int64_t k,
                  const uint8_t* packed, const float* wscales, int fmt6, int64_t n, void* y,
                  int y_dtype, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* DDG_H */
