/*
 * fp8blk -- fine-grained block-scaled FP8 quantization and block-scaled FP8
 * GEMM for AMD Instinct MI355X (gfx950).  C ABI.
 *
 * Pages cited (titles as published):
 *   [Fireworks-QAT] "DeepSeek R1 and V3 get quantization-aware fine-tuning on
 *                   Fireworks, keeping FP8 serving without the accuracy drop",
 *                   sections Synopsis and Interpretation.
 *   [DSV3-Blog5]    "DeepSeek-V3 Blog 5: Low-Precision Training - The FP8
 *                   Revolution in Large-Scale AI", sections "The Solution:
 *                   Block-Wise Quantization" and "Hardware Optimization:
 *                   Leveraging NVIDIA Tensor Cores for FP8".
 *   [FP8-DSV3-ru]   "FP8 в DeepSeek V3: как низкая точность ускоряет обучение
 *                   и инференс", sections "Как FP8 встроен в DeepSeek V3",
 *                   "Почему обычное округление не подходит", "Инференс с FP8",
 *                   "Почему FP8 требует scale factors".
 *   [prequant]      "fireworks-prequant 0.1.0", sections "Quick start" and
 *                   "Formats" (MXFP8: 1x32 blocks, E8M0 scales; the
 *                   routed-expert rule).
 *
 * Conventions shared by every entry point
 *   - Tensor pointers are DEVICE pointers (memory of the current HIP device)
 *     holding dense row-major matrices; the last index is contiguous.  bf16
 *     travels as uint16_t bit patterns, FP8 e4m3fn codes as uint8_t.
 *   - The caller allocates and owns every buffer; the library allocates
 *     nothing, keeps no per-call state and never synchronizes.  Work is
 *     enqueued on `stream` (a hipStream_t passed as void*, NULL = the
 *     default stream) and runs asynchronously.
 *   - Arguments are validated on the host before anything is enqueued; a
 *     nonzero fp8_status is returned and nothing is launched.  A launch
 *     failure reported by the runtime returns FP8_ERR_HIP.  Device-side
 *     faults caused by invalid pointers are not detectable here.
 *   - Matrices with zero rows or columns are valid and enqueue nothing.
 *   - Inputs must be finite (no Inf/NaN in bf16 data).
 *   - Results are deterministic: identical bytes for identical inputs,
 *     independent of stream and repetition.
 *   - The device must be gfx950 (MI355X/MI350X); other devices get
 *     FP8_ERR_UNSUPPORTED.
 */
#ifndef FP8BLK_H
#define FP8BLK_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define FP8BLK_ABI_VERSION 6

typedef enum {
  FP8_OK = 0,
  FP8_ERR_INVALID_ARG = 1, /* null pointer, unknown enum, bad rank          */
  FP8_ERR_SHAPE = 2,       /* negative or non-divisible dimension            */
  FP8_ERR_ALIGN = 3,       /* pointer not aligned as documented              */
  FP8_ERR_UNSUPPORTED = 4, /* block-kind combination or device not handled   */
  FP8_ERR_HIP = 5,         /* the HIP runtime reported an error              */
  FP8_ERR_TOO_LARGE = 6    /* needs more than the fixed no-allocation scratch */
} fp8_status;

/* Block geometry and scale type ([DSV3-Blog5] block-wise quantization;
 * [FP8-DSV3-ru]: 128x128 weight blocks with an fp32 scale inverse and
 * per-token 1x128 activation groups; [prequant]: MXFP8 = 1x32, E8M0). */
typedef enum {
  FP8_BLOCK_1x32_E8M0 = 0,   /* scale: uint8 E8M0 code, [rows][cols/32]        */
  FP8_BLOCK_1x128_F32 = 1,   /* scale: float, [rows][cols/128]                 */
  FP8_BLOCK_128x128_F32 = 2  /* scale: float, [rows/128][cols/128]             */
} fp8_block;

/* E8M0 exponent rule (the pages do not fix it).
 * CEIL : X = smallest integer with amax <= 448 * 2^X (no element saturates).
 * FLOOR: X = floor(log2 amax) - 8 (OCP MX rule; elements above 448*2^X
 *        saturate to +-448).  Both clamp X to [-127, 127]; amax == 0 gives
 *        X = -127.  The stored code is X + 127. */
typedef enum { FP8_E8M0_CEIL = 0, FP8_E8M0_FLOOR = 1 } fp8_e8m0_rule;

/* GEMM output element type. */
typedef enum { FP8_OUT_BF16 = 0, FP8_OUT_F32 = 1 } fp8_out;

/*
 * fp8_block_quantize -- block-wise FP8 quantization of a bf16 matrix.
 *
 * Defined by: [DSV3-Blog5] "The Solution: Block-Wise Quantization" (each
 * sub-matrix gets its own scaling factor); [FP8-DSV3-ru] "Почему обычное
 * округление не подходит" (128x128 weight blocks, scale inverse for
 * dequantization) and "Как FP8 встроен в DeepSeek V3" (online per-token,
 * per-128-channel activation quantization); [prequant] "Quick start" and
 * "Formats" (float8_e4m3fn weight + uint8 E8M0 weight_scale_inv, 1x32).
 *
 * For each block: amax = max |x|.
 *   fp32 kinds: s = RN32(amax / 448) is stored; q = e4m3(RN32(x / s));
 *               an all-zero block stores s = 0 and codes +-0.
 *   E8M0 kind : X from `rule`; code X + 127 is stored; q = e4m3(x * 2^-X).
 * e4m3(v): round to nearest even, saturate to +-448, keep the sign of zero.
 *
 * x     [rows x cols] bf16 (16-byte aligned).
 * q     [rows x cols] e4m3fn codes out (16-byte aligned).
 * scale out: uint8 [rows][cols/32] (1x32), float [rows][cols/128] (1x128,
 *       4-byte aligned), float [rows/128][cols/128] (128x128, 4-byte aligned).
 * xdq   optional (NULL = not written) [rows x cols] bf16 fake-quant output
 *       RN_bf16(RN32(decode(q) * scale)), 16-byte aligned.
 * rule  used by FP8_BLOCK_1x32_E8M0 only (ignored otherwise).
 * Shape: rows, cols >= 0, rows * cols <= 2^60; cols % 32 == 0 (1x32) or
 *        cols % 128 == 0; rows % 128 == 0 and rows / 128 <= 65535 for
 *        128x128.
 */
int fp8_block_quantize(const uint16_t* x, int64_t rows, int64_t cols, int kind, int rule,
                       uint8_t* q, void* scale, uint16_t* xdq, void* stream);

/*
 * fp8_block_quantize_batch -- several independent fp8_block_quantize calls
 * in one launch.
 *
 * Defined by: the same passages as fp8_block_quantize (each job is one such
 * call); a batch serves several tensors at once, for example a weight and
 * the activations of one projection ([FP8-DSV3-ru] "Как FP8 встроен в
 * DeepSeek V3": 128x128 weight blocks and 1x128 activation tiles) or a list
 * of routed expert projections ([prequant] "Formats").
 *
 * jobs   host array of `count` job descriptions (1 <= count <= 16; count 0
 *        enqueues nothing); each job has exactly the arguments, shape rules,
 *        alignment and outputs of fp8_block_quantize and gives the same
 *        bytes.  Jobs with zero rows or columns are skipped.  The jobs'
 *        buffers must not overlap one another.
 * Errors: the first invalid job's status is returned and nothing is
 *        launched; count outside [0, 16] is FP8_ERR_INVALID_ARG.
 */
typedef struct {
  const uint16_t* x;    /* [rows x cols] bf16 */
  int64_t rows;
  int64_t cols;
  int kind;             /* fp8_block */
  int rule;             /* fp8_e8m0_rule (1x32 only) */
  uint8_t* q;           /* [rows x cols] codes out */
  void* scale;          /* scales out, as for fp8_block_quantize */
  uint16_t* xdq;        /* optional fake-quant output, NULL = not written */
} fp8_quantize_job;

int fp8_block_quantize_batch(const fp8_quantize_job* jobs, int count, void* stream);

/*
 * fp8_block_dequantize -- block-scaled FP8 codes back to bf16.
 *
 * Defined by: [FP8-DSV3-ru] "Что такое FP8 простыми словами" and "Почему
 * FP8 требует scale factors" (FP8 weights are dequantized through the
 * block's inverse scale for higher-precision operations), "Практический
 * смысл для инференс-инфраструктуры" (FP8 weights converted to BF16 when a
 * backend needs it).
 *
 *   x = RN_bf16(RN32(decode(q) * scale))     (the fake-quant value)
 * with scale the block's fp32 value or 2^(E-127) for an E8M0 code E.
 * A product beyond the bf16 range rounds to +-inf (IEEE).
 *
 * q     [rows x cols] e4m3fn codes (16-byte aligned); NaN codes (0x7F,
 *       0xFF), which the quantizer never writes, give NaN.
 * scale as written by fp8_block_quantize for `kind` (uint8 E8M0 any
 *       alignment; fp32 4-byte aligned).
 * x     [rows x cols] bf16 out (16-byte aligned).
 * Shape: rows, cols >= 0; cols % 32 == 0 (1x32) or cols % 128 == 0;
 *        rows % 128 == 0 for 128x128; rows * cols / 8 <= 2^32 - 2^20.
 */
int fp8_block_dequantize(const uint8_t* q, const void* scale, int64_t rows, int64_t cols, int kind,
                         uint16_t* x, void* stream);

/*
 * fp8_fake_quant_merge -- QAT forward of a LoRA-adapted weight: merge
 * W + B.A in bf16, then fake-quantize the merged weight in 128x128 blocks.
 *
 * Defined by: [Fireworks-QAT] Synopsis and Interpretation (merged weights
 * are fake-quantized in the forward pass; LoRA factors stay bf16; merged
 * bf16 weights are converted to block-wise FP8 for serving); the 128x128
 * block with fp32 scale from [FP8-DSV3-ru].
 *
 *   acc = 0; for r = 0..R-1: acc = RN32(acc + B[n,r] * A[r,k])
 *   W'[n,k] = RN_bf16(RN32(W[n,k] + RN_bf16(acc)))
 * then exactly fp8_block_quantize(W', n, k, FP8_BLOCK_128x128_F32, ...).
 * W' itself is never written to memory.
 *
 * w      [n x k] bf16, lora_b [n x r] bf16, lora_a [r x k] bf16
 *        (w 16-byte aligned; lora_b, lora_a 4-byte aligned).
 * q      [n x k] codes out; scale float [n/128][k/128] out;
 * wdq    optional [n x k] bf16 fake-quant output (NULL = not written).
 * Shape: n % 128 == 0, k % 128 == 0, k <= 2^24, 1 <= r <= 64.
 */
int fp8_fake_quant_merge(const uint16_t* w, const uint16_t* lora_b, const uint16_t* lora_a,
                         int64_t n, int64_t k, int64_t r, uint8_t* q, float* scale,
                         uint16_t* wdq, void* stream);

/*
 * fp8_block_scaled_gemm -- Y = deq(A) . deq(B)^T with fp32 accumulation.
 *
 * Defined by: [DSV3-Blog5] "Hardware Optimization" (FP8 products on the
 * matrix units, intermediate results promoted to higher precision before
 * the final accumulation); [FP8-DSV3-ru] "Инференс с FP8" (FP8 matrix
 * multiplication on block-quantized operands).
 *
 * a_q [m x k] codes with a_scale; b_q [n x k] codes with b_scale (both
 * K-contiguous, as produced by fp8_block_quantize; 16-byte aligned;
 * E8M0 scale arrays 4-byte aligned, fp32 scale arrays 4-byte aligned).
 * Supported (a_kind, b_kind):
 *   (FP8_BLOCK_1x128_F32, FP8_BLOCK_128x128_F32): per 128-wide K chunk the
 *        FP8 partial product is formed on the matrix cores and added to the
 *        fp32 accumulator times sa[m][kb] * sb[n/128][kb];
 *   (FP8_BLOCK_1x32_E8M0, FP8_BLOCK_1x32_E8M0): MXFP8 x MXFP8, the
 *        power-of-two scales are applied inside the scaled matrix
 *        instruction and accumulation is continuous in fp32.
 * y      [m x n] out, bf16 (RN_bf16 of the fp32 result) or float, per y_type
 *        (16-byte aligned).
 * Shape: 0 <= m < 2^31, n % 128 == 0, k % 128 == 0, 0 < k <= 2^24 (m == 0 or
 *        n == 0 is a no-op).
 */
int fp8_block_scaled_gemm(const uint8_t* a_q, const void* a_scale, int a_kind,
                          const uint8_t* b_q, const void* b_scale, int b_kind,
                          int64_t m, int64_t n, int64_t k, void* y, int y_type, void* stream);

/*
 * fp8_grouped_gemm -- variable-M grouped GEMM over routed MoE experts.
 *
 * Defined by: the routed expert projections of [prequant] (MXFP8 weights,
 * "Formats" and the routed-expert rule) and the FP8 MoE activations of
 * [DSV3-Blog5] "Reducing Communication Overhead in MoE with FP8".
 *
 * Group g owns rows [off[g], off[g+1]) of A and expert matrix B[g]:
 *   Y[rows of g] = deq(A[rows of g]) . deq(B[g])^T, fp32 accumulation.
 * a_q [total_m x k] codes, a_kind = FP8_BLOCK_1x128_F32 (per-token scales
 *     float [total_m][k/128]);
 * b_q [groups x n x k] codes, b_kind = FP8_BLOCK_1x32_E8M0 (uint8
 *     [groups][n][k/32]) or FP8_BLOCK_128x128_F32 (float
 *     [groups][n/128][k/128]);
 * group_offsets: DEVICE int32 [groups+1], off[0] = 0, non-decreasing,
 *     off[groups] = total_m.  Not checked on the host; the kernel clamps
 *     each group's rows into [0, total_m] (and empty where off[g+1] <
 *     off[g]), so a violation leaves output rows unspecified but accesses
 *     nothing outside the buffers;
 * y [total_m x n] out, bf16 or float per y_type (16-byte aligned).
 * Shape: 1 <= groups <= 1024, 0 <= total_m < 2^31, n % 128 == 0,
 *        k % 128 == 0, 0 < k <= 2^24.
 */
int fp8_grouped_gemm(const uint8_t* a_q, const void* a_scale, int a_kind,
                     const uint8_t* b_q, const void* b_scale, int b_kind,
                     const int32_t* group_offsets, int64_t groups, int64_t total_m,
                     int64_t n, int64_t k, void* y, int y_type, void* stream);

/*
 * fp8_grouped_gemm_gather -- fp8_grouped_gemm whose A rows are gathered.
 *
 * Defined by: the MoE dispatch of [DSV3-Blog5] "Reducing Communication
 * Overhead in MoE with FP8" (routed tokens carry FP8 activations) and
 * [FP8-DSV3-ru] "Как FP8 связан с MoE-архитектурой DeepSeek V3" (each token
 * activates only some of the experts): each token's activations are
 * quantized once, per token in 1x128 tiles, and every expert reads the rows
 * of the tokens routed to it.
 *
 * Grouped row i (group g owns [off[g], off[g+1])) is
 *   Y[i] = deq(A[row_index[i]]) . deq(B[g])^T,   fp32 accumulation,
 * i.e. fp8_grouped_gemm on the rows A[row_index[0..total_m-1]], without
 * writing that permuted copy.
 * a_q [a_rows x k] codes, a_kind = FP8_BLOCK_1x128_F32 (float scales
 *     [a_rows][k/128]); a_rows * k < 2^32.
 * row_index: DEVICE int32 [total_m], values in [0, a_rows); 4-byte
 *     aligned.  Not checked on the host; the kernel clamps each value into
 *     [0, a_rows), so a violation gives unspecified rows but no access
 *     outside A or its scales.
 * Every other argument as for fp8_grouped_gemm.
 */
int fp8_grouped_gemm_gather(const uint8_t* a_q, const void* a_scale, int a_kind, int64_t a_rows,
                            const int32_t* row_index, const uint8_t* b_q, const void* b_scale, int b_kind,
                            const int32_t* group_offsets, int64_t groups, int64_t total_m, int64_t n, int64_t k,
                            void* y, int y_type, void* stream);

/*
 * fp8_lora_backward -- QAT backward for the LoRA factors.
 *
 * Defined by: [Fireworks-QAT] Synopsis and Interpretation (QAT trains the
 * LoRA factors in bf16 while the forward pass uses the fake-quantized
 * merged weight and activations).  The gradient rule is not printed there;
 * the fake-quant is taken as straight-through (identity Jacobian), so with
 * the forward Y = X_hat . W_hat^T, W_hat = fakequant(W + B.A):
 *   dW = dY^T . X_hat,   dB = dW . A^T,   dA = B^T . dW,
 * computed without forming dW as dB = dY^T . (X_hat . A^T) and
 * dA = (dY . B)^T . X_hat, products of bf16 values accumulated in fp32;
 * the rank-r intermediates are carried as the sum of two bf16 values
 * (16 significant bits).  Results are rounded once (RN_bf16) or kept fp32.
 *
 * dy     [m x n] bf16 output gradient (16-byte aligned);
 * x      [m x k] bf16 fake-quantized activations X_hat (16-byte aligned);
 * lora_b [n x r] bf16 (2-byte aligned); lora_a [r x k] bf16 (16-byte
 *        aligned);
 * workspace: DEVICE scratch of at least the size fp8_lora_backward_workspace
 *        reports for (m, n, k, r), 256-byte aligned, owned by the caller;
 *        its contents on entry do not matter and are garbage on exit;
 *        concurrent calls need separate workspaces;
 * d_lora_b [n x r], d_lora_a [r x k] out: bf16 (out_type FP8_OUT_BF16,
 *        2-byte aligned) or float (FP8_OUT_F32, 4-byte aligned).  m == 0
 *        writes zeros.  dy and x may be NULL when m == 0; lora_b and
 *        d_lora_b when n == 0; lora_a and d_lora_a when k == 0.
 * Shape: m >= 0, m < 2^31 - 64; n % 128 == 0, k % 128 == 0, n, k <= 2^24;
 *        1 <= r <= 64.  n == k == 0 enqueues nothing.
 */
int fp8_lora_backward(const uint16_t* dy, const uint16_t* x, const uint16_t* lora_b,
                      const uint16_t* lora_a, int64_t m, int64_t n, int64_t k, int64_t r,
                      void* workspace, size_t workspace_bytes, void* d_lora_b, void* d_lora_a,
                      int out_type, void* stream);

/* Workspace bytes fp8_lora_backward needs for (m, n, k, r), into *bytes
 * (host pointer).  Same shape checks and status codes as the call itself. */
int fp8_lora_backward_workspace(int64_t m, int64_t n, int64_t k, int64_t r, size_t* bytes);

/*
 * fp8_lora_backward_noalloc -- fp8_lora_backward without a workspace
 * argument and without any allocation, for callers that cannot allocate
 * device memory (code under stream or graph capture, tight serving loops,
 * harnesses that forbid allocation).
 *
 * Same computation, arguments (minus workspace / workspace_bytes), shape
 * rules, alignment and results as fp8_lora_backward: the output bytes are
 * identical.  The workspace is a fixed array of FP8BLK_NOALLOC_SCRATCH_BYTES
 * bytes per device, held by the library from first use until the process
 * ends; its contents on entry do not matter.  Problems whose workspace
 * (fp8_lora_backward_workspace) exceeds it return FP8_ERR_TOO_LARGE and
 * enqueue nothing (40 MiB: 8192 tokens at n = k = 7168 fit up to rank 64).
 * Every call on one device shares that device's array: calls that may
 * overlap on one device (other streams, other host threads) race and must
 * be serialized by the caller.  The array's address is looked up on the
 * first call on each device, with that device current; nothing is
 * allocated then either.
 */
#define FP8BLK_NOALLOC_SCRATCH_BYTES (40ull << 20)
int fp8_lora_backward_noalloc(const uint16_t* dy, const uint16_t* x, const uint16_t* lora_b,
                              const uint16_t* lora_a, int64_t m, int64_t n, int64_t k, int64_t r,
                              void* d_lora_b, void* d_lora_a, int out_type, void* stream);

/*
 * fp8_nvfp4_quantize -- NVFP4 prequantization: packed FP4 values with FP8
 * block scales.
 *
 * Defined by: [prequant] "Formats" (nvfp4: packed FP4 + FP8 block scales,
 * served at FP4) and the routed-expert rule below it.  The page gives no
 * layout; this library takes E2M1 elements (OCP Microscaling), 1x16 blocks
 * with e4m3fn scales, and an fp32 scale per tensor:
 *   A = max |x| over the tensor (or the caller's value), g = RN32(A / 2688)
 *   S = e4m3(RN32(a / RN32(6 g))), a = the block's amax (RNE, saturating;
 *       S = 0 when g = 0)
 *   m = RN32(e4m3(S) * g), code = e2m1(RN32(x / m)) (RNE, saturating at 6,
 *       sign kept; only the sign when m = 0)
 *   xdq = RN_bf16(RN32(e2m1(code) * m)).
 *
 * x      [rows x cols] bf16 (16-byte aligned); the rows form rows/rows_per_tensor
 *        stacked tensors of rows_per_tensor rows, each with its own A and g;
 * tensor_amax [tensors] float: written with A when amax_given == 0, read as
 *        A (finite, >= 0) when amax_given == 1 (4-byte aligned);
 * q      [rows x cols/2] bytes out, element 2j in the low nibble of byte j
 *        (8-byte aligned);
 * block_scale [rows x cols/16] e4m3fn codes out;
 * global_scale [tensors] float g out (4-byte aligned);
 * xdq    optional [rows x cols] bf16 fake-quant output (16-byte aligned).
 * Shape: cols % 16 == 0, rows % rows_per_tensor == 0, rows * cols / 8 <=
 *        2^32 - 2^20.  rows == 0 or cols == 0 enqueues nothing.
 */
int fp8_nvfp4_quantize(const uint16_t* x, int64_t rows, int64_t cols, int64_t rows_per_tensor,
                       float* tensor_amax, int amax_given, uint8_t* q, uint8_t* block_scale,
                       float* global_scale, uint16_t* xdq, void* stream);

/*
 * fp8_nvfp4_dequantize -- NVFP4 codes + scales -> bf16:
 *   x = RN_bf16(RN32(e2m1(code) * RN32(e4m3(S) * g))), the value
 * fp8_nvfp4_quantize writes to xdq.  Defined by: [prequant] "Formats"
 * (serving loads the packed weights); arguments and shape as there (q
 * 8-byte aligned, as fp8_nvfp4_quantize requires of its code buffer).
 */
int fp8_nvfp4_dequantize(const uint8_t* q, const uint8_t* block_scale, const float* global_scale,
                         int64_t rows, int64_t cols, int64_t rows_per_tensor, uint16_t* x, void* stream);

/* Static, human-readable text for a status code (never NULL). */
const char* fp8_status_string(int status);

/* FP8BLK_ABI_VERSION of the loaded library. */
int fp8_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* FP8BLK_H */
