// C-ABI entry points of the fp8blk library: argument validation, device
// checks and kernel dispatch.  The declarations and their contracts are in
// include/fp8blk.h.
#include "fp8blk.h"

#include <hip/hip_runtime.h>

#include <mutex>
#include <string.h>

#include "launch.h"

namespace {

constexpr int kMaxDevices = 64;

struct DeviceInfo {
  bool ok = false;
  bool supported = false;
  int num_cu = 0;
};

DeviceInfo g_dev[kMaxDevices];
std::once_flag g_once[kMaxDevices];

// Properties of the current device, read once per device.
int current_device(DeviceInfo** out) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return FP8_ERR_HIP;
  if (dev < 0 || dev >= kMaxDevices) return FP8_ERR_UNSUPPORTED;
  std::call_once(g_once[dev], [dev] {
    hipDeviceProp_t prop;
    if (hipGetDeviceProperties(&prop, dev) != hipSuccess) return;
    g_dev[dev].ok = true;
    g_dev[dev].num_cu = prop.multiProcessorCount;
    g_dev[dev].supported = strncmp(prop.gcnArchName, "gfx950", 6) == 0;
  });
  if (!g_dev[dev].ok) return FP8_ERR_HIP;
  if (!g_dev[dev].supported) return FP8_ERR_UNSUPPORTED;
  *out = &g_dev[dev];
  return FP8_OK;
}

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

// a * b <= lim for non-negative a, b, without overflowing int64.
bool product_at_most(int64_t a, int64_t b, int64_t lim) { return b == 0 || a <= lim / b; }

// Element counts beyond 2^60 are rejected before any size arithmetic.
constexpr int64_t kMaxElements = int64_t(1) << 60;
static_assert(FP8BLK_NOALLOC_SCRATCH_BYTES == (unsigned long long)fp8blk::kLoraScratchBytes,
              "header and library agree on the no-allocation scratch size");

// GEMM reductions: per-tile A/B offsets are 32-bit (256 rows x K bytes).
constexpr int64_t kMaxGemmK = int64_t(1) << 24;

int hip_status(hipError_t e) { return e == hipSuccess ? FP8_OK : FP8_ERR_HIP; }

bool valid_kind(int k) { return k == FP8_BLOCK_1x32_E8M0 || k == FP8_BLOCK_1x128_F32 || k == FP8_BLOCK_128x128_F32; }

// Scale pointer alignment: fp32 scales 4 bytes; E8M0 bytes read four at a
// time by the GEMMs, so 4 bytes there too (quantize writes single bytes).
uintptr_t scale_align(int kind, bool gemm) { return kind == FP8_BLOCK_1x32_E8M0 ? (gemm ? 4 : 1) : 4; }

}  // namespace

extern "C" {

int fp8_abi_version(void) { return FP8BLK_ABI_VERSION; }

const char* fp8_status_string(int s) {
  switch (s) {
    case FP8_OK: return "ok";
    case FP8_ERR_INVALID_ARG: return "invalid argument (null pointer, unknown enum or bad rank)";
    case FP8_ERR_SHAPE: return "invalid shape (negative or not a multiple of the block)";
    case FP8_ERR_ALIGN: return "pointer not aligned as required";
    case FP8_ERR_UNSUPPORTED: return "unsupported block-kind combination or device (gfx950 required)";
    case FP8_ERR_HIP: return "HIP runtime error";
    case FP8_ERR_TOO_LARGE: return "problem larger than the library's fixed no-allocation scratch buffer";
    default: return "unknown status";
  }
}

static int quantize_args(const uint16_t* x, int64_t rows, int64_t cols, int kind, int rule, const uint8_t* q,
                         const void* scale, const uint16_t* xdq) {
  if (!valid_kind(kind)) return FP8_ERR_INVALID_ARG;
  if (kind == FP8_BLOCK_1x32_E8M0 && rule != FP8_E8M0_CEIL && rule != FP8_E8M0_FLOOR) return FP8_ERR_INVALID_ARG;
  if (rows < 0 || cols < 0 || !product_at_most(rows, cols, kMaxElements)) return FP8_ERR_SHAPE;
  const int64_t bc = kind == FP8_BLOCK_1x32_E8M0 ? 32 : 128;
  if (cols % bc) return FP8_ERR_SHAPE;
  if (kind == FP8_BLOCK_128x128_F32 && rows % 128) return FP8_ERR_SHAPE;
  if (kind == FP8_BLOCK_128x128_F32 && rows / 128 > 65535) return FP8_ERR_SHAPE;
  if (rows == 0 || cols == 0) return FP8_OK;
  if (!x || !q || !scale) return FP8_ERR_INVALID_ARG;
  if (!aligned(x, 16) || !aligned(q, 16) || (xdq && !aligned(xdq, 16)) || !aligned(scale, scale_align(kind, false)))
    return FP8_ERR_ALIGN;
  return FP8_OK;
}

int fp8_block_quantize_batch(const fp8_quantize_job* jobs, int count, void* stream) {
  if (count < 0 || count > fp8blk::kMaxQuantJobs) return FP8_ERR_INVALID_ARG;
  if (count == 0) return FP8_OK;
  if (!jobs) return FP8_ERR_INVALID_ARG;
  fp8blk::QuantJobIn in[fp8blk::kMaxQuantJobs];
  int64_t wgs = 0;
  bool work = false;
  for (int i = 0; i < count; ++i) {
    const fp8_quantize_job& j = jobs[i];
    if (int st = quantize_args(j.x, j.rows, j.cols, j.kind, j.rule, j.q, j.scale, j.xdq)) return st;
    work = work || (j.rows > 0 && j.cols > 0);
    if (j.kind != FP8_BLOCK_128x128_F32 && j.rows * (j.cols / 8) > 0xFFF00000ll) return FP8_ERR_SHAPE;
    wgs += j.kind == FP8_BLOCK_128x128_F32 ? (j.rows / 128) * (j.cols / 128)
                                           : j.rows * j.cols / 8 / fp8blk::kQuantBatchRowsChunks + 1;
    in[i] = fp8blk::QuantJobIn{j.x, j.rows, j.cols, j.kind, j.rule == FP8_E8M0_FLOOR, j.q, j.scale, j.xdq};
  }
  if (wgs > 0x7FFFFFFFll) return FP8_ERR_SHAPE;
  if (!work) return FP8_OK;
  DeviceInfo* dev = nullptr;
  if (int st = current_device(&dev)) return st;
  return hip_status(fp8blk::launch_quant_batch(in, count, reinterpret_cast<hipStream_t>(stream)));
}

int fp8_block_quantize(const uint16_t* x, int64_t rows, int64_t cols, int kind, int rule, uint8_t* q, void* scale,
                       uint16_t* xdq, void* stream) {
  if (int st = quantize_args(x, rows, cols, kind, rule, q, scale, xdq)) return st;
  if (rows == 0 || cols == 0) return FP8_OK;
  DeviceInfo* dev = nullptr;
  if (int s = current_device(&dev)) return s;
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  if (kind == FP8_BLOCK_128x128_F32)
    return hip_status(fp8blk::launch_quant_128(x, rows, cols, q, static_cast<float*>(scale), xdq, st));
  return hip_status(fp8blk::launch_quant_rows(x, rows, cols, kind == FP8_BLOCK_1x32_E8M0 ? 32 : 128,
                                              rule == FP8_E8M0_FLOOR, q, scale, xdq, dev->num_cu, st));
}

int fp8_block_dequantize(const uint8_t* q, const void* scale, int64_t rows, int64_t cols, int kind, uint16_t* x,
                         void* stream) {
  if (!valid_kind(kind)) return FP8_ERR_INVALID_ARG;
  if (rows < 0 || cols < 0 || !product_at_most(rows, cols, kMaxElements)) return FP8_ERR_SHAPE;
  const int64_t bc = kind == FP8_BLOCK_1x32_E8M0 ? 32 : 128;
  if (cols % bc) return FP8_ERR_SHAPE;
  if (kind == FP8_BLOCK_128x128_F32 && rows % 128) return FP8_ERR_SHAPE;
  if (rows == 0 || cols == 0) return FP8_OK;
  if (rows * (cols / 8) > 0xFFF00000ll) return FP8_ERR_SHAPE;  // 32-bit chunk indices, with launch margin
  if (!q || !scale || !x) return FP8_ERR_INVALID_ARG;
  if (!aligned(q, 16) || !aligned(x, 16) || !aligned(scale, scale_align(kind, false))) return FP8_ERR_ALIGN;
  DeviceInfo* dev = nullptr;
  if (int s = current_device(&dev)) return s;
  return hip_status(fp8blk::launch_dequant(q, scale, rows, cols, kind, x, reinterpret_cast<hipStream_t>(stream)));
}

int fp8_fake_quant_merge(const uint16_t* w, const uint16_t* lora_b, const uint16_t* lora_a, int64_t n, int64_t k,
                         int64_t r, uint8_t* q, float* scale, uint16_t* wdq, void* stream) {
  if (r < 1 || r > 64) return FP8_ERR_INVALID_ARG;
  if (n < 0 || k < 0 || n % 128 || k % 128 || n / 128 > 65535 || k > (int64_t(1) << 24)) return FP8_ERR_SHAPE;
  if (n == 0 || k == 0) return FP8_OK;
  if (!w || !lora_b || !lora_a || !q || !scale) return FP8_ERR_INVALID_ARG;
  if (!aligned(w, 16) || !aligned(q, 16) || !aligned(scale, 4) || !aligned(lora_a, 4) || !aligned(lora_b, 4) ||
      (wdq && !aligned(wdq, 16)))
    return FP8_ERR_ALIGN;
  DeviceInfo* dev = nullptr;
  if (int s = current_device(&dev)) return s;
  return hip_status(fp8blk::launch_merge(w, lora_b, lora_a, n, k, r, q, scale, wdq, reinterpret_cast<hipStream_t>(stream)));
}

int fp8_block_scaled_gemm(const uint8_t* a_q, const void* a_scale, int a_kind, const uint8_t* b_q, const void* b_scale,
                          int b_kind, int64_t m, int64_t n, int64_t k, void* y, int y_type, void* stream) {
  if (!valid_kind(a_kind) || !valid_kind(b_kind)) return FP8_ERR_INVALID_ARG;
  if (y_type != FP8_OUT_BF16 && y_type != FP8_OUT_F32) return FP8_ERR_INVALID_ARG;
  const bool f32pair = a_kind == FP8_BLOCK_1x128_F32 && b_kind == FP8_BLOCK_128x128_F32;
  const bool mxpair = a_kind == FP8_BLOCK_1x32_E8M0 && b_kind == FP8_BLOCK_1x32_E8M0;
  if (!f32pair && !mxpair) return FP8_ERR_UNSUPPORTED;
  if (m < 0 || n < 0 || k < 0 || n % 128 || k % 128) return FP8_ERR_SHAPE;
  if (m > 0x7FFFFFFFll || n > 0x7FFFFFFFll || k > kMaxGemmK) return FP8_ERR_SHAPE;
  if ((m + 255) / 256 * (n / 128) > 0x7FFFFFFF) return FP8_ERR_SHAPE;
  if (m == 0 || n == 0) return FP8_OK;
  if (!y) return FP8_ERR_INVALID_ARG;
  if (k == 0) return FP8_ERR_SHAPE;  // an empty reduction is not a block-scaled product
  if (!a_q || !b_q || !a_scale || !b_scale) return FP8_ERR_INVALID_ARG;
  if (!aligned(a_q, 16) || !aligned(b_q, 16) || !aligned(a_scale, scale_align(a_kind, true)) ||
      !aligned(b_scale, scale_align(b_kind, true)) || !aligned(y, 16))
    return FP8_ERR_ALIGN;
  DeviceInfo* dev = nullptr;
  if (int s = current_device(&dev)) return s;
  return hip_status(fp8blk::launch_gemm(a_q, a_scale, a_kind, b_q, b_scale, b_kind, m, n, k, y,
                                        y_type == FP8_OUT_F32, dev->num_cu, reinterpret_cast<hipStream_t>(stream)));
}

static int grouped_common(const uint8_t* a_q, const void* a_scale, int a_kind, int64_t a_rows,
                          const int32_t* row_index, bool gather, const uint8_t* b_q, const void* b_scale, int b_kind,
                          const int32_t* group_offsets, int64_t groups, int64_t total_m, int64_t n, int64_t k, void* y,
                          int y_type, void* stream) {
  if (!valid_kind(a_kind) || !valid_kind(b_kind)) return FP8_ERR_INVALID_ARG;
  if (y_type != FP8_OUT_BF16 && y_type != FP8_OUT_F32) return FP8_ERR_INVALID_ARG;
  if (a_kind != FP8_BLOCK_1x128_F32 || (b_kind != FP8_BLOCK_1x32_E8M0 && b_kind != FP8_BLOCK_128x128_F32))
    return FP8_ERR_UNSUPPORTED;
  if (groups < 1 || groups > 1024) return FP8_ERR_INVALID_ARG;
  if (total_m < 0 || n < 0 || k <= 0 || n % 128 || k % 128) return FP8_ERR_SHAPE;
  if (n > 0x7FFFFFFFll || k > kMaxGemmK) return FP8_ERR_SHAPE;
  if (total_m > 0x7FFFFFFF || (total_m / 128 + groups) * (n / 128) > 0x7FFFFF00) return FP8_ERR_SHAPE;
  if (gather && (a_rows < 0 || a_rows * k > 0xFFFFFFFFll)) return FP8_ERR_SHAPE;  // 32-bit row offsets
  if (total_m == 0 || n == 0) return FP8_OK;
  if (gather && a_rows == 0) return FP8_ERR_SHAPE;
  if (!a_q || !a_scale || !b_q || !b_scale || !group_offsets || !y || (gather && !row_index))
    return FP8_ERR_INVALID_ARG;
  if (!aligned(a_q, 16) || !aligned(b_q, 16) || !aligned(a_scale, 4) || !aligned(b_scale, 4) ||
      !aligned(group_offsets, 4) || !aligned(y, 16) || (gather && !aligned(row_index, 4)))
    return FP8_ERR_ALIGN;
  DeviceInfo* dev = nullptr;
  if (int s = current_device(&dev)) return s;
  return hip_status(fp8blk::launch_grouped_gemm(a_q, a_scale, a_kind, gather ? row_index : nullptr, a_rows, b_q,
                                                b_scale, b_kind, group_offsets, groups, total_m, n, k, y,
                                                y_type == FP8_OUT_F32, dev->num_cu,
                                                reinterpret_cast<hipStream_t>(stream)));
}

int fp8_grouped_gemm(const uint8_t* a_q, const void* a_scale, int a_kind, const uint8_t* b_q, const void* b_scale,
                     int b_kind, const int32_t* group_offsets, int64_t groups, int64_t total_m, int64_t n, int64_t k,
                     void* y, int y_type, void* stream) {
  return grouped_common(a_q, a_scale, a_kind, total_m, nullptr, false, b_q, b_scale, b_kind, group_offsets, groups,
                        total_m, n, k, y, y_type, stream);
}

int fp8_grouped_gemm_gather(const uint8_t* a_q, const void* a_scale, int a_kind, int64_t a_rows,
                            const int32_t* row_index, const uint8_t* b_q, const void* b_scale, int b_kind,
                            const int32_t* group_offsets, int64_t groups, int64_t total_m, int64_t n, int64_t k,
                            void* y, int y_type, void* stream) {
  return grouped_common(a_q, a_scale, a_kind, a_rows, row_index, true, b_q, b_scale, b_kind, group_offsets, groups,
                        total_m, n, k, y, y_type, stream);
}

static int lora_shape(int64_t m, int64_t n, int64_t k, int64_t r) {
  if (r < 1 || r > 64) return FP8_ERR_INVALID_ARG;
  if (m < 0 || n < 0 || k < 0 || n % 128 || k % 128) return FP8_ERR_SHAPE;
  if (m > 0x7FFFFFFFll - 64 || n > (int64_t(1) << 24) || k > (int64_t(1) << 24)) return FP8_ERR_SHAPE;
  return FP8_OK;
}

int fp8_lora_backward_workspace(int64_t m, int64_t n, int64_t k, int64_t r, size_t* bytes) {
  if (!bytes) return FP8_ERR_INVALID_ARG;
  if (int s = lora_shape(m, n, k, r)) return s;
  *bytes = (size_t)fp8blk::lora_bwd_workspace_bytes(m, n, k, r);
  return FP8_OK;
}

// Arguments of both LoRA backward entry points except the workspace.
static int lora_args(const uint16_t* dy, const uint16_t* x, const uint16_t* lora_b, const uint16_t* lora_a, int64_t m,
                     int64_t n, int64_t k, int64_t r, const void* d_lora_b, const void* d_lora_a, int out_type) {
  if (out_type != FP8_OUT_BF16 && out_type != FP8_OUT_F32) return FP8_ERR_INVALID_ARG;
  if (int s = lora_shape(m, n, k, r)) return s;
  if (n == 0 && k == 0) return FP8_OK;
  if ((n > 0 && (!lora_b || !d_lora_b)) || (k > 0 && (!lora_a || !d_lora_a)) ||
      (m > 0 && ((n > 0 && !dy) || (k > 0 && !x))))
    return FP8_ERR_INVALID_ARG;
  const uintptr_t oa = out_type == FP8_OUT_F32 ? 4 : 2;
  if ((dy && !aligned(dy, 16)) || (x && !aligned(x, 16)) || (lora_a && !aligned(lora_a, 16)) ||
      (lora_b && !aligned(lora_b, 2)) || (d_lora_b && !aligned(d_lora_b, oa)) || (d_lora_a && !aligned(d_lora_a, oa)))
    return FP8_ERR_ALIGN;
  return FP8_OK;
}

int fp8_lora_backward(const uint16_t* dy, const uint16_t* x, const uint16_t* lora_b, const uint16_t* lora_a,
                      int64_t m, int64_t n, int64_t k, int64_t r, void* workspace, size_t workspace_bytes,
                      void* d_lora_b, void* d_lora_a, int out_type, void* stream) {
  if (int s = lora_args(dy, x, lora_b, lora_a, m, n, k, r, d_lora_b, d_lora_a, out_type)) return s;
  if (n == 0 && k == 0) return FP8_OK;
  if (!workspace) return FP8_ERR_INVALID_ARG;
  if (workspace_bytes < (size_t)fp8blk::lora_bwd_workspace_bytes(m, n, k, r)) return FP8_ERR_INVALID_ARG;
  if (!aligned(workspace, 256)) return FP8_ERR_ALIGN;
  DeviceInfo* dev = nullptr;
  if (int s = current_device(&dev)) return s;
  return hip_status(fp8blk::launch_lora_bwd(dy, x, lora_b, lora_a, m, n, k, r, workspace, d_lora_b, d_lora_a,
                                            out_type == FP8_OUT_F32, dev->num_cu,
                                            reinterpret_cast<hipStream_t>(stream)));
}

int fp8_lora_backward_noalloc(const uint16_t* dy, const uint16_t* x, const uint16_t* lora_b, const uint16_t* lora_a,
                              int64_t m, int64_t n, int64_t k, int64_t r, void* d_lora_b, void* d_lora_a,
                              int out_type, void* stream) {
  if (int s = lora_args(dy, x, lora_b, lora_a, m, n, k, r, d_lora_b, d_lora_a, out_type)) return s;
  if (n == 0 && k == 0) return FP8_OK;
  if (fp8blk::lora_bwd_workspace_bytes(m, n, k, r) > fp8blk::kLoraScratchBytes) return FP8_ERR_TOO_LARGE;
  DeviceInfo* dev = nullptr;
  if (int s = current_device(&dev)) return s;
  int id = 0;
  if (hipGetDevice(&id) != hipSuccess) return FP8_ERR_HIP;
  void* ws = nullptr;
  if (fp8blk::lora_bwd_scratch(id, &ws) != hipSuccess) return FP8_ERR_HIP;
  return hip_status(fp8blk::launch_lora_bwd(dy, x, lora_b, lora_a, m, n, k, r, ws, d_lora_b, d_lora_a,
                                            out_type == FP8_OUT_F32, dev->num_cu,
                                            reinterpret_cast<hipStream_t>(stream)));
}

static int nvfp4_shape(int64_t rows, int64_t cols, int64_t rows_per_tensor) {
  if (rows < 0 || cols < 0 || cols % 16 || !product_at_most(rows, cols, kMaxElements)) return FP8_ERR_SHAPE;
  if (rows_per_tensor < 1 || rows % rows_per_tensor) return FP8_ERR_SHAPE;
  if (rows * (cols / 8) > 0xFFF00000ll) return FP8_ERR_SHAPE;  // 32-bit chunk indices, with launch margin
  return FP8_OK;
}

int fp8_nvfp4_quantize(const uint16_t* x, int64_t rows, int64_t cols, int64_t rows_per_tensor, float* tensor_amax,
                       int amax_given, uint8_t* q, uint8_t* block_scale, float* global_scale, uint16_t* xdq,
                       void* stream) {
  if (amax_given != 0 && amax_given != 1) return FP8_ERR_INVALID_ARG;
  if (int s = nvfp4_shape(rows, cols, rows_per_tensor)) return s;
  if (rows == 0 || cols == 0) return FP8_OK;
  if (!x || !tensor_amax || !q || !block_scale || !global_scale) return FP8_ERR_INVALID_ARG;
  if (!aligned(x, 16) || !aligned(q, 8) || !aligned(tensor_amax, 4) || !aligned(global_scale, 4) ||
      (xdq && !aligned(xdq, 16)))
    return FP8_ERR_ALIGN;
  DeviceInfo* dev = nullptr;
  if (int s = current_device(&dev)) return s;
  return hip_status(fp8blk::launch_nvfp4_quant(x, rows, cols, rows_per_tensor, tensor_amax, amax_given == 1, q,
                                               block_scale, global_scale, xdq,
                                               reinterpret_cast<hipStream_t>(stream)));
}

int fp8_nvfp4_dequantize(const uint8_t* q, const uint8_t* block_scale, const float* global_scale, int64_t rows,
                         int64_t cols, int64_t rows_per_tensor, uint16_t* x, void* stream) {
  if (int s = nvfp4_shape(rows, cols, rows_per_tensor)) return s;
  if (rows == 0 || cols == 0) return FP8_OK;
  if (!q || !block_scale || !global_scale || !x) return FP8_ERR_INVALID_ARG;
  // codes are read a dword (half a 1x16 block) at a time; q keeps the 8-byte
  // alignment of fp8_nvfp4_quantize's code buffer
  if (!aligned(q, 8) || !aligned(global_scale, 4) || !aligned(x, 16)) return FP8_ERR_ALIGN;
  DeviceInfo* dev = nullptr;
  if (int s = current_device(&dev)) return s;
  return hip_status(fp8blk::launch_nvfp4_dequant(q, block_scale, global_scale, rows, cols, rows_per_tensor, x,
                                                 reinterpret_cast<hipStream_t>(stream)));
}

}  // extern "C"
