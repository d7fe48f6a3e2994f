// Kernel launchers of the fp8blk library (internal; arguments are already
// validated by abi.cpp).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fp8blk {

hipError_t launch_quant_rows(const uint16_t* x, int64_t rows, int64_t cols, int blk, bool floor_rule, uint8_t* q,
                             void* scale, uint16_t* xdq, int num_cu, hipStream_t stream);
hipError_t launch_quant_128(const uint16_t* x, int64_t rows, int64_t cols, uint8_t* q, float* scale, uint16_t* xdq,
                            hipStream_t stream);
// Batched quantize: jobs already validated (at most kMaxQuantJobs).
constexpr int kMaxQuantJobs = 16;
// 8-chunk groups a rows-kind (1x32, 1x128) batch workgroup covers in its one
// pass: 8 waves x 64 lanes x 2 chunks.
constexpr int64_t kQuantBatchRowsChunks = 1024;
struct QuantJobIn {
  const uint16_t* x;
  int64_t rows, cols;
  int kind;           // 0 = 1x32 E8M0, 1 = 1x128 fp32, 2 = 128x128 fp32
  bool floor_rule;
  uint8_t* q;
  void* scale;
  uint16_t* xdq;
};
struct QuantJob {
  const uint16_t* x;
  int64_t rows, cols;
  uint8_t* q;
  void* scale;
  uint16_t* xdq;
  int kind, floor_rule, cached, blocks_x, wg0, wgs;
};
struct QuantBatch {
  QuantJob job[kMaxQuantJobs];
  int count;
};
hipError_t launch_quant_batch(const QuantJobIn* jobs, int count, hipStream_t stream);
hipError_t launch_dequant(const uint8_t* q, const void* scale, int64_t rows, int64_t cols, int kind, uint16_t* x,
                          hipStream_t stream);
hipError_t launch_merge(const uint16_t* w, const uint16_t* lb, const uint16_t* la, int64_t n, int64_t k, int64_t r,
                        uint8_t* q, float* scale, uint16_t* wdq, hipStream_t stream);
hipError_t launch_gemm(const uint8_t* a, const void* sa, int a_kind, const uint8_t* b, const void* sb, int b_kind,
                       int64_t m, int64_t n, int64_t k, void* y, bool out_f32, int num_cu, hipStream_t stream);
hipError_t launch_grouped_gemm(const uint8_t* a, const void* sa, int a_kind, const int32_t* row_index,
                               int64_t a_rows, const uint8_t* b, const void* sb, int b_kind, const int32_t* offsets, int64_t groups,
                               int64_t total_m, int64_t n, int64_t k, void* y, bool out_f32, int num_cu,
                               hipStream_t stream);

int64_t lora_bwd_workspace_bytes(int64_t m, int64_t n, int64_t k, int64_t r);
// Fixed scratch of the no-allocation LoRA backward (one array per device):
// 40 MiB holds the workspace of 8192 tokens at hidden sizes 7168 and rank
// 64 (36.4 MiB).
constexpr int64_t kLoraScratchBytes = int64_t(40) << 20;
constexpr int kMaxScratchDevices = 64;
// The device address of `dev`'s scratch array (looked up once per device,
// with `dev` current).
hipError_t lora_bwd_scratch(int dev, void** ptr);
hipError_t launch_lora_bwd(const uint16_t* dy, const uint16_t* x, const uint16_t* lb, const uint16_t* la, int64_t m,
                           int64_t n, int64_t k, int64_t r, void* workspace, void* d_b, void* d_a, bool out_f32,
                           int num_cu, hipStream_t stream);

hipError_t launch_nvfp4_quant(const uint16_t* x, int64_t rows, int64_t cols, int64_t rpt, float* amax,
                              bool amax_given, uint8_t* q, uint8_t* bs, float* gs, uint16_t* xdq,
                              hipStream_t stream);
hipError_t launch_nvfp4_dequant(const uint8_t* q, const uint8_t* bs, const float* gs, int64_t rows, int64_t cols,
                                int64_t rpt, uint16_t* x, hipStream_t stream);

}  // namespace fp8blk
