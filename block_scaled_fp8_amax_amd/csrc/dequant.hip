// Block-scaled FP8 -> bf16 dequantization (gfx950).
//
// Method ("FP8 в DeepSeek V3", "Что такое FP8 простыми словами" and "Почему
// FP8 требует scale factors": FP8 weights are dequantized through the
// block's inverse scale when an operation needs higher precision;
// "Практический смысл для инференс-инфраструктуры": FP8 weights can be
// converted to BF16): x = RN_bf16(RN32(decode(q) * scale)), the same value
// as the fake-quant output of the quantizer.
//
// Layout: the code matrix is a flat array of 8-code chunks (8 bytes); a
// chunk never crosses a row (cols is a multiple of 32) nor a block, so it
// has a single scale.  A lane handles U chunks, each one 8-byte load of
// codes, one scale load, 4 packed fp8 -> fp32 conversions, 8 multiplies and
// one 16-byte bf16 store, so that every wave-wide store writes 1 KiB of
// contiguous memory.  One pass per workgroup over a grid that covers the
// matrix; small workgroups (2 waves, 2 chunks per lane) measured fastest.
#include "device.h"
#include "launch.h"

namespace fp8blk {

constexpr int kDqThreads = 128;   // 2 waves and 2 chunks per lane: 10% faster than
constexpr int kDqU = 2;           // 256 threads x 4 chunks on a 1x32 expert layer

// KIND: 0 = 1x32 E8M0, 1 = 1x128 fp32, 2 = 128x128 fp32 (the fp8_block values)
template <int KIND>
__global__ __launch_bounds__(kDqThreads) void dequant_kernel(const u32x2* __restrict__ q, uint32_t nchunks,
                                                             uint32_t cpr, int64_t cols, const void* __restrict__ scale,
                                                             u32x4* __restrict__ x) {
  const uint32_t first = blockIdx.x * (uint32_t)(kDqThreads * kDqU) + threadIdx.x;
  // codes and scales of every chunk loaded before any is used (indices past
  // the end read the last chunk and are not stored), so that no load waits
  // behind another
  u32x2 c[kDqU];
  float s[kDqU];
#pragma unroll
  for (int u = 0; u < kDqU; ++u) {
    const uint32_t i0 = first + u * kDqThreads;
    const uint32_t idx = i0 < nchunks ? i0 : nchunks - 1;
    c[u] = __builtin_nontemporal_load(q + idx);
    if constexpr (KIND == 0) {
      // row blocks never straddle rows, so the scales are in chunk order:
      // 4 chunks per 1x32 block
      s[u] = e8m0_val(reinterpret_cast<const uint8_t*>(scale)[idx >> 2]);
    } else if constexpr (KIND == 1) {
      s[u] = reinterpret_cast<const float*>(scale)[idx >> 4];   // 16 chunks per 1x128 tile
    } else {
      const uint32_t row = idx / cpr;                   // cpr = cols / 8 chunks per row
      const int64_t col = (int64_t)(idx - row * cpr) * 8;
      s[u] = reinterpret_cast<const float*>(scale)[(int64_t)(row / 128) * (cols / 128) + col / 128];
    }
  }
#pragma unroll
  for (int u = 0; u < kDqU; ++u) {
    const uint32_t idx = first + u * kDqThreads;
    if (idx >= nchunks) continue;
    float d[8];
    decode4_e4m3(c[u].x, d);
    decode4_e4m3(c[u].y, d + 4);
    const float su = s[u];
    const u32x4 o = {pack_bf16x2(d[0] * su, d[1] * su), pack_bf16x2(d[2] * su, d[3] * su),
                     pack_bf16x2(d[4] * su, d[5] * su), pack_bf16x2(d[6] * su, d[7] * su)};
    __builtin_nontemporal_store(o, x + idx);
  }
}

hipError_t launch_dequant(const uint8_t* q, const void* scale, int64_t rows, int64_t cols, int kind, uint16_t* x,
                          hipStream_t stream) {
  const uint32_t nchunks = (uint32_t)(rows * cols / 8);
  const uint32_t cpr = (uint32_t)(cols / 8);
  const uint32_t per_wg = kDqThreads * kDqU;
  const dim3 grid((nchunks + per_wg - 1) / per_wg);
  const u32x2* qv = reinterpret_cast<const u32x2*>(q);
  u32x4* xv = reinterpret_cast<u32x4*>(x);
  if (kind == 0)
    hipLaunchKernelGGL((dequant_kernel<0>), grid, dim3(kDqThreads), 0, stream, qv, nchunks, cpr, cols, scale, xv);
  else if (kind == 1)
    hipLaunchKernelGGL((dequant_kernel<1>), grid, dim3(kDqThreads), 0, stream, qv, nchunks, cpr, cols, scale, xv);
  else
    hipLaunchKernelGGL((dequant_kernel<2>), grid, dim3(kDqThreads), 0, stream, qv, nchunks, cpr, cols, scale, xv);
  return hipGetLastError();
}

}  // namespace fp8blk
