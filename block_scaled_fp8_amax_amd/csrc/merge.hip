// QAT forward: LoRA merge W + B.A in bf16 fused with 128x128 fake-quant.
//
// Method ("DeepSeek R1 and V3 get quantization-aware fine-tuning on
// Fireworks ...", Synopsis and Interpretation): the merged weight W + B.A
// is fake-quantized in the forward pass while the LoRA factors stay bf16;
// the FP8 weight format is DeepSeek-V3's 128x128 block with an fp32 scale
// inverse ("FP8 в DeepSeek V3", "Почему обычное округление не подходит").
//
// Arithmetic (sequential fp32 sum over the rank, one rounding per step):
//   acc = 0; for r: acc = fma(B[n,r], A[r,k], acc)   (bf16 x bf16 is exact)
//   W'  = RN_bf16(RN_bf16(acc) + W)                   (fp32 add, bf16 round)
// then the 128x128 quantizer of quantize.hip, on W' kept in registers: the
// merged weight is never written.
//
// Layout: one 256-thread workgroup per 128x128 block.  Wave w handles rows
// w, w+4, ..., lane l the two columns 2l, 2l+1, so a wave covers a whole
// 128-column block row with one dword per lane and B[n, :] is the same for
// every lane of the wave (an LDS broadcast).  Each lane holds its two
// columns of A (RMAX ranks, fp32) in registers.  The rank-r update costs
// 2r fused multiply-adds per lane per row; this kernel is bound by that
// vector-ALU work, not by HBM.
#include "device.h"
#include "launch.h"

namespace fp8blk {

template <int RMAX, bool DQ>
__global__ __launch_bounds__(256) void merge_128_kernel(const uint16_t* __restrict__ w, const uint16_t* __restrict__ lb,
                                                        const uint16_t* __restrict__ la, int64_t k, int r,
                                                        uint8_t* __restrict__ q, float* __restrict__ scale,
                                                        uint16_t* __restrict__ wdq) {
  __shared__ float sB[128][RMAX + 1];
  __shared__ uint32_t red[4];
  const int t = threadIdx.x;
  const int lane = t & 63;
  const int wv = t >> 6;
  const int64_t row0 = (int64_t)blockIdx.y * 128;
  const int64_t col = (int64_t)blockIdx.x * 128 + 2 * lane;

  // B block [128 x r] -> LDS as fp32.
  for (int i = t; i < 128 * r; i += 256) {
    const int rr = i / r, cc = i - rr * r;
    sB[rr][cc] = __uint_as_float((uint32_t)lb[(row0 + rr) * r + cc] << 16);
  }
  // A columns of this lane -> registers.
  float a0[RMAX], a1[RMAX];
#pragma unroll
  for (int i = 0; i < RMAX; ++i) {
    uint32_t pair = 0;
    if (i < r) pair = *reinterpret_cast<const uint32_t*>(la + (int64_t)i * k + col);
    a0[i] = bf_lo(pair);
    a1[i] = bf_hi(pair);
  }
  __syncthreads();

  // Merge 32 rows per wave; keep W' as packed bf16 pairs.
  uint32_t wp[32];
  uint32_t m = 0;
#pragma unroll 4
  for (int j = 0; j < 32; ++j) {
    const int rr = wv + 4 * j;
    const uint32_t w2 = __builtin_nontemporal_load(reinterpret_cast<const uint32_t*>(w + (row0 + rr) * k + col));
    float acc0 = 0.f, acc1 = 0.f;
#pragma unroll
    for (int i = 0; i < RMAX; ++i) {
      if (i < r) {
        const float b = sB[rr][i];
        acc0 = __builtin_fmaf(b, a0[i], acc0);
        acc1 = __builtin_fmaf(b, a1[i], acc1);
      }
    }
    const uint32_t d = pack_bf16x2(acc0, acc1);
    const uint32_t s2 = pack_bf16x2(bf_lo(w2) + bf_lo(d), bf_hi(w2) + bf_hi(d));
    wp[j] = s2;
    const uint32_t mm = absmax_bits<1>(&s2);
    m = m > mm ? m : mm;
  }
  m = wave_max(m);
  if (lane == 0) red[wv] = m;
  __syncthreads();
  m = red[0];
#pragma unroll
  for (int i = 1; i < 4; ++i) m = m > red[i] ? m : red[i];
  const F32Block fb = f32_block(m);

#pragma unroll 8
  for (int j = 0; j < 32; ++j) {
    const int rr = wv + 4 * j;
    const float q0 = f32_quot(bf_lo(wp[j]), fb);
    const float q1 = f32_quot(bf_hi(wp[j]), fb);
    const uint32_t c = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(q0, q1, 0, false) & 0xFFFFu;
    const int64_t off = (row0 + rr) * k + col;
    *reinterpret_cast<uint16_t*>(q + off) = (uint16_t)c;
    if constexpr (DQ) {
      const v2f d = __builtin_amdgcn_cvt_pk_f32_fp8((int)c, false);
      __builtin_nontemporal_store(pack_bf16x2(d[0] * fb.s, d[1] * fb.s), reinterpret_cast<uint32_t*>(wdq + off));
    }
  }
  if (t == 0) scale[(int64_t)blockIdx.y * (k / 128) + blockIdx.x] = fb.s;
}

hipError_t launch_merge(const uint16_t* w, const uint16_t* lb, const uint16_t* la, int64_t n, int64_t k, int64_t r,
                        uint8_t* q, float* scale, uint16_t* wdq, hipStream_t stream) {
  dim3 grid((unsigned)(k / 128), (unsigned)(n / 128));
  const int ri = (int)r;
#define FP8BLK_MERGE(RM)                                                                                       \
  do {                                                                                                         \
    if (wdq)                                                                                                   \
      hipLaunchKernelGGL((merge_128_kernel<RM, true>), grid, dim3(256), 0, stream, w, lb, la, k, ri, q, scale, \
                         wdq);                                                                                 \
    else                                                                                                       \
      hipLaunchKernelGGL((merge_128_kernel<RM, false>), grid, dim3(256), 0, stream, w, lb, la, k, ri, q,       \
                         scale, wdq);                                                                          \
  } while (0)
  if (r <= 16)
    FP8BLK_MERGE(16);
  else if (r <= 32)
    FP8BLK_MERGE(32);
  else
    FP8BLK_MERGE(64);
#undef FP8BLK_MERGE
  return hipGetLastError();
}

}  // namespace fp8blk
