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
// Layout: one 256-thread workgroup per 128x128 block; wave w owns rows
// 32w .. 32w+31.  A lane owns CPL consecutive columns (4 for ranks up to
// 16, 2 above), so LPR = 128/CPL lanes cover a block row and a wave-wide
// load covers 64/LPR rows.  All of the wave's W loads are issued first
// (the 128x128 bf16 block is held in registers, 32 dwords per lane).  B's
// block rows go to LDS as fp32 (read back as 16-byte broadcasts) and the
// lane's A columns to registers; ranks from r up to the template's RMAX
// are zero, which leaves the sequential sum unchanged bit for bit
// (acc + 0 * 0 = acc), so the rank loop has no branches.  The update costs
// RMAX fused multiply-adds per element on the vector ALU.
#include <type_traits>

#include "device.h"
#include "launch.h"

namespace fp8blk {

template <int RMAX, int CPL, bool DQ, bool CACHED>
__global__ __launch_bounds__(256) void merge_128_kernel(const uint16_t* __restrict__ w, const uint16_t* __restrict__ lb,
                                                        const uint16_t* __restrict__ la, int64_t k, int r,
                                                        uint8_t* __restrict__ q, float* __restrict__ scale,
                                                        uint16_t* __restrict__ wdq) {
  constexpr int LPR = 128 / CPL;   // lanes per block row
  constexpr int RPI = 64 / LPR;    // rows per wave-wide load
  constexpr int NJ = 32 / RPI;     // loads per lane
  constexpr int DW = CPL / 2;      // dwords per lane and row
  static_assert(CPL == 2 || CPL == 4, "columns per lane");
  static_assert(RMAX % 4 == 0, "rank padding");
  __shared__ __attribute__((aligned(16))) float sB[128 * RMAX];
  __shared__ uint32_t red[4];
  const int t = threadIdx.x;
  const int lane = t & 63;
  const int wv = t >> 6;
  const int lc = lane % LPR, lr = lane / LPR;
  const int64_t row0 = (int64_t)blockIdx.y * 128;
  const int64_t col = (int64_t)blockIdx.x * 128 + lc * CPL;
  // element offsets inside the block (a 128-row block spans 128 * k
  // elements, far below 2^32), relative to a wave-uniform base
  const int64_t blk = row0 * k + (int64_t)blockIdx.x * 128;
  const uint32_t lofs = (uint32_t)((wv * 32 + lr) * k + lc * CPL);
  const uint32_t jstep = (uint32_t)(RPI * k);
  const uint8_t* wb = reinterpret_cast<const uint8_t*>(w + blk);   // byte offsets 2 * o

  // 1. the wave's 32 rows of W, all loads in flight
  uint32_t wp[32];
#pragma unroll
  for (int j = 0; j < NJ; ++j) {
    const uint32_t o = lofs + j * jstep;
    if constexpr (DW == 2) {
      const u32x2 v = __builtin_nontemporal_load(reinterpret_cast<const u32x2*>(wb + 2 * o));
      wp[2 * j] = v.x;
      wp[2 * j + 1] = v.y;
    } else {
      wp[j] = __builtin_nontemporal_load(reinterpret_cast<const uint32_t*>(wb + 2 * o));
    }
  }
  // 2. B block [128 x r] -> LDS as fp32, ranks >= r zero
  for (int i = t; i < 128 * RMAX; i += 256) {
    const int rr = i / RMAX, cc = i % RMAX;
    sB[i] = cc < r ? __uint_as_float((uint32_t)lb[(row0 + rr) * r + cc] << 16) : 0.f;
  }
  // 3. this lane's columns of A -> registers, ranks >= r zero
  float a[RMAX][CPL];
#pragma unroll
  for (int i = 0; i < RMAX; ++i) {
    uint32_t v[DW];
#pragma unroll
    for (int d = 0; d < DW; ++d) v[d] = 0;
    if (i < r) {
      // dword loads: lora_a is only required to be 4-byte aligned
#pragma unroll
      for (int d = 0; d < DW; ++d) v[d] = *reinterpret_cast<const uint32_t*>(la + (int64_t)i * k + col + 2 * d);
    }
#pragma unroll
    for (int d = 0; d < DW; ++d) {
      a[i][2 * d] = bf_lo(v[d]);
      a[i][2 * d + 1] = bf_hi(v[d]);
    }
  }
  __syncthreads();

  // 4. merge in place: W' = RN_bf16(W + RN_bf16(sum_r B[n,r] A[r,k]))
  uint32_t m = 0;
#pragma unroll
  for (int j = 0; j < NJ; ++j) {
    const int rr = wv * 32 + j * RPI + lr;
    float acc[CPL];
#pragma unroll
    for (int c = 0; c < CPL; ++c) acc[c] = 0.f;
#pragma unroll
    for (int i = 0; i < RMAX; i += 4) {
      const float4 b4 = *reinterpret_cast<const float4*>(&sB[rr * RMAX + i]);
      const float bv[4] = {b4.x, b4.y, b4.z, b4.w};
#pragma unroll
      for (int u = 0; u < 4; ++u)
#pragma unroll
        for (int c = 0; c < CPL; ++c) acc[c] = __builtin_fmaf(bv[u], a[i + u][c], acc[c]);
    }
#pragma unroll
    for (int d = 0; d < DW; ++d) {
      const uint32_t dl = pack_bf16x2(acc[2 * d], acc[2 * d + 1]);
      const uint32_t w2 = wp[j * DW + d];
      const uint32_t s2 = pack_bf16x2(bf_lo(w2) + bf_lo(dl), bf_hi(w2) + bf_hi(dl));
      wp[j * DW + d] = s2;
      const uint32_t mm = absmax_bits<1>(&s2);
      m = m > mm ? m : mm;
    }
  }
  m = wave_max(m);
  if (lane == 0) red[wv] = m;
  __syncthreads();
  m = red[0];
#pragma unroll
  for (int i = 1; i < 4; ++i) m = m > red[i] ? m : red[i];
  const F32Block fb = f32_block(m);

  // 5. quantize the merged block and store codes (+ the fake-quant copy).
  // The block-uniform prescale of the quotient is only needed for tiny
  // blocks; the common case runs without it.
  uint8_t* qb = q + blk;
  uint8_t* db = reinterpret_cast<uint8_t*>(wdq + blk);                 // byte offsets 2 * o
  auto quantize_out = [&](auto tiny) {
    constexpr bool TINY = decltype(tiny)::value;
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
      const uint32_t o = lofs + j * jstep;
      uint32_t c[DW];
#pragma unroll
      for (int d = 0; d < DW; ++d) {
        const float q0 = TINY ? f32_quot(bf_lo(wp[j * DW + d]), fb) : f32_quot_unit(bf_lo(wp[j * DW + d]), fb);
        const float q1 = TINY ? f32_quot(bf_hi(wp[j * DW + d]), fb) : f32_quot_unit(bf_hi(wp[j * DW + d]), fb);
        c[d] = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(q0, q1, 0, false) & 0xFFFFu;
      }
      if constexpr (DW == 2)
        store_code<CACHED>(c[0] | (c[1] << 16), reinterpret_cast<uint32_t*>(qb + o));
      else
        *reinterpret_cast<uint16_t*>(qb + o) = (uint16_t)c[0];
      if constexpr (DQ) {
        uint32_t dv[DW];
#pragma unroll
        for (int d = 0; d < DW; ++d) {
          const v2f dq = __builtin_amdgcn_cvt_pk_f32_fp8((int)c[d], false);
          dv[d] = pack_bf16x2(dq[0] * fb.s, dq[1] * fb.s);
        }
        if constexpr (DW == 2)
          __builtin_nontemporal_store((u32x2){dv[0], dv[1]}, reinterpret_cast<u32x2*>(db + 2 * o));
        else
          __builtin_nontemporal_store(dv[0], reinterpret_cast<uint32_t*>(db + 2 * o));
      }
    }
  };
  if (fb.pre == 1.0f)
    quantize_out(std::false_type{});
  else
    quantize_out(std::true_type{});
  if (t == 0) scale[(int64_t)blockIdx.y * (k / 128) + blockIdx.x] = fb.s;
}

hipError_t launch_merge(const uint16_t* w, const uint16_t* lb, const uint16_t* la, int64_t n, int64_t k, int64_t r,
                        uint8_t* q, float* scale, uint16_t* wdq, hipStream_t stream) {
  dim3 grid((unsigned)(k / 128), (unsigned)(n / 128));
  const int ri = (int)r;
  const bool cached = n * k <= kCachedCodeBytes;
#define FP8BLK_MERGE(RM, CP)                                                                                         \
  do {                                                                                                               \
    if (wdq && cached)                                                                                               \
      hipLaunchKernelGGL((merge_128_kernel<RM, CP, true, true>), grid, dim3(256), 0, stream, w, lb, la, k, ri, q,    \
                         scale, wdq);                                                                                \
    else if (wdq)                                                                                                    \
      hipLaunchKernelGGL((merge_128_kernel<RM, CP, true, false>), grid, dim3(256), 0, stream, w, lb, la, k, ri, q,   \
                         scale, wdq);                                                                                \
    else if (cached)                                                                                                 \
      hipLaunchKernelGGL((merge_128_kernel<RM, CP, false, true>), grid, dim3(256), 0, stream, w, lb, la, k, ri, q,   \
                         scale, wdq);                                                                                \
    else                                                                                                             \
      hipLaunchKernelGGL((merge_128_kernel<RM, CP, false, false>), grid, dim3(256), 0, stream, w, lb, la, k, ri, q,  \
                         scale, wdq);                                                                                \
  } while (0)
  if (r <= 16)
    FP8BLK_MERGE(16, 4);
  else if (r <= 32)
    FP8BLK_MERGE(32, 2);
  else
    FP8BLK_MERGE(64, 2);
#undef FP8BLK_MERGE
  return hipGetLastError();
}

}  // namespace fp8blk
