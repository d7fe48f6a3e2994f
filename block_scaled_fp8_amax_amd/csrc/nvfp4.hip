// NVFP4 prequantization and dequantization (gfx950).
//
// Format ([prequant] "Formats": packed FP4 values with FP8 block scales,
// served at FP4): E2M1 elements two per byte (element 2j of a row in the low
// nibble of byte j), one e4m3fn scale per 1x16 block of a row, and one fp32
// scale g per tensor so that the e4m3 block scales cover the tensor's range:
//   A = max |x| over the tensor, g = RN32(A / 2688)        (2688 = 448 * 6)
//   S = e4m3(RN32(a / RN32(6 g)))   a = the block's amax, RNE, saturating
//   m = RN32(e4m3(S) * g);  code = e2m1(RN32(x / m)), RNE, saturating at 6,
//   sign kept; m = 0 leaves the sign alone
//   dequantized value RN_bf16(RN32(e2m1(code) * m)).
//
// Kernels:
//   nvfp4_zero_kernel / nvfp4_amax_kernel: per-tensor A as fp32 bits
//     (atomic max of non-negative floats ordered as integers; exact and
//     order-independent).  An amax workgroup streams 256 KiB in eight
//     rounds, the next round's loads in flight while the current one is
//     reduced (256 KiB per workgroup measured fastest: 128 KiB and 512 KiB
//     both ran about 12% slower).
//   nvfp4_quant_kernel: one lane per 1x16 block (two 16-byte loads, 8 bytes
//     of codes), two blocks per lane.  x / m is the correctly rounded
//     quotient from a correctly rounded reciprocal and one remainder
//     correction (Markstein), prescaled by 2^64 for m < 2^-60 (a branch
//     taken only by waves that hold such a block).
//     v_cvt_scalef32_pk_fp4_f32 with scale 1 rounds two fp32 values to E2M1
//     (nearest even, saturating, sign kept) into one byte; the fake-quant
//     output decodes with v_cvt_scalef32_pk_f32_fp4.
//   nvfp4_dequant_kernel: half a 1x16 block (8 codes, one dword) per lane,
//     two halves per lane 256 lanes apart, each to one 16-byte bf16 store, so
//     that every store instruction writes 1 KiB contiguous.  14% faster than
//     a whole block per lane (two stores 32 bytes apart per lane, which
//     cover each line only halfway per instruction); one half per lane was
//     9% slower than that, four and eight per lane 4% and 0% faster.
#include "device.h"
#include "launch.h"

namespace fp8blk {

namespace {

constexpr int kNvThreads = 256;     // zero and amax kernels
constexpr int kNvQThreads = 64;     // encode kernel (one wave: 2% faster than 256 threads)
constexpr int kNvDThreads = 256;    // dequantize kernel
constexpr int kNvU = 2;          // half 1x16 blocks per lane (dequantize)
constexpr int kAmU = 8;          // chunks per lane per round (amax)
constexpr int kAmRounds = 8;     // rounds per amax workgroup
constexpr float kGlobalDiv = 2688.0f;

__global__ __launch_bounds__(kNvThreads) void nvfp4_zero_kernel(uint32_t* amax_bits, uint32_t tensors) {
  const uint32_t i = blockIdx.x * kNvThreads + threadIdx.x;
  if (i < tensors) amax_bits[i] = 0u;
}

// Tensor t owns chunks [t * cpt, (t + 1) * cpt); workgroups of a tensor split
// its chunks (kAmRounds * kAmU per lane), each adds its max with one atomic.
__global__ __launch_bounds__(kNvThreads) void nvfp4_amax_kernel(const u32x4* __restrict__ x, uint32_t cpt,
                                                                uint32_t wpt, uint32_t* __restrict__ amax_bits) {
  __shared__ uint32_t red[kNvThreads / 64];
  const uint32_t t = blockIdx.x / wpt;
  const uint32_t wi = blockIdx.x - t * wpt;
  const u32x4* xt = x + (uint64_t)t * cpt;
  const uint32_t c0 = wi * (uint32_t)(kNvThreads * kAmU * kAmRounds) + threadIdx.x;
  uint32_t mx = 0;
  u32x4 v[kAmU];
#pragma unroll
  for (int u = 0; u < kAmU; ++u) {
    const uint32_t c = c0 + u * kNvThreads;
    v[u] = c < cpt ? __builtin_nontemporal_load(xt + c) : (u32x4){0u, 0u, 0u, 0u};
  }
  for (int rnd = 1; rnd <= kAmRounds; ++rnd) {
    u32x4 cur[kAmU];
#pragma unroll
    for (int u = 0; u < kAmU; ++u) cur[u] = v[u];
    if (rnd < kAmRounds) {
#pragma unroll
      for (int u = 0; u < kAmU; ++u) {
        const uint32_t c = c0 + (rnd * kAmU + u) * kNvThreads;
        v[u] = c < cpt ? __builtin_nontemporal_load(xt + c) : (u32x4){0u, 0u, 0u, 0u};
      }
    }
#pragma unroll
    for (int u = 0; u < kAmU; ++u) {
      const uint32_t w[4] = {cur[u].x, cur[u].y, cur[u].z, cur[u].w};
      const uint32_t b = absmax_bits<4>(w);
      mx = mx > b ? mx : b;
    }
  }
  mx = wave_max(mx);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = mx;
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t r = red[0];
#pragma unroll
    for (int i = 1; i < kNvThreads / 64; ++i) r = r > red[i] ? r : red[i];
    atomicMax(amax_bits + t, r << 16);
  }
}

// Four bytes of E2M1 code pairs times m, rounded to bf16: one 16-byte group.
__device__ __forceinline__ u32x4 fp4x8_times(uint32_t code, float m) {
  const v2f d0 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(code, 1.0f, 0);
  const v2f d1 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(code, 1.0f, 1);
  const v2f d2 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(code, 1.0f, 2);
  const v2f d3 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(code, 1.0f, 3);
  return (u32x4){pack_bf16x2(d0[0] * m, d0[1] * m), pack_bf16x2(d1[0] * m, d1[1] * m),
                 pack_bf16x2(d2[0] * m, d2[1] * m), pack_bf16x2(d3[0] * m, d3[1] * m)};
}

__device__ __forceinline__ float with_sign_of(float q, float x) {
  return __uint_as_float((__float_as_uint(q) & 0x7FFFFFFFu) | (__float_as_uint(x) & 0x80000000u));
}

// One lane per 1x16 block (two 16-byte loads); block index bi covers
// elements [16 bi, 16 bi + 16); codes are 8 bytes per block.
constexpr int kNvB = 2;   // blocks per lane

template <bool DQ>
__global__ __launch_bounds__(kNvQThreads) void nvfp4_quant_kernel(const u32x4* __restrict__ x, uint32_t nblocks,
                                                                 uint32_t bpt,
                                                                 const float* __restrict__ amax,
                                                                 u32x2* __restrict__ q, uint8_t* __restrict__ bs,
                                                                 float* __restrict__ gs, u32x4* __restrict__ xdq) {
  const uint32_t first = blockIdx.x * (uint32_t)(kNvQThreads * kNvB) + threadIdx.x;
  u32x4 v[kNvB][2];
#pragma unroll
  for (int u = 0; u < kNvB; ++u) {
    const uint32_t bi = first + u * kNvQThreads;
#pragma unroll
    for (int h = 0; h < 2; ++h)
      v[u][h] = bi < nblocks ? __builtin_nontemporal_load(x + 2 * bi + h) : (u32x4){0u, 0u, 0u, 0u};
  }
#pragma unroll
  for (int u = 0; u < kNvB; ++u) {
    const uint32_t bi = first + u * kNvQThreads;
    if (bi >= nblocks) continue;
    const uint32_t w[8] = {v[u][0].x, v[u][0].y, v[u][0].z, v[u][0].w, v[u][1].x, v[u][1].y, v[u][1].z, v[u][1].w};
    const uint32_t ab = absmax_bits<8>(w);
    const uint32_t t = bi / bpt;
    const float g = amax[t] / kGlobalDiv;
    const float t6 = 6.0f * g;
    const float a = __uint_as_float(ab << 16);
    const float ratio = t6 > 0.0f ? a / t6 : 0.0f;
    const uint32_t S = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(clamp448(ratio), 0.0f, 0, false) & 0xFFu;
    const float m = __builtin_amdgcn_cvt_pk_f32_fp8((int)S, false)[0] * g;
    float xe[16], qv[16];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      xe[2 * i] = bf_lo(w[i]);
      xe[2 * i + 1] = bf_hi(w[i]);
    }
    if (__builtin_amdgcn_ballot_w64(m < 0x1p-60f) == 0) {
      // no lane of the wave needs the prescale
      const float y = 1.0f / m;
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const float q0 = xe[e] * y;
        const float r = __builtin_fmaf(-q0, m, xe[e]);
        qv[e] = with_sign_of(__builtin_fmaf(r, y, q0), xe[e]);
      }
    } else if (m > 0.0f) {
      const float pre = m < 0x1p-60f ? 0x1p64f : 1.0f;
      const float mp = m * pre;
      const float y = 1.0f / mp;
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const float xp = xe[e] * pre;
        const float q0 = xp * y;
        const float r = __builtin_fmaf(-q0, mp, xp);
        qv[e] = with_sign_of(__builtin_fmaf(r, y, q0), xe[e]);
      }
    } else {
#pragma unroll
      for (int e = 0; e < 16; ++e) qv[e] = xe[e] * 0.0f;
    }
    uint32_t c0 = 0, c1 = 0;
    c0 = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(c0, qv[0], qv[1], 1.0f, 0);
    c0 = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(c0, qv[2], qv[3], 1.0f, 1);
    c0 = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(c0, qv[4], qv[5], 1.0f, 2);
    c0 = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(c0, qv[6], qv[7], 1.0f, 3);
    c1 = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(c1, qv[8], qv[9], 1.0f, 0);
    c1 = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(c1, qv[10], qv[11], 1.0f, 1);
    c1 = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(c1, qv[12], qv[13], 1.0f, 2);
    c1 = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(c1, qv[14], qv[15], 1.0f, 3);
    __builtin_nontemporal_store((u32x2){c0, c1}, q + bi);
    bs[bi] = (uint8_t)S;
    if (bi == t * bpt) gs[t] = g;
    if constexpr (DQ) {
      __builtin_nontemporal_store(fp4x8_times(c0, m), xdq + 2 * bi);
      __builtin_nontemporal_store(fp4x8_times(c1, m), xdq + 2 * bi + 1);
    }
  }
}

// Half h of the codes (dword h: elements 8h .. 8h+7, block h / 2) goes to
// the bf16 chunk x[h].
__global__ __launch_bounds__(kNvDThreads) void nvfp4_dequant_kernel(const uint32_t* __restrict__ q, uint32_t nhalves,
                                                                   uint32_t bpt,
                                                                   const uint8_t* __restrict__ bs,
                                                                   const float* __restrict__ gs,
                                                                   u32x4* __restrict__ x) {
  const uint32_t first = blockIdx.x * (uint32_t)(kNvDThreads * kNvU) + threadIdx.x;
  // codes, block scale and global scale of every half loaded before any is
  // used (2% faster than loading the scales after the branch); halves past
  // the end read the last half and are not stored
  uint32_t c[kNvU], sb[kNvU];
  float sg[kNvU];
#pragma unroll
  for (int u = 0; u < kNvU; ++u) {
    const uint32_t h0 = first + u * kNvDThreads;
    const uint32_t h = h0 < nhalves ? h0 : nhalves - 1;
    c[u] = __builtin_nontemporal_load(q + h);
    sb[u] = bs[h >> 1];
    sg[u] = gs[(h >> 1) / bpt];
  }
#pragma unroll
  for (int u = 0; u < kNvU; ++u) {
    const uint32_t h = first + u * kNvDThreads;
    if (h >= nhalves) continue;
    const float m = __builtin_amdgcn_cvt_pk_f32_fp8((int)sb[u], false)[0] * sg[u];
    __builtin_nontemporal_store(fp4x8_times(c[u], m), x + h);
  }
}

}  // namespace

hipError_t launch_nvfp4_quant(const uint16_t* x, int64_t rows, int64_t cols, int64_t rpt, float* amax,
                              bool amax_given, uint8_t* q, uint8_t* bs, float* gs, uint16_t* xdq,
                              hipStream_t stream) {
  const uint32_t nchunks = (uint32_t)(rows * cols / 8);
  const uint32_t cpr = (uint32_t)(cols / 8);
  const uint32_t tensors = (uint32_t)(rows / rpt);
  const u32x4* xv = reinterpret_cast<const u32x4*>(x);
  if (!amax_given) {
    uint32_t* ab = reinterpret_cast<uint32_t*>(amax);
    hipLaunchKernelGGL(nvfp4_zero_kernel, dim3((tensors + kNvThreads - 1) / kNvThreads), dim3(kNvThreads), 0,
                       stream, ab, tensors);
    const uint32_t cpt = (uint32_t)(rpt * cols / 8);
    const uint32_t per = kNvThreads * kAmU * kAmRounds;
    const uint32_t wpt = (cpt + per - 1) / per;
    hipLaunchKernelGGL(nvfp4_amax_kernel, dim3(tensors * wpt), dim3(kNvThreads), 0, stream, xv, cpt, wpt, ab);
  }
  const uint32_t nblocks = nchunks / 2, bpt = (uint32_t)(rpt * (cpr / 2));
  const uint32_t per_wg = kNvQThreads * kNvB;
  const dim3 grid((nblocks + per_wg - 1) / per_wg);
  u32x2* qv = reinterpret_cast<u32x2*>(q);
  if (xdq)
    hipLaunchKernelGGL((nvfp4_quant_kernel<true>), grid, dim3(kNvQThreads), 0, stream, xv, nblocks, bpt, amax, qv,
                       bs, gs, reinterpret_cast<u32x4*>(xdq));
  else
    hipLaunchKernelGGL((nvfp4_quant_kernel<false>), grid, dim3(kNvQThreads), 0, stream, xv, nblocks, bpt, amax, qv,
                       bs, gs, nullptr);
  return hipGetLastError();
}

hipError_t launch_nvfp4_dequant(const uint8_t* q, const uint8_t* bs, const float* gs, int64_t rows, int64_t cols,
                                int64_t rpt, uint16_t* x, hipStream_t stream) {
  const uint32_t nhalves = (uint32_t)(rows * cols / 8);
  const uint32_t per_wg = kNvDThreads * kNvU;
  hipLaunchKernelGGL(nvfp4_dequant_kernel, dim3((nhalves + per_wg - 1) / per_wg), dim3(kNvDThreads), 0, stream,
                     reinterpret_cast<const uint32_t*>(q), nhalves, (uint32_t)(rpt * cols / 16), bs, gs,
                     reinterpret_cast<u32x4*>(x));
  return hipGetLastError();
}

}  // namespace fp8blk
