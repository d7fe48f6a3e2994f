// Block-scaled FP8 GEMM and grouped (MoE expert) GEMM on gfx950 MFMA.
//
// Method: FP8 operands are multiplied on the matrix units and the partial
// results are promoted to a higher precision before the final accumulation
// ("DeepSeek-V3 Blog 5", "Hardware Optimization: Leveraging NVIDIA Tensor
// Cores for FP8"; matmul accumulation kept out of low precision, "FP8 в
// DeepSeek V3", "Какие операции нельзя бездумно переводить в FP8").  Here
// the partial product of every 128-wide K chunk comes from one
// v_mfma_*_16x16x128_f8f6f4 per 16x16 output tile and is folded into an
// fp32 accumulator with the chunk's fp32 scales (the per-K-block rescale);
// MXFP8 operands ("fireworks-prequant 0.1.0", "Formats") use the scaled form
// of the same instruction, which applies E8M0 scales per 32-wide K block in
// hardware.
//
// Operand modes (A is [M x K], B is [N x K], both K-contiguous):
//   kF32xF32 : A 1x128 fp32 scales, B 128x128 fp32 scales:
//              acc += P * (sa[m][kb] * sb[n/128][kb])
//   kMXxMX   : A and B 1x32 E8M0: acc = mfma_scale(A, B, acc, 2^Xa, 2^Xb)
//   kF32xMX  : A 1x128 fp32, B 1x32 E8M0 (grouped experts):
//              acc += mfma_scale(A, B, 0, 1, 2^Xb) * sa[m][kb]
//
// Tiling: a 256-thread workgroup computes a 128x128 tile of Y as a 2x2 grid
// of waves, each wave a 64x64 block of 4x4 MFMA tiles.  K advances 128 at a
// time through double-buffered LDS tiles (rows padded to 144 bytes so that
// the 16-byte fragment reads of 8 consecutive rows hit distinct banks).
//
// MFMA operand layout (measured on gfx950 with single-element probes): for
// 16x16x128 lane l holds row (l % 16) and, within the 128-wide K chunk,
// bytes [16g, 16g+16) in its first 16 bytes and [64+16g, 64+16g+16) in its
// last 16 (g = l / 16).  The scale operand of lane L applies to row L % 16
// and the 32-wide K block L / 16.  The 16x16 fp32 result gives lane l
// column l % 16 and rows 4*(l/16) + v, v = 0..3.
#include "device.h"
#include "launch.h"

namespace fp8blk {

constexpr int kBM = 128, kBN = 128, kBK = 128;
constexpr int kLdsStride = 144;

enum { kF32xF32 = 0, kMXxMX = 1, kF32xMX = 2 };

struct GemmParams {
  const uint8_t* a;
  const void* sa;
  const uint8_t* b;
  const void* sb;
  void* y;
  const int32_t* offsets;  // grouped only
  int64_t m, n, k;
  int64_t b_group_stride;   // bytes of B per group
  int64_t sb_group_stride;  // scale elements of B per group
  int groups;
  int m_slots;              // grouped: upper bound on m-tiles
};

template <int MODE>
struct ScaleKinds {
  static constexpr bool a_mx = (MODE == kMXxMX);
  static constexpr bool b_mx = (MODE != kF32xF32);
};

__device__ __forceinline__ v8i make_frag(const uint4& lo, const uint4& hi) {
  v8i r;
  r[0] = (int)lo.x; r[1] = (int)lo.y; r[2] = (int)lo.z; r[3] = (int)lo.w;
  r[4] = (int)hi.x; r[5] = (int)hi.y; r[6] = (int)hi.z; r[7] = (int)hi.w;
  return r;
}

// Locate the tile of a grouped problem: slot -> (group, first row, rows).
// Every workgroup rebuilds the prefix of m-tiles per group in LDS.
// `scratch` is LDS of at least 2 * 1025 ints that is free until the caller's
// next barrier.
__device__ __forceinline__ bool grouped_tile(const int32_t* __restrict__ off, int groups, int slot, int* scratch,
                                             int* g_out, int64_t* row0, int* rows) {
  int* s_off = scratch;
  int* s_pref = scratch + 1025;
  const int t = threadIdx.x;
  for (int g = t; g <= groups; g += 256) s_off[g] = off[g];
  __syncthreads();
  // tiles per group, then an inclusive scan (groups <= 1024)
  for (int g = t; g < groups; g += 256) s_pref[g + 1] = (s_off[g + 1] - s_off[g] + kBM - 1) / kBM;
  if (t == 0) s_pref[0] = 0;
  __syncthreads();
  for (int d = 1; d < groups; d <<= 1) {
    int v[4];
    int cnt = 0;
    for (int g = t; g < groups; g += 256) v[cnt++] = (g >= d) ? s_pref[g + 1 - d] : 0;
    __syncthreads();
    cnt = 0;
    for (int g = t; g < groups; g += 256) s_pref[g + 1] += v[cnt++];
    __syncthreads();
  }
  if (slot >= s_pref[groups]) return false;
  int lo = 0, hi = groups - 1;  // find g with s_pref[g] <= slot < s_pref[g+1]
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (s_pref[mid] <= slot) lo = mid; else hi = mid - 1;
  }
  const int g = lo;
  *g_out = g;
  *row0 = (int64_t)s_off[g] + (int64_t)(slot - s_pref[g]) * kBM;
  const int64_t left = (int64_t)s_off[g + 1] - *row0;
  *rows = (int)(left < kBM ? left : kBM);
  return true;
}

template <int MODE, bool OUT_F32, bool GROUPED>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2))) void gemm_kernel(GemmParams p) {
  using SK = ScaleKinds<MODE>;
  __shared__ __attribute__((aligned(16))) uint8_t sA[2][kBM * kLdsStride];
  __shared__ __attribute__((aligned(16))) uint8_t sB[2][kBN * kLdsStride];
  __shared__ __attribute__((aligned(16))) uint32_t sSA[2][kBM];  // fp32 bits or 4 E8M0 bytes per row
  __shared__ __attribute__((aligned(16))) uint32_t sSB[2][kBN];  // 4 E8M0 bytes per column (MX B)

  const int t = threadIdx.x;
  const int lane = t & 63;
  const int wave = t >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int64_t K = p.k;
  const int KB = (int)(K / kBK);

  // ---- tile coordinates
  int64_t m0;
  int mrows;
  const int64_t n0 = (int64_t)blockIdx.y * kBN;
  const uint8_t* bq = p.b;
  const uint8_t* sbq8 = reinterpret_cast<const uint8_t*>(p.sb);
  const float* sbf = reinterpret_cast<const float*>(p.sb);
  if constexpr (GROUPED) {
    int g;
    // sA[1] is first written after the barrier that follows store_tile(0)
    if (!grouped_tile(p.offsets, p.groups, (int)blockIdx.x, reinterpret_cast<int*>(&sA[1][0]), &g, &m0, &mrows))
      return;
    bq += (int64_t)g * p.b_group_stride;
    sbq8 += (int64_t)g * p.sb_group_stride;
    sbf += (int64_t)g * p.sb_group_stride;
  } else {
    m0 = (int64_t)blockIdx.x * kBM;
    const int64_t left = p.m - m0;
    mrows = (int)(left < kBM ? left : kBM);
  }
  const uint8_t* aq = p.a + m0 * K;

  // ---- global -> register staging: 4 A chunks + 4 B chunks of 16 B per thread
  const int ld_row = t >> 3;       // 0..31
  const int ld_c = (t & 7) * 16;   // byte offset in the 128-byte K chunk
  uint4 ra[4], rb[4];
  uint32_t rsa = 0, rsb = 0;
  float sb_k = 0.f;

  auto load_tile = [&](int kb) {
    const int64_t koff = (int64_t)kb * kBK + ld_c;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int r = ld_row + 32 * j;
      ra[j] = r < mrows ? *reinterpret_cast<const uint4*>(aq + (int64_t)r * K + koff) : make_uint4(0, 0, 0, 0);
      rb[j] = *reinterpret_cast<const uint4*>(bq + (n0 + r) * K + koff);
    }
    if (t < kBM) {
      if constexpr (SK::a_mx)
        rsa = t < mrows ? *reinterpret_cast<const uint32_t*>(reinterpret_cast<const uint8_t*>(p.sa) +
                                                             (m0 + t) * (K / 32) + 4 * kb)
                        : 0u;
      else
        rsa = t < mrows ? __float_as_uint(reinterpret_cast<const float*>(p.sa)[(m0 + t) * KB + kb]) : 0u;
    } else if constexpr (SK::b_mx) {
      const int c = t - kBM;
      rsb = *reinterpret_cast<const uint32_t*>(sbq8 + (n0 + c) * (K / 32) + 4 * kb);
    }
  };
  auto store_tile = [&](int buf) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int r = ld_row + 32 * j;
      *reinterpret_cast<uint4*>(&sA[buf][r * kLdsStride + ld_c]) = ra[j];
      *reinterpret_cast<uint4*>(&sB[buf][r * kLdsStride + ld_c]) = rb[j];
    }
    if (t < kBM) sSA[buf][t] = rsa;
    else if constexpr (SK::b_mx) sSB[buf][t - kBM] = rsb;
  };

  v4f acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = (v4f){0.f, 0.f, 0.f, 0.f};

  const int fr = lane & 15;          // fragment row / column
  const int fg = (lane >> 4) * 16;   // K byte offset of the lane group

  load_tile(0);
  store_tile(0);
  __syncthreads();

  for (int kb = 0; kb < KB; ++kb) {
    const int buf = kb & 1;
    if (kb + 1 < KB) load_tile(kb + 1);
    if constexpr (MODE == kF32xF32) sb_k = sbf[(n0 / 128) * KB + kb];

    // A fragments and per-row scales of this wave's 4 m-subtiles
    v8i af[4];
    float sc[4][4];
    int xa[4];
#pragma unroll
    for (int mi = 0; mi < 4; ++mi) {
      const int ar = wm * 64 + mi * 16 + fr;
      const uint8_t* base = &sA[buf][ar * kLdsStride + fg];
      af[mi] = make_frag(*reinterpret_cast<const uint4*>(base), *reinterpret_cast<const uint4*>(base + 64));
      if constexpr (SK::a_mx) {
        xa[mi] = (int)((sSA[buf][ar] >> (8 * (lane >> 4))) & 0xFFu);
      } else {
        const uint4 s4 = *reinterpret_cast<const uint4*>(&sSA[buf][wm * 64 + mi * 16 + 4 * (lane >> 4)]);
        sc[mi][0] = __uint_as_float(s4.x);
        sc[mi][1] = __uint_as_float(s4.y);
        sc[mi][2] = __uint_as_float(s4.z);
        sc[mi][3] = __uint_as_float(s4.w);
        if constexpr (MODE == kF32xF32) {
#pragma unroll
          for (int v = 0; v < 4; ++v) sc[mi][v] *= sb_k;
        }
      }
    }
#pragma unroll
    for (int ni = 0; ni < 4; ++ni) {
      const int bc = wn * 64 + ni * 16 + fr;
      const uint8_t* base = &sB[buf][bc * kLdsStride + fg];
      const v8i bfr = make_frag(*reinterpret_cast<const uint4*>(base), *reinterpret_cast<const uint4*>(base + 64));
      int xb = 127;
      if constexpr (SK::b_mx) xb = (int)((sSB[buf][bc] >> (8 * (lane >> 4))) & 0xFFu);
#pragma unroll
      for (int mi = 0; mi < 4; ++mi) {
        if constexpr (MODE == kMXxMX) {
          acc[mi][ni] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(af[mi], bfr, acc[mi][ni], 0, 0, 0, xa[mi],
                                                                         0, xb);
        } else {
          const v4f zero = {0.f, 0.f, 0.f, 0.f};
          v4f pp;
          if constexpr (MODE == kF32xMX)
            pp = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(af[mi], bfr, zero, 0, 0, 0, 127, 0, xb);
          else
            pp = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(af[mi], bfr, zero, 0, 0, 0, 0, 0, 0);
#pragma unroll
          for (int v = 0; v < 4; ++v) acc[mi][ni][v] = __builtin_fmaf(pp[v], sc[mi][v], acc[mi][ni][v]);
        }
      }
    }
    if (kb + 1 < KB) store_tile(buf ^ 1);
    __syncthreads();
  }

  // ---- epilogue
  const int64_t N = p.n;
#pragma unroll
  for (int mi = 0; mi < 4; ++mi) {
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int r = wm * 64 + mi * 16 + 4 * (lane >> 4) + v;
      if (r < mrows) {
        const int64_t row = m0 + r;
#pragma unroll
        for (int ni = 0; ni < 4; ++ni) {
          const int64_t col = n0 + wn * 64 + ni * 16 + fr;
          const float val = acc[mi][ni][v];
          if constexpr (OUT_F32) {
            reinterpret_cast<float*>(p.y)[row * N + col] = val;
          } else {
            const uint32_t b2 = pack_bf16x2(val, 0.f);
            reinterpret_cast<uint16_t*>(p.y)[row * N + col] = (uint16_t)(b2 & 0xFFFFu);
          }
        }
      }
    }
  }
}

template <int MODE, bool GROUPED>
static void launch_mode(const GemmParams& p, dim3 grid, bool out_f32, hipStream_t stream) {
  if (out_f32)
    hipLaunchKernelGGL((gemm_kernel<MODE, true, GROUPED>), grid, dim3(256), 0, stream, p);
  else
    hipLaunchKernelGGL((gemm_kernel<MODE, false, GROUPED>), grid, dim3(256), 0, stream, p);
}

hipError_t launch_gemm(const uint8_t* a, const void* sa, int a_kind, const uint8_t* b, const void* sb, int b_kind,
                       int64_t m, int64_t n, int64_t k, void* y, bool out_f32, hipStream_t stream) {
  GemmParams p{};
  p.a = a; p.sa = sa; p.b = b; p.sb = sb; p.y = y;
  p.m = m; p.n = n; p.k = k;
  dim3 grid((unsigned)((m + kBM - 1) / kBM), (unsigned)(n / kBN));
  if (a_kind == 1 && b_kind == 2)
    launch_mode<kF32xF32, false>(p, grid, out_f32, stream);
  else
    launch_mode<kMXxMX, false>(p, grid, out_f32, stream);
  return hipGetLastError();
}

hipError_t launch_grouped_gemm(const uint8_t* a, const void* sa, int a_kind, const uint8_t* b, const void* sb,
                               int b_kind, const int32_t* offsets, int64_t groups, int64_t total_m, int64_t n,
                               int64_t k, void* y, bool out_f32, hipStream_t stream) {
  (void)a_kind;
  GemmParams p{};
  p.a = a; p.sa = sa; p.b = b; p.sb = sb; p.y = y;
  p.offsets = offsets;
  p.m = total_m; p.n = n; p.k = k;
  p.groups = (int)groups;
  p.b_group_stride = n * k;
  const int64_t slots = total_m / kBM + groups;
  p.m_slots = (int)slots;
  dim3 grid((unsigned)slots, (unsigned)(n / kBN));
  if (b_kind == 0) {
    p.sb_group_stride = n * (k / 32);
    launch_mode<kF32xMX, true>(p, grid, out_f32, stream);
  } else {
    p.sb_group_stride = (n / 128) * (k / 128);
    launch_mode<kF32xF32, true>(p, grid, out_f32, stream);
  }
  return hipGetLastError();
}

}  // namespace fp8blk
