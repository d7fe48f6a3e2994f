// Block-wise FP8 quantization kernels (gfx950).
//
// Method: per block amax -> scale -> round-to-nearest-even, saturating
// e4m3fn encode ("DeepSeek-V3 Blog 5", "The Solution: Block-Wise
// Quantization"; "FP8 в DeepSeek V3", 128x128 weight blocks with an fp32
// scale inverse and per-token 1x128 activation groups; "fireworks-prequant
// 0.1.0", MXFP8 1x32 blocks with E8M0 scales).
//
// Two kernels:
//   quant_rows  : 1x32 and 1x128 blocks.  Both run along the contiguous
//                 dimension and the column count is a multiple of the block,
//                 so the matrix is a flat array of consecutive blocks and the
//                 scale array is in block order.  One 16-byte load per lane
//                 holds 8 bf16; a block is 4 (1x32) or 16 (1x128) adjacent
//                 lanes, reduced with DPP lane permutations.  Each wave
//                 handles U = 2 chunks per lane (2 KiB of bf16 in flight
//                 per wave) and a workgroup is one wave, one pass per
//                 workgroup: the grid covers the whole matrix, so retiring
//                 workgroups are replaced by new ones whose loads are issued
//                 at once (measured faster than a capped grid walking the
//                 matrix in a grid-stride loop, which serializes each wave's
//                 loads behind its stores, and than 4 chunks per lane or
//                 256-thread workgroups: 7.5% on a 1x32 expert-layer
//                 prequant, 2% on 1x128 activations).
//   quant_128   : 128x128 blocks, one 512-thread workgroup per block; every
//                 thread keeps its 32 elements in registers between the amax
//                 pass and the encode pass, so the block is read once.
// Codes go out with ordinary stores when the code matrix fits in half the
// Infinity Cache (CACHED), with nontemporal stores otherwise; the bf16
// fake-quant copy is always nontemporal.
#include "device.h"
#include "launch.h"

namespace fp8blk {

constexpr int kQRowsThreads = 64;
constexpr int kQRowsU = 2;

// Encode the 8 bf16 values of one chunk; returns the codes as two dwords and
// (if DQ) writes the bf16 fake-quant values to dq[0..3].
template <bool F32SCALE, bool FLOOR, bool DQ>
__device__ __forceinline__ u32x2 encode_chunk(const u32x4& v, const F32Block& fb, float inv, float sval,
                                              u32x4* dq) {
  const uint32_t w[4] = {v.x, v.y, v.z, v.w};
  float f[8];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    float lo = bf_lo(w[i]), hi = bf_hi(w[i]);
    if constexpr (F32SCALE) {
      f[2 * i] = f32_quot(lo, fb);
      f[2 * i + 1] = f32_quot(hi, fb);
    } else {
      f[2 * i] = lo * inv;        // exact power-of-two scaling
      f[2 * i + 1] = hi * inv;
      if constexpr (FLOOR) {
        f[2 * i] = clamp448(f[2 * i]);
        f[2 * i + 1] = clamp448(f[2 * i + 1]);
      }
    }
  }
  u32x2 c;
  c.x = cvt4_e4m3(f[0], f[1], f[2], f[3]);
  c.y = cvt4_e4m3(f[4], f[5], f[6], f[7]);
  if constexpr (DQ) {
    float d[8];
    decode4_e4m3(c.x, d);
    decode4_e4m3(c.y, d + 4);
    u32x4 o;
    o.x = pack_bf16x2(d[0] * sval, d[1] * sval);
    o.y = pack_bf16x2(d[2] * sval, d[3] * sval);
    o.z = pack_bf16x2(d[4] * sval, d[5] * sval);
    o.w = pack_bf16x2(d[6] * sval, d[7] * sval);
    *dq = o;
  }
  return c;
}

// BLK = 32 (E8M0 scales) or 128 (fp32 scales).  Wave `wave` of `nwaves`
// takes the passes wave, wave + nwaves, ... of 64 * kQRowsU chunks.
template <int BLK, bool FLOOR, bool DQ, bool CACHED>
__device__ __forceinline__ void quant_rows_body(const u32x4* __restrict__ x, int64_t nchunks, u32x2* __restrict__ q,
                                                void* __restrict__ scale, u32x4* __restrict__ xdq, int64_t wave,
                                                int64_t nwaves, int lane) {
  constexpr int LANES = BLK / 8;
  constexpr bool F32SCALE = (BLK == 128);
  for (int64_t base = wave * 64 * kQRowsU; base < nchunks; base += nwaves * 64 * kQRowsU) {
    u32x4 v[kQRowsU];
#pragma unroll
    for (int u = 0; u < kQRowsU; ++u) {
      const int64_t idx = base + u * 64 + lane;
      v[u] = idx < nchunks ? __builtin_nontemporal_load(x + idx) : (u32x4){0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int u = 0; u < kQRowsU; ++u) {
      const int64_t idx = base + u * 64 + lane;
      const uint32_t w[4] = {v[u].x, v[u].y, v[u].z, v[u].w};
      const uint32_t amax = group_max<LANES>(absmax_bits<4>(w));
      F32Block fb;
      float inv = 0.f, sval;
      uint32_t code = 0;
      if constexpr (F32SCALE) {
        fb = f32_block(amax);
        sval = fb.s;
      } else {
        code = e8m0_code<FLOOR>(amax);
        inv = e8m0_inv(code);
        sval = e8m0_val(code);
      }
      u32x4 dqv;
      const u32x2 c = encode_chunk<F32SCALE, FLOOR, DQ>(v[u], fb, inv, sval, &dqv);
      if (idx < nchunks) {
        store_code<CACHED>(c, q + idx);
        if constexpr (DQ) __builtin_nontemporal_store(dqv, xdq + idx);
        if ((lane & (LANES - 1)) == 0) {
          if constexpr (F32SCALE)
            reinterpret_cast<float*>(scale)[idx / LANES] = fb.s;
          else
            reinterpret_cast<uint8_t*>(scale)[idx / LANES] = (uint8_t)code;
        }
      }
    }
  }
}

template <int BLK, bool FLOOR, bool DQ, bool CACHED>
__global__ __launch_bounds__(kQRowsThreads) void quant_rows_kernel(const u32x4* __restrict__ x, int64_t nchunks,
                                                                   u32x2* __restrict__ q, void* __restrict__ scale,
                                                                   u32x4* __restrict__ xdq) {
  quant_rows_body<BLK, FLOOR, DQ, CACHED>(x, nchunks, q, scale, xdq,
                                          (int64_t)blockIdx.x * (kQRowsThreads / 64) + (threadIdx.x >> 6),
                                          (int64_t)gridDim.x * (kQRowsThreads / 64), (int)(threadIdx.x & 63));
}

// 128x128 block (bx, by) by a 512-thread workgroup: thread t covers column
// chunk (t % 16) * 8 of rows (t / 16) + 32 * i, i = 0..3; red is 8 words of
// LDS.
template <bool DQ, bool CACHED>
__device__ __forceinline__ void quant_128_body(const uint16_t* __restrict__ x, int64_t cols, uint8_t* __restrict__ q,
                                               float* __restrict__ scale, uint16_t* __restrict__ xdq, int64_t bx,
                                               int64_t by, uint32_t* red) {
  const int t = threadIdx.x;
  const int64_t r0 = by * 128 + (t >> 4);
  const int64_t c0 = bx * 128 + (t & 15) * 8;
  u32x4 v[4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
    v[i] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(x + (r0 + 32 * i) * cols + c0));
  uint32_t m = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint32_t w[4] = {v[i].x, v[i].y, v[i].z, v[i].w};
    const uint32_t mi = absmax_bits<4>(w);
    m = m > mi ? m : mi;
  }
  m = wave_max(m);
  if ((t & 63) == 0) red[t >> 6] = m;
  __syncthreads();
  m = red[0];
#pragma unroll
  for (int i = 1; i < 8; ++i) m = m > red[i] ? m : red[i];
  const F32Block fb = f32_block(m);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    u32x4 dqv;
    const u32x2 c = encode_chunk<true, false, DQ>(v[i], fb, 0.f, fb.s, &dqv);
    const int64_t off = (r0 + 32 * i) * cols + c0;
    store_code<CACHED>(c, reinterpret_cast<u32x2*>(q + off));
    if constexpr (DQ) __builtin_nontemporal_store(dqv, reinterpret_cast<u32x4*>(xdq + off));
  }
  if (t == 0) scale[by * (cols / 128) + bx] = fb.s;
}

template <bool DQ, bool CACHED>
__global__ __launch_bounds__(512) void quant_128_kernel(const uint16_t* __restrict__ x, int64_t cols,
                                                        uint8_t* __restrict__ q, float* __restrict__ scale,
                                                        uint16_t* __restrict__ xdq) {
  __shared__ uint32_t red[8];
  quant_128_body<DQ, CACHED>(x, cols, q, scale, xdq, blockIdx.x, blockIdx.y, red);
}

// ------------------------------------------------------------ batched jobs

// Several independent quantizations in one launch of 512-thread
// workgroups: job j owns workgroups [wg0, wg0 + wgs).  A 128x128 job runs one
// workgroup per block; a 1x32 / 1x128 job runs the rows body over its
// workgroups' 8 waves each.  Every job's bytes equal those of its own launch
// (a block never spans two waves, whatever the grouping into workgroups).
__global__ __launch_bounds__(512) void quant_batch_kernel(QuantBatch b) {
  __shared__ uint32_t red[8];
  int j = 0;
  while (j + 1 < b.count && (int)blockIdx.x >= b.job[j + 1].wg0) ++j;
  const QuantJob& J = b.job[j];
  const int local = (int)blockIdx.x - J.wg0;
  const bool dq = J.xdq != nullptr;
  if (J.kind == 2) {
    const int64_t bx = local % J.blocks_x, by = local / J.blocks_x;
    if (dq && J.cached) quant_128_body<true, true>(J.x, J.cols, J.q, static_cast<float*>(J.scale), J.xdq, bx, by, red);
    else if (dq) quant_128_body<true, false>(J.x, J.cols, J.q, static_cast<float*>(J.scale), J.xdq, bx, by, red);
    else if (J.cached) quant_128_body<false, true>(J.x, J.cols, J.q, static_cast<float*>(J.scale), J.xdq, bx, by, red);
    else quant_128_body<false, false>(J.x, J.cols, J.q, static_cast<float*>(J.scale), J.xdq, bx, by, red);
    return;
  }
  const u32x4* xv = reinterpret_cast<const u32x4*>(J.x);
  u32x2* qv = reinterpret_cast<u32x2*>(J.q);
  u32x4* dv = reinterpret_cast<u32x4*>(J.xdq);
  const int64_t n = J.rows * J.cols / 8;
  const int64_t wave = (int64_t)local * 8 + (threadIdx.x >> 6), nwaves = (int64_t)J.wgs * 8;
  const int lane = (int)(threadIdx.x & 63);
#define FP8BLK_ROWS(B, F)                                                                  \
  do {                                                                                     \
    if (dq && J.cached) quant_rows_body<B, F, true, true>(xv, n, qv, J.scale, dv, wave, nwaves, lane);      \
    else if (dq) quant_rows_body<B, F, true, false>(xv, n, qv, J.scale, dv, wave, nwaves, lane);           \
    else if (J.cached) quant_rows_body<B, F, false, true>(xv, n, qv, J.scale, dv, wave, nwaves, lane);     \
    else quant_rows_body<B, F, false, false>(xv, n, qv, J.scale, dv, wave, nwaves, lane);                  \
  } while (0)
  if (J.kind == 1)
    FP8BLK_ROWS(128, false);
  else if (J.floor_rule)
    FP8BLK_ROWS(32, true);
  else
    FP8BLK_ROWS(32, false);
#undef FP8BLK_ROWS
}

// ------------------------------------------------------------------ launchers

static int rows_grid(int64_t nchunks, int num_cu) {
  const int64_t per_block = (int64_t)(kQRowsThreads / 64) * 64 * kQRowsU;  // chunks per workgroup pass
  int64_t need = (nchunks + per_block - 1) / per_block;
  (void)num_cu;
  const int64_t cap = int64_t(1) << 30;   // the loop below covers any remainder
  if (need > cap) need = cap;
  if (need < 1) need = 1;
  return (int)need;
}

template <int BLK, bool FLOOR>
static void launch_rows(int grid, const u32x4* xv, int64_t nchunks, u32x2* qv, void* scale, u32x4* dv, bool cached,
                        hipStream_t stream) {
  if (dv && cached)
    hipLaunchKernelGGL((quant_rows_kernel<BLK, FLOOR, true, true>), dim3(grid), dim3(kQRowsThreads), 0, stream, xv,
                       nchunks, qv, scale, dv);
  else if (dv)
    hipLaunchKernelGGL((quant_rows_kernel<BLK, FLOOR, true, false>), dim3(grid), dim3(kQRowsThreads), 0, stream, xv,
                       nchunks, qv, scale, dv);
  else if (cached)
    hipLaunchKernelGGL((quant_rows_kernel<BLK, FLOOR, false, true>), dim3(grid), dim3(kQRowsThreads), 0, stream, xv,
                       nchunks, qv, scale, dv);
  else
    hipLaunchKernelGGL((quant_rows_kernel<BLK, FLOOR, false, false>), dim3(grid), dim3(kQRowsThreads), 0, stream, xv,
                       nchunks, qv, scale, dv);
}

hipError_t launch_quant_rows(const uint16_t* x, int64_t rows, int64_t cols, int blk, bool floor_rule, uint8_t* q,
                             void* scale, uint16_t* xdq, int num_cu, hipStream_t stream) {
  const int64_t nchunks = rows * cols / 8;
  const int grid = rows_grid(nchunks, num_cu);
  const u32x4* xv = reinterpret_cast<const u32x4*>(x);
  u32x2* qv = reinterpret_cast<u32x2*>(q);
  u32x4* dv = reinterpret_cast<u32x4*>(xdq);
  const bool cached = rows * cols <= kCachedCodeBytes;
  if (blk == 128)
    launch_rows<128, false>(grid, xv, nchunks, qv, scale, dv, cached, stream);
  else if (floor_rule)
    launch_rows<32, true>(grid, xv, nchunks, qv, scale, dv, cached, stream);
  else
    launch_rows<32, false>(grid, xv, nchunks, qv, scale, dv, cached, stream);
  return hipGetLastError();
}

hipError_t launch_quant_128(const uint16_t* x, int64_t rows, int64_t cols, uint8_t* q, float* scale, uint16_t* xdq,
                            hipStream_t stream) {
  dim3 grid((unsigned)(cols / 128), (unsigned)(rows / 128));
  const bool cached = rows * cols <= kCachedCodeBytes;
  if (xdq && cached)
    hipLaunchKernelGGL((quant_128_kernel<true, true>), grid, dim3(512), 0, stream, x, cols, q, scale, xdq);
  else if (xdq)
    hipLaunchKernelGGL((quant_128_kernel<true, false>), grid, dim3(512), 0, stream, x, cols, q, scale, xdq);
  else if (cached)
    hipLaunchKernelGGL((quant_128_kernel<false, true>), grid, dim3(512), 0, stream, x, cols, q, scale, xdq);
  else
    hipLaunchKernelGGL((quant_128_kernel<false, false>), grid, dim3(512), 0, stream, x, cols, q, scale, xdq);
  return hipGetLastError();
}

hipError_t launch_quant_batch(const QuantJobIn* jobs, int count, hipStream_t stream) {
  QuantBatch b;
  int wg = 0, n = 0;
  for (int i = 0; i < count; ++i) {
    const QuantJobIn& in = jobs[i];
    if (in.rows == 0 || in.cols == 0) continue;
    QuantJob& J = b.job[n++];
    J.x = in.x;
    J.rows = in.rows;
    J.cols = in.cols;
    J.q = in.q;
    J.scale = in.scale;
    J.xdq = in.xdq;
    J.kind = in.kind;
    J.floor_rule = in.floor_rule ? 1 : 0;
    J.cached = in.rows * in.cols <= kCachedCodeBytes ? 1 : 0;
    J.blocks_x = (int)(in.cols / 128);
    J.wg0 = wg;
    if (in.kind == 2) {
      J.wgs = (int)((in.rows / 128) * (in.cols / 128));
    } else {
      static_assert(kQuantBatchRowsChunks == 8 * 64 * kQRowsU, "chunks of one pass of a batch workgroup");
      J.wgs = (int)((in.rows * in.cols / 8 + kQuantBatchRowsChunks - 1) / kQuantBatchRowsChunks);
    }
    wg += J.wgs;
  }
  b.count = n;
  if (n == 0) return hipSuccess;
  hipLaunchKernelGGL(quant_batch_kernel, dim3(wg), dim3(512), 0, stream, b);
  return hipGetLastError();
}

}  // namespace fp8blk
