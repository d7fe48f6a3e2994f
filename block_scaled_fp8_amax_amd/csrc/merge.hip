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
// load covers 64/LPR rows.  Every load of the workgroup's block is issued
// up front, in the order B block, A columns, W rows (the 128x128 bf16 block
// is held in registers, 32 dwords per lane), so that B's LDS stores wait
// only for B and the merge of each W row only for that row; the barrier
// after the LDS stores waits on LDS alone.  B's block rows go to LDS as
// fp32 (read back as 16-byte broadcasts) and the lane's A columns to
// registers; ranks from r up to the template's RMAX are zero, which leaves
// the sequential sum unchanged bit for bit (acc + 0 * 0 = acc), so the rank
// loop has no branches.  The loads of B and A are issued for every rank at
// a rank clamped below r and zeroed afterwards: a load under a branch
// waited for everything in flight, which serialized the 8 B loads of a
// thread behind the W block (rank 16: 60.0 to 54.0 us, rank 64: 324 to
// 202 us at 7168x7168).  A rank equal to the template's RMAX (FULL) needs
// no clamp and no zeroing: 1-3% faster.  The update costs RMAX fused
// multiply-adds per element on the vector ALU.
#include <type_traits>

#include "device.h"
#include "launch.h"

namespace fp8blk {

template <int RMAX, int CPL, bool DQ, bool CACHED, bool FULL>
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
  const uint8_t* wb = reinterpret_cast<const uint8_t*>(w + blk);

  // Loads in the order B block, A columns, W rows, with compiler barriers
  // between the groups: B's LDS stores then wait only for B, and the merge
  // waits for each W row as it arrives.
  // A rank-r block of B (r == RMAX) is 128 * RMAX contiguous bf16: thread
  // t takes dwords [t * BPT / 2, (t + 1) * BPT / 2) of it.  Otherwise
  // thread t takes elements t, t + 256, ... of the RMAX-padded block.
  constexpr int BPT = 128 * RMAX / 256;   // B elements per thread
  uint32_t braw[BPT];
  // (every load is issued, at a clamped rank below r, so that none waits
  // behind a branch; ranks >= r are then zeroed)
  if constexpr (FULL) {
    const uint32_t* bblk = reinterpret_cast<const uint32_t*>(lb + row0 * RMAX);   // wave-uniform
#pragma unroll
    for (int n = 0; n < BPT / 2; ++n) braw[n] = bblk[t * (BPT / 2) + n];
  } else {
#pragma unroll
    for (int n = 0; n < BPT; ++n) {
      const int i = t + 256 * n;
      const int rr = i / RMAX, cc = i % RMAX;
      braw[n] = (uint32_t)lb[(row0 + rr) * r + (cc < r ? cc : r - 1)];
    }
  }
  asm volatile("" ::: "memory");
  // A's rows as 32-bit byte offsets from the block's wave-uniform column
  // base (rank * k * 2 < 2^31 for k <= 2^24, r <= 64), so that each load
  // takes a scalar base and one vector add
  uint32_t araw[RMAX][DW];
  const uint8_t* la_blk = reinterpret_cast<const uint8_t*>(la + (int64_t)blockIdx.x * 128);
  const uint32_t lcol_b = (uint32_t)(lc * CPL * 2);
#pragma unroll
  for (int i = 0; i < RMAX; ++i) {
    const int ic = FULL ? i : (i < r ? i : r - 1);
    const uint32_t ao = (uint32_t)ic * (uint32_t)k * 2u + lcol_b;
    // dword loads: lora_a is only required to be 4-byte aligned
#pragma unroll
    for (int d = 0; d < DW; ++d) araw[i][d] = *reinterpret_cast<const uint32_t*>(la_blk + ao + 4 * d);
  }
  asm volatile("" ::: "memory");
  uint32_t wp[32];
#pragma unroll
  for (int j = 0; j < NJ; ++j) {
    const uint32_t ob = 2 * lofs + j * (2 * jstep);   // byte offset of the lane's bf16
    if constexpr (DW == 2) {
      const u32x2 v = __builtin_nontemporal_load(reinterpret_cast<const u32x2*>(wb + ob));
      wp[2 * j] = v.x;
      wp[2 * j + 1] = v.y;
    } else {
      wp[j] = __builtin_nontemporal_load(reinterpret_cast<const uint32_t*>(wb + ob));
    }
  }
  asm volatile("" ::: "memory");
  if constexpr (FULL) {
#pragma unroll
    for (int n = 0; n < BPT / 2; ++n) {
      sB[t * BPT + 2 * n] = bf_lo(braw[n]);
      sB[t * BPT + 2 * n + 1] = bf_hi(braw[n]);
    }
  } else {
#pragma unroll
    for (int n = 0; n < BPT; ++n) {
      const int cc = (t + 256 * n) % RMAX;
      sB[t + 256 * n] = cc < r ? __uint_as_float(braw[n] << 16) : 0.f;
    }
  }
  float a[RMAX][CPL];
#pragma unroll
  for (int i = 0; i < RMAX; ++i)
#pragma unroll
    for (int d = 0; d < DW; ++d) {
      a[i][2 * d] = (FULL || i < r) ? bf_lo(araw[i][d]) : 0.f;
      a[i][2 * d + 1] = (FULL || i < r) ? bf_hi(araw[i][d]) : 0.f;
    }
  // B's LDS stores land before the barrier; the W loads may stay in flight
  // (__syncthreads would wait for them as well)
  __builtin_amdgcn_s_waitcnt(0xC07F);
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");

  // 4. merge in place: W' = RN_bf16(W + RN_bf16(sum_r B[n,r] A[r,k])).
  // The block amax runs on the packed bf16 magnitudes, one 16-bit max per
  // half of a dword, and the two halves meet once at the end.
  v2u16 m2 = {0, 0};
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
      // RN_bf16(acc) as an fp32 directly: the bf16 lands in the high half
      // of the conversion's result, above a zero low half
      const float d0 = __uint_as_float(pack_bf16x2(0.f, acc[2 * d]));
      const float d1 = __uint_as_float(pack_bf16x2(0.f, acc[2 * d + 1]));
      const uint32_t w2 = wp[j * DW + d];
      const uint32_t s2 = pack_bf16x2(bf_lo(w2) + d0, bf_hi(w2) + d1);
      wp[j * DW + d] = s2;
      m2 = __builtin_elementwise_max(m2, __builtin_bit_cast(v2u16, s2 & 0x7FFF7FFFu));
    }
  }
  uint32_t m = m2[0] > m2[1] ? (uint32_t)m2[0] : (uint32_t)m2[1];
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
      const uint32_t o = lofs + j * jstep;   // element (= code byte) offset; bf16 at 2 * o
      // the lane's codes in one dword: the first pair in the low half, the
      // second (4 columns per lane) in the high half of the same register
      uint32_t cw;
#pragma unroll
      for (int d = 0; d < DW; ++d) {
        const float q0 = TINY ? f32_quot(bf_lo(wp[j * DW + d]), fb) : f32_quot_unit(bf_lo(wp[j * DW + d]), fb);
        const float q1 = TINY ? f32_quot(bf_hi(wp[j * DW + d]), fb) : f32_quot_unit(bf_hi(wp[j * DW + d]), fb);
        // the low pair's conversion keeps the register's high half, which
        // the second pair then overwrites: any prior content will do
        if (d == 0)
          cw = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(q0, q1, __float_as_int(q0), false);
        else
          cw = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(q0, q1, (int)cw, true);
      }
      if constexpr (DW == 2)
        store_code<CACHED>(cw, reinterpret_cast<uint32_t*>(qb + o));
      else
        *reinterpret_cast<uint16_t*>(qb + o) = (uint16_t)cw;
      if constexpr (DQ) {
        uint32_t dv[DW];
#pragma unroll
        for (int d = 0; d < DW; ++d) {
          const v2f dq = d == 0 ? __builtin_amdgcn_cvt_pk_f32_fp8((int)cw, false)
                                : __builtin_amdgcn_cvt_pk_f32_fp8((int)cw, true);
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
#define FP8BLK_MERGE1(RM, CP, FU)                                                                                    \
  do {                                                                                                               \
    if (wdq && cached)                                                                                               \
      hipLaunchKernelGGL((merge_128_kernel<RM, CP, true, true, FU>), grid, dim3(256), 0, stream, w, lb, la, k, ri,  \
                         q, scale, wdq);                                                                             \
    else if (wdq)                                                                                                    \
      hipLaunchKernelGGL((merge_128_kernel<RM, CP, true, false, FU>), grid, dim3(256), 0, stream, w, lb, la, k, ri, \
                         q, scale, wdq);                                                                             \
    else if (cached)                                                                                                 \
      hipLaunchKernelGGL((merge_128_kernel<RM, CP, false, true, FU>), grid, dim3(256), 0, stream, w, lb, la, k, ri, \
                         q, scale, wdq);                                                                             \
    else                                                                                                             \
      hipLaunchKernelGGL((merge_128_kernel<RM, CP, false, false, FU>), grid, dim3(256), 0, stream, w, lb, la, k,    \
                         ri, q, scale, wdq);                                                                         \
  } while (0)
#define FP8BLK_MERGE(RM, CP)                  \
  do {                                        \
    if (ri == RM) FP8BLK_MERGE1(RM, CP, true); \
    else FP8BLK_MERGE1(RM, CP, false);         \
  } while (0)
  if (r <= 16)
    FP8BLK_MERGE(16, 4);
  else if (r <= 32)
    FP8BLK_MERGE(32, 2);
  else
    FP8BLK_MERGE(64, 2);
#undef FP8BLK_MERGE
#undef FP8BLK_MERGE1
  return hipGetLastError();
}

}  // namespace fp8blk
