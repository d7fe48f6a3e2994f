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
// Tiling (template): a workgroup of (BM/64) x (BN/64) waves computes a
// BM x BN tile, each wave a 64x64 block of 4x4 MFMA tiles.  K advances 128
// bytes at a time through a STAGES-deep ring of LDS stages filled by direct
// global->LDS loads (global_load_lds_dwordx4): every wave-wide load writes
// 1 KiB of LDS contiguously, 8 tile rows of 128 bytes.  Within a row the
// 16-byte K chunk c sits in slot c ^ swz(row), so that the 16-byte fragment
// reads of 16 consecutive rows touch distinct banks; the XOR is applied on
// the global-address side of the load.  One barrier per K step: the loads
// for step kb+STAGES-1 are issued right after it, into the slot that was
// read at step kb-1.  The loads are inline assembly so that the compiler
// does not insert a full memory wait before every LDS read; vmcnt is
// managed here.
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

constexpr int kBK = 128;

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
  int tiles_m, tiles_n;     // dense: tile grid (launched 1-D)
  int band;                 // dense: m-tiles per band of the tile order (0 = row of tiles)
};

// Dense tile order.  Workgroup i is dispatched to XCD i % 8 and the XCDs
// have separate L2 caches, so consecutive tile indices are given to one XCD
// (a contiguous range of 1/8 of the tiles each), and tiles are numbered
// column by column inside bands of `band` m-tiles, which makes each XCD's
// range a compact band x (range/band) block of the output.
__device__ __forceinline__ void dense_tile(const GemmParams& p, int* tm, int* tn) {
  const int nwg = p.tiles_m * p.tiles_n;
  int id = blockIdx.x;
  if ((nwg & 7) == 0) id = (id & 7) * (nwg >> 3) + (id >> 3);
  const int band = p.band > 0 ? p.band : p.tiles_m;
  const int per_band = band * p.tiles_n;
  const int b = id / per_band, r = id - b * per_band;
  const int rows_here = (b + 1) * band <= p.tiles_m ? band : p.tiles_m - b * band;
  *tm = b * band + r % rows_here;
  *tn = r / rows_here;
}

__device__ __forceinline__ v8i make_frag(const u32x4& lo, const u32x4& hi) {
  v8i r;
  r[0] = (int)lo.x; r[1] = (int)lo.y; r[2] = (int)lo.z; r[3] = (int)lo.w;
  r[4] = (int)hi.x; r[5] = (int)hi.y; r[6] = (int)hi.z; r[7] = (int)hi.w;
  return r;
}

// Slot pattern of tile row r: rows of equal parity get distinct XOR patterns
// across 16 consecutive rows.
__device__ __forceinline__ int swz(int r) { return (r >> 1) & 7; }

// Direct global->LDS loads.  `lds` must be wave-uniform; lane i writes
// lds + 16*i (dwordx4) or lds + 4*i (dword).  Completion is tracked by vmcnt.
__device__ __forceinline__ void dma16(const void* base, uint32_t voff, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %2\n\tglobal_load_lds_dwordx4 %0, %1" ::"v"(voff), "s"(base), "s"(lds) : "memory");
}
__device__ __forceinline__ void dma4(const void* base, uint32_t voff, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %2\n\tglobal_load_lds_dword %0, %1" ::"v"(voff), "s"(base), "s"(lds) : "memory");
}

// s_waitcnt vmcnt(n) for a wave-uniform n (clamped to 15); other counters
// untouched.
__device__ __forceinline__ void wait_vmcnt(int n) {
  switch (n) {
    case 0: __builtin_amdgcn_s_waitcnt(0x0F70); break;
    case 1: __builtin_amdgcn_s_waitcnt(0x0F71); break;
    case 2: __builtin_amdgcn_s_waitcnt(0x0F72); break;
    case 3: __builtin_amdgcn_s_waitcnt(0x0F73); break;
    case 4: __builtin_amdgcn_s_waitcnt(0x0F74); break;
    case 5: __builtin_amdgcn_s_waitcnt(0x0F75); break;
    case 6: __builtin_amdgcn_s_waitcnt(0x0F76); break;
    case 7: __builtin_amdgcn_s_waitcnt(0x0F77); break;
    case 8: __builtin_amdgcn_s_waitcnt(0x0F78); break;
    case 9: __builtin_amdgcn_s_waitcnt(0x0F79); break;
    case 10: __builtin_amdgcn_s_waitcnt(0x0F7A); break;
    case 11: __builtin_amdgcn_s_waitcnt(0x0F7B); break;
    case 12: __builtin_amdgcn_s_waitcnt(0x0F7C); break;
    case 13: __builtin_amdgcn_s_waitcnt(0x0F7D); break;
    case 14: __builtin_amdgcn_s_waitcnt(0x0F7E); break;
    default: __builtin_amdgcn_s_waitcnt(0x0F7F); break;
  }
}

// Locate the tile of a grouped problem: slot -> (group, first row, rows).
// Every workgroup rebuilds the prefix of m-tiles per group in LDS.
// `scratch` is LDS of at least 2 * 1025 ints.
template <int BM>
__device__ __forceinline__ bool grouped_tile(const int32_t* __restrict__ off, int groups, int slot, int* scratch,
                                             int nthreads, int* g_out, int64_t* row0, int* rows) {
  int* s_off = scratch;
  int* s_pref = scratch + 1025;
  const int t = threadIdx.x;
  for (int g = t; g <= groups; g += nthreads) s_off[g] = off[g];
  __syncthreads();
  for (int g = t; g < groups; g += nthreads) s_pref[g + 1] = (s_off[g + 1] - s_off[g] + BM - 1) / BM;
  if (t == 0) s_pref[0] = 0;
  __syncthreads();
  for (int d = 1; d < groups; d <<= 1) {  // inclusive scan of s_pref[1..groups]
    int v[4];
    int cnt = 0;
    for (int g = t; g < groups; g += nthreads) v[cnt++] = (g >= d) ? s_pref[g + 1 - d] : 0;
    __syncthreads();
    cnt = 0;
    for (int g = t; g < groups; g += nthreads) s_pref[g + 1] += v[cnt++];
    __syncthreads();
  }
  if (slot >= s_pref[groups]) return false;
  int lo = 0, hi = groups - 1;  // g with s_pref[g] <= slot < s_pref[g+1]
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (s_pref[mid] <= slot) lo = mid; else hi = mid - 1;
  }
  const int g = lo;
  *g_out = g;
  *row0 = (int64_t)s_off[g] + (int64_t)(slot - s_pref[g]) * BM;
  const int64_t left = (int64_t)s_off[g + 1] - *row0;
  *rows = (int)(left < BM ? left : BM);
  return true;
}

template <int BM, int BN, int STAGES>
struct Layout {
  static constexpr int kA = BM * kBK;           // bytes of A per stage
  static constexpr int kB = BN * kBK;
  static constexpr int kSA = BM * 4;            // A scales (fp32 or 4 E8M0 bytes) per row
  static constexpr int kSB = BN * 4;            // B E8M0 scales per column
  static constexpr int kStage = kA + kB + kSA + kSB;
  static constexpr int kTileStride = BN + 4;    // fp32 epilogue staging row stride
  static constexpr int kEpi = BM * kTileStride * 4;
  static constexpr int kBytes = (STAGES * kStage > kEpi ? STAGES * kStage : kEpi);
};

template <int MODE, bool OUT_F32, bool GROUPED, int BM, int BN, int STAGES>
__global__ __launch_bounds__((BM / 64) * (BN / 64) * 64) void gemm_kernel(GemmParams p) {
  constexpr int WN = BN / 64, NT = (BM / 64) * WN * 64, NW = NT / 64;
  constexpr bool A_MX = (MODE == kMXxMX);
  constexpr bool B_MX = (MODE != kF32xF32);
  using L = Layout<BM, BN, STAGES>;
  static_assert(BM % 64 == 0 && BN % 64 == 0, "tile");
  static_assert((BM / 8) % NW == 0 && (BN / 8) % NW == 0, "load split");
  __shared__ __attribute__((aligned(16))) uint8_t smem[L::kBytes];

  const int t = threadIdx.x;
  const int lane = t & 63;
  const int wave = __builtin_amdgcn_readfirstlane(t >> 6);
  const int wm = wave / WN, wn = wave % WN;
  const int64_t K = p.k;
  const int KB = (int)(K / kBK);

  // ---- tile coordinates
  int64_t m0;
  int mrows;
  int64_t n0;
  const uint8_t* bq = p.b;
  const uint8_t* sbq8 = reinterpret_cast<const uint8_t*>(p.sb);
  const float* sbf = reinterpret_cast<const float*>(p.sb);
  if constexpr (GROUPED) {
    int g;
    if (!grouped_tile<BM>(p.offsets, p.groups, (int)blockIdx.x, reinterpret_cast<int*>(smem), NT, &g, &m0, &mrows))
      return;
    g = __builtin_amdgcn_readfirstlane(g);
    m0 = (int64_t)__builtin_amdgcn_readfirstlane((int)m0);
    mrows = __builtin_amdgcn_readfirstlane(mrows);
    bq += (int64_t)g * p.b_group_stride;
    sbq8 += (int64_t)g * p.sb_group_stride;
    sbf += (int64_t)g * p.sb_group_stride;
    n0 = (int64_t)blockIdx.y * BN;
    __syncthreads();   // the scratch above is stage 0, written by the prologue
  } else {
    int tm, tn;
    dense_tile(p, &tm, &tn);
    m0 = (int64_t)tm * BM;
    n0 = (int64_t)tn * BN;
    const int64_t left = p.m - m0;
    mrows = (int)(left < BM ? left : BM);
  }
  const uint8_t* aq = p.a + m0 * K;
  const uint8_t* bt = bq + n0 * K;
  const uint32_t lds0 = (uint32_t)(uintptr_t)smem;

  // ---- per-lane byte offsets of the direct loads from the tile base, without
  // the K step.  Rows past the end of A re-read the last valid row; their
  // results are never stored.
  constexpr int A_LOADS = BM / 8 / NW;   // 1 KiB wave-wide loads per wave per stage
  constexpr int B_LOADS = BN / 8 / NW;
  uint32_t a_off[A_LOADS], b_off[B_LOADS];
  {
    const int sub = lane >> 3;           // row within the 8-row block
    const int slot = lane & 7;
#pragma unroll
    for (int j = 0; j < A_LOADS; ++j) {
      const int r = (j * NW + wave) * 8 + sub;
      const int rr = r < mrows ? r : mrows - 1;
      a_off[j] = (uint32_t)(rr * K) + (uint32_t)((slot ^ swz(r)) * 16);
    }
#pragma unroll
    for (int j = 0; j < B_LOADS; ++j) {
      const int r = (j * NW + wave) * 8 + sub;
      b_off[j] = (uint32_t)(r * K) + (uint32_t)((slot ^ swz(r)) * 16);
    }
  }
  // Scale loads: waves 0 .. BM/64-1 load the A row scales (one dword per row);
  // for E8M0 B the next BN/64 waves load the column scales (4 bytes each);
  // for a 128x128 fp32 B the next wave loads the block's single scale with
  // every lane (a broadcast copy), so that no ordinary vector load, whose
  // wait would also drain the in-flight stages, is needed in the loop.
  constexpr int SA_WAVES = BM / 64;
  constexpr int SB_WAVES = B_MX ? BN / 64 : 1;
  static_assert(SA_WAVES + SB_WAVES <= NW, "scale loaders");
  const bool sa_loader = wave < SA_WAVES;
  const bool sb_loader = wave >= SA_WAVES && wave < SA_WAVES + SB_WAVES;
  uint32_t s_off = 0;
  const void* sb_base = B_MX ? static_cast<const void*>(sbq8) : static_cast<const void*>(sbf);
  if (sa_loader) {
    const int r = wave * 64 + lane;
    const int64_t rr = m0 + (r < mrows ? r : mrows - 1);
    s_off = A_MX ? (uint32_t)(rr * (K / 32)) : (uint32_t)(rr * KB * 4);
  } else if (sb_loader) {
    if constexpr (B_MX) {
      const int c = (wave - SA_WAVES) * 64 + lane;
      s_off = (uint32_t)((n0 + c) * (K / 32));
    } else {
      s_off = (uint32_t)((n0 / 128) * KB * 4);
    }
  }
  const int loads_per_stage = A_LOADS + B_LOADS + ((sa_loader || sb_loader) ? 1 : 0);

  auto issue = [&](int kb, int stage) {
    const uint32_t sbase = lds0 + stage * L::kStage;
    const uint32_t koff = (uint32_t)kb * kBK;
#pragma unroll
    for (int j = 0; j < A_LOADS; ++j) dma16(aq, a_off[j] + koff, sbase + (j * NW + wave) * 1024);
#pragma unroll
    for (int j = 0; j < B_LOADS; ++j) dma16(bt, b_off[j] + koff, sbase + L::kA + (j * NW + wave) * 1024);
    if (sa_loader)
      dma4(p.sa, s_off + (uint32_t)kb * 4, sbase + L::kA + L::kB + wave * 256);
    else if (sb_loader)
      dma4(sb_base, s_off + (uint32_t)kb * 4, sbase + L::kA + L::kB + L::kSA + (wave - SA_WAVES) * 256);
  };

  v4f acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = (v4f){0.f, 0.f, 0.f, 0.f};

  const int fr = lane & 15;       // fragment row / column
  const int fg = lane >> 4;       // K chunk of the lane group (and chunk + 4)

  // prologue: stages 0 .. STAGES-2
#pragma unroll
  for (int s = 0; s < STAGES - 1; ++s)
    if (s < KB) issue(s, s);

  for (int kb = 0; kb < KB; ++kb) {
    const int stage = kb % STAGES;
    // this wave's loads of the later stages may stay in flight
    int later = KB - 1 - kb;
    later = later < STAGES - 2 ? later : STAGES - 2;
    wait_vmcnt(later * loads_per_stage);
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");   // keep LDS reads of this step below the barrier
    if (kb + STAGES - 1 < KB) issue(kb + STAGES - 1, (kb + STAGES - 1) % STAGES);

    const uint8_t* sA = smem + stage * L::kStage;
    const uint8_t* sB = sA + L::kA;
    const uint32_t* sSA = reinterpret_cast<const uint32_t*>(sA + L::kA + L::kB);
    const uint32_t* sSB = sSA + BM;
    float sb_k = 1.f;
    if constexpr (MODE == kF32xF32) sb_k = __uint_as_float(sSB[0]);

    v8i af[4];
    float sc[4][4];
    int xa[4];
#pragma unroll
    for (int mi = 0; mi < 4; ++mi) {
      const int ar = wm * 64 + mi * 16 + fr;
      const uint8_t* rowp = sA + ar * kBK;
      const int s0 = (fg ^ swz(ar)) * 16;
      af[mi] = make_frag(*reinterpret_cast<const u32x4*>(rowp + s0), *reinterpret_cast<const u32x4*>(rowp + (s0 ^ 64)));
      if constexpr (A_MX) {
        xa[mi] = (int)((sSA[ar] >> (8 * fg)) & 0xFFu);
      } else {
        const u32x4 s4 = *reinterpret_cast<const u32x4*>(&sSA[wm * 64 + mi * 16 + 4 * fg]);
        sc[mi][0] = __uint_as_float(s4.x) * sb_k;
        sc[mi][1] = __uint_as_float(s4.y) * sb_k;
        sc[mi][2] = __uint_as_float(s4.z) * sb_k;
        sc[mi][3] = __uint_as_float(s4.w) * sb_k;
      }
    }
    v4f part[2][4];
#pragma unroll
    for (int ni = 0; ni < 4; ++ni) {
      const int bc = wn * 64 + ni * 16 + fr;
      const uint8_t* rowp = sB + bc * kBK;
      const int s0 = (fg ^ swz(bc)) * 16;
      const v8i bfr = make_frag(*reinterpret_cast<const u32x4*>(rowp + s0), *reinterpret_cast<const u32x4*>(rowp + (s0 ^ 64)));
      int xb = 127;
      if constexpr (B_MX) xb = (int)((sSB[bc] >> (8 * fg)) & 0xFFu);
#pragma unroll
      for (int mi = 0; mi < 4; ++mi) {
        if constexpr (MODE == kMXxMX) {
          acc[mi][ni] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(af[mi], bfr, acc[mi][ni], 0, 0, 0, xa[mi],
                                                                         0, xb);
        } else {
          const v4f zero = {0.f, 0.f, 0.f, 0.f};
          if constexpr (MODE == kF32xMX)
            part[ni & 1][mi] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(af[mi], bfr, zero, 0, 0, 0, 127, 0, xb);
          else
            part[ni & 1][mi] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(af[mi], bfr, zero, 0, 0, 0, 0, 0, 0);
        }
      }
      if constexpr (MODE != kMXxMX) {
        if (ni > 0) {
#pragma unroll
          for (int mi = 0; mi < 4; ++mi)
#pragma unroll
            for (int v = 0; v < 4; ++v)
              acc[mi][ni - 1][v] = __builtin_fmaf(part[(ni - 1) & 1][mi][v], sc[mi][v], acc[mi][ni - 1][v]);
        }
      }
    }
    if constexpr (MODE != kMXxMX) {
#pragma unroll
      for (int mi = 0; mi < 4; ++mi)
#pragma unroll
        for (int v = 0; v < 4; ++v) acc[mi][3][v] = __builtin_fmaf(part[1][mi][v], sc[mi][v], acc[mi][3][v]);
    }
  }

  // ---- epilogue: stage the tile in LDS, then write whole rows with 16-byte
  // stores (8 bf16 or 4 fp32 per lane).
  __syncthreads();
  float* stile = reinterpret_cast<float*>(smem);
  constexpr int TS = L::kTileStride;
#pragma unroll
  for (int mi = 0; mi < 4; ++mi)
#pragma unroll
    for (int ni = 0; ni < 4; ++ni)
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int r = wm * 64 + mi * 16 + 4 * fg + v;
        const int c = wn * 64 + ni * 16 + fr;
        stile[r * TS + c] = acc[mi][ni][v];
      }
  __syncthreads();
  const int64_t N = p.n;
  if constexpr (OUT_F32) {
    constexpr int LPR = BN / 4;              // lanes per row
    constexpr int RPP = NT / LPR;            // rows per pass
#pragma unroll 4
    for (int it = 0; it < BM / RPP; ++it) {
      const int r = it * RPP + t / LPR;
      const int c = (t % LPR) * 4;
      if (r < mrows) {
        const float4 v = *reinterpret_cast<const float4*>(&stile[r * TS + c]);
        *reinterpret_cast<float4*>(reinterpret_cast<float*>(p.y) + (m0 + r) * N + n0 + c) = v;
      }
    }
  } else {
    constexpr int LPR = BN / 8;
    constexpr int RPP = NT / LPR;
#pragma unroll 4
    for (int it = 0; it < BM / RPP; ++it) {
      const int r = it * RPP + t / LPR;
      const int c = (t % LPR) * 8;
      if (r < mrows) {
        const float4 v0 = *reinterpret_cast<const float4*>(&stile[r * TS + c]);
        const float4 v1 = *reinterpret_cast<const float4*>(&stile[r * TS + c + 4]);
        u32x4 o;
        o.x = pack_bf16x2(v0.x, v0.y);
        o.y = pack_bf16x2(v0.z, v0.w);
        o.z = pack_bf16x2(v1.x, v1.y);
        o.w = pack_bf16x2(v1.z, v1.w);
        *reinterpret_cast<u32x4*>(reinterpret_cast<uint16_t*>(p.y) + (m0 + r) * N + n0 + c) = o;
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Dense kernel with a ping-pong schedule.  256x128 tile, 8 waves; wave w and
// wave w+4 share a SIMD.  Waves 0-3 (group 0) own output columns 0-63 and
// waves 4-7 (group 1) columns 64-127; wave w % 4 selects a 64-row slice.
// Every K step is split into two half-steps separated by a workgroup
// barrier.  In each half-step one group runs its "memory" phase (LDS reads
// of its fragments for the next step and its share of the direct loads of
// a future stage) while the other group runs its "compute" phase (16 MFMAs
// and the fp32 promotion), so the matrix cores of every SIMD are fed by one
// wave while its partner waits on memory:
//   half-step 2kb   : group 0 memory(kb)   | group 1 compute(kb-1)
//   half-step 2kb+1 : group 0 compute(kb)  | group 1 memory(kb)
// Group 0 loads the A tile and the A scales, group 1 the B tile and the B
// scales.  A stage is read at half-steps 2kb and 2kb+1 and refilled from
// half-step 2kb+6 on (3 stages).
template <int MODE, bool OUT_F32>
__global__ __launch_bounds__(512) void gemm_pp_kernel(GemmParams p) {
  constexpr int BM = 256, BN = 128, STAGES = 3, NW = 8;
  constexpr bool A_MX = (MODE == kMXxMX);
  constexpr bool B_MX = (MODE != kF32xF32);
  using L = Layout<BM, BN, STAGES>;
  __shared__ __attribute__((aligned(16))) uint8_t smem[L::kBytes];

  const int t = threadIdx.x;
  const int lane = t & 63;
  const int wave = __builtin_amdgcn_readfirstlane(t >> 6);
  const int grp = wave >> 2;          // 0: A loader, 1: B loader
  const int gw = wave & 3;            // wave within the group
  const int wm = gw, wn = grp;        // 64x64 output block of this wave
  const int64_t K = p.k;
  const int KB = (int)(K / kBK);

  int tm, tn;
  dense_tile(p, &tm, &tn);
  const int64_t m0 = (int64_t)tm * BM, n0 = (int64_t)tn * BN;
  const int mrows = (int)((p.m - m0) < BM ? (p.m - m0) : BM);
  const uint8_t* aq = p.a + m0 * K;
  const uint8_t* bt = p.b + n0 * K;
  const uint32_t lds0 = (uint32_t)(uintptr_t)smem;

  // ---- this wave's share of every stage.  The 8-row blocks of the A and B
  // tiles are dealt to the 8 waves in turn (block rb goes to wave rb % 8), so
  // each group issues half of the tile loads in its memory phase: 4 x 1 KiB
  // of A and 2 x 1 KiB of B per wave.  Group 0 also loads the A scales,
  // group 1 the B scales.
  constexpr int A_PER = BM / 8 / NW, B_PER = BN / 8 / NW;
  uint32_t a_off[A_PER], b_off[B_PER];
  {
    const int sub = lane >> 3, slot = lane & 7;
#pragma unroll
    for (int j = 0; j < A_PER; ++j) {
      const int r = (j * NW + wave) * 8 + sub;
      const int rr = r < mrows ? r : mrows - 1;
      a_off[j] = (uint32_t)(rr * K) + (uint32_t)((slot ^ swz(r)) * 16);
    }
#pragma unroll
    for (int j = 0; j < B_PER; ++j) {
      const int r = (j * NW + wave) * 8 + sub;
      b_off[j] = (uint32_t)(r * K) + (uint32_t)((slot ^ swz(r)) * 16);
    }
  }
  // every wave issues exactly one scale load per stage (group 1 waves 2-3
  // repeat the loads of waves 0-1, writing identical bytes), so that the
  // per-wave load count is a compile-time constant of the group
  uint32_t s_off = 0, s_lds = 0;
  const void* s_base = nullptr;
  if (grp == 0) {
    const int r = gw * 64 + lane;
    const int64_t rr = m0 + (r < mrows ? r : mrows - 1);
    s_off = A_MX ? (uint32_t)(rr * (K / 32)) : (uint32_t)(rr * KB * 4);
    s_lds = L::kA + L::kB + gw * 256;
    s_base = p.sa;
  } else if (B_MX) {
    const int cw = gw & (BN / 64 - 1);
    s_off = (uint32_t)((n0 + cw * 64 + lane) * (K / 32));
    s_lds = L::kA + L::kB + L::kSA + cw * 256;
    s_base = p.sb;
  } else {
    s_off = (uint32_t)((n0 / 128) * KB * 4);
    s_lds = L::kA + L::kB + L::kSA;
    s_base = p.sb;
  }
  auto issue = [&](int kb) {
    const uint32_t sbase = lds0 + (kb % STAGES) * L::kStage;
    const uint32_t koff = (uint32_t)kb * kBK;
#pragma unroll
    for (int j = 0; j < A_PER; ++j) dma16(aq, a_off[j] + koff, sbase + (j * NW + wave) * 1024);
#pragma unroll
    for (int j = 0; j < B_PER; ++j) dma16(bt, b_off[j] + koff, sbase + L::kA + (j * NW + wave) * 1024);
    dma4(s_base, s_off + (uint32_t)kb * 4, sbase + s_lds);
  };

  v4f acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = (v4f){0.f, 0.f, 0.f, 0.f};

  const int fr = lane & 15;
  const int fg = lane >> 4;
  v8i af[4], bfr[4];
  float sc[4][4];
  float sbk = 1.f;
  int xa[4], xb[4];

  // memory phase: fragments and scales of step kb into registers
  auto mem_phase = [&](int kb) {
    const uint8_t* sA = smem + (kb % STAGES) * L::kStage;
    const uint8_t* sB = sA + L::kA;
    const uint32_t* sSA = reinterpret_cast<const uint32_t*>(sA + L::kA + L::kB);
    const uint32_t* sSB = sSA + BM;
#pragma unroll
    for (int mi = 0; mi < 4; ++mi) {
      const int ar = wm * 64 + mi * 16 + fr;
      const uint8_t* rowp = sA + ar * kBK;
      const int s0 = (fg ^ swz(ar)) * 16;
      af[mi] = make_frag(*reinterpret_cast<const u32x4*>(rowp + s0), *reinterpret_cast<const u32x4*>(rowp + (s0 ^ 64)));
      if constexpr (A_MX) {
        xa[mi] = (int)((sSA[ar] >> (8 * fg)) & 0xFFu);
      } else {
        const u32x4 s4 = *reinterpret_cast<const u32x4*>(&sSA[wm * 64 + mi * 16 + 4 * fg]);
        sc[mi][0] = __uint_as_float(s4.x);
        sc[mi][1] = __uint_as_float(s4.y);
        sc[mi][2] = __uint_as_float(s4.z);
        sc[mi][3] = __uint_as_float(s4.w);
      }
    }
#pragma unroll
    for (int ni = 0; ni < 4; ++ni) {
      const int bc = wn * 64 + ni * 16 + fr;
      const uint8_t* rowp = sB + bc * kBK;
      const int s0 = (fg ^ swz(bc)) * 16;
      bfr[ni] = make_frag(*reinterpret_cast<const u32x4*>(rowp + s0), *reinterpret_cast<const u32x4*>(rowp + (s0 ^ 64)));
      if constexpr (B_MX) xb[ni] = (int)((sSB[bc] >> (8 * fg)) & 0xFFu);
    }
    if constexpr (MODE == kF32xF32) sbk = __uint_as_float(sSB[0]);
    if (kb + STAGES - 1 < KB) issue(kb + STAGES - 1);
    __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0): the stage may be refilled after the next barrier
  };

  // compute phase: 16 MFMAs and the promotion of their partial products.
  // The fold of subtile column ni-1 is interleaved with the MFMAs of column
  // ni (one MFMA, then the four multiply-adds of a partial issued four MFMAs
  // earlier), so the wave never waits on a just-issued MFMA.
  auto compute_phase = [&]() {
    v4f part[2][4];
#pragma unroll
    for (int ni = 0; ni < 4; ++ni) {
      if (MODE == kF32xF32 && ni == 1) {
#pragma unroll
        for (int mi = 0; mi < 4; ++mi)
#pragma unroll
          for (int v = 0; v < 4; ++v) sc[mi][v] *= sbk;
      }
#pragma unroll
      for (int mi = 0; mi < 4; ++mi) {
        if constexpr (MODE == kMXxMX) {
          acc[mi][ni] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(af[mi], bfr[ni], acc[mi][ni], 0, 0, 0,
                                                                         xa[mi], 0, xb[ni]);
        } else {
          const v4f zero = {0.f, 0.f, 0.f, 0.f};
          if constexpr (MODE == kF32xMX)
            part[ni & 1][mi] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(af[mi], bfr[ni], zero, 0, 0, 0, 127,
                                                                                0, xb[ni]);
          else
            part[ni & 1][mi] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(af[mi], bfr[ni], zero, 0, 0, 0, 0, 0, 0);
          if (ni > 0) {
#pragma unroll
            for (int v = 0; v < 4; ++v)
              acc[mi][ni - 1][v] = __builtin_fmaf(part[(ni - 1) & 1][mi][v], sc[mi][v], acc[mi][ni - 1][v]);
          }
        }
      }
    }
    if constexpr (MODE != kMXxMX) {
#pragma unroll
      for (int mi = 0; mi < 4; ++mi)
#pragma unroll
        for (int v = 0; v < 4; ++v) acc[mi][3][v] = __builtin_fmaf(part[1][mi][v], sc[mi][v], acc[mi][3][v]);
      // instruction order for the scheduler: 4 MFMAs (with the 16 scale
      // products), then 12 x (1 MFMA, 4 multiply-adds), then the last 16
      // multiply-adds
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        if (MODE == kF32xF32) __builtin_amdgcn_sched_group_barrier(0x002, 4, 0);
      }
#pragma unroll
      for (int i = 0; i < 12; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x002, 4, 0);
      }
      __builtin_amdgcn_sched_group_barrier(0x002, 16, 0);
    }
  };

  // prologue: stages 0 .. STAGES-2
  for (int s = 0; s < STAGES - 1 && s < KB; ++s) issue(s);

  // wait until this wave's share of stage kb has landed (the next stage may
  // stay in flight); then the barrier makes every share visible
  auto wait_stage = [&](int kb, int per_stage) {
    if (kb + 1 < KB) wait_vmcnt(per_stage); else wait_vmcnt(0);
  };
  auto half_barrier = [&]() {
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_sched_barrier(0);
    asm volatile("" ::: "memory");
  };
  if (grp == 0) {
    constexpr int PER = A_PER + B_PER + 1;
    for (int kb = 0; kb < KB; ++kb) {
      wait_stage(kb, PER);
      half_barrier();              // half-step 2kb: memory
      mem_phase(kb);
      half_barrier();              // half-step 2kb+1: compute
      compute_phase();
    }
    half_barrier();                // half-step 2KB
  } else {
    constexpr int PER = A_PER + B_PER + 1;
    wait_stage(0, PER);
    half_barrier();                // half-step 0
    for (int kb = 0; kb < KB; ++kb) {
      half_barrier();              // half-step 2kb+1: memory
      mem_phase(kb);
      if (kb + 1 < KB) wait_stage(kb + 1, PER);
      half_barrier();              // half-step 2kb+2: compute
      compute_phase();
    }
  }

  // ---- epilogue (as in gemm_kernel)
  __syncthreads();
  float* stile = reinterpret_cast<float*>(smem);
  constexpr int TS = L::kTileStride;
#pragma unroll
  for (int mi = 0; mi < 4; ++mi)
#pragma unroll
    for (int ni = 0; ni < 4; ++ni)
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int r = wm * 64 + mi * 16 + 4 * fg + v;
        const int c = wn * 64 + ni * 16 + fr;
        stile[r * TS + c] = acc[mi][ni][v];
      }
  __syncthreads();
  const int64_t N = p.n;
  constexpr int NT = NW * 64;
  if constexpr (OUT_F32) {
    constexpr int LPR = BN / 4, RPP = NT / LPR;
#pragma unroll 4
    for (int it = 0; it < BM / RPP; ++it) {
      const int r = it * RPP + t / LPR;
      const int c = (t % LPR) * 4;
      if (r < mrows) {
        const float4 v = *reinterpret_cast<const float4*>(&stile[r * TS + c]);
        *reinterpret_cast<float4*>(reinterpret_cast<float*>(p.y) + (m0 + r) * N + n0 + c) = v;
      }
    }
  } else {
    constexpr int LPR = BN / 8, RPP = NT / LPR;
#pragma unroll 4
    for (int it = 0; it < BM / RPP; ++it) {
      const int r = it * RPP + t / LPR;
      const int c = (t % LPR) * 8;
      if (r < mrows) {
        const float4 v0 = *reinterpret_cast<const float4*>(&stile[r * TS + c]);
        const float4 v1 = *reinterpret_cast<const float4*>(&stile[r * TS + c + 4]);
        u32x4 o;
        o.x = pack_bf16x2(v0.x, v0.y);
        o.y = pack_bf16x2(v0.z, v0.w);
        o.z = pack_bf16x2(v1.x, v1.y);
        o.w = pack_bf16x2(v1.z, v1.w);
        *reinterpret_cast<u32x4*>(reinterpret_cast<uint16_t*>(p.y) + (m0 + r) * N + n0 + c) = o;
      }
    }
  }
}

template <int MODE, bool GROUPED, int BM, int BN, int STAGES>
static void launch_mode(const GemmParams& p, dim3 grid, bool out_f32, hipStream_t stream) {
  constexpr int NT = (BM / 64) * (BN / 64) * 64;
  if (out_f32)
    hipLaunchKernelGGL((gemm_kernel<MODE, true, GROUPED, BM, BN, STAGES>), grid, dim3(NT), 0, stream, p);
  else
    hipLaunchKernelGGL((gemm_kernel<MODE, false, GROUPED, BM, BN, STAGES>), grid, dim3(NT), 0, stream, p);
}

// Dense: 256x128 tiles, 8 waves, 3 stages (148.5 KiB of LDS, one workgroup
// per CU); a tile moves 48 KiB per K step for 8.4 MFLOP.
constexpr int kDenseBM = 256, kDenseBN = 128, kDenseStages = 3, kDenseBand = 4;
// Grouped: 128x128 tiles (groups are often only ~100-200 rows), 4 waves,
// 2 stages (~66 KiB, two workgroups per CU).
constexpr int kGroupBM = 128, kGroupBN = 128, kGroupStages = 2;

hipError_t launch_gemm(const uint8_t* a, const void* sa, int a_kind, const uint8_t* b, const void* sb, int b_kind,
                       int64_t m, int64_t n, int64_t k, void* y, bool out_f32, hipStream_t stream) {
  GemmParams p{};
  p.a = a; p.sa = sa; p.b = b; p.sb = sb; p.y = y;
  p.m = m; p.n = n; p.k = k;
  p.tiles_m = (int)((m + kDenseBM - 1) / kDenseBM);
  p.tiles_n = (int)(n / kDenseBN);
  p.band = kDenseBand;
  dim3 grid((unsigned)(p.tiles_m * p.tiles_n));
  const bool f32 = a_kind == 1 && b_kind == 2;
  if (f32 && out_f32)
    hipLaunchKernelGGL((gemm_pp_kernel<kF32xF32, true>), grid, dim3(512), 0, stream, p);
  else if (f32)
    hipLaunchKernelGGL((gemm_pp_kernel<kF32xF32, false>), grid, dim3(512), 0, stream, p);
  else if (out_f32)
    hipLaunchKernelGGL((gemm_pp_kernel<kMXxMX, true>), grid, dim3(512), 0, stream, p);
  else
    hipLaunchKernelGGL((gemm_pp_kernel<kMXxMX, false>), grid, dim3(512), 0, stream, p);
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
  const int64_t slots = total_m / kGroupBM + groups;
  dim3 grid((unsigned)slots, (unsigned)(n / kGroupBN));
  if (b_kind == 0) {
    p.sb_group_stride = n * (k / 32);
    launch_mode<kF32xMX, true, kGroupBM, kGroupBN, kGroupStages>(p, grid, out_f32, stream);
  } else {
    p.sb_group_stride = (n / 128) * (k / 128);
    launch_mode<kF32xF32, true, kGroupBM, kGroupBN, kGroupStages>(p, grid, out_f32, stream);
  }
  return hipGetLastError();
}

}  // namespace fp8blk
