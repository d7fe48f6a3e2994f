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
// Tiling: a workgroup of 8 waves computes a BM x BN tile (128x256, or
// 256x128 when N is not a multiple of 256), each wave a 64x64 block of 4x4
// MFMA tiles.  K advances
// 128 bytes at a time through a 3-deep ring of LDS stages filled by direct
// global->LDS loads (global_load_lds_dwordx4): every wave-wide load writes
// 1 KiB of LDS contiguously, 8 tile rows of 128 bytes.  Within a row the
// 16-byte K chunk c sits in slot c ^ swz(row), so that the 16-byte fragment
// reads of 16 consecutive rows touch distinct banks; the XOR is applied on
// the global-address side of the load.  The loads are inline assembly so
// that the compiler does not insert a full memory wait before every LDS
// read; vmcnt is managed here.
//
// MFMA operand layout (measured on gfx950 with single-element probes): for
// 16x16x128 lane l holds row (l % 16) and, within the 128-wide K chunk,
// bytes [16g, 16g+16) in its first 16 bytes and [64+16g, 64+16g+16) in its
// last 16 (g = l / 16).  The scale operand of lane L applies to row L % 16
// and the 32-wide K block L / 16.  The 16x16 fp32 result gives lane l
// column l % 16 and rows 4*(l/16) + v, v = 0..3.
#include <type_traits>

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
  const int32_t* row_index; // grouped only: A row read for each grouped row (null = the row itself)
  int64_t a_rows;           // gathered grouped only: rows of A (row_index values are clamped below it)
  int64_t m, n, k;
  int64_t b_group_stride;   // bytes of B per group
  int64_t sb_group_stride;  // scale elements of B per group
  int groups;
  int tiles_m, tiles_n;     // tile grid (grouped: tiles_m unused, n-tiles per group)
  int band;                 // m-tiles per band of the tile order (0 = one band)
};

// Dense tile order.  Workgroup b runs on XCD b % 8 and the XCDs have
// separate L2 caches, so each XCD takes a contiguous 1/8 of the tile
// indices, handed to its workgroups in turn (slot b / 8 takes indices
// slot, slot + W, ... of the range, W = workgroups per XCD); tiles are
// numbered column by column inside bands of `band` m-tiles, which makes
// the tiles an XCD runs at once a compact band x (W/band) block.
__device__ __forceinline__ int dense_tile_id(const GemmParams& p, int it) {
  const int T = p.tiles_m * p.tiles_n;
  const int x = (int)(blockIdx.x & 7), wsz = (int)(gridDim.x >> 3);
  const int q = T >> 3, rem = T & 7;
  const int cnt = q + (x < rem ? 1 : 0), start = x * q + (x < rem ? x : rem);
  const int j = (int)(blockIdx.x >> 3) + it * wsz;
  return j < cnt ? start + j : -1;
}
__device__ __forceinline__ void dense_tile(const GemmParams& p, int id, int* tm, int* tn) {
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

// Tiles per CU in one window of the grouped order (one window per XCD in
// turn): 2 measured 1.3% faster than 1 on the MoE down projection and equal
// on gate||up; 4 was 0.6% slower on gate||up.
constexpr int kWinTiles = 2;

// Grouped tile order.  Every workgroup builds, in LDS, the number of
// m-tiles of each group (ceil(M_g / BM)) and their prefix sums over the
// groups in zig-zag order (below); a group's tiles are numbered after those
// of the groups before it in that order, banded inside the group like the
// dense order.  Consecutive runs of tiles ("windows", kWinTiles tiles
// per CU of an XCD) share A rows and B columns; window w runs on XCD
// w mod 8, so each XCD sees a mix of large (compute-bound) and small
// (memory-bound) groups.  The grid is persistent: one workgroup per CU;
// workgroup b (XCD b mod 8, slot b / 8) takes positions slot, slot + W, ...
// (W workgroups per XCD) of every window of its XCD in turn.
// The offsets are not checked on the host.  Group g's rows are taken as
// [lo, hi) with lo = off[g] and hi = off[g+1] clamped into [0, total_m] and
// hi >= lo, so offsets that break the contract give unspecified output rows
// but no access outside A, its scales or Y.
__device__ __forceinline__ int clamp_int(int v, int lo, int hi) { return v < lo ? lo : (v > hi ? hi : v); }
__device__ __forceinline__ void group_rows(const GemmParams& p, int g, int* lo, int* hi) {
  const int total = (int)p.m;
  *lo = clamp_int(p.offsets[g], 0, total);
  *hi = clamp_int(p.offsets[g + 1], *lo, total);
}

// Groups are taken in zig-zag order of their index (0, G-1, 1, G-2, ...):
// when the group sizes rise or fall with the index, as with experts
// numbered by popularity, large groups (compute-bound tiles that reuse
// their weights) then run beside small ones (tiles that stream their
// weights once), instead of all large groups first and all small ones
// last (Zipf-routed MoE GEMMs: gate||up 4.78 to 4.70 ms, down projection
// 2.64 to 2.60 ms, bit-identical).  Position q holds group zigzag_group(q).
__device__ __forceinline__ int zigzag_group(int q, int groups) { return (q & 1) ? groups - 1 - (q >> 1) : (q >> 1); }

// s_incl: LDS of `groups` ints, s_incl[q] = m-tiles of the groups at
// positions 0..q (the m-tiles before position q are s_incl[q - 1], 0 for
// q = 0); returns the tile count.
template <int BM>
__device__ __forceinline__ int grouped_prefix(const GemmParams& p, int* s_incl, int nthreads) {
  const int groups = p.groups;
  const int t = threadIdx.x;
  for (int q = t; q < groups; q += nthreads) {
    int lo, hi;
    group_rows(p, zigzag_group(q, groups), &lo, &hi);
    s_incl[q] = (hi - lo + BM - 1) / BM;
  }
  __syncthreads();
  for (int d = 1; d < groups; d <<= 1) {  // inclusive scan
    int v[4];
    int cnt = 0;
    for (int g = t; g < groups; g += nthreads) v[cnt++] = (g >= d) ? s_incl[g - d] : 0;
    __syncthreads();
    cnt = 0;
    for (int g = t; g < groups; g += nthreads) s_incl[g] += v[cnt++];
    __syncthreads();
  }
  return s_incl[groups - 1] * p.tiles_n;
}

// Tile L (< the tile count) -> group, first row, rows, n-tile.
template <int BM>
__device__ __forceinline__ void grouped_locate(const GemmParams& p, const int* s_incl, int L,
                                               int* g_out, int64_t* row0, int* rows, int* tn_out) {
  const int tiles_n = p.tiles_n;
  const int slot = L / tiles_n;
  int lo = 0, hi = p.groups - 1;  // position q with s_incl[q - 1] <= slot < s_incl[q]
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (s_incl[mid - 1] <= slot) lo = mid; else hi = mid - 1;
  }
  const int qpos = lo;
  const int g = zigzag_group(qpos, p.groups);
  const int before = qpos > 0 ? s_incl[qpos - 1] : 0;
  const int tmg = s_incl[qpos] - before;
  const int r = L - before * tiles_n;
  const int band = p.band > 0 && p.band < tmg ? p.band : tmg;
  const int per_band = band * tiles_n;
  const int b = r / per_band, rr = r - b * per_band;
  const int rows_here = (b + 1) * band <= tmg ? band : tmg - b * band;
  const int tm = b * band + rr % rows_here;
  *g_out = g;
  *tn_out = rr / rows_here;
  int row_lo, row_hi;
  group_rows(p, g, &row_lo, &row_hi);
  *row0 = (int64_t)row_lo + (int64_t)tm * BM;
  const int64_t left = (int64_t)row_hi - *row0;
  *rows = (int)(left < BM ? left : BM);
}

// Row scales of A (and column scales of an E8M0-scaled B) are loaded in
// chunks of several K steps, 4 bytes per row and step: one fp32 scale, or
// the four E8M0 scales of the step's 1x32 blocks.  A chunk of SC steps is
// laid out as [block of 64/SC rows][K step][64/SC rows] x 4 bytes, so that
// one 64-lane dword load fills one block.  E8M0 B scales whose 4-step
// pieces are 16-byte aligned (K a multiple of 512, scale array 16-byte
// aligned) are loaded instead 16 bytes per column and lane, a chunk laid
// out as [column][K step] x 4 bytes: one load per 64 columns and 4 steps
// in place of 4 dword loads that each touch 16 scale rows (on the grouped
// MoE GEMM the dword loads cost 10% against no B-scale loads at all, the
// 16-byte loads about 5%).
constexpr int kLdsMax = 160 * 1024;
constexpr int kGroupTable = 1024 * 4;           // grouped: m-tile prefix of up to 1024 groups
// (1024 and not 1025 ints: with 3 stages, both 4-step scale rings and the
// table, a 128x256 or 256x128 tile fills the 160 KiB of LDS exactly)

// LDS bytes of a kernel with 3 stages and chunks of sa (A) and sb (B) steps
constexpr int pp_lds_bytes(int bm, int bn, bool b_mx, bool grouped, int sa, int sb) {
  return 3 * (bm * 128 + bn * 128 + (b_mx ? 0 : 256)) + 2 * bm * sa * 4 + (b_mx ? 2 * bn * sb * 4 : 0) +
         (grouped ? kGroupTable : 4);
}
// Chunk lengths: 4 K steps where they fit, else 2 (B first)
template <int BM, int BN, bool B_MX, bool GROUPED>
struct ChunkSteps {
  static constexpr int B = pp_lds_bytes(BM, BN, B_MX, GROUPED, 4, 4) <= kLdsMax ? 4 : 2;
  static constexpr int A = pp_lds_bytes(BM, BN, B_MX, GROUPED, 4, B) <= kLdsMax ? 4 : 2;
  static_assert(pp_lds_bytes(BM, BN, B_MX, GROUPED, A, B) <= kLdsMax, "LDS");
};

template <int BM, int BN, int STAGES, bool B_MX, int SCA, int SCB>
struct Layout {
  static constexpr int kA = BM * kBK;           // bytes of A per stage
  static constexpr int kB = BN * kBK;
  static constexpr int kSB = B_MX ? 0 : 256;    // fp32 B scales: one per 128-column block, in 64/(BN/128) lanes
  static constexpr int kStage = kA + kB + kSB;
  // after the stages, a ring of 2 A-scale chunks, then (E8M0 B) a ring of
  // 2 B-scale chunks
  static constexpr int kRingA = STAGES * kStage;
  static constexpr int kChunkA = BM * SCA * 4;
  static constexpr int kRingB = kRingA + 2 * kChunkA;
  static constexpr int kChunkB = B_MX ? BN * SCB * 4 : 0;
  static constexpr int kMain = kRingB + 2 * kChunkB;
  static constexpr int kTileStride = BN + 4;    // fp32 epilogue staging row stride
  static constexpr int kEpi = BM * kTileStride * 4;
  static constexpr int kBytes = (kMain > kEpi ? kMain : kEpi);
};

// ---------------------------------------------------------------------------
// Ping-pong kernel.  8 waves; wave w and wave w+4 share a SIMD.  Waves 0-3
// (group 0) own the left half of the tile's columns and waves 4-7 (group 1)
// the right half; within a group, wave w % 4 selects a 64x64 block.  Every
// K step is split into two half-steps separated by a workgroup barrier.  In
// each half-step one group runs its "memory" phase (LDS reads of its
// fragments for the next step and its share of the direct loads of a
// future stage) while the other group runs its "compute" phase (16 MFMAs
// and the fp32 promotion), so the matrix cores of every SIMD are fed by one
// wave while its partner waits on memory:
//   half-step 2kb   : group 0 memory(kb)   | group 1 compute(kb-1)
//   half-step 2kb+1 : group 0 compute(kb)  | group 1 memory(kb)
// The 8-row blocks of the A and B tiles are dealt to the 8 waves in turn,
// so each memory phase issues half of a stage's loads.  Group 0 also loads
// the A scales, a chunk of several K steps at a time into a ring of two
// chunks (the chunk starting at step kb is issued with the loads of stage
// kb), group 1 the B scales (E8M0 B in chunks too).  A stage is read at
// half-steps 2kb and 2kb+1 and refilled from half-step 2kb+6 on (3 stages).
template <int MODE, bool OUT_F32, bool GROUPED, int BM, int BN, bool BVEC>
__global__ __launch_bounds__(512) void gemm_pp_kernel(GemmParams p) {
  constexpr int STAGES = 3, NW = 8;
  constexpr int WMB = BM / 64;                 // 64-row blocks of the tile
  constexpr int GNB = BN / 128;                // 64-column blocks per group
  static_assert(WMB * GNB == 4, "each group is 4 waves of 64x64");
  constexpr bool A_MX = (MODE == kMXxMX);
  constexpr bool B_MX = (MODE != kF32xF32);
  constexpr int SLB = 64 / (BN / 128);         // fp32 B scales: lanes per 128-column block
  // K steps per scale chunk; rows (columns) per scale load; loads per
  // wave and chunk (group 0 loads A's chunks, group 1 B's)
  constexpr int SCA = ChunkSteps<BM, BN, B_MX, GROUPED>::A;
  constexpr int SCB = ChunkSteps<BM, BN, B_MX, GROUPED>::B;
  constexpr int RPLA = 64 / SCA, RPLB = 64 / SCB;
  constexpr int LPWA = BM / RPLA / 4, LPWB = B_MX ? BN / RPLB / 4 : 1;
  using L = Layout<BM, BN, STAGES, B_MX, SCA, SCB>;
  // BVEC: E8M0 B scales taken 16 bytes (4 K steps) per column and lane
  static_assert(!BVEC || (B_MX && SCB == 4 && BN % 64 == 0), "vector B-scale chunks");
  __shared__ __attribute__((aligned(16))) uint8_t smem[L::kBytes];
  __shared__ int s_grp[GROUPED ? kGroupTable / 4 : 1];   // grouped: m-tile prefix

  const int t = threadIdx.x;
  const int lane = t & 63;
  const int wave = __builtin_amdgcn_readfirstlane(t >> 6);
  const int grp = wave >> 2;          // ping-pong group
  const int gw = wave & 3;            // wave within the group
  const int wm = gw % WMB;            // 64x64 output block of this wave
  const int wn = grp * GNB + gw / WMB;
  const int64_t K = p.k;
  const int KB = (int)(K / kBK);
  int n_tiles = 1;
  if constexpr (GROUPED) n_tiles = grouped_prefix<BM>(p, s_grp, NW * 64);

  // this workgroup's tiles in turn (persistent grid)
  for (int it = 0;; ++it) {
  // ---- tile coordinates
  int64_t m0, n0;
  int mrows;
  const uint8_t* bq = p.b;
  const uint8_t* sb8 = reinterpret_cast<const uint8_t*>(p.sb);
  if constexpr (GROUPED) {
    const int wsz = (int)(gridDim.x >> 3);                    // CUs of an XCD (a window holds kWinTiles per CU)
    const int tile = ((it / kWinTiles) * 8 + (int)(blockIdx.x & 7)) * (kWinTiles * wsz) + (it % kWinTiles) * wsz +
                     (int)(blockIdx.x >> 3);
    if (tile >= n_tiles) break;
    int g, tn;
    grouped_locate<BM>(p, s_grp, tile, &g, &m0, &mrows, &tn);
    g = __builtin_amdgcn_readfirstlane(g);
    tn = __builtin_amdgcn_readfirstlane(tn);
    m0 = (int64_t)__builtin_amdgcn_readfirstlane((int)m0);
    mrows = __builtin_amdgcn_readfirstlane(mrows);
    n0 = (int64_t)tn * BN;
    bq += (int64_t)g * p.b_group_stride;
    sb8 += (int64_t)g * p.sb_group_stride * (B_MX ? 1 : 4);
  } else {
    const int id = dense_tile_id(p, it);
    if (id < 0) break;
    int tm, tn;
    dense_tile(p, id, &tm, &tn);
    m0 = (int64_t)tm * BM;
    n0 = (int64_t)tn * BN;
    mrows = (int)((p.m - m0) < BM ? (p.m - m0) : BM);
  }
  // A rows: tile row r reads row m0 + r of A, or, for a gathered grouped
  // problem, row row_index[m0 + r] (offsets then count from A's base; the
  // library checks that A's rows * K fit in 32 bits).
  const bool gather = GROUPED && p.row_index != nullptr;
  auto a_row = [&](int r) -> int64_t {
    return gather ? (int64_t)clamp_int(p.row_index[m0 + r], 0, (int)p.a_rows - 1) : (int64_t)r;
  };
  const uint8_t* aq = gather ? p.a : p.a + m0 * K;
  const uint8_t* bt = bq + n0 * K;
  const uint32_t lds0 = (uint32_t)(uintptr_t)smem;

  // ---- this wave's share of every stage.  Rows past the end of A re-read
  // the last valid row; their results are never stored.
  constexpr int A_PER = BM / 8 / NW, B_PER = BN / 8 / NW;
  uint32_t a_off[A_PER], b_off[B_PER];
  {
    const int sub = lane >> 3, slot = lane & 7;
#pragma unroll
    for (int j = 0; j < A_PER; ++j) {
      const int r = (j * NW + wave) * 8 + sub;
      const int rr = r < mrows ? r : mrows - 1;
      a_off[j] = (uint32_t)(a_row(rr) * K) + (uint32_t)((slot ^ swz(r)) * 16);
    }
#pragma unroll
    for (int j = 0; j < B_PER; ++j) {
      const int r = (j * NW + wave) * 8 + sub;
      b_off[j] = (uint32_t)(r * K) + (uint32_t)((slot ^ swz(r)) * 16);
    }
  }
  // Scale chunks.  Group 0 loads A's, group 1 (E8M0 B) B's, one chunk of
  // SC K steps at a time: load j of wave gw covers the block j * 4 + gw of
  // 64 / SC rows (columns), lane l reading row l % (64 / SC) of the block at
  // step l / (64 / SC) of the chunk.  A load thus touches 16 or 32 rows of
  // the scale array instead of 64, and the rows are what costs (they are
  // K / 128 or K / 32 bytes apart).  Rows past the end of A re-read the last
  // valid row, steps past K the last step.
  constexpr int LPW = LPWA > LPWB ? LPWA : LPWB;
  const int64_t a_row_bytes = A_MX ? K / 32 : (int64_t)KB * 4;
  const uint8_t* c_base;
  uint32_t c_off[LPW];
  uint32_t c_ring;
  int c_steps, c_rows, c_loads;
  if (grp == 0) {
    c_base = reinterpret_cast<const uint8_t*>(p.sa) + (gather ? 0 : m0 * a_row_bytes);
#pragma unroll
    for (int j = 0; j < LPW; ++j) {
      const int r = (j * 4 + gw) * RPLA + lane % RPLA;
      const int rr = r < mrows ? r : mrows - 1;
      c_off[j] = (uint32_t)(a_row(rr) * a_row_bytes);
    }
    c_ring = L::kRingA;
    c_steps = SCA; c_rows = RPLA; c_loads = LPWA;
  } else {
    c_base = sb8 + n0 * (K / 32);
    if constexpr (BVEC) {
      c_off[0] = (uint32_t)((gw * 64 + lane) * (K / 32));
      c_loads = gw < BN / 64 ? 1 : 0;
    } else {
#pragma unroll
      for (int j = 0; j < LPW; ++j) c_off[j] = (uint32_t)(((j * 4 + gw) * RPLB + lane % RPLB) * (K / 32));
      c_loads = B_MX ? LPWB : 0;
    }
    c_ring = L::kRingB;
    c_steps = SCB; c_rows = RPLB;
  }
  const uint32_t c_chunk = grp == 0 ? L::kChunkA : L::kChunkB;
  auto issue_chunk = [&](int c) {
    const uint32_t cbase = lds0 + c_ring + (c & 1) * c_chunk;
    if (BVEC && grp == 1) {
      if (c_loads) dma16(c_base, c_off[0] + (uint32_t)c * 16, cbase + gw * 1024);
      return;
    }
    int ks = c * c_steps + lane / c_rows;
    ks = ks < KB ? ks : KB - 1;
#pragma unroll
    for (int j = 0; j < LPW; ++j)
      if (j < c_loads) dma4(c_base, c_off[j] + (uint32_t)ks * 4, cbase + (j * 4 + gw) * 256);
  };
  // fp32 B scales, one load per stage by group 1.  Scale bases are per
  // tile, offsets small.
  uint32_t s_off = 0, s_lds = 0;
  const uint8_t* s_base = nullptr;
  bool s_load = false;
  if (grp == 0 || B_MX) {
  } else {
    // one fp32 scale per 128-column block and K step: one wave loads every
    // block's, lane l the scale of block l / SLB, so a block's scale is
    // read from LDS at a wave-uniform address (a broadcast)
    s_load = gw == 0;
    s_base = sb8 + (n0 / 128) * (int64_t)KB * 4;
    s_off = (uint32_t)((lane / SLB) * KB * 4);
    s_lds = L::kA + L::kB;
  }
  constexpr int PER = A_PER + B_PER + 1;
  // load i (0 .. PER-1) of this wave's share of stage kb
  auto issue_one = [&](int kb, int i) {
    const uint32_t sbase = lds0 + (kb % STAGES) * L::kStage;
    const uint32_t koff = (uint32_t)kb * kBK;
    if (i < A_PER)
      dma16(aq, a_off[i] + koff, sbase + (i * NW + wave) * 1024);
    else if (i < A_PER + B_PER)
      dma16(bt, b_off[i - A_PER] + koff, sbase + L::kA + ((i - A_PER) * NW + wave) * 1024);
    else if (s_load)
      dma4(s_base, s_off + (uint32_t)kb * 4, sbase + s_lds);
  };
  // a stage's loads, then the scale chunk that starts at stage kb: issued
  // before any load of the next stage, it has landed once stage kb has
  // (loads complete in order).  Issued last rather than first, the chunk's
  // scattered rows do not delay the stage's data.
  auto issue = [&](int kb) {
#pragma unroll
    for (int i = 0; i < PER; ++i) issue_one(kb, i);
    if (kb % c_steps == 0) issue_chunk(kb / c_steps);
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

  // memory phase: fragments and scales of step kb into registers, with this
  // wave's loads of stage kb+2 interleaved between the fragment reads (a
  // load waiting on the address unit then does not hold back LDS reads)
  auto mem_phase = [&](int kb, auto do_load_t) {
    constexpr bool do_load = decltype(do_load_t)::value;
    const uint8_t* sA = smem + (kb % STAGES) * L::kStage;
    const uint8_t* sB = sA + L::kA;
    const uint32_t* sSB = reinterpret_cast<const uint32_t*>(sA + L::kA + L::kB);
    // scales of A row r at step kb: sSCA[(r / RPLA) * 64 + r % RPLA], of B
    // column c: sSCB[(c / RPLB) * 64 + c % RPLB]
    const uint32_t* sSCA = reinterpret_cast<const uint32_t*>(smem + L::kRingA + ((kb / SCA) & 1) * L::kChunkA) + (kb % SCA) * RPLA;
    const uint32_t* sSCB = reinterpret_cast<const uint32_t*>(smem + L::kRingB + ((kb / SCB) & 1) * L::kChunkB) + (kb % SCB) * RPLB;
    const uint32_t* sSCBv = reinterpret_cast<const uint32_t*>(smem + L::kRingB + ((kb / SCB) & 1) * L::kChunkB) + (kb % SCB);
#pragma unroll
    for (int mi = 0; mi < 4; ++mi) {
      const int ar = wm * 64 + mi * 16 + fr;
      const uint8_t* rowp = sA + ar * kBK;
      const int s0 = (fg ^ swz(ar)) * 16;
      af[mi] = make_frag(*reinterpret_cast<const u32x4*>(rowp + s0), *reinterpret_cast<const u32x4*>(rowp + (s0 ^ 64)));
      if constexpr (do_load) issue_one(kb + STAGES - 1, mi);
      if constexpr (A_MX) {
        xa[mi] = (int)((sSCA[(ar / RPLA) * 64 + ar % RPLA] >> (8 * fg)) & 0xFFu);
      } else {
        const int r0 = wm * 64 + mi * 16 + 4 * fg;   // 4 rows in one block of RPLA (>= 16) rows
        const u32x4 s4 = *reinterpret_cast<const u32x4*>(&sSCA[(r0 / RPLA) * 64 + r0 % RPLA]);
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
      if constexpr (do_load) {
        if (4 + ni < PER) issue_one(kb + STAGES - 1, 4 + ni);
      }
      if constexpr (BVEC) xb[ni] = (int)((sSCBv[bc * SCB] >> (8 * fg)) & 0xFFu);
      else if constexpr (B_MX) xb[ni] = (int)((sSCB[(bc / RPLB) * 64 + bc % RPLB] >> (8 * fg)) & 0xFFu);
    }
    if constexpr (MODE == kF32xF32) sbk = __uint_as_float(sSB[(wn >> 1) * SLB]);
    if constexpr (do_load) {
#pragma unroll
      for (int i = 8; i < PER; ++i) issue_one(kb + STAGES - 1, i);
    }
    if constexpr (do_load) {
      if ((kb + STAGES - 1) % c_steps == 0) issue_chunk((kb + STAGES - 1) / c_steps);
    }
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
          else  // literal zero scale operands: the compiler emits the plain (unscaled)
                // v_mfma_f32_16x16x128_f8f6f4; the neutral E8M0 scale 127 gives the scaled
                // form with scale registers, measured 11% slower in this kernel (C2, C3)
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
  // (BVEC: a B-scale chunk issued behind stage kb+1 may stay in flight too)
  auto wait_stage = [&](int kb) {
    if (kb + 1 >= KB) wait_vmcnt(0);
    else if (s_load) wait_vmcnt(PER);
    else if (BVEC && grp == 1 && c_loads && (kb + 1) % SCB == 0) wait_vmcnt(PER);
    else wait_vmcnt(PER - 1);
  };
  auto half_barrier = [&]() {
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_sched_barrier(0);
    asm volatile("" ::: "memory");
  };
  // The loops are split where the loads of later stages run out, so that
  // the loop bodies carry no branch around the loads.
  const int kl = KB > STAGES - 1 ? KB - (STAGES - 1) : 0;
  if (grp == 0) {
    auto step = [&](int kb, auto do_load) {
      wait_stage(kb);
      half_barrier();              // half-step 2kb: memory
      mem_phase(kb, do_load);
      half_barrier();              // half-step 2kb+1: compute
      compute_phase();
    };
    for (int kb = 0; kb < kl; ++kb) step(kb, std::true_type{});
    for (int kb = kl; kb < KB; ++kb) step(kb, std::false_type{});
    half_barrier();                // half-step 2KB
  } else {
    wait_stage(0);
    half_barrier();                // half-step 0
    // Grouped kernels: group 1's memory phase runs at raised wave priority,
    // so that its LDS reads and loads issue ahead of the partner wave's
    // promotion arithmetic on the same SIMD (bit-identical; MoE gate||up
    // -4.3%, down projection -3.1%; the same on group 0, or on the dense
    // kernels, gained nothing or lost up to 3.5%).
    auto step = [&](int kb, auto do_load) {
      half_barrier();              // half-step 2kb+1: memory
      if constexpr (GROUPED) __builtin_amdgcn_s_setprio(1);
      mem_phase(kb, do_load);
      if constexpr (GROUPED) __builtin_amdgcn_s_setprio(0);
      if (kb + 1 < KB) wait_stage(kb + 1);
      half_barrier();              // half-step 2kb+2: compute
      compute_phase();
    };
    for (int kb = 0; kb < kl; ++kb) step(kb, std::true_type{});
    for (int kb = kl; kb < KB; ++kb) step(kb, std::false_type{});
  }

  // ---- epilogue: stage the tile in LDS, then write whole rows with 16-byte
  // stores (8 bf16 or 4 fp32 per lane)
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
  __syncthreads();   // the next tile's loads reuse this LDS
  }  // tile loop
}

template <int MODE, bool GROUPED, int BM, int BN, bool BVEC = false>
static void launch_pp(const GemmParams& p, dim3 grid, bool out_f32, hipStream_t stream) {
  if (out_f32)
    hipLaunchKernelGGL((gemm_pp_kernel<MODE, true, GROUPED, BM, BN, BVEC>), grid, dim3(512), 0, stream, p);
  else
    hipLaunchKernelGGL((gemm_pp_kernel<MODE, false, GROUPED, BM, BN, BVEC>), grid, dim3(512), 0, stream, p);
}
// E8M0 B scales in 16-byte pieces: every column's chunk of 4 K steps is
// 16-byte aligned and inside its row when K is a multiple of 512 and the
// scale array is 16-byte aligned
static bool b_scales_vec(const void* sb, int64_t k) { return k % 512 == 0 && (uintptr_t)sb % 16 == 0; }

// Dense: 128x256 tiles (256x128 when n is not a multiple of 256), 3 stages
// (151 or 153.5 KiB of LDS with the A-scale ring, one workgroup per CU); a tile moves 48 KiB per K step
// for 8.4 MFLOP.  Bands of 4 m-tiles.
constexpr int kDenseBand = 4;
// Grouped: the same tiles (m-tiles of 128 rows also waste less on small
// groups); bands of 8 m-tiles.
constexpr int kGroupBand = 8;

hipError_t launch_gemm(const uint8_t* a, const void* sa, int a_kind, const uint8_t* b, const void* sb, int b_kind,
                       int64_t m, int64_t n, int64_t k, void* y, bool out_f32, int num_cu, hipStream_t stream) {
  GemmParams p{};
  p.a = a; p.sa = sa; p.b = b; p.sb = sb; p.y = y;
  p.m = m; p.n = n; p.k = k;
  const bool wide = n % 256 == 0;
  p.tiles_m = (int)(wide ? (m + 127) / 128 : (m + 255) / 256);
  p.tiles_n = (int)(wide ? n / 256 : n / 128);
  p.band = kDenseBand;
  // persistent: at most one workgroup per CU (the kernel's LDS admits one),
  // a multiple of the 8 XCDs
  const int64_t tiles = (int64_t)p.tiles_m * p.tiles_n;
  const int64_t full = num_cu >= 8 ? num_cu / 8 * 8 : 8;
  const int64_t wgs = tiles < full ? (tiles + 7) / 8 * 8 : full;
  dim3 grid((unsigned)wgs);
  if (a_kind == 1 && b_kind == 2) {
    if (wide) launch_pp<kF32xF32, false, 128, 256>(p, grid, out_f32, stream);
    else launch_pp<kF32xF32, false, 256, 128>(p, grid, out_f32, stream);
  } else if (b_scales_vec(sb, k)) {
    if (wide) launch_pp<kMXxMX, false, 128, 256, true>(p, grid, out_f32, stream);
    else launch_pp<kMXxMX, false, 256, 128, true>(p, grid, out_f32, stream);
  } else {
    if (wide) launch_pp<kMXxMX, false, 128, 256>(p, grid, out_f32, stream);
    else launch_pp<kMXxMX, false, 256, 128>(p, grid, out_f32, stream);
  }
  return hipGetLastError();
}

hipError_t launch_grouped_gemm(const uint8_t* a, const void* sa, int a_kind, const int32_t* row_index,
                               int64_t a_rows, const uint8_t* b, const void* sb, int b_kind, const int32_t* offsets, int64_t groups,
                               int64_t total_m, int64_t n, int64_t k, void* y, bool out_f32, int num_cu,
                               hipStream_t stream) {
  (void)a_kind;
  GemmParams p{};
  p.a = a; p.sa = sa; p.b = b; p.sb = sb; p.y = y;
  p.offsets = offsets;
  p.row_index = row_index;
  p.a_rows = a_rows;
  p.m = total_m; p.n = n; p.k = k;
  p.groups = (int)groups;
  p.b_group_stride = n * k;
  p.sb_group_stride = b_kind == 0 ? n * (k / 32) : (n / 128) * (k / 128);
  p.band = kGroupBand;
  const bool wide = n % 256 == 0;
  p.tiles_n = (int)(wide ? n / 256 : n / 128);
  // persistent: one workgroup per CU (the kernel's LDS admits one), a
  // multiple of the 8 XCDs
  const int wgs = num_cu >= 8 ? num_cu / 8 * 8 : 8;
  dim3 grid((unsigned)wgs);
  if (b_kind == 0 && b_scales_vec(sb, k)) {
    if (wide) launch_pp<kF32xMX, true, 128, 256, true>(p, grid, out_f32, stream);
    else launch_pp<kF32xMX, true, 256, 128, true>(p, grid, out_f32, stream);
  } else if (b_kind == 0) {
    if (wide) launch_pp<kF32xMX, true, 128, 256>(p, grid, out_f32, stream);
    else launch_pp<kF32xMX, true, 256, 128>(p, grid, out_f32, stream);
  } else {
    if (wide) launch_pp<kF32xF32, true, 128, 256>(p, grid, out_f32, stream);
    else launch_pp<kF32xF32, true, 256, 128>(p, grid, out_f32, stream);
  }
  return hipGetLastError();
}

}  // namespace fp8blk
