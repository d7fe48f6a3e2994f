// QAT backward for the LoRA factors (gfx950).
//
// Method ([Fireworks-QAT] Synopsis and Interpretation): in QAT the forward
// pass runs on the fake-quantized merged weight W_hat = fakequant(W + B.A)
// and fake-quantized activations X_hat, while B, A and their gradients stay
// in bf16.  With the fake-quant passed straight through, the weight
// gradient is dW = dY^T . X_hat and
//     dB = dW . A^T = dY^T . (X_hat . A^T) = dY^T . P,     P = X_hat . A^T
//     dA = B^T . dW = (dY . B)^T . X_hat = Q^T . X_hat,    Q = dY . B
// so dW [N x K] is never formed: two skinny products over the hidden
// dimensions and two reductions over the tokens.
//
// Kernels (one stream, in order):
//   prep    B^T, zero-padded to RP = 16 * CT rows, into the workspace (the
//           MFMA operands need the reduced index contiguous per lane).
//   proj    P and Q for 32 tokens per workgroup.  Four waves split the
//           hidden dimension in 128-wide blocks; each wave runs two 16-token
//           MFMA tiles (v_mfma_f32_16x16x32_bf16) against the A / B^T
//           fragments, the four partial sums meet in LDS.  P and Q leave as
//           an unevaluated sum hi + lo of two bf16 values (16 significant
//           bits), already in the lane layout the reduction loads.
//   reduce  dB^T and dA partials over one slice of 32-token blocks.  A wave
//           owns 128 columns of dY (or X_hat) and loads, per block, 8 rows
//           of 16 bytes per lane; the 8x8 bf16 block a lane holds is
//           transposed in registers (v_perm_b32), so that the token index
//           becomes the reduced MFMA index.  hi and lo operands feed the same
//           fp32 accumulator.  Two row groups of 4 waves per workgroup add
//           through LDS; each workgroup writes one fp32 partial.
//   finish  sum of the slice partials in slice order, rounded to bf16 (or
//           kept fp32): deterministic, no atomics.
//
// Reduced-index assignment: an MFMA sums over 32 values of its reduced
// index, 8 per lane group; which hidden or token index each (lane group,
// element) pair stands for is free as long as both operands agree, and both
// operands are loaded with the same assignment below.
#include <mutex>

#include "device.h"
#include "launch.h"

// Scratch of fp8_lora_backward_noalloc: the workspace of the kernels below
// in a fixed device array, for callers that cannot allocate.  Each GPU the
// library runs on holds its own copy until the process ends.  Host code
// never uses the name itself (on the host it is a stand-in, not a device
// address): lora_bwd_scratch looks up the address once per device.
static __device__ __align__(256) uint8_t scratch[fp8blk::kLoraScratchBytes];

namespace fp8blk {

namespace {
struct ScratchSlot {
  std::once_flag once;
  hipError_t err = hipSuccess;
  void* ptr = nullptr;
};
ScratchSlot g_scratch[kMaxScratchDevices];
}  // namespace

hipError_t lora_bwd_scratch(int dev, void** ptr) {
  if (dev < 0 || dev >= kMaxScratchDevices) return hipErrorInvalidDevice;
  ScratchSlot& s = g_scratch[dev];
  // runs with `dev` current (the caller's device), once per device
  std::call_once(s.once, [&s] { s.err = hipGetSymbolAddress(&s.ptr, HIP_SYMBOL(scratch)); });
  if (s.err != hipSuccess) return s.err;
  *ptr = s.ptr;
  return hipSuccess;
}

namespace {

typedef __bf16 v8bf __attribute__((ext_vector_type(8)));

constexpr int kPrepThreads = 256;
constexpr int kProjThreads = 256;   // 4 waves, 32 tokens (ranks above 32; rank <= 32: 8 waves, 64 tokens)
constexpr int kRedThreads = 512;    // 4 column waves x 2 row groups
constexpr int kRedCols = 512;       // columns per reduction workgroup
constexpr int kFinThreads = 256;
constexpr int kRedTargetWG = 256;   // reduction workgroups aimed at (slices x column groups)

struct LoraBwdParams {
  const uint16_t* dy;   // [m][n]
  const uint16_t* x;    // [m][k]
  const uint16_t* lb;   // [n][r]
  const uint16_t* la;   // [r][k]
  uint16_t* bt;         // [rp][n] workspace
  u32x4* pf;            // P fragments [mb][ct][hi, lo][64 lanes]
  u32x4* qf;            // Q fragments
  float* part_b;        // [slices][n][rp]
  float* part_a;        // [slices][rp][k]
  void* d_b;            // [n][r]
  void* d_a;            // [r][k]
  int64_t m;
  int n, k, r;
  int mb;               // 32-token blocks
  int slices, bps;      // slices of bps blocks
  int out_f32;
};

__device__ __forceinline__ v4f mfma_bf16(u32x4 a, u32x4 b, v4f c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(v8bf, a), __builtin_bit_cast(v8bf, b), c, 0, 0,
                                                 0);
}

__device__ __forceinline__ u32x4 ld16(const uint16_t* p) { return *reinterpret_cast<const u32x4*>(p); }

constexpr u32x4 kZero4 = {0u, 0u, 0u, 0u};

// Row c of the padded B^T (blockIdx.y = c < rp) is column c of B, zero for
// c >= r; blockIdx.x covers n.
__global__ __launch_bounds__(kPrepThreads) void lora_prep_kernel(LoraBwdParams p) {
  const int c = (int)blockIdx.y;
  const int64_t nn = (int64_t)blockIdx.x * kPrepThreads + threadIdx.x;
  if (nn >= p.n) return;
  p.bt[(int64_t)c * p.n + nn] = c < p.r ? p.lb[nn * p.r + c] : (uint16_t)0;
}

// P (blockIdx.y == 0: X_hat against A) or Q (blockIdx.y == 1: dY against
// B^T) for tokens [16 T * blockIdx.x, +16 T): NWV waves, each T 16-token
// tiles over the 128-wide blocks w, w + NWV, ... of the hidden dimension.
template <int CT, int T>
__global__ __launch_bounds__(T == 4 ? 512 : 256) void lora_proj_kernel(LoraBwdParams p) {
  constexpr int NWV = T == 4 ? 8 : 4;
  __shared__ float red[NWV][T][CT][4][64];
  const bool isq = blockIdx.y != 0;
  const uint16_t* src = isq ? p.dy : p.x;
  const int64_t ld = isq ? p.n : p.k;
  const uint16_t* sm = isq ? p.bt : p.la;
  const int sm_rows = isq ? 16 * CT : p.r;
  u32x4* frag = isq ? p.qf : p.pf;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int fr = lane & 15, fg = lane >> 4;
  const int64_t m0 = (int64_t)blockIdx.x * (16 * T);
  const int nkb = (int)(ld / 128);

  // Lane (fr, fg) of tile t reads token m0 + 16t + fr; of fragment ct, row
  // 16ct + fr of the small operand.  MFMA j of a 128-wide block covers
  // hidden indices 32j + 8fg + e, e = 0..7, in both operands.
  const uint16_t* xr[T];
  bool xv[T];
#pragma unroll
  for (int t = 0; t < T; ++t) {
    const int64_t row = m0 + 16 * t + fr;
    xv[t] = row < p.m;
    xr[t] = src + (xv[t] ? row : 0) * ld + 8 * fg;
  }
  const uint16_t* sr[CT];
  bool sv[CT];
#pragma unroll
  for (int ct = 0; ct < CT; ++ct) {
    const int c = 16 * ct + fr;
    sv[ct] = c < sm_rows;
    sr[ct] = sm + (int64_t)(sv[ct] ? c : 0) * ld + 8 * fg;
  }

  v4f acc[T][CT];
#pragma unroll
  for (int t = 0; t < T; ++t)
#pragma unroll
    for (int ct = 0; ct < CT; ++ct) acc[t][ct] = (v4f){0.f, 0.f, 0.f, 0.f};

  u32x4 xa[T][4], sa[CT][4];
  auto load = [&](int kb) {
#pragma unroll
    for (int t = 0; t < T; ++t)
#pragma unroll
      for (int j = 0; j < 4; ++j) xa[t][j] = xv[t] ? ld16(xr[t] + kb * 128 + 32 * j) : kZero4;
#pragma unroll
    for (int ct = 0; ct < CT; ++ct)
#pragma unroll
      for (int j = 0; j < 4; ++j) sa[ct][j] = sv[ct] ? ld16(sr[ct] + kb * 128 + 32 * j) : kZero4;
  };
  int kb = w;
  if (kb < nkb) load(kb);
  while (kb < nkb) {
    u32x4 xc[T][4], sc[CT][4];
#pragma unroll
    for (int t = 0; t < T; ++t)
#pragma unroll
      for (int j = 0; j < 4; ++j) xc[t][j] = xa[t][j];
#pragma unroll
    for (int ct = 0; ct < CT; ++ct)
#pragma unroll
      for (int j = 0; j < 4; ++j) sc[ct][j] = sa[ct][j];
    kb += NWV;
    if (kb < nkb) load(kb);
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int t = 0; t < T; ++t)
#pragma unroll
        for (int ct = 0; ct < CT; ++ct) acc[t][ct] = mfma_bf16(xc[t][j], sc[ct][j], acc[t][ct]);
  }

  // acc[t][ct] lane l holds token m0 + 16t + 4(l/16) + v, column 16ct + l%16.
#pragma unroll
  for (int t = 0; t < T; ++t)
#pragma unroll
    for (int ct = 0; ct < CT; ++ct)
#pragma unroll
      for (int v = 0; v < 4; ++v) red[w][t][ct][v][lane] = acc[t][ct][v];
  __syncthreads();

  // Fragment lane L = (column L%16, group L/16) holds tokens 8(L/16) + e of
  // the block, e = 0..7; thread (L, ep) forms elements 2ep and 2ep + 1.
  // With T = 4 the workgroup writes two 32-token blocks: waves 4b .. 4b+3
  // form block b.
  const int L = threadIdx.x & 63, ep = (threadIdx.x >> 6) & 3, b = (threadIdx.x >> 6) >> 2;
  const int cc = L & 15, G = L >> 4;
  const int64_t blk = (int64_t)blockIdx.x * (T / 2) + b;
  if (blk >= p.mb) return;
  uint32_t* fw = reinterpret_cast<uint32_t*>(frag);
#pragma unroll
  for (int ct = 0; ct < CT; ++ct) {
    float s[2];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int ml = 32 * b + 8 * G + 2 * ep + h;
      const int t = ml >> 4, g = (ml & 15) >> 2, v = ml & 3, sl = 16 * g + cc;
      float a = red[0][t][ct][v][sl];
#pragma unroll
      for (int ww = 1; ww < NWV; ++ww) a += red[ww][t][ct][v][sl];
      s[h] = a;
    }
    const uint32_t hi = pack_bf16x2(s[0], s[1]);
    const uint32_t lo = pack_bf16x2(s[0] - bf_lo(hi), s[1] - bf_hi(hi));
    const int64_t base = ((blk * CT + ct) * 2) * 256 + L * 4 + ep;
    fw[base] = hi;
    fw[base + 256] = lo;
  }
}

// Reduction over one slice of 32-token blocks: dB^T partial (dY with P) for
// column groups [0, cgb) and dA partial (X_hat with Q) after them.
template <int CT>
__global__ __launch_bounds__(kRedThreads) void lora_reduce_kernel(LoraBwdParams p, int cgb) {
  __shared__ float xch[4][CT][8][4][64];
  const int s = blockIdx.x % p.slices;
  const int cga = blockIdx.x / p.slices;
  const bool isa = cga >= cgb;
  const int cg = isa ? cga - cgb : cga;
  const uint16_t* src = isa ? p.x : p.dy;
  const int cols = isa ? p.k : p.n;
  const u32x4* frag = isa ? p.qf : p.pf;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int nw = w & 3, mg = w >> 2;
  const int fr = lane & 15, fg = lane >> 4;
  const int c0 = cg * kRedCols + nw * 128;
  const bool active = c0 < cols;

  v4f acc[CT][8];
#pragma unroll
  for (int ct = 0; ct < CT; ++ct)
#pragma unroll
    for (int j = 0; j < 8; ++j) acc[ct][j] = (v4f){0.f, 0.f, 0.f, 0.f};

  const int mb_end = min((s + 1) * p.bps, p.mb);
  // Lane (fr, fg) reads tokens 32mb + 8fg + t, t = 0..7, columns c0 + 8fr + j.
  const uint16_t* colp = src + c0 + 8 * fr;
  u32x4 d[8];
  auto load = [&](int mb) {
    const int64_t row0 = (int64_t)mb * 32 + 8 * fg;
#pragma unroll
    for (int t = 0; t < 8; ++t) d[t] = row0 + t < p.m ? ld16(colp + (row0 + t) * cols) : kZero4;
  };
  // Rank 64 holds 128 accumulators per lane: no room for a second row
  // buffer there, so the next block is loaded ahead only for CT < 4.
  constexpr bool kAhead = CT < 4;
  int mb = s * p.bps + mg;
  if (kAhead && active && mb < mb_end) load(mb);
  while (active && mb < mb_end) {
    u32x4 dc[8];
    if constexpr (!kAhead) load(mb);
#pragma unroll
    for (int t = 0; t < 8; ++t) dc[t] = d[t];
    u32x4 fh[CT], fl[CT];
#pragma unroll
    for (int ct = 0; ct < CT; ++ct) {
      fh[ct] = frag[((int64_t)mb * CT + ct) * 128 + lane];
      fl[ct] = frag[((int64_t)mb * CT + ct) * 128 + 64 + lane];
    }
    mb += 2;
    if (kAhead && mb < mb_end) load(mb);
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      // element e of the operand = token 8fg + e, column c0 + 8fr + j
      const uint32_t sel = (j & 1) ? 0x07060302u : 0x05040100u;
      u32x4 b;
#pragma unroll
      for (int dd = 0; dd < 4; ++dd) b[dd] = __builtin_amdgcn_perm(dc[2 * dd + 1][j >> 1], dc[2 * dd][j >> 1], sel);
#pragma unroll
      for (int ct = 0; ct < CT; ++ct) {
        acc[ct][j] = mfma_bf16(fh[ct], b, acc[ct][j]);
        acc[ct][j] = mfma_bf16(fl[ct], b, acc[ct][j]);
      }
    }
  }

  if (mg == 1) {
#pragma unroll
    for (int ct = 0; ct < CT; ++ct)
#pragma unroll
      for (int j = 0; j < 8; ++j)
#pragma unroll
        for (int v = 0; v < 4; ++v) xch[nw][ct][j][v][lane] = acc[ct][j][v];
  }
  __syncthreads();
  if (mg != 0 || !active) return;
  constexpr int RP = 16 * CT;
  // acc[ct][j] lane l: rank index 16ct + 4(l/16) + v, column c0 + 8(l%16) + j.
  if (!isa) {
    float* out = p.part_b + (int64_t)s * p.n * RP;
#pragma unroll
    for (int ct = 0; ct < CT; ++ct)
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        v4f o;
#pragma unroll
        for (int v = 0; v < 4; ++v) o[v] = acc[ct][j][v] + xch[nw][ct][j][v][lane];
        *reinterpret_cast<v4f*>(out + (int64_t)(c0 + 8 * fr + j) * RP + 16 * ct + 4 * fg) = o;
      }
  } else {
    float* out = p.part_a + (int64_t)s * RP * p.k;
#pragma unroll
    for (int ct = 0; ct < CT; ++ct)
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        v4f o0, o1;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          o0[j] = acc[ct][j][v] + xch[nw][ct][j][v][lane];
          o1[j] = acc[ct][j + 4][v] + xch[nw][ct][j + 4][v][lane];
        }
        float* q = out + (int64_t)(16 * ct + 4 * fg + v) * p.k + c0 + 8 * fr;
        *reinterpret_cast<v4f*>(q) = o0;
        *reinterpret_cast<v4f*>(q + 4) = o1;
      }
  }
}

// Workgroups [0, nbb) sum dB: thread x is partial row x >> rp_log2 (= n),
// rank x & (rp - 1) (rp is a power of two).  Workgroups nbb + c * kba + j
// sum row c of dA, columns [kFinThreads * j, +kFinThreads).  Slices are
// added in order, so the result does not depend on the launch.
__global__ __launch_bounds__(kFinThreads) void lora_finish_kernel(LoraBwdParams p, int rp_log2, int nbb, int kba) {
  const int rp = 1 << rp_log2;
  float acc = 0.f;
  if ((int)blockIdx.x < nbb) {
    const int64_t x = (int64_t)blockIdx.x * kFinThreads + threadIdx.x;
    const int64_t nn = x >> rp_log2;
    const int c = (int)(x & (rp - 1));
    if (nn >= p.n || c >= p.r) return;
    for (int s = 0; s < p.slices; ++s) acc += p.part_b[(((int64_t)s * p.n + nn) << rp_log2) + c];
    const int64_t o = nn * p.r + c;
    if (p.out_f32)
      reinterpret_cast<float*>(p.d_b)[o] = acc;
    else
      reinterpret_cast<uint16_t*>(p.d_b)[o] = (uint16_t)(pack_bf16x2(acc, 0.f) & 0xFFFFu);
  } else {
    const int b = (int)blockIdx.x - nbb;
    const int c = b / kba;
    const int64_t kk = (int64_t)(b - c * kba) * kFinThreads + threadIdx.x;
    if (kk >= p.k) return;
    for (int s = 0; s < p.slices; ++s) acc += p.part_a[((int64_t)s * rp + c) * p.k + kk];
    const int64_t o = (int64_t)c * p.k + kk;
    if (p.out_f32)
      reinterpret_cast<float*>(p.d_a)[o] = acc;
    else
      reinterpret_cast<uint16_t*>(p.d_a)[o] = (uint16_t)(pack_bf16x2(acc, 0.f) & 0xFFFFu);
  }
}

struct LoraPlan {
  int ct, rp, mb, cgb, cga, slices, bps;
  int64_t off_bt, off_pf, off_qf, off_pb, off_pa, bytes;
};

int64_t align256(int64_t v) { return (v + 255) & ~int64_t(255); }

LoraPlan plan(int64_t m, int64_t n, int64_t k, int64_t r) {
  LoraPlan pl;
  pl.ct = r <= 16 ? 1 : r <= 32 ? 2 : 4;
  pl.rp = 16 * pl.ct;
  pl.mb = (int)((m + 31) / 32);
  pl.cgb = (int)((n + kRedCols - 1) / kRedCols);
  pl.cga = (int)((k + kRedCols - 1) / kRedCols);
  const int cgs = pl.cgb + pl.cga > 0 ? pl.cgb + pl.cga : 1;
  int target = kRedTargetWG / cgs;
  if (target < 1) target = 1;
  pl.bps = pl.mb > 0 ? (pl.mb + target - 1) / target : 0;
  if (pl.bps > 0 && pl.bps < 2) pl.bps = 2;  // one block per row group at least
  pl.slices = pl.bps > 0 ? (pl.mb + pl.bps - 1) / pl.bps : 1;
  const int64_t frag_bytes = (int64_t)pl.mb * pl.ct * 2 * 1024;
  pl.off_bt = 0;
  pl.off_pf = align256(pl.off_bt + (int64_t)pl.rp * n * 2);
  pl.off_qf = align256(pl.off_pf + frag_bytes);
  pl.off_pb = align256(pl.off_qf + frag_bytes);
  pl.off_pa = align256(pl.off_pb + (int64_t)pl.slices * n * pl.rp * 4);
  pl.bytes = align256(pl.off_pa + (int64_t)pl.slices * pl.rp * k * 4);
  return pl;
}

template <int CT>
hipError_t launch_ct(const LoraBwdParams& p, const LoraPlan& pl, int num_cu, hipStream_t stream) {
  (void)num_cu;
  if (pl.rp * (int64_t)p.n > 0) {
    const int64_t g = ((int64_t)p.n + kPrepThreads - 1) / kPrepThreads;
    hipLaunchKernelGGL(lora_prep_kernel, dim3((unsigned)g, (unsigned)pl.rp), dim3(kPrepThreads), 0, stream, p);
  }
  if (pl.mb > 0)
  {
    if constexpr (CT <= 2)
      hipLaunchKernelGGL((lora_proj_kernel<CT, 4>), dim3((pl.mb + 1) / 2, 2), dim3(512), 0, stream, p);
    else
      hipLaunchKernelGGL((lora_proj_kernel<CT, 2>), dim3(pl.mb, 2), dim3(kProjThreads), 0, stream, p);
  }
  if (pl.cgb + pl.cga > 0)
    hipLaunchKernelGGL((lora_reduce_kernel<CT>), dim3((pl.cgb + pl.cga) * pl.slices), dim3(kRedThreads), 0, stream,
                       p, pl.cgb);
  const int64_t outs = (int64_t)p.r * (p.n + p.k);
  if (outs > 0) {
    const int64_t nbb = ((int64_t)p.n * pl.rp + kFinThreads - 1) / kFinThreads;
    const int64_t kba = ((int64_t)p.k + kFinThreads - 1) / kFinThreads;
    const int rp_log2 = pl.rp == 16 ? 4 : pl.rp == 32 ? 5 : 6;
    hipLaunchKernelGGL(lora_finish_kernel, dim3((unsigned)(nbb + (int64_t)p.r * kba)), dim3(kFinThreads), 0, stream, p,
                       rp_log2, (int)nbb, (int)kba);
  }
  return hipGetLastError();
}

}  // namespace

int64_t lora_bwd_workspace_bytes(int64_t m, int64_t n, int64_t k, int64_t r) { return plan(m, n, k, r).bytes; }

hipError_t launch_lora_bwd(const uint16_t* dy, const uint16_t* x, const uint16_t* lb, const uint16_t* la, int64_t m,
                           int64_t n, int64_t k, int64_t r, void* workspace, void* d_b, void* d_a, bool out_f32,
                           int num_cu, hipStream_t stream) {
  const LoraPlan pl = plan(m, n, k, r);
  char* ws = static_cast<char*>(workspace);
  LoraBwdParams p;
  p.dy = dy;
  p.x = x;
  p.lb = lb;
  p.la = la;
  p.bt = reinterpret_cast<uint16_t*>(ws + pl.off_bt);
  p.pf = reinterpret_cast<u32x4*>(ws + pl.off_pf);
  p.qf = reinterpret_cast<u32x4*>(ws + pl.off_qf);
  p.part_b = reinterpret_cast<float*>(ws + pl.off_pb);
  p.part_a = reinterpret_cast<float*>(ws + pl.off_pa);
  p.d_b = d_b;
  p.d_a = d_a;
  p.m = m;
  p.n = (int)n;
  p.k = (int)k;
  p.r = (int)r;
  p.mb = pl.mb;
  p.slices = pl.slices;
  p.bps = pl.bps;
  p.out_f32 = out_f32 ? 1 : 0;
  if (pl.ct == 1) return launch_ct<1>(p, pl, num_cu, stream);
  if (pl.ct == 2) return launch_ct<2>(p, pl, num_cu, stream);
  return launch_ct<4>(p, pl, num_cu, stream);
}

}  // namespace fp8blk
