// Router scores over the whole expert pool (LongCat-Flash Technical Report
// notes, Key claims [§2.1, §2.4]): logits[t][e] = sum_h x[t][h] * w_router[e][h]
// with fp32 router weights and an fp32 result.
//
// bf16 activations (H % 64 == 0): matrix cores.  Each fp32 weight w is split
// exactly into three bf16 planes, w = hi + mid + lo (hi: w truncated to bf16,
// mid: the remainder truncated, lo: what is left; see split3).  x is bf16, so every product
// x*hi, x*mid, x*lo is exact in the fp32 accumulator of
// v_mfma_f32_16x16x32_bf16: three matrix-core passes give fp32-accurate
// scores at bf16 matrix-core rate instead of the fp32 vector rate.
//   block: 128 tokens x 64 experts; compute wave w owns experts [16w, 16w+16)
//   for all 128 tokens; K in 64-element stages; x tile (128 B rows, bf16) and
//   the raw fp32 weight tile (256 B rows) are filled by global_load_lds_dwordx4
//   from four loader waves into a 5-stage LDS ring; the split happens in
//   registers on the fragment read.  XCD-aware order: the 12 expert tiles of
//   one token tile run on one XCD.
// Large bf16 batches take 256 x 96 tiles (router_wide), and with weights split
// once beforehand (router_split) the same tiles read the planes instead of
// splitting (router_wide_planes): bitwise the same logits.
// bf16 activations with T <= 64 and H % 256 == 0 (decode): 16 experts x 16
// tokens per block, H split over the block's 8 waves (router_small below).
// fp32 activations (or H % 64 != 0, or x or the weights not 16-byte aligned):
// an LDS-tiled FMA kernel, 64 tokens x 64 experts per block, K step 16, a 4x4
// patch per thread.  Any T, E, H.
#include "moe_internal.h"

namespace moe {
namespace {

constexpr int kTM = 64, kTN = 64, kTK = 16, kThreads = 256;


template <typename TX>
__global__ __launch_bounds__(kThreads) void router_fma(const TX* __restrict__ x,
                                                       const float* __restrict__ w, int T, int H,
                                                       int E, float* __restrict__ logits) {
  __shared__ float As[kTK][kTM + 4];
  __shared__ float Bs[kTK][kTN + 4];
  const int m0 = blockIdx.y * kTM, n0 = blockIdx.x * kTN;
  const int tx = threadIdx.x % 16, ty = threadIdx.x / 16;
  // Each thread stages column kk = tid % kTK of rows tid / kTK + RS j of
  // both tiles at every K step; the next step's values are fetched into
  // registers while the current step is multiplied.
  constexpr int NL = kTM * kTK / kThreads, RS = kThreads / kTK;
  static_assert(kTM == kTN && kThreads % kTK == 0 && NL * kThreads == kTM * kTK,
                "tile elements split evenly over the threads");
  const int kk = threadIdx.x % kTK, r0 = threadIdx.x / kTK;
  float rx[NL], rw[NL];
  auto fetch = [&](int k0) {
    const bool kin = k0 + kk < H;
#pragma unroll
    for (int j = 0; j < NL; ++j) {
      const int r = r0 + RS * j;
      rx[j] = (m0 + r < T && kin) ? ld_f32(x + (size_t)(m0 + r) * H + k0 + kk) : 0.0f;
      rw[j] = (n0 + r < E && kin) ? w[(size_t)(n0 + r) * H + k0 + kk] : 0.0f;
    }
  };
  float acc[4][4] = {};
  fetch(0);
  for (int k0 = 0; k0 < H; k0 += kTK) {
#pragma unroll
    for (int j = 0; j < NL; ++j) {
      As[kk][r0 + RS * j] = rx[j];
      Bs[kk][r0 + RS * j] = rw[j];
    }
    __syncthreads();
    if (k0 + kTK < H) fetch(k0 + kTK);
#pragma unroll
    for (int k = 0; k < kTK; ++k) {
      float a[4], b[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        a[i] = As[k][ty * 4 + i];
        b[i] = Bs[k][tx * 4 + i];
      }
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = fmaf(a[i], b[j], acc[i][j]);
    }
    __syncthreads();
  }
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int t = m0 + ty * 4 + i, e = n0 + tx * 4 + j;
      if (t < T && e < E) logits[(size_t)t * E + e] = acc[i][j];
    }
}

// ----------------------------------------------------- matrix-core path --
constexpr int kRM = 128, kRN = 64, kRK = 64;
constexpr int kAStage = kRM * kRK * 2;          // 16 KB of x
constexpr int kBStage = kRN * kRK * 4;          // 16 KB of fp32 weights
constexpr int kRStageBytes = kAStage + kBStage;

typedef __attribute__((address_space(3))) void lds_void;

// x tile rows: 8 chunks of 16 B, XOR-swizzled by row & 7 as in the expert GEMM.
__device__ __forceinline__ int swz8(int row, int chunk) { return chunk ^ (row & 7); }
// weight tile rows: 16 chunks of 16 B (fp32), swizzled by the row's low 4 bits.
__device__ __forceinline__ int swz16(int row, int chunk) { return chunk ^ (row & 15); }

// Three bf16 planes of 8 fp32 weights, w = hi + mid + lo exactly, by
// truncation: hi is w with its low 16 bits cleared (w's top 8 significant
// bits, a bf16 value); r = w - hi is exact (at most 16 significant bits);
// mid is r with its low 16 bits cleared; lo = r - mid is exact with at most 8
// significant bits, so a bf16 value too (for |w| >= 2^-110; below that the
// remainders are subnormal and lo loses at most 2^-133 absolutely, as a
// round-to-nearest split would).  Each plane's bf16 bits are the high
// halves of w, r and lo, packed two per register with one byte permute --
// about 5.5 VALU operations per weight against 7.5 for round-to-nearest
// conversions (measured: the split is ~70 of the prefill router's 228 us).
__device__ __forceinline__ uint32_t high_halves(float a, float b) {
  // bytes 2-3 of a into bytes 0-1, bytes 2-3 of b into bytes 2-3
  return __builtin_amdgcn_perm(__float_as_uint(b), __float_as_uint(a), 0x07060302u);
}
__device__ __forceinline__ float clear_low16(float v) {
  return __uint_as_float(__float_as_uint(v) & 0xFFFF0000u);
}
__device__ __forceinline__ void split3(const f32x4& v0, const f32x4& v1, bf16x8& hi, bf16x8& mid,
                                       bf16x8& lo) {
  float w[8], r[8], l[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    w[i] = i < 4 ? v0[i] : v1[i - 4];
    r[i] = w[i] - clear_low16(w[i]);
    l[i] = r[i] - clear_low16(r[i]);
  }
  uint32_t h[4], m[4], o[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    h[j] = high_halves(w[2 * j], w[2 * j + 1]);
    m[j] = high_halves(r[2 * j], r[2 * j + 1]);
    o[j] = high_halves(l[2 * j], l[2 * j + 1]);
  }
  hi = __builtin_bit_cast(bf16x8, h);
  mid = __builtin_bit_cast(bf16x8, m);
  lo = __builtin_bit_cast(bf16x8, o);
}

// 8 waves per block: waves 4-7 only issue the global->LDS loads of each
// stage (x rows 8 per instruction, weight rows 4 per instruction), waves 0-3
// only read fragments, split the weights and issue MFMAs -- a stalled load
// issue then holds a loader, not a matrix core.  Every step issues the same
// loads (past the end they read one fixed line into a stage no one reads
// again), so every wait count is a constant.  The 12 expert tiles of one
// token tile run on one XCD and re-read its x rows from L2; they start their
// K sweeps at two offsets (by tile parity) so that they do not all wait on
// the same miss.  Two offsets measured 2-8 % faster than one per tile.
constexpr int kRThreads = 512;
constexpr int kRS = 5;                          // ring stages (160 KB)

__global__ __launch_bounds__(kRThreads, 1) void router_mfma(const bf16* __restrict__ x,
                                                            const float* __restrict__ w, int T,
                                                            int H, int E, int NTE,
                                                            float* __restrict__ logits) {
  __shared__ __attribute__((aligned(1024))) char smem[kRS * kRStageBytes];
  const int b = blockIdx.x;
  const int xcd = b & 7, slot = b >> 3;
  const int mt = (slot / NTE) * 8 + xcd;
  const int nt = slot % NTE;
  const int m0 = mt * kRM, n0 = nt * kRN;
  if (m0 >= T) return;
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int KT = H / kRK;
  const int k_start = ((nt & 1) * KT) / 2;   // two offsets (see above)

  if (wave >= 4) {
    const int l = wave - 4;
    const bf16* a_src[4];
    const float* b_src[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int ra = (l + 4 * q) * 8 + (lane >> 3);
      a_src[q] = x + (size_t)min(m0 + ra, T - 1) * H + swz8(ra, lane & 7) * 8;
      const int rb = (l + 4 * q) * 4 + (lane >> 4);
      b_src[q] = w + (size_t)min(n0 + rb, E - 1) * H + swz16(rb, lane & 15) * 4;
    }
    auto issue = [&](int kt) {
      char* sb = smem + (kt % kRS) * kRStageBytes;
      int ks = kt + k_start;
      ks = ks >= KT ? ks - KT : ks;
      const int k0 = kt < KT ? ks * kRK : 0;
#pragma unroll
      for (int q = 0; q < 4; ++q)
        __builtin_amdgcn_global_load_lds((const void*)(a_src[q] + k0),
                                         (lds_void*)(sb + (l + 4 * q) * 1024), 16, 0, 0);
#pragma unroll
      for (int q = 0; q < 4; ++q)
        __builtin_amdgcn_global_load_lds((const void*)(b_src[q] + k0),
                                         (lds_void*)(sb + kAStage + (l + 4 * q) * 1024), 16, 0,
                                         0);
    };
    for (int kt = 0; kt < kRS - 1; ++kt) issue(kt);
    for (int kt = 0; kt < KT; ++kt) {
      wait_vmcnt<8 * (kRS - 2)>();   // step kt has landed (in-order completion)
      lds_barrier();                 // publish it; every wave is done with step kt - 1
      issue(kt + kRS - 1);           // into the stage step kt - 1 used
    }
    wait_vmcnt<0>();
    lds_barrier();   // the LDS is free for the output tile
    lds_barrier();   // the tile is written
    return;
  }

  f32x4 acc[kRM / 16];
#pragma unroll
  for (int i = 0; i < kRM / 16; ++i) acc[i] = f32x4{0, 0, 0, 0};
  const int rB = 16 * wave + (lane & 15);
  for (int kt = 0; kt < KT; ++kt) {
    lds_barrier();
    const char* As = smem + (kt % kRS) * kRStageBytes;
    const char* Bs = As + kAStage;
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
      // this lane's 8 k values: k = 32kk + 8(lane/16) .. +8 -> fp32 chunks 2c, 2c+1
      const int c = kk * 8 + (lane >> 4) * 2;
      const f32x4 v0 = *(const f32x4*)(Bs + rB * 256 + swz16(rB, c) * 16);
      const f32x4 v1 = *(const f32x4*)(Bs + rB * 256 + swz16(rB, c + 1) * 16);
      bf16x8 bh, bm, bl;
      split3(v0, v1, bh, bm, bl);
      const int ch = kk * 4 + (lane >> 4);
#pragma unroll
      for (int rb = 0; rb < kRM / 16; ++rb) {
        const int rA = rb * 16 + (lane & 15);
        const bf16x8 a = *(const bf16x8*)(As + rA * 128 + swz8(rA, ch) * 16);
        acc[rb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, bl, acc[rb], 0, 0, 0);
        acc[rb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, bm, acc[rb], 0, 0, 0);
        acc[rb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, bh, acc[rb], 0, 0, 0);
      }
    }
  }
  // Output through LDS: [128 tokens][64 experts] fp32 (row pitch 272 B), then
  // 16 bytes per lane to logits -- whole 256 B row pieces per 16 lanes
  // instead of one 4-byte value per lane per store instruction.
  constexpr int kPitch = kRN * 4 + 16;
  static_assert(kRM * kPitch <= kRS * kRStageBytes, "output tile fits the ring");
  lds_barrier();   // loads landed, fragments read: the LDS is free
#pragma unroll
  for (int rb = 0; rb < kRM / 16; ++rb)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = rb * 16 + 4 * (lane >> 4) + i;
      *(float*)(smem + r * kPitch + (16 * wave + (lane & 15)) * 4) = acc[rb][i];
    }
  lds_barrier();   // the four compute waves' values are in the tile
  // whole 16-byte pieces: in range and 16-byte aligned
  const bool full = n0 + kRN <= E && (E & 3) == 0 && ((uintptr_t)logits & 15) == 0;
  for (int j = threadIdx.x; j < kRM * (kRN / 4); j += 256) {
    const int r = j / (kRN / 4), cq = j % (kRN / 4);
    if (m0 + r >= T) continue;
    const f32x4 v = *(const f32x4*)(smem + r * kPitch + cq * 16);
    float* dst = logits + (size_t)(m0 + r) * E + n0 + 4 * cq;
    if (full) {
      *(f32x4*)dst = v;
    } else {
#pragma unroll
      for (int u = 0; u < 4; ++u)
        if (n0 + 4 * cq + u < E) dst[u] = v[u];
    }
  }
}

// ------------------------------------------------ wide tiles (prefill) --
// Large batches: 256 tokens x 96 experts per block, K steps of 32.  The 128 x
// 64 tiles above move 32 KB from L2 into LDS per 3.1 MFLOP step, and that
// traffic, not the matrix cores, bounds them; a 256 x 96 tile moves 28 KB
// per 4.7 MFLOP step (1.7x fewer bytes per flop), and at 768 experts the
// 8192-token layer is exactly 256 blocks, one per CU.  A 64-element K step
// would leave room for only two 56 KB stages, so the step is 32: x rows are
// 64 B in LDS (4 chunks, swizzled by (row >> 1) & 3 so that any 8
// consecutive rows' chunk c land in 8 distinct 16-byte bank groups) and
// weight rows 128 B (8 chunks, swizzled by row & 7).  Compute wave (wr, wc)
// owns tokens [128 wr, +128) x experts [48 wc, +48): 8 x 3 16 x 16 blocks,
// and splits its 3 weight column blocks into the three bf16 planes per step.
// The loaders issue the weight halves of the fill before the x halves (the
// weights come from the last-level cache or HBM; x from L2), as the expert
// GEMM does.  Every compute and loader wave helps write the output tile.
constexpr int kWM = 256, kWN = 96, kWK = 32;
constexpr int kWAStage = kWM * kWK * 2;           // 16 KB of x
constexpr int kWBStage = kWN * kWK * 4;           // 12 KB of fp32 weights
constexpr int kWStageBytes = kWAStage + kWBStage;
constexpr int kWS = 5;                            // ring stages (140 KB)
constexpr int kWQa = kWAStage / 1024 / 4;         // x loads per loader per step (4)
constexpr int kWQb = kWBStage / 1024 / 4;         // weight loads per loader per step (3)
constexpr int kWQ = kWQa + kWQb;
constexpr int kWPitch = kWN * 4 + 16;             // output tile row pitch (bytes)
static_assert(kWM * kWPitch <= kWS * kWStageBytes, "output tile fits the ring");
static_assert((kWS - 2) * kWQ < 64, "vmcnt range");

__device__ __forceinline__ int swz4(int row, int chunk) { return chunk ^ ((row >> 1) & 3); }

// Ring steps 0..kWS-2 after the split fill: step kt's x loads have the fill's
// later x loads and kt whole steps behind them.
template <int KT0, class F>
__device__ __forceinline__ void wide_head(int KT, F& issue) {
  if constexpr (KT0 < kWS - 1) {
    if (KT0 >= KT) return;
    wait_vmcnt<(kWS - 2 - KT0) * kWQa + KT0 * kWQ>();
    lds_barrier();
    issue(KT0 + kWS - 1);
    wide_head<KT0 + 1>(KT, issue);
  }
}

__global__ __launch_bounds__(kRThreads, 1) void router_wide(const bf16* __restrict__ x,
                                                            const float* __restrict__ w, int T,
                                                            int H, int E, int NTE,
                                                            float* __restrict__ logits) {
  __shared__ __attribute__((aligned(1024))) char smem[kWS * kWStageBytes];
  const int b = blockIdx.x;
  const int xcd = b & 7, slot = b >> 3;
  const int mt = (slot / NTE) * 8 + xcd;   // the expert tiles of a token tile share an XCD
  const int nt = slot % NTE;
  const int m0 = mt * kWM, n0 = nt * kWN;
  if (m0 >= T) return;
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int KT = H / kWK;
  const int k_start = ((nt & 1) * KT) / 2;   // two K offsets by tile parity

  if (wave >= 4) {
    const int l = wave - 4;
    const bf16* a_src[kWQa];
    const float* b_src[kWQb];
    // instruction q of loader l covers x rows 16 (l + 4q) .. +16 (4 lanes a
    // row) and weight rows 8 (l + 4q) .. +8 (8 lanes a row); lane j's 16
    // bytes land at byte 16 j of the instruction's 1 KB.
#pragma unroll
    for (int q = 0; q < kWQa; ++q) {
      const int ra = (l + 4 * q) * 16 + (lane >> 2);
      a_src[q] = x + (size_t)min(m0 + ra, T - 1) * H + swz4(ra, lane & 3) * 8;
    }
#pragma unroll
    for (int q = 0; q < kWQb; ++q) {
      const int rb = (l + 4 * q) * 8 + (lane >> 3);
      b_src[q] = w + (size_t)min(n0 + rb, E - 1) * H + swz8(rb, lane & 7) * 4;
    }
    auto k_of = [&](int kt) {
      int ks = kt + k_start;
      ks = ks >= KT ? ks - KT : ks;
      return kt < KT ? ks * kWK : 0;
    };
    auto issue_a = [&](int kt) {
      char* sb = smem + (kt % kWS) * kWStageBytes;
      const int k0 = k_of(kt);
#pragma unroll
      for (int q = 0; q < kWQa; ++q)
        __builtin_amdgcn_global_load_lds((const void*)(a_src[q] + k0),
                                         (lds_void*)(sb + (l + 4 * q) * 1024), 16, 0, 0);
    };
    auto issue_b = [&](int kt) {
      char* sb = smem + (kt % kWS) * kWStageBytes;
      const int k0 = k_of(kt);
#pragma unroll
      for (int q = 0; q < kWQb; ++q)
        __builtin_amdgcn_global_load_lds((const void*)(b_src[q] + k0),
                                         (lds_void*)(sb + kWAStage + (l + 4 * q) * 1024), 16, 0,
                                         0);
    };
    auto issue = [&](int kt) {
      issue_a(kt);
      issue_b(kt);
    };
    for (int kt = 0; kt < kWS - 1; ++kt) issue_b(kt);
    for (int kt = 0; kt < kWS - 1; ++kt) issue_a(kt);
    wide_head<0>(KT, issue);
    for (int kt = kWS - 1; kt < KT; ++kt) {
      wait_vmcnt<(kWS - 2) * kWQ>();   // step kt has landed (in-order completion)
      lds_barrier();                   // publish it; every wave is done with step kt - 1
      issue(kt + kWS - 1);             // into the stage step kt - 1 used
    }
    wait_vmcnt<0>();
    lds_barrier();   // the LDS is free for the output tile
  } else {
    const int wr = wave >> 1, wc = wave & 1;
    f32x4 acc[8][3];
#pragma unroll
    for (int rb = 0; rb < 8; ++rb)
#pragma unroll
      for (int cb = 0; cb < 3; ++cb) acc[rb][cb] = f32x4{0, 0, 0, 0};
    for (int kt = 0; kt < KT; ++kt) {
      lds_barrier();
      const char* As = smem + (kt % kWS) * kWStageBytes;
      const char* Bs = As + kWAStage;
      // lane l: k elements 8 (l >> 4) .. + 8 of the step = x chunk l >> 4,
      // fp32 weight chunks 2 (l >> 4) and 2 (l >> 4) + 1
      const int c = lane >> 4;
      bf16x8 bh[3], bm[3], bl[3];
#pragma unroll
      for (int cb = 0; cb < 3; ++cb) {
        const int rB = 48 * wc + 16 * cb + (lane & 15);
        const f32x4 v0 = *(const f32x4*)(Bs + rB * 128 + swz8(rB, 2 * c) * 16);
        const f32x4 v1 = *(const f32x4*)(Bs + rB * 128 + swz8(rB, 2 * c + 1) * 16);
        split3(v0, v1, bh[cb], bm[cb], bl[cb]);
      }
#pragma unroll
      for (int rb = 0; rb < 8; ++rb) {
        const int rA = 128 * wr + 16 * rb + (lane & 15);
        const bf16x8 a = *(const bf16x8*)(As + rA * 64 + swz4(rA, c) * 16);
#pragma unroll
        for (int cb = 0; cb < 3; ++cb) {
          acc[rb][cb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, bl[cb], acc[rb][cb], 0, 0, 0);
          acc[rb][cb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, bm[cb], acc[rb][cb], 0, 0, 0);
          acc[rb][cb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, bh[cb], acc[rb][cb], 0, 0, 0);
        }
      }
    }
    lds_barrier();   // loads landed, fragments read: the LDS is free
    // acc[rb][cb] element i: token 128 wr + 16 rb + 4 (l >> 4) + i,
    // expert 48 wc + 16 cb + (l & 15)
#pragma unroll
    for (int rb = 0; rb < 8; ++rb)
#pragma unroll
      for (int cb = 0; cb < 3; ++cb)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int r = 128 * wr + 16 * rb + 4 * (lane >> 4) + i;
          *(float*)(smem + r * kWPitch + (48 * wc + 16 * cb + (lane & 15)) * 4) = acc[rb][cb][i];
        }
  }
  lds_barrier();   // the output tile is complete
  // all 8 waves store it, 16 bytes per lane, whole 16-byte pieces when the
  // tile is in range and aligned
  const bool full = n0 + kWN <= E && (E & 3) == 0 && ((uintptr_t)logits & 15) == 0;
  constexpr int kQuads = kWN / 4;
  for (int j = threadIdx.x; j < kWM * kQuads; j += kRThreads) {
    const int r = j / kQuads, cq = j - r * kQuads;
    if (m0 + r >= T) continue;
    const f32x4 v = *(const f32x4*)(smem + r * kWPitch + cq * 16);
    float* dst = logits + (size_t)(m0 + r) * E + n0 + 4 * cq;
    if (full) {
      *(f32x4*)dst = v;
    } else {
#pragma unroll
      for (int u = 0; u < 4; ++u)
        if (n0 + 4 * cq + u < E) dst[u] = v[u];
    }
  }
}

// ------------------------------------- wide tiles on pre-split weights --
// The same tiles and the same matrix-core operations in the same order as
// router_wide, on weights split once into their three bf16 planes
// (router_split below: planes[p][e][h], p = hi, mid, lo), so that the
// compute waves only read fragments and multiply.  A stage is 16 KB of x and
// 18 KB of planes (288 plane rows of 64 B, swizzled like the x rows); four
// stages fit.  Loader waves 4-5 stream x (8 loads a step each), waves 6-7 the
// planes (9 each): each loader waits only on its own loads, so the two
// operands need no split fill.  Measured on the 8192-token layer: 233 -> 189
// us (16384 tokens: 441 -> 359 us).
constexpr int kPBStage = 3 * kWN * kWK * 2;       // 18 KB of planes
constexpr int kPStageBytes = kWAStage + kPBStage;
constexpr int kPS = 4;                            // ring stages (136 KB)
constexpr int kPQa = kWAStage / 1024 / 2;         // x loads per x loader per step (8)
constexpr int kPQb = kPBStage / 1024 / 2;         // plane loads per plane loader per step (9)
static_assert(kWM * kWPitch <= kPS * kPStageBytes, "output tile fits the ring");
static_assert((kPS - 2) * kPQb < 64, "vmcnt range");

template <int Q, class F>
__device__ __forceinline__ void planes_loader(int KT, F& issue) {
  for (int kt = 0; kt < kPS - 1; ++kt) issue(kt);
  for (int kt = 0; kt < KT; ++kt) {
    wait_vmcnt<(kPS - 2) * Q>();   // step kt has landed (in-order completion)
    lds_barrier();                 // publish it; every wave is done with step kt - 1
    issue(kt + kPS - 1);           // into the stage step kt - 1 used
  }
  wait_vmcnt<0>();
  lds_barrier();   // the LDS is free for the output tile
}

// Compute waves.  Eight (two per SIMD, 64 tokens x 48 experts each, so that
// one wave's fragment reads overlap the other's matrix-core work) measured
// the same as four: 190 vs 189 us on the 8192-token layer.
constexpr int kPCW = 4;
constexpr int kPThreads = (kPCW + 4) * kWave;
constexpr int kPRows = kWM / (kPCW / 2);           // tokens per compute wave
__global__ __launch_bounds__(kPThreads, 1) void router_wide_planes(
    const bf16* __restrict__ x, const bf16* __restrict__ planes, int T, int H, int E, int NTE,
    float* __restrict__ logits) {
  __shared__ __attribute__((aligned(1024))) char smem[kPS * kPStageBytes];
  const int b = blockIdx.x;
  const int xcd = b & 7, slot = b >> 3;
  const int mt = (slot / NTE) * 8 + xcd;   // the expert tiles of a token tile share an XCD
  const int nt = slot % NTE;
  const int m0 = mt * kWM, n0 = nt * kWN;
  if (m0 >= T) return;
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int KT = H / kWK;
  const int k_start = ((nt & 1) * KT) / 2;   // two K offsets by tile parity
  auto k_of = [&](int kt) {
    int ks = kt + k_start;
    ks = ks >= KT ? ks - KT : ks;
    return kt < KT ? ks * kWK : 0;
  };

  if (wave >= kPCW + 2) {
    // instruction q of plane loader l covers plane rows 16 (l + 2q) .. +16
    // (4 lanes a row; 96 rows a plane, so one plane per instruction)
    const int l = wave - kPCW - 2;
    const bf16* src[kPQb];
#pragma unroll
    for (int q = 0; q < kPQb; ++q) {
      const int pr = (l + 2 * q) * 16 + (lane >> 2);
      const int p = pr / kWN, r = pr - p * kWN;
      src[q] = planes + ((size_t)p * E + min(n0 + r, E - 1)) * H + swz4(pr, lane & 3) * 8;
    }
    auto issue = [&](int kt) {
      char* sb = smem + (kt % kPS) * kPStageBytes + kWAStage;
      const int k0 = k_of(kt);
#pragma unroll
      for (int q = 0; q < kPQb; ++q)
        __builtin_amdgcn_global_load_lds((const void*)(src[q] + k0),
                                         (lds_void*)(sb + (l + 2 * q) * 1024), 16, 0, 0);
    };
    planes_loader<kPQb>(KT, issue);
  } else if (wave >= kPCW) {
    // instruction q of x loader l covers x rows 16 (l + 2q) .. +16
    const int l = wave - kPCW;
    const bf16* src[kPQa];
#pragma unroll
    for (int q = 0; q < kPQa; ++q) {
      const int ra = (l + 2 * q) * 16 + (lane >> 2);
      src[q] = x + (size_t)min(m0 + ra, T - 1) * H + swz4(ra, lane & 3) * 8;
    }
    auto issue = [&](int kt) {
      char* sb = smem + (kt % kPS) * kPStageBytes;
      const int k0 = k_of(kt);
#pragma unroll
      for (int q = 0; q < kPQa; ++q)
        __builtin_amdgcn_global_load_lds((const void*)(src[q] + k0),
                                         (lds_void*)(sb + (l + 2 * q) * 1024), 16, 0, 0);
    };
    planes_loader<kPQa>(KT, issue);
  } else {
    constexpr int RB = kPRows / 16;
    const int wr = wave >> 1, wc = wave & 1;
    f32x4 acc[RB][3];
#pragma unroll
    for (int rb = 0; rb < RB; ++rb)
#pragma unroll
      for (int cb = 0; cb < 3; ++cb) acc[rb][cb] = f32x4{0, 0, 0, 0};
    for (int kt = 0; kt < KT; ++kt) {
      lds_barrier();
      const char* As = smem + (kt % kPS) * kPStageBytes;
      const char* Bs = As + kWAStage;
      const int c = lane >> 4;   // k elements 8c .. 8c + 8 of the step
      bf16x8 bp[3][3];           // [plane][column block]
#pragma unroll
      for (int p = 0; p < 3; ++p)
#pragma unroll
        for (int cb = 0; cb < 3; ++cb) {
          const int pr = p * kWN + 48 * wc + 16 * cb + (lane & 15);
          bp[p][cb] = *(const bf16x8*)(Bs + pr * 64 + swz4(pr, c) * 16);
        }
#pragma unroll
      for (int rb = 0; rb < RB; ++rb) {
        const int rA = kPRows * wr + 16 * rb + (lane & 15);
        const bf16x8 a = *(const bf16x8*)(As + rA * 64 + swz4(rA, c) * 16);
#pragma unroll
        for (int cb = 0; cb < 3; ++cb) {
          acc[rb][cb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, bp[2][cb], acc[rb][cb], 0, 0, 0);
          acc[rb][cb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, bp[1][cb], acc[rb][cb], 0, 0, 0);
          acc[rb][cb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, bp[0][cb], acc[rb][cb], 0, 0, 0);
        }
      }
    }
    lds_barrier();   // loads landed, fragments read: the LDS is free
#pragma unroll
    for (int rb = 0; rb < RB; ++rb)
#pragma unroll
      for (int cb = 0; cb < 3; ++cb)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int r = kPRows * wr + 16 * rb + 4 * (lane >> 4) + i;
          *(float*)(smem + r * kWPitch + (48 * wc + 16 * cb + (lane & 15)) * 4) = acc[rb][cb][i];
        }
  }
  lds_barrier();   // the output tile is complete
  const bool full = n0 + kWN <= E && (E & 3) == 0 && ((uintptr_t)logits & 15) == 0;
  constexpr int kQuads = kWN / 4;
  for (int j = threadIdx.x; j < kWM * kQuads; j += kPThreads) {
    const int r = j / kQuads, cq = j - r * kQuads;
    if (m0 + r >= T) continue;
    const f32x4 v = *(const f32x4*)(smem + r * kWPitch + cq * 16);
    float* dst = logits + (size_t)(m0 + r) * E + n0 + 4 * cq;
    if (full) {
      *(f32x4*)dst = v;
    } else {
#pragma unroll
      for (int u = 0; u < 4; ++u)
        if (n0 + 4 * cq + u < E) dst[u] = v[u];
    }
  }
}

// planes[p][e][h] (p = hi, mid, lo) of the fp32 router weights, split3 of
// every 8 consecutive weights of a row (H % 8 == 0).
__global__ __launch_bounds__(256) void router_split(const float* __restrict__ w, long long n8,
                                                    long long plane, bf16* __restrict__ planes) {
  const long long i = (long long)blockIdx.x * 256 + threadIdx.x;
  if (i >= n8) return;
  const f32x4 v0 = *(const f32x4*)(w + 8 * i);
  const f32x4 v1 = *(const f32x4*)(w + 8 * i + 4);
  bf16x8 hi, mid, lo;
  split3(v0, v1, hi, mid, lo);
  *(bf16x8*)(planes + 8 * i) = hi;
  *(bf16x8*)(planes + plane + 8 * i) = mid;
  *(bf16x8*)(planes + 2 * plane + 8 * i) = lo;
}

// ------------------------------------------------- few tokens (decode) --
// With T <= 64 the 128 x 64 tiles above leave a dozen blocks for the whole
// chip, each streaming 64 experts' weights over all of H.  Here a block takes
// 16 experts and all T tokens, and its 8 waves split H into 8 ranges.  Each
// wave loads its fragments straight from global memory (nothing is reused
// inside the block), splits the weights into the three bf16 planes and
// accumulates; the 8 partial tiles are then added through LDS in wave order,
// a fixed order, so the result is bitwise reproducible.
constexpr int kSmallT = 64;       // the most tokens this kernel takes
constexpr int kSmallTB = 16;      // tokens per block (one MFMA row block)
constexpr int kSmallN = 16;       // experts per block
constexpr int kSmallWaves = 8;    // K ranges
constexpr int kSmallU = 4;        // 32-element k slices in flight per wave

// Block = 16 experts x 16 tokens; its 8 waves each own one eighth of H, and
// their partial tiles are added through LDS in a fixed order.  The token
// groups of one expert tile run on one XCD (blockIdx mod 8), so the
// weights are fetched from HBM once and re-read from L2.  At 64 tokens x
// 768 experts that is 192 blocks; one block per 16 experts (all 64 tokens,
// 48 blocks) left most CUs idle: 38 -> 21 us.  Sixteen waves per block
// (half the K range each) measured slower (22.7 vs 20.5 us).
__global__ __launch_bounds__(kSmallWaves * kWave) void router_small(const bf16* __restrict__ x,
                                                                    const float* __restrict__ w,
                                                                    int T, int H, int E, int NTE,
                                                                    int NQ,
                                                                    float* __restrict__ logits) {
  __shared__ float part[kSmallWaves][kSmallTB][kSmallN];
  const int b = blockIdx.x;
  const int xcd = b & 7, slot = b >> 3;
  const int tq = slot % NQ, nt = (slot / NQ) * 8 + xcd;
  if (nt >= NTE) return;
  const int n0 = nt * kSmallN, t0 = tq * kSmallTB;
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = threadIdx.x / kWave;
  const int kr = H / kSmallWaves;   // a multiple of 32 (H % 256 == 0)
  const int kbeg = wave * kr;
  // v_mfma_f32_16x16x32_bf16 fragments: lane l holds row / column l & 15 and
  // k elements 8 (l >> 4) .. + 8 of a 32-element slice.  Tokens past T and
  // experts past E are clamped and their results dropped.
  const float* wrow = w + (size_t)min(n0 + (lane & 15), E - 1) * H + kbeg + 8 * (lane >> 4);
  const bf16* xrow = x + (size_t)min(t0 + (lane & 15), T - 1) * H + kbeg + 8 * (lane >> 4);
  f32x4 acc = f32x4{0, 0, 0, 0};
  for (int k = 0; k < kr; k += 32 * kSmallU) {
    f32x4 w0[kSmallU], w1[kSmallU];
    bf16x8 xa[kSmallU];
#pragma unroll
    for (int u = 0; u < kSmallU; ++u) {
      const int kk = min(k + 32 * u, kr - 32);   // past the range: a valid slice, not used
      w0[u] = *(const f32x4*)(wrow + kk);
      w1[u] = *(const f32x4*)(wrow + kk + 4);
      xa[u] = *(const bf16x8*)(xrow + kk);
    }
#pragma unroll
    for (int u = 0; u < kSmallU; ++u) {
      if (k + 32 * u >= kr) break;   // wave-uniform
      bf16x8 bh, bm, bl;
      split3(w0[u], w1[u], bh, bm, bl);
      acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(xa[u], bl, acc, 0, 0, 0);
      acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(xa[u], bm, acc, 0, 0, 0);
      acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(xa[u], bh, acc, 0, 0, 0);
    }
  }
  // acc element i: token t0 + 4 (l >> 4) + i, expert n0 + (l & 15)
#pragma unroll
  for (int i = 0; i < 4; ++i) part[wave][4 * (lane >> 4) + i][lane & 15] = acc[i];
  __syncthreads();
  for (int j = threadIdx.x; j < kSmallTB * kSmallN; j += kSmallWaves * kWave) {
    const int t = j / kSmallN, c = j % kSmallN;
    float sum = 0.0f;
#pragma unroll
    for (int v = 0; v < kSmallWaves; ++v) sum += part[v][t][c];
    if (t0 + t < T && n0 + c < E) logits[(size_t)(t0 + t) * E + n0 + c] = sum;
  }
}

}  // namespace

hipError_t launch_router_split(const float* w, int E, int H, void* planes, hipStream_t s) {
  const long long n8 = (long long)E * H / 8;
  MOE_LAUNCH("router_split", s,
             router_split<<<(unsigned)ceil_div(n8, 256), 256, 0, s>>>(w, n8, (long long)E * H,
                                                                      (bf16*)planes));
  return hipGetLastError();
}

hipError_t launch_router_logits(const void* x, int dtype, const float* w, const void* planes,
                                int T, int H, int E, float* logits, hipStream_t s) {
  // the matrix-core kernels move x and the weights in 16-byte pieces; other
  // alignments (the API takes element-aligned pointers) go to the FMA kernel
  const bool mfma = dtype == MOE_BF16 && (((uintptr_t)x | (uintptr_t)w) & 15) == 0;
  if (mfma && T <= kSmallT && H % (kSmallWaves * 32) == 0) {
    const int nte = ceil_div(E, kSmallN), nq = ceil_div(T, kSmallTB);
    MOE_LAUNCH("router_logits", s,
               router_small<<<8 * nq * ceil_div(nte, 8), kSmallWaves * kWave, 0, s>>>(
                   (const bf16*)x, w, T, H, E, nte, nq, logits));
    return hipGetLastError();
  }
  if (mfma && H % kWK == 0 &&
      (long long)ceil_div(T, kWM) * ceil_div(E, kWN) >= 256) {   // enough wide tiles for every CU
    const int nte = (E + kWN - 1) / kWN;
    const unsigned groups = ceil_div(ceil_div(T, kWM), 8);
    if (planes) {
      MOE_LAUNCH("router_logits", s,
                 router_wide_planes<<<groups * 8 * nte, kPThreads, 0, s>>>(
                     (const bf16*)x, (const bf16*)planes, T, H, E, nte, logits));
      return hipGetLastError();
    }
    MOE_LAUNCH("router_logits", s,
               router_wide<<<groups * 8 * nte, kRThreads, 0, s>>>((const bf16*)x, w, T, H, E,
                                                                  nte, logits));
    return hipGetLastError();
  }
  if (mfma && H % kRK == 0) {
    const int nte = (E + kRN - 1) / kRN;
    const unsigned groups = ceil_div(ceil_div(T, kRM), 8);
    MOE_LAUNCH("router_logits", s,
               router_mfma<<<groups * 8 * nte, kRThreads, 0, s>>>((const bf16*)x, w, T, H, E,
                                                                  nte, logits));
    return hipGetLastError();
  }
  dim3 grid(ceil_div(E, kTN), ceil_div(T, kTM));
  if (dtype == MOE_BF16)
    MOE_LAUNCH("router_logits", s,
               router_fma<bf16><<<grid, kThreads, 0, s>>>((const bf16*)x, w, T, H, E, logits));
  else
    MOE_LAUNCH("router_logits", s,
               router_fma<float><<<grid, kThreads, 0, s>>>((const float*)x, w, T, H, E, logits));
  return hipGetLastError();
}

}  // namespace moe
