// FFN experts on expert-grouped rows (LongCat-Flash Technical Report notes,
// Key claims [§2.4]: fine-grained FFN experts, intermediate 2048 at hidden
// 6144; SwiGLU form):
//   hh = silu(X W_g^T) * (X W_u^T),  Y = hh W_d^T,  per expert, empty experts skipped.
//
// Work list.  A small kernel turns offsets[] into m-tiles (expert, first row,
// rows <= BM); the GEMM grids are sized on the host from the capacity bound
// (rows_cap / BM + n_ffn m-tiles) and blocks past the real count exit.
//
// bf16 path (gfx950 matrix cores, v_mfma_f32_16x16x32_bf16, fp32 accumulate):
//   - one block = one m-tile (all of the expert's rows, up to BM) x BN rows
//     of the weight matrix, so every weight tile is fetched from HBM once when
//     an expert's rows fit one m-tile -- the regime of the full-scale layer,
//     where the weights (not the MFMA rate) bound the time.  BN = 128, or,
//     chosen per block, 256 (gate/up, partial tiles of 2-5 row groups) and
//     192 (down, 2-7 groups): the activation rows every column tile re-reads
//     from L2 then cost less per weight byte (see launch_expert_ffn);
//   - wave w owns BN / 4 weight rows (16-column MFMA blocks) and every row
//     block of the m-tile; 32-row groups past the expert's rows are skipped;
//   - 8 waves: four compute waves (fragment reads + MFMA only) and four
//     loader waves that stream 64-element K steps by global->LDS DMA into a
//     ring of 3 to 8 steps;
//   - LDS rows are 128 B with the 16-byte chunks XOR-swizzled by row & 7 so
//     that the fragment reads (16 rows x one chunk per 16 lanes) are free of
//     bank conflicts: timed on gfx950 they run as fast as linear
//     ds_read_b128 (an unswizzled layout is 2.4x slower);
//   - gate/up: weight rows are paired so that a lane holds gate column j and
//     up column j in the same accumulator slot, and silu(g)*u is applied in
//     registers before hh is stored (bf16);
//   - a block's fill issues the weight halves of its first steps before the
//     activation halves (HBM latency first; ~1 % per GEMM, measured);
//   - gate/up can read its activation rows straight from x through row_src
//     (the row gather): the DMA takes any 16-byte-aligned row address, so
//     the dispatch copy into x_perm is not needed;
//   - the output tile is staged in LDS and stored 16 bytes per lane (whole
//     128-byte lines), not one 2-byte value per lane per instruction;
//   - block -> tile order is XCD-aware: consecutive blocks land on the 8 XCDs
//     in turn, so all column tiles of one m-tile run on one XCD and re-read
//     the m-tile's activation rows from that XCD's L2; the column tiles start
//     their K sweeps at a few different offsets, so that those re-reads are L2
//     hits rather than 32 simultaneous waits on one miss.
#include "moe_internal.h"

namespace moe {
namespace {

constexpr int kThreads = 256;        // fp32 path and the small kernels
constexpr int kGemmThreads = 512;    // bf16 GEMM: 4 compute + 4 loader waves
constexpr int kBK = 64;                 // k elements per pipeline step
constexpr int kRowBytes = kBK * 2;      // 128 B per LDS row of a step
constexpr int kBN = 128;                // weight rows per block (the narrow tiles)
constexpr int kBNWide = 192;            // down: wide tiles
constexpr int kWideGroups = 0x0FC;      // bits 2..7: the down GEMM's 192-row tiles
constexpr int kBNGateUpWide = 256;      // gate/up: 128 hh columns per tile
constexpr int kWideGroupsGateUp = 0x03C;   // bits 2..5: 256-row tiles (a 3-stage ring fits)
constexpr int kBmBf16 = 256;
constexpr int kBmF32 = 32;

// Chunk swizzle of a 128 B LDS row: 16 lanes reading one 16-byte chunk of 16
// consecutive rows (the MFMA fragment read) hit distinct banks.
__device__ __forceinline__ int swz(int row, int chunk) { return chunk ^ (row & 7); }

// ------------------------------------------------------------ work list --
// Rows are clamped to [0, rows_cap) and the list to max_tiles entries, so a
// malformed offsets[] can shrink the work but never index past the buffers.
__global__ __launch_bounds__(1024) void ffn_tiles(const int32_t* __restrict__ offsets, int n_ffn,
                                                  int bm, int rows_cap, int max_tiles,
                                                  int4* __restrict__ tiles,
                                                  int* __restrict__ ntiles) {
  __shared__ int part[1024];
  const int tid = threadIdx.x;
  const int per = (n_ffn + 1023) / 1024;
  const int lo = min(n_ffn, tid * per), hi = min(n_ffn, lo + per);
  auto span = [&](int e, int& r0, int& m) {
    r0 = min(max(offsets[e], 0), rows_cap);
    m = min(max(offsets[e + 1], r0), rows_cap) - r0;
  };
  int s = 0;
  for (int e = lo; e < hi; ++e) {
    int r0, m;
    span(e, r0, m);
    s += (m + bm - 1) / bm;
  }
  part[tid] = s;
  __syncthreads();
  for (int off = 1; off < 1024; off <<= 1) {
    int v = tid >= off ? part[tid - off] : 0;
    __syncthreads();
    part[tid] += v;
    __syncthreads();
  }
  int pos = part[tid] - s;
  for (int e = lo; e < hi; ++e) {
    int r0, m;
    span(e, r0, m);
    for (int j = 0; j * bm < m && pos < max_tiles; ++j)
      tiles[pos++] = make_int4(e, r0 + j * bm, min(bm, m - j * bm), 0);
  }
  if (tid == 1023) *ntiles = min(part[1023], max_tiles);
}

// -------------------------------------------------------- bf16 MFMA GEMM --
// GATEUP: A = x_perm [.][H], W = w13 [N][2I][H], C = hh [.][I]   (KD = H, NT = I/64)
// down  : A = hh     [.][I], W = w2  [N][H][I],  C = y_perm [.][H] (KD = I, NT = H/128)
constexpr int kLdsBytes = 160 * 1024;

// Producer/consumer pipeline, 8 waves (2 per SIMD).
//   - Waves 4-7 (loaders) only issue loads: global_load_lds_dwordx4, 1 KB
//     (8 rows x 128 B) per instruction straight into an LDS ring of S steps,
//     as deep as the 160 KB allow (8 steps at G = 1 down to 3 at G = 8).
//   - Waves 0-3 (compute) only read fragments from LDS and issue MFMAs.
// One barrier per step joins all eight.  Under load a 1 KB vector-memory
// instruction occupies the wave that issues it for ~40-70 cycles; with the
// roles split those stalls fall on a loader, and the compute wave sharing its
// SIMD keeps the matrix core busy.  Writing LDS by DMA (rather than through
// VGPRs and ds_write) keeps the loader's per-step work to issuing loads.
typedef __attribute__((address_space(3))) void lds_void;
constexpr int kCachePolicyNT = 2;   // non-temporal: weights are streamed once

template <int G, int BN = kBN>
struct Ring {
  static constexpr int kABytes = 32 * G * kRowBytes;   // A tile of one step
  static constexpr int kStageBytes = kABytes + BN * kRowBytes;
  static constexpr int kQa = G;                        // A loads per loader per step
  static constexpr int kQb = BN / 8 / 4;               // B loads per loader per step (4 or 6)
  static constexpr int kQ = kQa + kQb;
  static constexpr int kFit = kLdsBytes / kStageBytes;
  static constexpr int S = kFit > 8 ? 8 : kFit;
  static_assert(S >= 3, "three steps in the ring");
  static_assert((S - 2) * kQ < 64, "vmcnt range");
};

struct TileSrc {
  const bf16* a_rows;   // the m-tile's activation rows (see a_pitch / a_step)
  const int32_t* gather;   // non-null: row r of the tile is row gather[r] / gK of a_rows
  int gK, gT;              // (clamped to [0, gT)), i.e. a token row of x
  int rows;             // live rows of the m-tile
  const bf16* w;        // this expert's weight matrix (row stride KD)
  int nt, I;            // column tile, intermediate size (gate/up pairing)
  bool gateup;
  int a_pitch;          // elements between activation rows
  int a_step;           // elements between K steps of one row block
};

// Weight row held in row r (0..BN-1) of the block's weight tile.  Gate/up:
// rows 32p + [0,16) are gate rows j, 32p + [16,32) the up rows of the same j
// (BN / 2 hh columns per tile), so that one lane ends up with gate column j
// and up column j.
template <int BN>
__device__ __forceinline__ int weight_row(const TileSrc& t, int r) {
  if (t.gateup) {
    const int j = t.nt * (BN / 2) + 16 * (r >> 5) + (r & 15);
    return (r & 16) ? t.I + j : j;
  }
  return t.nt * BN + r;
}

// Steps 0..S-2 of the loader's sweep, after the split fill: step kt's
// activation loads have the fill's later activation loads (S - 2 - kt steps
// of QA) and kt whole steps (Q each) behind them.  From step S - 1 on, S - 2
// whole steps are.
template <int S, int QA, int Q, int KT0, class F>
__device__ __forceinline__ void ring_head(int KT, F& issue) {
  if constexpr (KT0 < S - 1) {
    if (KT0 >= KT) return;
    wait_vmcnt<(S - 2 - KT0) * QA + KT0 * Q>();
    lds_barrier();
    issue(KT0 + S - 1);
    ring_head<S, QA, Q, KT0 + 1>(KT, issue);
  }
}

// Loader l (0..3) moves 8-row groups l, l+4, ... of both tiles; lane j of an
// instruction fetches the 16-byte chunk that lands at byte 16 j of the group,
// i.e. chunk swz(row, j & 7) of row 8 g + (j >> 3).  Every step issues the
// same loads -- past the end they read one fixed line into a stage no one
// reads again -- so every wait count is a constant.  The sweep starts at
// k_start and wraps around.
template <int G, bool GATHER, int BN>
__device__ __forceinline__ void ffn_loader(char* smem, const TileSrc& t, int KD, int k_start,
                                           int l, int lane) {
  using R = Ring<G, BN>;
  constexpr int S = R::S, kQ = R::kQ;
  const int KT = KD / kBK;
  const int lr = lane >> 3, lc = lane & 7;
  const bf16* src[kQ];
  // Row gather.  Loader l's lanes need the indices of 8 G rows, 8 per group.
  //   G <= 4: the rows of a group are wave-uniform, so the indices come in by
  //     scalar loads (32 scalar registers at most), waited on with lgkmcnt
  //     apart from the DMA's vmcnt, and each lane selects its row's only
  //     after the fill's weight loads are out: the index latency hides behind
  //     them.  A per-lane vector load would be ordered with the DMA, and the
  //     compiler would drain every DMA before its first use.
  //   G > 4: too many registers for that; one vector load per lane (lane j:
  //     group j / 8, row j % 8) is waited on before any DMA is issued and
  //     shuffled to the lanes that need it -- one round trip per block.
  constexpr bool kScalarIdx = R::kQa <= 4;
  int tok[R::kQa];
  int raw[kScalarIdx ? R::kQa : 1][8];
  if constexpr (GATHER && kScalarIdx) {
#pragma unroll
    for (int i = 0; i < R::kQa; ++i)
#pragma unroll
      for (int j = 0; j < 8; ++j) raw[i][j] = t.gather[min((l + 4 * i) * 8 + j, t.rows - 1)];
  }
  if constexpr (GATHER && !kScalarIdx) {
    const int gi = min(lane >> 3, R::kQa - 1);
    const int v = t.gather[min((l + 4 * gi) * 8 + (lane & 7), t.rows - 1)];
#pragma unroll
    for (int i = 0; i < R::kQa; ++i) tok[i] = __shfl(v, i * 8 + lr);
    __builtin_amdgcn_sched_barrier(0);   // no DMA may be moved above that wait
  }
#pragma unroll
  for (int i = 0; i < R::kQb; ++i) {
    const int r = (l + 4 * i) * 8 + lr;
    src[R::kQa + i] = t.w + (size_t)weight_row<BN>(t, r) * KD + swz(r, lc) * 8;
  }
  auto stage = [&](int kt) { return smem + (kt % S) * R::kStageBytes; };
  auto k_of = [&](int kt) { const int ks = kt + k_start; return ks >= KT ? ks - KT : ks; };
  auto issue_a = [&](int kt) {
    const bool real = kt < KT;
    const size_t ka = real ? (size_t)k_of(kt) * t.a_step : 0;
#pragma unroll
    for (int i = 0; i < R::kQa; ++i)
      __builtin_amdgcn_global_load_lds((const void*)(real ? src[i] + ka : t.w),
                                       (lds_void*)(stage(kt) + (l + 4 * i) * 1024), 16, 0, 0);
  };
  auto issue_b = [&](int kt) {
    const bool real = kt < KT;
    const int k0 = real ? k_of(kt) * kBK : 0;
#pragma unroll
    for (int i = 0; i < R::kQb; ++i)
      __builtin_amdgcn_global_load_lds((const void*)(real ? src[R::kQa + i] + k0 : t.w),
                                       (lds_void*)(stage(kt) + R::kABytes + (l + 4 * i) * 1024),
                                       16, 0, kCachePolicyNT);
  };
  auto issue = [&](int kt) {
    issue_a(kt);
    issue_b(kt);
  };
  // Fill: the weight halves of the first S - 1 steps go out first (HBM, the
  // longest wait), then their activation halves, whose addresses may still be
  // waiting on the row-gather index loads.
  for (int kt = 0; kt < S - 1; ++kt) issue_b(kt);
  if constexpr (GATHER && kScalarIdx) {
#pragma unroll
    for (int i = 0; i < R::kQa; ++i) {
      int v = raw[i][0];
#pragma unroll
      for (int j = 1; j < 8; ++j) v = lr == j ? raw[i][j] : v;
      tok[i] = v;
    }
  }
#pragma unroll
  for (int i = 0; i < R::kQa; ++i) {
    const int r = (l + 4 * i) * 8 + lr;        // rows past the tile: clamped (never used)
    const int ar = GATHER ? min(max(tok[i], 0) / t.gK, t.gT - 1) : min(r, t.rows - 1);
    src[i] = t.a_rows + (size_t)ar * t.a_pitch + swz(r, lc) * 8;
  }
  for (int kt = 0; kt < S - 1; ++kt) issue_a(kt);
  ring_head<S, R::kQa, kQ, 0>(KT, issue);
  for (int kt = S - 1; kt < KT; ++kt) {
    wait_vmcnt<(S - 2) * kQ>();   // step kt has landed (in-order completion)
    lds_barrier();                // publish step kt; every wave is done with step kt - 1
    issue(kt + S - 1);            // into the stage step kt - 1 used
  }
  wait_vmcnt<0>();   // the past-the-end loads land before the block exits
}

// The compute waves' K sweep: step kt reads stage kt % S.
template <int G, int BN, class Compute>
__device__ __forceinline__ void ffn_consumer(char* smem, int KD, Compute&& compute) {
  using R = Ring<G, BN>;
  const int KT = KD / kBK;
  for (int kt = 0; kt < KT; ++kt) {
    lds_barrier();
    const char* As = smem + (kt % R::S) * R::kStageBytes;
    compute(As, As + R::kABytes);
  }
}

// Partial tiles: wave w owns weight rows [16 CB w, +16 CB) (CB 16-column MFMA
// blocks: 2 of a 128-row tile, 3 of a 192-row one) and all 32G live rows.
template <int G, int CB>
struct ColumnSplit {
  f32x4 (&acc)[kBmBf16 / 16][CB];
  int wave, lane;
  __device__ __forceinline__ void operator()(const char* As, const char* Bs) const {
#pragma unroll
    for (int kk = 0; kk < kBK / 32; ++kk) {
      const int ch = kk * 4 + (lane >> 4);
      bf16x8 b[CB];
#pragma unroll
      for (int cb = 0; cb < CB; ++cb) {
        const int rB = 16 * CB * wave + 16 * cb + (lane & 15);
        b[cb] = *(const bf16x8*)(Bs + rB * kRowBytes + swz(rB, ch) * 16);
      }
      bf16x8 a[2 * G];
#pragma unroll
      for (int rb = 0; rb < 2 * G; ++rb) {
        const int rA = rb * 16 + (lane & 15);
        a[rb] = *(const bf16x8*)(As + rA * kRowBytes + swz(rA, ch) * 16);
      }
#pragma unroll
      for (int rb = 0; rb < 2 * G; ++rb)
#pragma unroll
        for (int cb = 0; cb < CB; ++cb)
          acc[rb][cb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[rb], b[cb], acc[rb][cb], 0, 0, 0);
    }
  }
};

// Full 256-row tiles (experts with many rows: compute-bound): the four waves
// tile the 256 x 128 block 2 x 2 -- wave (wr, wc) owns rows [128 wr, +128)
// and weight rows [64 wc, +64) -- reading 96 KB of LDS fragments per step for
// 64 MFMAs per wave instead of the 144 KB the column split needs.
struct Quadrant {
  f32x4 (&acc)[8][4];
  int wave, lane;
  __device__ __forceinline__ void operator()(const char* As, const char* Bs) const {
    const int wr = wave >> 1, wc = wave & 1;
#pragma unroll
    for (int kk = 0; kk < kBK / 32; ++kk) {
      const int ch = kk * 4 + (lane >> 4);
      bf16x8 b[4];
#pragma unroll
      for (int cb = 0; cb < 4; ++cb) {
        const int rB = 64 * wc + 16 * cb + (lane & 15);
        b[cb] = *(const bf16x8*)(Bs + rB * kRowBytes + swz(rB, ch) * 16);
      }
#pragma unroll
      for (int rb = 0; rb < 8; ++rb) {
        const int rA = 128 * wr + rb * 16 + (lane & 15);
        const bf16x8 a = *(const bf16x8*)(As + rA * kRowBytes + swz(rA, ch) * 16);
#pragma unroll
        for (int cb = 0; cb < 4; ++cb)
          acc[rb][cb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b[cb], acc[rb][cb], 0, 0, 0);
      }
    }
  }
};

// Epilogue through LDS.  Written straight from the accumulators, the output
// takes one 2-byte value per lane per store instruction (32-64 instructions
// per wave), and each of those waits its turn in the CU's memory pipeline
// behind the other blocks' streams -- on the full-scale layer that cost more
// than the K loop's own stalls.  Instead the values go to an LDS tile
// [rows][NC] (row pitch NC * 2 + 16 bytes), and the tile leaves with
// 16 bytes per lane, whole 128-byte lines of output per instruction.  The
// stores are non-temporal: HBM writes interleaved with the weight stream cost
// read bandwidth, and streaming them out is ~2% faster per GEMM (measured).
// The hh tile is written m-tile-blocked (each tile's rows x 64 columns
// contiguous), so the down GEMM reads each K step of it as one block.
template <int NC>
struct OutTile {
  static constexpr int kPitch = NC * 2 + 16;
  static constexpr int kChunks = NC / 8;        // 16-byte chunks per row
  char* t;
  __device__ __forceinline__ void put(int r, int c, float v) const {
    *(bf16*)(t + r * kPitch + c * 2) = (bf16)v;
  }
  // rows 0..rows-1 of the tile to dst + r * pitch; tid: 0..255 over the four
  // compute waves
  __device__ __forceinline__ void flush(bf16* __restrict__ dst, size_t pitch, int rows,
                                        int tid) const {
    for (int j = tid; j < rows * kChunks; j += 256) {
      const int r = j / kChunks, c = j - r * kChunks;
      const i32x4 v = *(const i32x4*)(t + r * kPitch + c * 16);
      __builtin_nontemporal_store(v, (i32x4*)(dst + r * pitch + c * 8));
    }
  }
  // hh, m-tile-blocked: column block b (64 columns) of the m-tile's rows sits
  // contiguously at dst + b * rows * 64; this tile holds blocks b0 ..
  // b0 + NC / 64 - 1.
  __device__ __forceinline__ void flush_blocked(bf16* __restrict__ dst, int b0, int rows,
                                                int tid) const {
    for (int j = tid; j < rows * kChunks; j += 256) {
      const int r = j / kChunks, c = j - r * kChunks;
      const i32x4 v = *(const i32x4*)(t + r * kPitch + c * 16);
      bf16* blk = dst + (size_t)(b0 + (c >> 3)) * rows * 64;
      __builtin_nontemporal_store(v, (i32x4*)(blk + r * 64 + (c & 7) * 8));
    }
  }
};
static_assert(kBmBf16 * OutTile<kBN>::kPitch <= kLdsBytes, "output tile fits LDS");
static_assert(224 * OutTile<kBNWide>::kPitch <= kLdsBytes, "partial output tile fits LDS");

__device__ __forceinline__ float silu_mul(float g, float u) { return g / (1.0f + expf(-g)) * u; }

// A ring of at least three stages fits LDS for G groups of 32 rows and BN
// weight rows (192-row tiles: up to 7 groups).
constexpr bool ring_fits(int G, int BN) {
  return kLdsBytes / (32 * G * kRowBytes + BN * kRowBytes) >= 3;
}

// One block's work: rows [row0, row0 + rows) of expert e against column
// tile nt (of NT) of BN weight rows.
template <bool GATEUP, int BN>
__device__ __forceinline__ void ffn_block(char* smem, const bf16* __restrict__ A,
                                          const int32_t* __restrict__ gather, int gK, int gT,
                                          const bf16* __restrict__ W, int e, int row0, int rows,
                                          int nt, int NT, int KD, int I, int H,
                                          bf16* __restrict__ C) {
  constexpr int BM = kBmBf16;
  static_assert(BM == 256, "instances cover 8 groups of 32 rows");
  constexpr int CB = BN / 64;   // 16-column MFMA blocks per compute wave (partial tiles)
  const int groups = (rows + 31) >> 5;
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);   // wave-uniform

  const size_t wrows = GATEUP ? (size_t)2 * I : (size_t)H;
  // Activation rows: x_perm is row-major [rows][H], or (gather) the rows are
  // token rows of x picked through row_src, each a contiguous 2H-byte row all
  // the same, so the DMA loads them in place and no grouped copy is made; hh
  // is m-tile-blocked: rows [row0, row0 + rows) of column block j (64
  // columns, one K step of the down GEMM) sit contiguously at
  // row0 * I + j * rows * 64.
  const TileSrc src{gather ? A : A + (size_t)row0 * KD, gather ? gather + row0 : nullptr, gK, gT,
                    rows, W + (size_t)e * wrows * KD, nt, I, GATEUP,
                    GATEUP ? KD : kBK, GATEUP ? kBK : rows * kBK};
  // The column tiles of one m-tile run side by side on one XCD and read the
  // same activation rows.  Swept in lockstep, every one of them waits on the
  // same L2 miss at every step; spread over the whole K range, the m-tile's
  // rows are all live at once and crowd L2.  Tiles start their K sweep (and
  // wrap around) at one of a few offsets, by column tile: four for full
  // 256-row tiles (3 MB of activation rows), two for the partial tiles of
  // gate/up (~1.5 MB at the prefill shape; one, three or four were slower or
  // equal), four for down's 192-row tiles (2.57 -> 2.54 ms on prefill
  // against two, which was 1.4 % faster than one), and one for down's other
  // partial tiles, whose m-tile is a few hundred KB.  Measured against one offset per
  // column tile: prefill gate/up 5.38 -> 5.23 ms, down 2.90 -> 2.88 ms, and
  // 7-14 % on experts of 2048-16384 rows.  Tiles of one 32-row group (decode)
  // keep one offset per column tile, which measured 0.4 % faster there.
  const int KT = KD / kBK;
  const int n_start = rows == kBmBf16 ? 4 : rows <= 32 ? NT : GATEUP ? 2 : BN != kBN ? 4 : 1;
  const int k_start = ((nt % n_start) * KT) / n_start;

  if (wave >= 4) {   // loader waves
    switch (groups) {
#define MOE_CASE(g) \
      case g:                                                                  \
        if constexpr (ring_fits(g, BN)) {                                      \
          if (GATEUP && src.gather)                                            \
            ffn_loader<g, GATEUP, BN>(smem, src, KD, k_start, wave - 4, lane); \
          else                                                                 \
            ffn_loader<g, false, BN>(smem, src, KD, k_start, wave - 4, lane);  \
        }                                                                      \
        break;
      MOE_CASE(1) MOE_CASE(2) MOE_CASE(3) MOE_CASE(4)
      MOE_CASE(5) MOE_CASE(6) MOE_CASE(7) MOE_CASE(8)
#undef MOE_CASE
      default: break;
    }
    // Two more barriers, matching the compute waves': the LDS is free for the
    // output tile (every load has landed), then the tile is written.
    lds_barrier();
    lds_barrier();
    return;
  }

  // Output tile: gate/up 64 hh columns, down BN y columns of this column tile.
  constexpr int NC = GATEUP ? BN / 2 : BN;
  const OutTile<NC> out{smem};
  const int c = lane & 15, q = lane >> 4;
  if (BN == kBN && rows == BM) {
    f32x4 acc[8][4];
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) acc[i][j] = f32x4{0, 0, 0, 0};
    ffn_consumer<8, kBN>(smem, KD, Quadrant{acc, wave, lane});
    lds_barrier();   // loads landed, fragments read: the LDS is free
    // lane holds C[128 wr + 16 rb + 4 q + i][weight row 64 wc + 16 cb + c]
    const int wr = wave >> 1, wc = wave & 1;
#pragma unroll
    for (int rb = 0; rb < 8; ++rb)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = 128 * wr + rb * 16 + 4 * q + i;
        if (GATEUP) {
          // weight rows 64 wc + [0,16) gate / [16,32) up of one column block, then the next
#pragma unroll
          for (int p = 0; p < 2; ++p)
            out.put(r, 32 * wc + 16 * p + c, silu_mul(acc[rb][2 * p][i], acc[rb][2 * p + 1][i]));
        } else {
#pragma unroll
          for (int cb = 0; cb < 4; ++cb) out.put(r, 64 * wc + 16 * cb + c, acc[rb][cb][i]);
        }
      }
  } else {
    f32x4 acc[BM / 16][CB];
#pragma unroll
    for (int i = 0; i < BM / 16; ++i)
#pragma unroll
      for (int j = 0; j < CB; ++j) acc[i][j] = f32x4{0, 0, 0, 0};
    // K loop instantiated per number of live 32-row groups: branch-free, only
    // the live rows are loaded and only their MFMAs issued.
    switch (groups) {
#define MOE_CASE(g)                                                                 \
      case g:                                                                       \
        if constexpr (ring_fits(g, BN))                                             \
          ffn_consumer<g, BN>(smem, KD, ColumnSplit<g, CB>{acc, wave, lane});       \
        break;
      MOE_CASE(1) MOE_CASE(2) MOE_CASE(3) MOE_CASE(4)
      MOE_CASE(5) MOE_CASE(6) MOE_CASE(7) MOE_CASE(8)
#undef MOE_CASE
      default: break;
    }
    lds_barrier();   // loads landed, fragments read: the LDS is free
    // lane holds C[16 rb + 4 q + i][weight row 16 CB wave + 16 cb + c]
#pragma unroll
    for (int rb = 0; rb < BM / 16; ++rb) {
      if (rb * 16 >= rows) continue;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = rb * 16 + 4 * q + i;
        if constexpr (GATEUP) {
          // column blocks 2p (gate) and 2p + 1 (up) of hh columns 16 (CB/2) wave + 16 p + c
#pragma unroll
          for (int p = 0; p < CB / 2; ++p)
            out.put(r, 16 * (CB / 2) * wave + 16 * p + c,
                    silu_mul(acc[rb][2 * p][i], acc[rb][2 * p + 1][i]));
        } else {
#pragma unroll
          for (int cb = 0; cb < CB; ++cb) out.put(r, 16 * CB * wave + 16 * cb + c, acc[rb][cb][i]);
        }
      }
    }
  }
  lds_barrier();   // the four compute waves' values are in the tile
  if (GATEUP)   // hh, m-tile-blocked in 64-column blocks (one down K step each)
    out.flush_blocked(C + (size_t)row0 * I, nt * (NC / 64), rows, threadIdx.x);
  else          // y_perm, row-major
    out.flush(C + (size_t)row0 * H + nt * NC, H, rows, threadIdx.x);
}

// One launch per GEMM.  Block -> (m-tile, column slot), XCD-aware: the slots
// of one m-tile run on one XCD and share its activation rows through that
// XCD's L2.  Slots count 128-row column tiles; an m-tile whose number of
// 32-row groups has its bit set in wide_mask takes the wider tiles (BNW
// rows) instead, and its slots past N / BNW exit at once -- cheaper than a
// second launch for the other tiles (measured: an empty second launch cost
// 57 us, and two serial launches each drain their own tail; gate/up on the
// 8192-token layer 5.1-5.2 -> 4.55 ms).  WIDE = false compiles the 128-row
// path alone, for layers with no wide tiles: the kernel with both paths
// measured 1.5 % slower there (the 16384-token skewed layer's gate/up).
template <bool GATEUP, bool WIDE>
__global__ __launch_bounds__(kGemmThreads, 1) void ffn_mfma_bf16(
    const bf16* __restrict__ A, const int32_t* __restrict__ gather, int gK, int gT,
    const bf16* __restrict__ W, const int4* __restrict__ tiles, const int* __restrict__ ntiles,
    int KD, int I, int H, int NT, int wide_mask, bf16* __restrict__ C) {
  __shared__ __attribute__((aligned(1024))) char smem[kLdsBytes];
  constexpr int BNW = GATEUP ? kBNGateUpWide : kBNWide;
  const int b = blockIdx.x;
  const int xcd = b & 7, slot = b >> 3;
  const int mt = (slot / NT) * 8 + xcd;
  const int nt = slot % NT;
  if (mt >= *ntiles) return;
  const int4 tile = tiles[mt];
  const int e = tile.x, row0 = tile.y, rows = tile.z;
  const int groups = (rows + 31) >> 5;
  if constexpr (WIDE) {
    if (((wide_mask >> groups) & 1) && ring_fits(groups, BNW)) {
      const int ntw = (GATEUP ? 2 * I : H) / BNW;
      if (nt >= ntw) return;
      ffn_block<GATEUP, BNW>(smem, A, gather, gK, gT, W, e, row0, rows, nt, ntw, KD, I, H, C);
      return;
    }
  }
  ffn_block<GATEUP, kBN>(smem, A, gather, gK, gT, W, e, row0, rows, nt, NT, KD, I, H, C);
}

// ------------------------------------------------------------ fp32 path --
// Plain LDS-tiled FMA kernels for fp32 layers (exact fp32 products, fp32
// accumulation); any H and I.  Tile: 32 rows x 32 outputs, K step 32.
template <bool GATEUP>
__global__ __launch_bounds__(kThreads) void ffn_f32(const float* __restrict__ A,
                                                    const int32_t* __restrict__ gather, int gK,
                                                    int gT,
                                                    const float* __restrict__ W,
                                                    const int4* __restrict__ tiles,
                                                    const int* __restrict__ ntiles, int KD, int I,
                                                    int H, float* __restrict__ C) {
  constexpr int TM = 32, TN = 32, TK = 32;
  constexpr int NB = GATEUP ? 2 * TN : TN;   // weight rows per tile
  __shared__ float As[TK][TM + 1];
  __shared__ float Bs[TK][NB + 1];
  const int mt = blockIdx.y;
  if (mt >= *ntiles) return;
  const int4 tile = tiles[mt];
  const int e = tile.x, row0 = tile.y, rows = tile.z;
  const int n0 = blockIdx.x * TN;
  const int NOUT = GATEUP ? I : H;
  const size_t wrows = GATEUP ? (size_t)2 * I : (size_t)H;
  const float* wexp = W + (size_t)e * wrows * KD;
  const int tx = threadIdx.x % 16, ty = threadIdx.x / 16;   // outputs: rows ty*2+{0,1}, cols tx*2+{0,1}
  float acc[2][2][2] = {};
  for (int k0 = 0; k0 < KD; k0 += TK) {
    for (int i = threadIdx.x; i < TM * TK; i += kThreads) {
      const int r = i / TK, k = i % TK;
      if (r < rows && k0 + k < KD) {
        const int ar = gather ? min(max(gather[row0 + r], 0) / gK, gT - 1) : row0 + r;
        As[k][r] = A[(size_t)ar * KD + k0 + k];
      } else {
        As[k][r] = 0.0f;
      }
    }
    for (int i = threadIdx.x; i < NB * TK; i += kThreads) {
      const int c = i / TK, k = i % TK;
      int n = n0 + (c % TN);
      int wr = (GATEUP && c >= TN) ? I + n : n;
      Bs[k][c] = (n < NOUT && k0 + k < KD) ? wexp[(size_t)wr * KD + k0 + k] : 0.0f;
    }
    __syncthreads();
    for (int k = 0; k < TK; ++k) {
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const float a = As[k][ty * 2 + i];
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          acc[i][j][0] = fmaf(a, Bs[k][tx * 2 + j], acc[i][j][0]);
          if (GATEUP) acc[i][j][1] = fmaf(a, Bs[k][TN + tx * 2 + j], acc[i][j][1]);
        }
      }
    }
    __syncthreads();
  }
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int r = ty * 2 + i, n = n0 + tx * 2 + j;
      if (r >= rows || n >= NOUT) continue;
      float v = acc[i][j][0];
      if (GATEUP) v = v / (1.0f + expf(-v)) * acc[i][j][1];
      C[(size_t)(row0 + r) * NOUT + n] = v;
    }
}

inline size_t align256(size_t b) { return (b + 255) & ~(size_t)255; }
inline int ffn_bm(int dtype) { return dtype == MOE_BF16 ? kBmBf16 : kBmF32; }
inline size_t max_mtiles(int rows_cap, int n_ffn, int bm) { return (size_t)rows_cap / bm + n_ffn + 8; }

}  // namespace

size_t ffn_ws_bytes(int rows_cap, int n_ffn, int I, int dtype) {
  const int es = dtype == MOE_BF16 ? 2 : 4;
  return 256 + align256(max_mtiles(rows_cap, n_ffn, ffn_bm(dtype)) * sizeof(int4)) +
         align256((size_t)rows_cap * I * es);
}

hipError_t launch_expert_ffn(const void* x_perm, const int32_t* gather, int gK, int gT,
                             const int32_t* offsets, int rows_cap, int n_ffn, int H, int I,
                             const void* w13, const void* w2, int dtype, void* y_perm, void* ws,
                             hipStream_t s) {
  const int bm = ffn_bm(dtype);
  const size_t mtmax = max_mtiles(rows_cap, n_ffn, bm);
  int* ntiles = (int*)ws;
  int4* tiles = (int4*)((char*)ws + 256);
  void* hh = (char*)ws + 256 + align256(mtmax * sizeof(int4));
  MOE_LAUNCH("ffn_tiles", s,
             ffn_tiles<<<1, 1024, 0, s>>>(offsets, n_ffn, bm, rows_cap, (int)mtmax, tiles,
                                          ntiles));
  if (dtype == MOE_BF16) {
    const unsigned groups = ceil_div(mtmax, 8);
    const int nt1 = I / 64, nt2 = H / kBN;
    // Partial m-tiles take wider weight tiles, which cut the activation
    // traffic from L2 per weight byte:
    //   gate/up: 256 rows (128 hh columns) for tiles of 2-5 groups, whose
    //     3-stage ring still fits;
    //   down: 192 rows for tiles of 2-7 groups (4-5 stages).
    // Single-group tiles keep the 128-row tiles' deeper rings, and the
    // others do not fit.  Measured on the 8192-token layer: gate/up 5.31 ->
    // 5.08 ms and down 2.83 -> 2.51 ms as two launches per GEMM, gate/up
    // 4.55 ms as one; 256-row down tiles (3 stages) took 2.82 ms.  On the
    // 16384-token skewed layer (full tiles next to light experts' partial
    // ones) 0.19 ms faster.  Where the average FFN expert would have under
    // 32 rows even if every pick went to one (decode), every tile is a
    // single group and the kernel without the wide path is launched.
    const bool enough_rows = (long long)rows_cap >= 32LL * n_ffn;
    const int wide_gu = enough_rows && (2 * I) % kBNGateUpWide == 0 ? kWideGroupsGateUp : 0;
    const int wide_dn = enough_rows && H % kBNWide == 0 ? kWideGroups : 0;
#define MOE_GEMMS(W)                                                                     \
    MOE_LAUNCH("ffn_gateup_bf16", s,                                                       \
               ffn_mfma_bf16<true, W><<<groups * 8 * nt1, kGemmThreads, 0, s>>>(           \
                   (const bf16*)x_perm, gather, gK, gT, (const bf16*)w13, tiles, ntiles, H, \
                   I, H, nt1, wide_gu, (bf16*)hh));                                       \
    MOE_LAUNCH("ffn_down_bf16", s,                                                         \
               ffn_mfma_bf16<false, W><<<groups * 8 * nt2, kGemmThreads, 0, s>>>(          \
                   (const bf16*)hh, nullptr, 1, 1, (const bf16*)w2, tiles, ntiles, I, I, H, \
                   nt2, wide_dn, (bf16*)y_perm))
    if (wide_gu || wide_dn) {
      MOE_GEMMS(true);
    } else {
      MOE_GEMMS(false);
    }
#undef MOE_GEMMS
  } else {
    dim3 g1(ceil_div(I, 32), (unsigned)mtmax), g2(ceil_div(H, 32), (unsigned)mtmax);
    MOE_LAUNCH("ffn_gateup_f32", s,
               ffn_f32<true><<<g1, kThreads, 0, s>>>((const float*)x_perm, gather, gK, gT,
                                                     (const float*)w13, tiles, ntiles, H, I, H,
                                                     (float*)hh));
    MOE_LAUNCH("ffn_down_f32", s,
               ffn_f32<false><<<g2, kThreads, 0, s>>>((const float*)hh, nullptr, 1, 1,
                                                      (const float*)w2, tiles, ntiles, I, I, H,
                                                      (float*)y_perm));
  }
  return hipGetLastError();
}

}  // namespace moe
