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
//     hits rather than 32 simultaneous waits on one miss;
//   - the full 256-row m-tiles of experts that hold at least 256 rows (the
//     compute-bound regime) go to a kernel of their own, launched before the
//     other tiles of each GEMM: 256 x 256 blocks whose eight waves all compute
//     (the dense kernel, below).
#include <algorithm>
#include <mutex>

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
// Rows are clamped to [0, rows_cap) and the lists to their capacities, so a
// malformed offsets[] can shrink the work but never index past the buffers.
// Entry: (expert, first row, rows, m-tiles of that expert).  With full != 0,
// the m-tiles that hold bm rows go to full[] (the dense kernel's list) and
// only each expert's last, partial m-tile to tiles[].  tiles[] holds first
// the m-tiles of more than narrow_rows rows, then those of at most
// narrow_rows (narrow_rows = 0: all in the first part); counts: ntiles[0] =
// all of them, ntiles[3] = the first part, ntiles[4] = the second.
__global__ __launch_bounds__(1024) void ffn_tiles(const int32_t* __restrict__ offsets, int n_ffn,
                                                  int bm, int rows_cap, int max_tiles,
                                                  int4* __restrict__ tiles,
                                                  int* __restrict__ ntiles, int max_full,
                                                  int4* __restrict__ full,
                                                  int* __restrict__ nfull, int narrow_rows) {
  __shared__ int part[3][1024];
  __shared__ int full_experts;
  const int tid = threadIdx.x;
  const int per = (n_ffn + 1023) / 1024;
  const int lo = min(n_ffn, tid * per), hi = min(n_ffn, lo + per);
  auto span = [&](int e, int& r0, int& m) {
    r0 = min(max(offsets[e], 0), rows_cap);
    m = min(max(offsets[e + 1], r0), rows_cap) - r0;
  };
  if (tid == 0) full_experts = 0;
  __syncthreads();
  // only an expert's last m-tile can be short: it is narrow when it holds
  // at most narrow_rows rows
  auto n_narrow = [&](int m) { return m > 0 && m % bm != 0 && m % bm <= narrow_rows ? 1 : 0; };
  int s = 0, f = 0, n = 0, fe = 0;
  for (int e = lo; e < hi; ++e) {
    int r0, m;
    span(e, r0, m);
    const int nf = full ? m / bm : 0, nn = n_narrow(m);
    f += nf;
    n += nn;
    fe += nf > 0 ? 1 : 0;
    s += (m + bm - 1) / bm - nf - nn;
  }
  part[0][tid] = s;
  part[1][tid] = f;
  part[2][tid] = n;
  if (fe) atomicAdd(&full_experts, fe);
  __syncthreads();
  for (int off = 1; off < 1024; off <<= 1) {
    const int v0 = tid >= off ? part[0][tid - off] : 0;
    const int v1 = tid >= off ? part[1][tid - off] : 0;
    const int v2 = tid >= off ? part[2][tid - off] : 0;
    __syncthreads();
    part[0][tid] += v0;
    part[1][tid] += v1;
    part[2][tid] += v2;
    __syncthreads();
  }
  // With full m-tiles split off, each part of tiles[] lists the experts in
  // reverse order: the dense kernel has just read the experts' weights in
  // expert order, so the last ones are the likeliest to still sit in the
  // last-level cache when the other m-tiles read them again.
  const int nw = min(part[0][1023], max_tiles);
  const int nn = min(part[2][1023], max_tiles - nw);
  int pos = part[0][tid] - s, fpos = part[1][tid] - f, npos = part[2][tid] - n;
  for (int e = lo; e < hi; ++e) {
    int r0, m;
    span(e, r0, m);
    const int mt = (m + bm - 1) / bm, nf = full ? m / bm : 0, nar = n_narrow(m);
    for (int j = 0; j < mt; ++j) {
      const int4 t = make_int4(e, r0 + j * bm, min(bm, m - j * bm), mt);
      if (j < nf) {
        if (fpos < max_full) full[fpos++] = t;
      } else if (nar && j == mt - 1) {
        if (npos < nn) tiles[nw + (full ? nn - 1 - npos : npos)] = t;
        ++npos;
      } else {
        if (pos < nw) tiles[full ? nw - 1 - pos : pos] = t;
        ++pos;
      }
    }
  }
  if (tid == 1023) {
    ntiles[0] = nw + nn;
    ntiles[3] = nw;
    ntiles[4] = nn;
    if (full) {
      nfull[0] = min(part[1][1023], max_full);
      nfull[1] = full_experts;   // experts holding full m-tiles
    }
  }
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
// Weights are loaded non-temporally when one m-tile holds all of the expert's
// rows (read once: streamed past the caches) and with the default policy when
// it has several (its other m-tiles read the same weights again, and the
// caches keep them: the 256 MB last-level cache holds a heavy expert's 75 MB).
// Non-temporal weights of a 16,384-row expert made every m-tile fetch them from
// HBM again (measured: the weight loads alone took 575 us of a 1014 us gate/up
// GEMM).
constexpr int kCachePolicyNT = 2;
// Buffer descriptor word 3 for raw 32-bit buffer loads on gfx9 parts (data
// format 32, no swizzle, no index stride).
constexpr int kBufferFlags = 0x00020000;

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
  bool stream_w;        // the expert has one m-tile: weights non-temporal
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
    for (int i = 0; i < R::kQb; ++i) {
      const void* g = real ? src[R::kQa + i] + k0 : t.w;
      lds_void* d = (lds_void*)(stage(kt) + R::kABytes + (l + 4 * i) * 1024);
      if (t.stream_w)
        __builtin_amdgcn_global_load_lds(g, d, 16, 0, kCachePolicyNT);
      else
        __builtin_amdgcn_global_load_lds(g, d, 16, 0, 0);
    }
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

// One K step (two 32-wide k blocks) of one compute wave's tile: R row blocks
// (A rows a_row0 + 16 rb) x C column blocks (weight rows b_row0 + 16 cb) of
// 16 x 16, v_mfma_f32_16x16x32_bf16 with fp32 accumulators.
// The fragment reads are software-pipelined: the step runs as groups of two
// row blocks (2 C MFMAs), and the A fragments of the next group, and at the
// first group the second k block's B fragments, are read from LDS before the
// current group's MFMAs issue, so each read has a whole group of MFMAs to
// land in.  (Read just in time, one wait per two row blocks exposed the LDS
// latency eight times per K step; the MFMA rate of full tiles was ~40 % of
// peak.)  Each group starts by waiting for every outstanding LDS read
// (lgkmcnt(0): only its own fragments are then in flight), so the pipeline
// holds even where the compiler's own waits are that coarse, as they are in
// the full tiles' loop of the kernels with wide tiles.  The sched_barriers
// keep the compiler from sinking the reads to their uses.
struct NoHook {
  __device__ __forceinline__ void operator()(int) const {}
};

// hook(g) runs at the start of MFMA group g, after that group's reads are out
// (the dense kernel issues one of its next step's global->LDS loads there).
// ONE_B: one set of B fragment registers, reloaded at the first group of the
// second k block (one exposed LDS latency per step, 4 C fewer registers).
// SWAP: the B fragments feed the MFMA's first operand, so each 16 x 16 block
// of acc holds the transposed product: lane (q = lane / 16, c = lane % 16)
// gets B rows 4 q .. 4 q + 3 of the block against A row c.
template <int R, int C, class Acc, class Hook = NoHook, bool ONE_B = false, bool SWAP = false>
__device__ __forceinline__ void mma_step(const char* As, const char* Bs, int a_row0, int b_row0,
                                         int lane, Acc& acc, const Hook& hook = Hook{}) {
  constexpr int kRG = R % 2 == 0 ? 2 : 1;   // row blocks per group
  constexpr int kNG = 2 * R / kRG;          // groups per step (both k blocks)
  const int lr = lane & 15, lq = lane >> 4;
  auto a_frag = [&](int kk, int rb) {
    const int rA = a_row0 + 16 * rb + lr;
    return *(const bf16x8*)(As + rA * kRowBytes + swz(rA, kk * 4 + lq) * 16);
  };
  auto b_frag = [&](int kk, int cb) {
    const int rB = b_row0 + 16 * cb + lr;
    return *(const bf16x8*)(Bs + rB * kRowBytes + swz(rB, kk * 4 + lq) * 16);
  };
  bf16x8 b[ONE_B ? 1 : 2][C];
  bf16x8 a[2][kRG];
#pragma unroll
  for (int cb = 0; cb < C; ++cb) b[0][cb] = b_frag(0, cb);
#pragma unroll
  for (int r = 0; r < kRG; ++r) a[0][r] = a_frag(0, r);
#pragma unroll
  for (int g = 0; g < kNG; ++g) {
    const int kk = (g * kRG) / R, rb0 = (g * kRG) % R;
    // this group's fragments, read one group ago, have landed; the reads
    // issued next get the whole group's MFMAs to land in
    __builtin_amdgcn_s_waitcnt((0x3F & 0xF) | ((0x3F >> 4) << 14) | (0x7 << 4) | (0x0 << 8));
    __builtin_amdgcn_sched_barrier(0);
    if (g + 1 < kNG) {
      const int kn = ((g + 1) * kRG) / R, rn = ((g + 1) * kRG) % R;
#pragma unroll
      for (int r = 0; r < kRG; ++r) a[(g + 1) & 1][r] = a_frag(kn, rn + r);
    }
    if constexpr (ONE_B) {
      if (g == kNG / 2) {
#pragma unroll
        for (int cb = 0; cb < C; ++cb) b[0][cb] = b_frag(1, cb);
      }
    } else if (g == 0) {
#pragma unroll
      for (int cb = 0; cb < C; ++cb) b[1][cb] = b_frag(1, cb);
    }
    hook(g);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int r = 0; r < kRG; ++r)
#pragma unroll
      for (int cb = 0; cb < C; ++cb)
        acc[rb0 + r][cb] =
            SWAP ? __builtin_amdgcn_mfma_f32_16x16x32_bf16(b[ONE_B ? 0 : kk][cb], a[g & 1][r],
                                                           acc[rb0 + r][cb], 0, 0, 0)
                 : __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[g & 1][r], b[ONE_B ? 0 : kk][cb],
                                                           acc[rb0 + r][cb], 0, 0, 0);
    __builtin_amdgcn_sched_barrier(0);
  }
}

// Partial tiles: wave w owns weight rows [16 CB w, +16 CB) (CB 16-column MFMA
// blocks: 2 of a 128-row tile, 3 of a 192-row one, 4 of a 256-row one) and
// all 32G live rows.
template <int G, int CB>
struct ColumnSplit {
  f32x4 (&acc)[kBmBf16 / 16][CB];
  int wave, lane;
  __device__ __forceinline__ void operator()(const char* As, const char* Bs) const {
    mma_step<2 * G, CB>(As, Bs, 0, 16 * CB * wave, lane, acc);
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
    mma_step<8, 4>(As, Bs, 128 * (wave >> 1), 64 * (wave & 1), lane, acc);
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

// The K loops a kernel compiles for G live row groups at tile width BN: the
// wide tiles serve exactly the group counts of the kernel's WIDE_MASK and
// the 128-row tiles the others.  Only what can run is compiled: with every
// combination in one kernel, the compiler's wait-count analysis gave up on
// the full tiles' loop and waited for all outstanding LDS reads before each
// MFMA group, which undid the fragment-read pipelining there.
constexpr bool compiled(int G, int BN, int WIDE_MASK) {
  return ring_fits(G, BN) && (BN == kBN ? !((WIDE_MASK >> G) & 1) : ((WIDE_MASK >> G) & 1));
}

// One block's work: rows [row0, row0 + rows) of expert e against column
// tile nt (of NT) of BN weight rows.
template <bool GATEUP, int BN, int WIDE_MASK>
__device__ __forceinline__ void ffn_block(char* smem, const bf16* __restrict__ A,
                                          const int32_t* __restrict__ gather, int gK, int gT,
                                          const bf16* __restrict__ W, int e, int row0, int rows,
                                          bool stream_w, int nt, int NT, int KD, int I, int H,
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
                    rows, W + (size_t)e * wrows * KD, nt, I, GATEUP, stream_w,
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
        if constexpr (compiled(g, BN, WIDE_MASK)) {                            \
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
        if constexpr (compiled(g, BN, WIDE_MASK))                                   \
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
// 32-row groups has its bit set in WIDE_MASK takes the wider tiles (BNW
// rows) instead, and its slots past N / BNW exit at once -- cheaper than a
// second launch for the other tiles (measured: an empty second launch cost
// 57 us, and two serial launches each drain their own tail; gate/up on the
// 8192-token layer 5.1-5.2 -> 4.55 ms).  WIDE_MASK = 0 compiles the 128-row
// path alone, for layers with no wide tiles: the kernel with both paths
// measured 1.5 % slower there (the 16384-token skewed layer's gate/up).
template <bool GATEUP, int WIDE_MASK>
__global__ __launch_bounds__(kGemmThreads, 1) void ffn_mfma_bf16(
    const bf16* __restrict__ A, const int32_t* __restrict__ gather, int gK, int gT,
    const bf16* __restrict__ W, const int4* __restrict__ tiles, const int* __restrict__ ntiles,
    int KD, int I, int H, int NT, bf16* __restrict__ C) {
  __shared__ __attribute__((aligned(1024))) char smem[kLdsBytes];
  constexpr int BNW = GATEUP ? kBNGateUpWide : kBNWide;
  const int b = blockIdx.x;
  const int xcd = b & 7, slot = b >> 3;
  const int mt = (slot / NT) * 8 + xcd;
  const int nt = slot % NT;
  if (mt >= *ntiles) return;
  const int4 tile = tiles[mt];
  const int e = tile.x, row0 = tile.y, rows = tile.z;
  const bool stream_w = tile.w <= 1;
  const int groups = (rows + 31) >> 5;
  if constexpr (WIDE_MASK != 0) {
    if ((WIDE_MASK >> groups) & 1) {
      const int ntw = (GATEUP ? 2 * I : H) / BNW;
      if (nt >= ntw) return;
      ffn_block<GATEUP, BNW, WIDE_MASK>(smem, A, gather, gK, gT, W, e, row0, rows, stream_w, nt,
                                         ntw, KD, I, H, C);
      return;
    }
  }
  ffn_block<GATEUP, kBN, WIDE_MASK>(smem, A, gather, gK, gT, W, e, row0, rows, stream_w, nt, NT,
                                     KD, I, H, C);
}

// ------------------------------------------------- dense full-tile GEMM --
// Full m-tiles (256 rows of one expert: the experts that hold many tokens,
// compute-bound) in 256 x 256 blocks, a launch of their own before the other
// tiles: half the activation bytes per flop of the 256 x 128 quadrant path.
// On one 16,384-row expert the quadrant path's loads alone took 70 % of its
// time and its MFMAs alone 50 % (timing-only builds); this kernel takes
// ~0.75 ms for the gate/up GEMM against ~0.90 ms.
//   - 8 waves, 2 per SIMD; wave (wr, wc) = (w / 4, w % 4) computes rows
//     [128 wr, +128) x weight rows [64 wc, +64) (128 accumulator registers);
//   - no loader waves: each wave issues 8 of a K step's 64 global->LDS loads
//     (A: 32 groups of 8 rows, B: 32 groups) among the MFMA groups of an
//     earlier step, as buffer loads (32-bit per-lane offsets, the K step in
//     the scalar offset);
//   - weight tiles in a ring of three slots (loaded two steps ahead),
//     activation tiles in a ring of two (one step ahead), five separately
//     declared LDS arrays: the compiler can tell that the loads into one do
//     not touch the reads of another, so no fragment read waits for a load
//     in flight (with one array it made every read wait for the wave's
//     newest load).  With two stages of both (every load one step ahead)
//     the step-end wait was exposed.  Measured on the skewed layer (full
//     tiles, same box): gate/up 3.34 ms with two stages of both, 3.13-3.16
//     with the activation tiles two steps ahead, 3.03 with the weight tiles
//     two steps ahead and the cache-policy branch gone (below); down 1.75 ->
//     1.67-1.69 ms;
//   - the output leaves straight from the accumulators, 16 bytes per lane
//     (the MFMAs take the weight tile as their first operand, and the weight
//     rows are ordered so that a lane holds 8 consecutive output columns);
//   - measured and not kept: 32-wide K steps with four stages in four arrays
//     (64-byte rows: 0.93 ms), super-items of 8 m-tiles x 4 weight tiles per
//     XCD from k = 0 (heavy expert 0.78 ms, but the 64-expert layer's full
//     tiles 20 % slower); the two waves of a SIMD issuing their loads in
//     different MFMA groups (3-8 % slower); weight loads before activation
//     loads with two stages (12 % slower);
//   - gate/up pairing and the m-tile-blocked hh layout as in the other path;
//     weights always loaded with the default cache policy (the expert's
//     other m-tiles read them again; a choice per block made the compiler
//     lose track of which slots had loads in flight).
constexpr int kDenseBN = 256;
constexpr int kDenseSlot = 32 * 1024;   // one operand tile of a K step: 256 rows x 128 B
static_assert(5 * kDenseSlot <= kLdsBytes, "three A slots and two B slots");

// Weight row held in row r of a dense tile (column tile nt).  Wave column wc
// owns tile rows [64 wc, +64): 16-row blocks cb = 0..3, and after the
// swapped MFMA a lane holds rows 4 q .. 4 q + 3 of each block.  Those rows
// are ordered so that the lane's values are 8 consecutive output columns:
//   gate/up: blocks 2p (gate) and 2p + 1 (up) of hh columns
//     nt * 128 + 32 wc + 8 q + 4 p + i;
//   down: block cb row 4 q + i is y column nt * 256 + 64 wc + 32 (cb / 2) +
//     8 q + 4 (cb % 2) + i.
__device__ __forceinline__ int dense_weight_row(bool gateup, int r, int nt, int I) {
  const int wc = r >> 6, cb = (r >> 4) & 3, q = (r >> 2) & 3, i = r & 3;
  if (gateup) {
    const int j = nt * 128 + 32 * wc + 8 * q + 4 * (cb >> 1) + i;
    return (cb & 1) ? I + j : j;
  }
  return nt * 256 + 64 * wc + 32 * (cb >> 1) + 8 * q + 4 * (cb & 1) + i;
}

// One (full m-tile, 256-row weight tile nt) item of the dense kernel.
// LDS: the weight tile of a K step (256 weight rows x 64 k, 32 KB) in a ring
// of three slots w0-w2, the activation tile (256 rows) in a ring of two,
// a0-a1, five arrays of 32 KB declared apart.  During step kt's MFMAs each
// wave issues its share of step kt + 1's activation tile (two loads in each
// of MFMA groups 0 and 1) and of step kt + 2's weight tile (one load in each
// of groups 2-5), and at the end of the step waits for all but those last
// weight loads: the weights have more than a step to land, the activation
// rows most of one.
template <bool GATEUP>
__device__ __forceinline__ void dense_item(char* w0, char* w1, char* w2, char* a0, char* a1,
                                           const bf16* __restrict__ A,
                                           const int32_t* __restrict__ gather, int gK, int gT,
                                           const bf16* __restrict__ W, int4 tile, int nt,
                                           int KD, int I, int H, bf16* __restrict__ C) {
  const int e = tile.x, row0 = tile.y;
  constexpr int BM = kBmBf16;
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int wr = wave >> 2, wc = wave & 3;
  const int KT = KD / kBK;
  const int k_start = ((nt % 4) * KT) / 4;
  const size_t wrows = GATEUP ? (size_t)2 * I : (size_t)H;
  const bf16* a_rows = gather ? A : A + (size_t)row0 * KD;
  const int32_t* g = gather ? gather + row0 : nullptr;
  const int a_pitch = GATEUP ? KD : kBK, a_step = GATEUP ? kBK : BM * kBK;
  const bf16* w = W + (size_t)e * wrows * KD;
  // this wave's load groups: A and B groups wave + 8 i, i < 4; lane j of a
  // group's load fetches chunk swz(row, j & 7) of row 8 g + (j >> 3).  Buffer
  // loads: a 32-bit per-lane byte offset from the tile's base (token rows of
  // x, grouped rows or the m-tile's hh; one expert's weight rows) and a
  // scalar one for the K step.
  const int lr = lane >> 3, lc = lane & 7;
  uint32_t aoff[4], boff[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int r = (wave + 8 * i) * 8 + lr;
    const int ar = g ? min(max(g[r], 0) / gK, gT - 1) : r;
    aoff[i] = ((uint32_t)ar * (uint32_t)a_pitch + swz(r, lc) * 8) * 2;
    boff[i] = ((uint32_t)dense_weight_row(GATEUP, r, nt, I) * (uint32_t)KD + swz(r, lc) * 8) * 2;
  }
  const __amdgpu_buffer_rsrc_t rs_a =
      __builtin_amdgcn_make_buffer_rsrc((void*)a_rows, (short)0, 0x7fffffff, kBufferFlags);
  const __amdgpu_buffer_rsrc_t rs_b =
      __builtin_amdgcn_make_buffer_rsrc((void*)w, (short)0, 0x7fffffff, kBufferFlags);
  // (kt < KT + 2: past the end it wraps into the sweep again)
  auto k_of = [&](int kt) {
    int ks = kt + k_start;
    ks = ks >= KT ? ks - KT : ks;
    return ks >= KT ? ks - KT : ks;
  };
  auto load_a = [&](char* dst, int kt, int u) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rs_a, (lds_void*)(dst + (wave + 8 * u) * 1024), 16,
                                             aoff[u], (uint32_t)k_of(kt) * (a_step * 2), 0, 0);
  };
  auto load_b = [&](char* dst, int kt, int u) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rs_b, (lds_void*)(dst + (wave + 8 * u) * 1024), 16,
                                             boff[u], (uint32_t)k_of(kt) * (kBK * 2), 0, 0);
  };
  f32x4 acc[8][4];
#pragma unroll
  for (int i = 0; i < 8; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f32x4{0, 0, 0, 0};
  // Every step issues the same loads -- past the end of the sweep they read
  // real rows again into a slot no step reads -- so the wait count is one
  // constant and the compiler's view of which slots have loads in flight
  // is the same on every path.
  // step kt reads weight slot kt % 3 and activation slot kt % 2
  auto step = [&](const char* ws, const char* as, char* ad, char* wd, int kt) {
    auto hook = [&](int grp) {
      if (grp < 2) {
        load_a(ad, kt + 1, 2 * grp);
        load_a(ad, kt + 1, 2 * grp + 1);
      } else if (grp < 6) {
        load_b(wd, kt + 2, grp - 2);
      }
    };
    mma_step<8, 4, decltype(acc), decltype(hook), true, true>(as, ws, 128 * wr, 64 * wc, lane,
                                                              acc, hook);
    wait_vmcnt<4>();   // everything but step kt + 2's weight loads has landed
    lds_barrier();     // ... for every wave; every wave is done with ws and as
  };
#pragma unroll
  for (int u = 0; u < 4; ++u) load_b(w0, 0, u);
#pragma unroll
  for (int u = 0; u < 4; ++u) load_a(a0, 0, u);
#pragma unroll
  for (int u = 0; u < 4; ++u) load_b(w1, 1, u);
  wait_vmcnt<4>();
  lds_barrier();
  // Six steps per pass.  The passes are straight-line code and the last
  // steps nest, so that the compiler sees which slots can have loads in
  // flight at every fragment read (with a guard on each step it assumed any
  // step could be skipped, and with a branch between two cache policies in
  // the loads it merged the two paths' views; either way it waited for every
  // load before some of the reads).
  int kt = 0;
  for (; kt + 6 <= KT; kt += 6) {
    step(w0, a0, a1, w2, kt);
    step(w1, a1, a0, w0, kt + 1);
    step(w2, a0, a1, w1, kt + 2);
    step(w0, a1, a0, w2, kt + 3);
    step(w1, a0, a1, w0, kt + 4);
    step(w2, a1, a0, w1, kt + 5);
  }
  if (kt < KT) {
    step(w0, a0, a1, w2, kt);
    if (kt + 1 < KT) {
      step(w1, a1, a0, w0, kt + 1);
      if (kt + 2 < KT) {
        step(w2, a0, a1, w1, kt + 2);
        if (kt + 3 < KT) {
          step(w0, a1, a0, w2, kt + 3);
          if (kt + 4 < KT) step(w1, a0, a1, w0, kt + 4);
        }
      }
    }
  }
  wait_vmcnt<0>();   // the past-the-end loads land before the block's LDS is released
  // Epilogue straight from the accumulators: lane holds m-tile row
  // 128 wr + 16 rb + c and 8 consecutive output columns per store.
  const int c = lane & 15, q = lane >> 4;
#pragma unroll
  for (int rb = 0; rb < 8; ++rb) {
    const int r = 128 * wr + 16 * rb + c;
    if (GATEUP) {
      // hh, m-tile-blocked: 64-column block j of the m-tile's 256 rows at
      // row0 * I + j * 256 * 64
      const int col = nt * 128 + 32 * wc + 8 * q;
      bf16x8 v;
#pragma unroll
      for (int p = 0; p < 2; ++p)
#pragma unroll
        for (int i = 0; i < 4; ++i)
          v[4 * p + i] = (bf16)silu_mul(acc[rb][2 * p][i], acc[rb][2 * p + 1][i]);
      __builtin_nontemporal_store(
          v, (bf16x8*)(C + (size_t)row0 * I + (size_t)(col >> 6) * BM * 64 + r * 64 + (col & 63)));
    } else {
#pragma unroll
      for (int p = 0; p < 2; ++p) {
        const int col = nt * 256 + 64 * wc + 32 * p + 8 * q;
        bf16x8 v;
#pragma unroll
        for (int h = 0; h < 2; ++h)
#pragma unroll
          for (int i = 0; i < 4; ++i) v[4 * h + i] = (bf16)acc[rb][2 * p + h][i];
        __builtin_nontemporal_store(v, (bf16x8*)(C + (size_t)(row0 + r) * H + col));
      }
    }
  }
}

// One block per item, XCD-aware (block i on XCD i % 8; the column tiles of
// one m-tile share that XCD's L2, and their K sweeps start at four offsets
// so that they do not all wait on one miss).  The grid is sized from the
// capacity bound of full m-tiles; blocks past the real count exit.
template <bool GATEUP>
__global__ __launch_bounds__(kGemmThreads, 1) void ffn_dense_bf16(
    const bf16* __restrict__ A, const int32_t* __restrict__ gather, int gK, int gT,
    const bf16* __restrict__ W, const int4* __restrict__ full, const int* __restrict__ nfull,
    int KD, int I, int H, int NT, bf16* __restrict__ C) {
  __shared__ __attribute__((aligned(1024))) char w0[kDenseSlot];
  __shared__ __attribute__((aligned(1024))) char w1[kDenseSlot];
  __shared__ __attribute__((aligned(1024))) char w2[kDenseSlot];
  __shared__ __attribute__((aligned(1024))) char a0[kDenseSlot];
  __shared__ __attribute__((aligned(1024))) char a1[kDenseSlot];
  const int b = blockIdx.x;
  const int xcd = b & 7, slot = b >> 3;
  const int mt = (slot / NT) * 8 + xcd;
  const int nt = slot % NT;
  if (mt >= nfull[0]) return;
  dense_item<GATEUP>(w0, w1, w2, a0, a1, A, gather, gK, gT, W, full[mt], nt, KD, I, H, C);
}

// ----------------------- down GEMM: 512-row weight tiles, at most 128 rows --
// The down GEMM's last m-tiles of at most 4 row groups (at most 128 rows:
// half of the full-scale prefill layer's experts) against 512-row weight
// tiles, in a launch of their own between the dense kernel and the main
// one.  Every column tile re-reads the m-tile's hh rows from L2, and those
// loads hold the same per-CU request slots as the weight stream: at 192
// weight rows per tile every weight byte brings two thirds of a byte of
// them, at 512 a quarter.  Accumulators for 128 rows x 512 weight rows need
// eight compute waves, 64 weight rows each; the loads stay on four waves of
// their own (12 waves, 3 per SIMD, 168 registers each), so that a stalled
// 1 KB DMA issue never holds a matrix core.  Two 80 KB stages in two
// separately declared arrays, one step in flight, one barrier per step.
// Measured on 64 experts of 128 rows at the prefill shape: 297-304 us
// against 340-350 us for the main kernel's 192-row tiles.  (The same kernel
// for gate/up, K = 6144, was 7-11 % slower than the main kernel's 256-row
// tiles and is not used there.)
constexpr int kW12Threads = 768;
constexpr int kW12BN = 512;
constexpr int kW12Stage = 80 * 1024;
constexpr int kW12MaxRows = 128;
static_assert(64 * OutTile<kW12BN>::kPitch <= kW12Stage, "half the output tile fits a stage");

template <int G>
__device__ __forceinline__ void down512_item(char* s0, char* s1, const bf16* __restrict__ hh,
                                             const bf16* __restrict__ W, int4 tile, int nt,
                                             int I, int H, bf16* __restrict__ C) {
  constexpr int BN = kW12BN, R = 2 * G;
  constexpr int NA = 4 * G;                  // 8-row hh groups of a step
  constexpr int QB = BN / 8 / 4;             // weight groups per loader per step (16)
  using Out = OutTile<BN>;
  const int e = tile.x, row0 = tile.y, rows = tile.z;
  const bool stream_w = tile.w <= 1;
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int KT = I / kBK;
  const int k_start = ((nt % 2) * KT) / 2;
  auto k_of = [&](int kt) { const int ks = kt + k_start; return ks >= KT ? ks - KT : ks; };
  if (wave >= 8) {
    // Loader l moves hh groups l + 4 i (i < G) and weight groups l + 4 j
    // (j < 16) of every step; lane q fetches chunk swz(row, q & 7) of row
    // 8 g + (q >> 3).  Buffer loads: a 32-bit per-lane byte offset and a
    // scalar one.  hh is m-tile-blocked: K step k of row r at
    // row0 * I + k * rows * 64 + r * 64.  A loader's weight groups are 32
    // weight rows apart.
    const int l = wave - 8, lr = lane >> 3, lc = lane & 7;
    uint32_t voff_a[G];
#pragma unroll
    for (int i = 0; i < G; ++i) {
      const int r = 8 * (l + 4 * i) + lr;   // rows past the tile: clamped, never stored
      voff_a[i] = ((uint32_t)min(r, rows - 1) * kBK + swz(r, lc) * 8) * 2;
    }
    const int rb0 = 8 * l + lr;
    const uint32_t voff_b = ((uint32_t)(nt * BN + rb0) * (uint32_t)I + swz(rb0, lc) * 8) * 2;
    const uint32_t b_stride = 32u * (uint32_t)I * 2;
    const uint32_t a_step = (uint32_t)rows * kBK * 2;
    const __amdgpu_buffer_rsrc_t rs_a = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(hh + (size_t)row0 * I), (short)0, 0x7fffffff, kBufferFlags);
    const __amdgpu_buffer_rsrc_t rs_w = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(W + (size_t)e * H * I), (short)0, 0x7fffffff, kBufferFlags);
    auto issue = [&](int kt, char* dst) {
      const uint32_t k = (uint32_t)k_of(kt);
#pragma unroll
      for (int j = 0; j < QB; ++j) {   // weights first: the HBM wait
        lds_void* d = (lds_void*)(dst + (NA + l + 4 * j) * 1024);
        const uint32_t so = k * (kBK * 2) + (uint32_t)j * b_stride;
        if (stream_w)
          __builtin_amdgcn_raw_ptr_buffer_load_lds(rs_w, d, 16, voff_b, so, 0, kCachePolicyNT);
        else
          __builtin_amdgcn_raw_ptr_buffer_load_lds(rs_w, d, 16, voff_b, so, 0, 0);
      }
#pragma unroll
      for (int i = 0; i < G; ++i)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rs_a, (lds_void*)(dst + (l + 4 * i) * 1024),
                                                 16, voff_a[i], k * a_step, 0, 0);
    };
    issue(0, s0);
    for (int kt = 0; kt < KT; ++kt) {
      wait_vmcnt<0>();   // step kt has landed (the only one in flight)
      lds_barrier();     // publish it; the compute waves are done with step kt - 1
      if (kt + 1 < KT) issue(kt + 1, (kt + 1) & 1 ? s1 : s0);
    }
    lds_barrier();       // the compute waves are done: the stages take the output
    lds_barrier();       // ... which is now written
  } else {
    f32x4 acc[R][4];
#pragma unroll
    for (int i = 0; i < R; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) acc[i][j] = f32x4{0, 0, 0, 0};
    for (int kt = 0; kt < KT; ++kt) {
      lds_barrier();
      const char* src = kt & 1 ? s1 : s0;
      mma_step<R, 4, decltype(acc), NoHook, (G == 4)>(src, src + NA * 1024, 0, 64 * wave, lane,
                                                       acc);
    }
    lds_barrier();       // every wave is done reading the stages
    // rows [0, 64) through s0, [64, 128) through s1
    const int c = lane & 15, q = lane >> 4;
#pragma unroll
    for (int rb = 0; rb < R; ++rb) {
      const Out out{rb < 4 ? s0 : s1};
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int cb = 0; cb < 4; ++cb)
          out.put((rb & 3) * 16 + 4 * q + i, 64 * wave + 16 * cb + c, acc[rb][cb][i]);
    }
    lds_barrier();
  }
  for (int j = threadIdx.x; j < rows * Out::kChunks; j += kW12Threads) {
    const int r = j / Out::kChunks, cc = j - r * Out::kChunks;
    const i32x4 v = *(const i32x4*)((r < 64 ? s0 : s1) + (r & 63) * Out::kPitch + cc * 16);
    __builtin_nontemporal_store(v, (i32x4*)(C + (size_t)(row0 + r) * H + nt * BN + cc * 8));
  }
}

// One block per (narrow m-tile, 512-row weight tile), XCD-aware as the other
// GEMM kernels.  The narrow m-tiles are tiles[nwide[0] ..] (nnarrow[0] of
// them); the grid is sized from the capacity bound (one per expert), surplus
// blocks exit.
__global__ __launch_bounds__(kW12Threads, 1) void ffn_down512_bf16(
    const bf16* __restrict__ hh, const bf16* __restrict__ W, const int4* __restrict__ tiles,
    const int* __restrict__ nwide, const int* __restrict__ nnarrow, int I, int H, int NT,
    bf16* __restrict__ C) {
  __shared__ __attribute__((aligned(1024))) char s0[kW12Stage];
  __shared__ __attribute__((aligned(1024))) char s1[kW12Stage];
  const int b = blockIdx.x;
  const int xcd = b & 7, slot = b >> 3;
  const int mt = (slot / NT) * 8 + xcd;
  const int nt = slot % NT;
  if (mt >= *nnarrow) return;
  const int4 tile = tiles[*nwide + mt];
  switch ((tile.z + 31) >> 5) {
    case 1: down512_item<1>(s0, s1, hh, W, tile, nt, I, H, C); break;
    case 2: down512_item<2>(s0, s1, hh, W, tile, nt, I, H, C); break;
    case 3: down512_item<3>(s0, s1, hh, W, tile, nt, I, H, C); break;
    case 4: down512_item<4>(s0, s1, hh, W, tile, nt, I, H, C); break;
    default: break;
  }
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
  // Each thread stages the same tile elements at every K step: column
  // kk = tid % TK of rows tid / TK + RS j.  Their row addresses (the gather
  // resolved once) are set up before the loop, and the next step's values
  // are fetched into registers while the current step is multiplied.
  constexpr int NA = TM * TK / kThreads, NW = NB * TK / kThreads;
  static_assert(kThreads % TK == 0 && NA * kThreads == TM * TK && NW * kThreads == NB * TK,
                "tile elements split evenly over the threads");
  const int kk = threadIdx.x % TK, r0 = threadIdx.x / TK;
  constexpr int RS = kThreads / TK;   // rows apart between a thread's elements
  const float* arow[NA];
  const float* wrow[NW];
#pragma unroll
  for (int j = 0; j < NA; ++j) {
    const int r = r0 + RS * j;
    const int ar = r >= rows ? -1 : gather ? min(max(gather[row0 + r], 0) / gK, gT - 1) : row0 + r;
    arow[j] = ar < 0 ? nullptr : A + (size_t)ar * KD + kk;
  }
#pragma unroll
  for (int j = 0; j < NW; ++j) {
    const int c = r0 + RS * j;
    const int n = n0 + (c % TN);
    const int wr = (GATEUP && c >= TN) ? I + n : n;
    wrow[j] = n < NOUT ? wexp + (size_t)wr * KD + kk : nullptr;
  }
  float ra[NA], rw[NW];
  auto fetch = [&](int k0) {
    const bool kin = k0 + kk < KD;
#pragma unroll
    for (int j = 0; j < NA; ++j) ra[j] = (arow[j] && kin) ? arow[j][k0] : 0.0f;
#pragma unroll
    for (int j = 0; j < NW; ++j) rw[j] = (wrow[j] && kin) ? wrow[j][k0] : 0.0f;
  };
  float acc[2][2][2] = {};
  fetch(0);
  for (int k0 = 0; k0 < KD; k0 += TK) {
#pragma unroll
    for (int j = 0; j < NA; ++j) As[kk][r0 + RS * j] = ra[j];
#pragma unroll
    for (int j = 0; j < NW; ++j) Bs[kk][r0 + RS * j] = rw[j];
    __syncthreads();
    if (k0 + TK < KD) fetch(k0 + TK);
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
inline size_t max_full(int rows_cap) { return (size_t)rows_cap / kBmBf16 + 1; }
// Full m-tiles go to the dense kernel when both GEMMs' weight rows split
// into its 256-row tiles (bf16 only).
inline bool dense_shapes(int dtype, int H, int I) {
  return dtype == MOE_BF16 && (2 * I) % kDenseBN == 0 && H % kDenseBN == 0;
}

}  // namespace

// The workspace of moe_expert_ffn_gather_noalloc: one fixed array per GPU,
// alive until the process ends.  Host code never uses the name `scratch`
// (a host-side stand-in); it uses the device address looked up once per
// device with that device current.
static __device__ __align__(256) char scratch[MOE_EXPERT_FFN_NOALLOC_SCRATCH_BYTES];

namespace {
constexpr int kMaxDevices = 256;
std::mutex g_scratch_mu;
void* g_scratch_addr[kMaxDevices];
}  // namespace

hipError_t noalloc_scratch(void** addr) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  if (!g_scratch_addr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    g_scratch_addr[dev] = p;
  }
  *addr = g_scratch_addr[dev];
  return hipSuccess;
}

// Workspace: [0, 256) the two tile counts; the tile list; the full-tile
// list (bf16); hh [rows_cap][I].
size_t ffn_ws_bytes(int rows_cap, int n_ffn, int I, int dtype) {
  const int es = dtype == MOE_BF16 ? 2 : 4;
  return 256 + align256(max_mtiles(rows_cap, n_ffn, ffn_bm(dtype)) * sizeof(int4)) +
         (dtype == MOE_BF16 ? align256(max_full(rows_cap) * sizeof(int4)) : 0) +
         align256((size_t)rows_cap * I * es);
}

hipError_t launch_expert_ffn(const void* x_perm, const int32_t* gather, int gK, int gT,
                             const int32_t* offsets, int rows_cap, int n_ffn, int H, int I,
                             const void* w13, const void* w2, int dtype, void* y_perm, void* ws,
                             hipStream_t s) {
  const int bm = ffn_bm(dtype);
  const size_t mtmax = max_mtiles(rows_cap, n_ffn, bm);
  const size_t fmax = dtype == MOE_BF16 ? max_full(rows_cap) : 0;
  int* ntiles = (int*)ws;
  int* nfull = (int*)ws + 1;
  int4* tiles = (int4*)((char*)ws + 256);
  int4* full = (int4*)((char*)tiles + align256(mtmax * sizeof(int4)));
  void* hh = (char*)full + align256(fmax * sizeof(int4));
  // An expert holds at most one row per token: the gather path knows the
  // tokens, so a batch of fewer than 256 tokens has no full m-tile.
  const int rows_per_expert = gather ? min(rows_cap, gT) : rows_cap;
  // (and the dense kernel's 31-bit buffer byte offsets must reach: token
  // rows of x and the weights of one expert)
  const bool dense = dense_shapes(dtype, H, I) && rows_per_expert >= kBmBf16 &&
                     (size_t)(gather ? gT : kBmBf16) * H * 2 < ((size_t)1 << 31) &&
                     (size_t)2 * I * H * 2 < ((size_t)1 << 31);
  // Where the average FFN expert would have under 32 rows even if every
  // pick went to one (decode), every tile is a single group: the 128-row
  // tiles' deep rings stream the weights best, and neither the wide tiles
  // nor the 512-row down tiles are used.  The 512-row kernel's buffer loads
  // take 31-bit byte offsets within one expert's w2 and one m-tile's hh.
  const bool enough_rows = (long long)rows_cap >= 32LL * n_ffn;
  const bool down512 = dtype == MOE_BF16 && enough_rows && H % kW12BN == 0 &&
                       (size_t)H * I * 2 < ((size_t)1 << 31);
  MOE_LAUNCH("ffn_tiles", s,
             ffn_tiles<<<1, 1024, 0, s>>>(offsets, n_ffn, bm, rows_cap, (int)mtmax, tiles,
                                          ntiles, (int)fmax, dense ? full : nullptr, nfull,
                                          down512 ? kW12MaxRows : 0));
  if (dtype == MOE_BF16) {
    // with the full m-tiles in the dense kernel, at most one m-tile per
    // expert is left for this one
    const unsigned groups = ceil_div(dense ? std::min(mtmax, (size_t)n_ffn) : mtmax, 8);
    const int nt1 = I / 64, nt2 = H / kBN;
    const unsigned dense_groups = ceil_div(fmax, 8) * 8;   // full m-tiles, rounded to 8 XCDs
    if (dense) {
      const unsigned dense_grid = dense_groups * (2 * I / kDenseBN);
      // the full m-tiles: 256 x 256 blocks, before the other tiles
      MOE_LAUNCH("ffn_gateup_dense_bf16", s,
                 ffn_dense_bf16<true><<<dense_grid, kGemmThreads, 0, s>>>(
                                                (const bf16*)x_perm, gather, gK, gT,
                                                (const bf16*)w13, full, nfull, H, I, H,
                                                2 * I / kDenseBN, (bf16*)hh));
    }
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
    const bool wide_gu = enough_rows && (2 * I) % kBNGateUpWide == 0;
    const bool wide_dn = enough_rows && H % kBNWide == 0;
    const unsigned grid_gu = groups * 8 * nt1, grid_dn = groups * 8 * nt2;
    if (wide_gu)
      MOE_LAUNCH("ffn_gateup_bf16", s,
                 ffn_mfma_bf16<true, kWideGroupsGateUp><<<grid_gu, kGemmThreads, 0, s>>>(
                     (const bf16*)x_perm, gather, gK, gT, (const bf16*)w13, tiles, ntiles, H, I,
                     H, nt1, (bf16*)hh));
    else
      MOE_LAUNCH("ffn_gateup_bf16", s,
                 ffn_mfma_bf16<true, 0><<<grid_gu, kGemmThreads, 0, s>>>(
                     (const bf16*)x_perm, gather, gK, gT, (const bf16*)w13, tiles, ntiles, H, I,
                     H, nt1, (bf16*)hh));
    if (dense)
      MOE_LAUNCH("ffn_down_dense_bf16", s,
                 ffn_dense_bf16<false><<<dense_groups * (H / kDenseBN), kGemmThreads, 0, s>>>(
                                              (const bf16*)hh, nullptr, 1, 1, (const bf16*)w2,
                                              full, nfull, I, I, H, H / kDenseBN,
                                              (bf16*)y_perm));
    // the down GEMM's narrow m-tiles (at most 128 rows) in 512-row tiles;
    // the main kernel takes the first part of tiles[] (ntiles[3] of them)
    if (down512)
      MOE_LAUNCH("ffn_down_narrow_bf16", s,
                 ffn_down512_bf16<<<ceil_div(std::min(mtmax, (size_t)n_ffn), 8) * 8 *
                                        (H / kW12BN),
                                    kW12Threads, 0, s>>>(
                     (const bf16*)hh, (const bf16*)w2, tiles, ntiles + 3, ntiles + 4, I, H,
                     H / kW12BN, (bf16*)y_perm));
    if (wide_dn)
      MOE_LAUNCH("ffn_down_bf16", s,
                 ffn_mfma_bf16<false, kWideGroups><<<grid_dn, kGemmThreads, 0, s>>>(
                     (const bf16*)hh, nullptr, 1, 1, (const bf16*)w2, tiles, ntiles + 3, I, I, H,
                     nt2, (bf16*)y_perm));
    else
      MOE_LAUNCH("ffn_down_bf16", s,
                 ffn_mfma_bf16<false, 0><<<grid_dn, kGemmThreads, 0, s>>>(
                     (const bf16*)hh, nullptr, 1, 1, (const bf16*)w2, tiles, ntiles + 3, I, I, H,
                     nt2, (bf16*)y_perm));
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
