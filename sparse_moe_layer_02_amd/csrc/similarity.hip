// Router weight similarity: the pairwise cosine similarity of the experts'
// router weight vectors, the diagnostic the LongCat-Flash report watches for
// router stability (Technical Report notes, Key claims and Method [§3.1.3
// Router Stability]: high similarity marks a router that the load-balance
// term has collapsed).
//
//   dot[i][j] = sum_h w[i][h] * w[j][h]        (the Gram matrix of w_router)
//   sim[i][j] = dot[i][j] / (|w_i| * |w_j|), 0 when either norm is 0
//   mean      = average of sim[i][j] over i != j
//
// Three kernels on one stream:
//   1. sim_gram: upper-triangle 64 x 64 tiles of the Gram matrix on fp32
//      matrix cores (v_mfma_f32_16x16x4_f32), K split over blockIdx.y so that
//      a 768-row router fills the chip; each split writes its partial tile.
//   2. sim_finish: four blocks per triangle tile (16 rows each) sum the
//      partials in split order, divide by the row norms (from the diagonal
//      partials), write the tile and its mirror image, and their share of the
//      off-diagonal sum (fp64).
//   3. sim_mean: one block sums those shares in a fixed order.
// No atomics: the result is bitwise reproducible, and sim[i][j] and
// sim[j][i] are computed from the same partials, so sim is exactly symmetric.
#include "moe_internal.h"

namespace moe {
namespace {

constexpr int kSimTile = 64;     // output tile edge
constexpr int kSimK = 32;        // k per LDS stage (128-byte row pieces)
constexpr int kSimPitch = 36;    // LDS row pitch in floats: 16 rows x b128 reads hit 16 bank quads
constexpr int kSimThreads = 256; // 4 waves, 2 x 2 over the tile, 32 x 32 each
constexpr int kSimTargetBlocks = 640;
constexpr int kFinRows = 16;                          // tile rows per finishing block
constexpr int kFinBlocks = kSimTile / kFinRows;       // finishing blocks per tile
constexpr int kFinPer = kFinRows * kSimTile / 256;    // elements per finishing thread

typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f4;

struct SimPlan {
  int nt;       // tiles per side
  int ntri;     // upper-triangle tiles
  int splits;   // K splits
  int kchunk;   // floats of K per split (multiple of kSimK)
  size_t part_off, sum_off, bytes;
};

inline size_t align256(size_t v) { return (v + 255) & ~size_t(255); }

SimPlan sim_plan(int E, int H) {
  SimPlan p;
  p.nt = (E + kSimTile - 1) / kSimTile;
  p.ntri = p.nt * (p.nt + 1) / 2;
  const int steps = (H + kSimK - 1) / kSimK;
  int want = (kSimTargetBlocks + p.ntri - 1) / p.ntri;
  want = want < 1 ? 1 : (want > steps ? steps : want);
  const int per = (steps + want - 1) / want;
  p.kchunk = per * kSimK;
  p.splits = (steps + per - 1) / per;
  p.part_off = 0;
  p.sum_off = align256((size_t)p.splits * p.ntri * kSimTile * kSimTile * sizeof(float));
  p.bytes = p.sum_off + align256((size_t)p.ntri * kFinBlocks * sizeof(double));
  return p;
}

// Upper-triangle tile index of (ti, tj), ti <= tj, row-major over ti.
__device__ __forceinline__ int tri_index(int ti, int tj, int nt) {
  return ti * nt - ti * (ti - 1) / 2 + (tj - ti);
}

__global__ __launch_bounds__(kSimThreads) void sim_gram(const float* __restrict__ w, int E, int H,
                                                        int nt, int kchunk,
                                                        float* __restrict__ part) {
  __shared__ float lds[2][2][kSimTile * kSimPitch];  // [buffer][A/B][row * pitch + k]
  // Tile (ti, tj) from the linear triangle index.
  int p = blockIdx.x, ti = 0;
  while (p >= nt - ti) { p -= nt - ti; ++ti; }
  const int tj = ti + p;
  const int split = blockIdx.y;
  const int k_begin = split * kchunk;
  const int k_end = min(H, k_begin + kchunk);
  const int nsteps = (k_end - k_begin + kSimK - 1) / kSimK;

  const int tid = threadIdx.x;
  const int lrow = tid >> 3;          // 0..31; rows lrow and lrow + 32
  const int lcol = (tid & 7) * 4;     // float offset in the 32-float stage
  const int rowA0 = ti * kSimTile, rowB0 = tj * kSimTile;

  f4 ra[2], rb[2];
  auto load = [&](int step) {
    const int k = k_begin + step * kSimK + lcol;
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      const int r = lrow + 32 * q;
      const f4 z = {0.f, 0.f, 0.f, 0.f};
      ra[q] = (rowA0 + r < E && k < k_end) ? *(const f4*)(w + (size_t)(rowA0 + r) * H + k) : z;
      rb[q] = (rowB0 + r < E && k < k_end) ? *(const f4*)(w + (size_t)(rowB0 + r) * H + k) : z;
    }
  };
  auto store = [&](int buf) {
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      const int r = lrow + 32 * q;
      *(f4*)&lds[buf][0][r * kSimPitch + lcol] = ra[q];
      *(f4*)&lds[buf][1][r * kSimPitch + lcol] = rb[q];
    }
  };

  const int wave = tid >> 6, lane = tid & 63;
  const int wm = (wave >> 1) * 32, wn = (wave & 1) * 32;  // wave's 32 x 32 sub-tile
  const int fr = lane & 15, fg = lane >> 4;               // fragment row, k group
  f32x4 acc[2][2];
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int b = 0; b < 2; ++b) acc[a][b] = f32x4{0.f, 0.f, 0.f, 0.f};

  load(0);
  store(0);
  __syncthreads();
  for (int s = 0; s < nsteps; ++s) {
    const int buf = s & 1;
    if (s + 1 < nsteps) load(s + 1);
    // The MFMA's lane group g supplies k index g of each 4-k product; here it
    // supplies k = 16 * half + 4 * g + j for product j, the same mapping on
    // both operands, so every k of the stage enters each dot product once.
#pragma unroll
    for (int half = 0; half < 2; ++half) {
      f4 fa[2], fb[2];
#pragma unroll
      for (int m = 0; m < 2; ++m)
        fa[m] = *(const f4*)&lds[buf][0][(wm + 16 * m + fr) * kSimPitch + 16 * half + 4 * fg];
#pragma unroll
      for (int n = 0; n < 2; ++n)
        fb[n] = *(const f4*)&lds[buf][1][(wn + 16 * n + fr) * kSimPitch + 16 * half + 4 * fg];
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int m = 0; m < 2; ++m)
#pragma unroll
          for (int n = 0; n < 2; ++n)
            acc[m][n] = __builtin_amdgcn_mfma_f32_16x16x4f32(fa[m][j], fb[n][j], acc[m][n], 0, 0, 0);
    }
    if (s + 1 < nsteps) store(buf ^ 1);
    __syncthreads();
  }

  // acc[m][n] lane layout: element r is tile row wm + 16m + 4*fg + r (an A
  // row), column wn + 16n + fr (a B row).
  float* out = part + ((size_t)split * (gridDim.x) + blockIdx.x) * (kSimTile * kSimTile);
#pragma unroll
  for (int m = 0; m < 2; ++m)
#pragma unroll
    for (int n = 0; n < 2; ++n)
#pragma unroll
      for (int r = 0; r < 4; ++r)
        out[(wm + 16 * m + 4 * fg + r) * kSimTile + wn + 16 * n + fr] = acc[m][n][r];
}

// Block (tile, y) finishes rows 16y..16y+15 of triangle tile (ti, tj): sums
// the K-split partials in split order, takes the row norms it needs from the
// diagonal tiles' partials (every block sums them in the same order, so a
// norm is bitwise the same wherever it is used), writes cos for its part of
// tile (ti, tj) and, through LDS, the mirror image in tile (tj, ti), and
// leaves its share of the off-diagonal sum (fp64) in part_sum.  Inside a
// diagonal tile (a, b) and (b, a) both take the partial at (min, max), so sim
// is exactly symmetric.

__global__ __launch_bounds__(256) void sim_finish(const float* __restrict__ part, int E, int nt,
                                                  int splits, float* __restrict__ sim,
                                                  double* __restrict__ part_sum) {
  constexpr int kT2 = kSimTile * kSimTile;
  __shared__ float norm_a[kFinRows], norm_b[kSimTile];
  __shared__ float tile[kFinRows][kSimTile + 1];
  __shared__ double red[256];
  const int ntri = gridDim.x;
  int p = blockIdx.x, ti = 0;
  while (p >= nt - ti) { p -= nt - ti; ++ti; }
  const int tj = ti + p;
  const int a0 = blockIdx.y * kFinRows;
  const int tid = threadIdx.x;
  const size_t split_stride = (size_t)ntri * kT2;
  if (tid < kFinRows + kSimTile) {
    const bool is_a = tid < kFinRows;
    const int a = is_a ? a0 + tid : tid - kFinRows;
    const int t = is_a ? ti : tj;
    const float* d = part + (size_t)tri_index(t, t, nt) * kT2 + a * kSimTile + a;
    float g = 0.f;
    for (int sp = 0; sp < splits; ++sp) g += d[sp * split_stride];
    if (is_a) norm_a[tid] = sqrtf(g);
    else norm_b[a] = sqrtf(g);
  }
  __syncthreads();

  const bool diag = ti == tj;
  const float* src = part + (size_t)blockIdx.x * kT2;
  int off_e[kFinPer];
  float g[kFinPer];
#pragma unroll
  for (int q = 0; q < kFinPer; ++q) {
    const int e = tid + 256 * q;
    const int a = a0 + e / kSimTile, b = e % kSimTile;
    off_e[q] = diag ? min(a, b) * kSimTile + max(a, b) : a * kSimTile + b;
    g[q] = 0.f;
  }
  for (int sp = 0; sp < splits; ++sp)
#pragma unroll
    for (int q = 0; q < kFinPer; ++q) g[q] += src[sp * split_stride + off_e[q]];

  double off = 0.0;
#pragma unroll
  for (int q = 0; q < kFinPer; ++q) {
    const int e = tid + 256 * q;
    const int ra = e / kSimTile, b = e % kSimTile;
    const int i = ti * kSimTile + a0 + ra, j = tj * kSimTile + b;
    const float na = norm_a[ra], nb = norm_b[b];
    const float c = (na > 0.f && nb > 0.f) ? g[q] / (na * nb) : 0.f;
    tile[ra][b] = c;
    if (i < E && j < E) {
      sim[(size_t)i * E + j] = c;
      if (i != j) off += diag ? (double)c : 2.0 * (double)c;
    }
  }
  if (!diag) {
    __syncthreads();
#pragma unroll
    for (int q = 0; q < kFinPer; ++q) {
      const int e = tid + 256 * q;
      const int b = e / kFinRows, ra = e % kFinRows;
      const int i = ti * kSimTile + a0 + ra, j = tj * kSimTile + b;
      if (i < E && j < E) sim[(size_t)j * E + i] = tile[ra][b];
    }
  }
  red[tid] = off;
  __syncthreads();
  for (int w = 128; w > 0; w >>= 1) {
    if (tid < w) red[tid] += red[tid + w];
    __syncthreads();
  }
  if (tid == 0) part_sum[blockIdx.x * gridDim.y + blockIdx.y] = red[0];
}

__global__ __launch_bounds__(256) void sim_mean(const double* __restrict__ part_sum, int n,
                                                int E, float* __restrict__ mean) {
  __shared__ double red[256];
  double s = 0.0;
  for (int i = threadIdx.x; i < n; i += 256) s += part_sum[i];
  red[threadIdx.x] = s;
  __syncthreads();
  for (int w = 128; w > 0; w >>= 1) {
    if ((int)threadIdx.x < w) red[threadIdx.x] += red[threadIdx.x + w];
    __syncthreads();
  }
  if (threadIdx.x == 0) *mean = E > 1 ? (float)(red[0] / ((double)E * (double)(E - 1))) : 0.f;
}

}  // namespace

size_t similarity_ws_bytes(int E, int H) { return sim_plan(E, H).bytes; }

hipError_t launch_router_similarity(const float* w, int E, int H, float* sim, float* mean,
                                    void* ws, hipStream_t s) {
  const SimPlan p = sim_plan(E, H);
  char* base = (char*)ws;
  float* part = (float*)(base + p.part_off);
  double* part_sum = (double*)(base + p.sum_off);
  MOE_LAUNCH("sim_gram", s,
             sim_gram<<<dim3(p.ntri, p.splits), kSimThreads, 0, s>>>(w, E, H, p.nt, p.kchunk, part));
  MOE_LAUNCH("sim_finish", s,
             sim_finish<<<dim3(p.ntri, kFinBlocks), 256, 0, s>>>(part, E, p.nt, p.splits, sim,
                                                                 part_sum));
  MOE_LAUNCH("sim_mean", s, sim_mean<<<1, 256, 0, s>>>(part_sum, p.ntri * kFinBlocks, E, mean));
  return hipGetLastError();
}

}  // namespace moe
