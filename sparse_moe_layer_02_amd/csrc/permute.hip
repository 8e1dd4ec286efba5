// Dispatch on one GPU (LongCat-Flash Technical Report notes, Key claims
// [§2.2]: the dispatch half of dispatch/combine): every FFN selection (t, k)
// gets a row in an expert-major buffer; inside one expert, rows follow the
// token order.  The order must not depend on atomic arrival, so ranks are
// computed from bitmasks:
//   block b = tokens [64b, 64b+64), one wave; lane l is token 64b+l.
//   mask[e] (LDS, 64 bits) = OR of (1 << l) over the lanes that chose e.
//   A token chooses an expert at most once, so
//     rank of (t, e) inside block b = popcount(mask[e] & lanes below l),
//     cnt[e][b]                      = popcount(mask[e]).
//   row(t, e) = offsets[e] + sum_{b' < b} cnt[e][b'] + rank.
// Kernels: hist (cnt), scan over blocks per expert, scan over experts
// (offsets), scatter (slot_row, row_src), and, when a grouped copy is asked
// for, gather (x rows, one read of x[t] feeding all of its rows).
#include "moe_internal.h"

namespace moe {
namespace {

constexpr int kBlockTokens = 64;

// LDS mask table of one wave: one 64-bit word per FFN expert.
__device__ __forceinline__ void build_masks(unsigned long long* mask, const int32_t* idx, int T,
                                            int K, int n_ffn, int blk) {
  const int lane = threadIdx.x;
  for (int e = lane; e < n_ffn; e += kWave) mask[e] = 0ull;
  __syncthreads();
  const int t = blk * kBlockTokens + lane;
  if (t < T) {
    const int32_t* row = idx + (size_t)t * K;
    for (int k = 0; k < K; ++k) {
      int e = row[k];
      if ((unsigned)e < (unsigned)n_ffn) atomicOr(&mask[e], 1ull << lane);
    }
  }
  __syncthreads();
}

__global__ __launch_bounds__(kWave) void perm_hist(const int32_t* __restrict__ idx, int T, int K,
                                                   int n_ffn, int nblk,
                                                   int32_t* __restrict__ cnt) {
  extern __shared__ unsigned long long mask[];
  const int blk = blockIdx.x;
  build_masks(mask, idx, T, K, n_ffn, blk);
  for (int e = threadIdx.x; e < n_ffn; e += kWave)
    cnt[(size_t)e * nblk + blk] = __popcll(mask[e]);
}

// One wave per expert: exclusive scan of cnt[e][0..nblk) in place; tot[e].
__global__ __launch_bounds__(256) void perm_scan_blocks(int32_t* __restrict__ cnt, int nblk,
                                                        int n_ffn, int32_t* __restrict__ tot) {
  const int lane = threadIdx.x & (kWave - 1);
  const int e = blockIdx.x * (blockDim.x / kWave) + threadIdx.x / kWave;
  if (e >= n_ffn) return;
  int32_t* row = cnt + (size_t)e * nblk;
  int carry = 0;
  for (int base = 0; base < nblk; base += kWave) {
    const int b = base + lane;
    const int v = b < nblk ? row[b] : 0;
    int incl = v;
#pragma unroll
    for (int off = 1; off < kWave; off <<= 1) {
      int o = __shfl_up(incl, off);
      if (lane >= off) incl += o;
    }
    if (b < nblk) row[b] = carry + incl - v;
    carry += __shfl(incl, kWave - 1);
  }
  if (lane == 0) tot[e] = carry;
}

// One block: offsets = exclusive scan of tot over experts, offsets[n] = total.
__global__ __launch_bounds__(1024) void perm_scan_experts(const int32_t* __restrict__ tot,
                                                          int n_ffn,
                                                          int32_t* __restrict__ offsets) {
  __shared__ int part[1024];
  const int tid = threadIdx.x;
  const int per = (n_ffn + 1023) / 1024;
  const int lo = min(n_ffn, tid * per), hi = min(n_ffn, lo + per);
  int s = 0;
  for (int e = lo; e < hi; ++e) s += tot[e];
  part[tid] = s;
  __syncthreads();
  for (int off = 1; off < 1024; off <<= 1) {
    int v = tid >= off ? part[tid - off] : 0;
    __syncthreads();
    part[tid] += v;
    __syncthreads();
  }
  int run = part[tid] - s;  // exclusive prefix of this thread's chunk
  for (int e = lo; e < hi; ++e) {
    offsets[e] = run;
    run += tot[e];
  }
  if (tid == 1023) offsets[n_ffn] = part[1023];
}

__global__ __launch_bounds__(kWave) void perm_scatter(const int32_t* __restrict__ idx, int T,
                                                      int K, int n_ffn, int nblk,
                                                      const int32_t* __restrict__ pre,
                                                      const int32_t* __restrict__ offsets,
                                                      int32_t* __restrict__ row_src,
                                                      int32_t* __restrict__ slot_row) {
  extern __shared__ unsigned long long mask[];
  const int blk = blockIdx.x;
  build_masks(mask, idx, T, K, n_ffn, blk);
  const int lane = threadIdx.x;
  const int t = blk * kBlockTokens + lane;
  if (t >= T) return;
  const unsigned long long below = (1ull << lane) - 1ull;
  for (int k = 0; k < K; ++k) {
    const int s = t * K + k;
    const int e = idx[s];
    if ((unsigned)e < (unsigned)n_ffn) {   // other ids: not an FFN pick
      const int row = offsets[e] + pre[(size_t)e * nblk + blk] + __popcll(mask[e] & below);
      slot_row[s] = row;
      row_src[row] = s;
    } else {
      slot_row[s] = -1;
    }
  }
}

// T <= 64 (decode): the tokens are one 64-token block, so the histogram,
// both scans and the scatter fit one workgroup -- one launch instead of four
// (the four cost ~27 us at 64 tokens, almost all launch latency).  Wave 0
// (lane = token) builds the masks and scatters; all 1024 threads scan the
// experts.  The rows are those of the general path: offsets[e] +
// popcount(mask[e] & lanes below).  LDS: n_ffn masks, then n_ffn offsets.
__global__ __launch_bounds__(1024) void perm_small(const int32_t* __restrict__ idx, int T, int K,
                                                   int n_ffn, int32_t* __restrict__ offsets,
                                                   int32_t* __restrict__ row_src,
                                                   int32_t* __restrict__ slot_row) {
  extern __shared__ unsigned long long mask[];
  int* off = (int*)(mask + n_ffn);
  __shared__ int part[1024];
  const int tid = threadIdx.x;
  for (int e = tid; e < n_ffn; e += 1024) mask[e] = 0ull;
  __syncthreads();
  if (tid < kWave && tid < T) {
    const int32_t* row = idx + (size_t)tid * K;
    for (int k = 0; k < K; ++k) {
      const int e = row[k];
      if ((unsigned)e < (unsigned)n_ffn) atomicOr(&mask[e], 1ull << tid);
    }
  }
  __syncthreads();
  // exclusive scan of the per-expert counts: a chunk of experts per thread
  const int per = (n_ffn + 1023) / 1024;
  const int lo = min(n_ffn, tid * per), hi = min(n_ffn, lo + per);
  int sum = 0;
  for (int e = lo; e < hi; ++e) sum += __popcll(mask[e]);
  part[tid] = sum;
  __syncthreads();
  for (int o = 1; o < 1024; o <<= 1) {
    const int v = tid >= o ? part[tid - o] : 0;
    __syncthreads();
    part[tid] += v;
    __syncthreads();
  }
  int run = part[tid] - sum;
  for (int e = lo; e < hi; ++e) {
    off[e] = run;
    offsets[e] = run;
    run += __popcll(mask[e]);
  }
  if (tid == 1023) offsets[n_ffn] = part[1023];
  __syncthreads();
  if (tid < kWave && tid < T) {
    const unsigned long long below = (1ull << tid) - 1ull;
    for (int k = 0; k < K; ++k) {
      const int s = tid * K + k;
      const int e = idx[s];
      if ((unsigned)e < (unsigned)n_ffn) {
        const int r = off[e] + __popcll(mask[e] & below);
        slot_row[s] = r;
        row_src[r] = s;
      } else {
        slot_row[s] = -1;
      }
    }
  }
}

// One block per token: x[t] is read once and written to each of its FFN rows.
template <int VEC_PER_THREAD>
__global__ __launch_bounds__(256) void perm_gather(const i32x4* __restrict__ x, int row_vecs,
                                                   int K, const int32_t* __restrict__ slot_row,
                                                   i32x4* __restrict__ x_perm) {
  const int t = blockIdx.x;
  const i32x4* src = x + (size_t)t * row_vecs;
  i32x4 v[VEC_PER_THREAD];
#pragma unroll
  for (int j = 0; j < VEC_PER_THREAD; ++j) {
    int c = threadIdx.x + 256 * j;
    if (c < row_vecs) v[j] = src[c];
  }
  for (int k = 0; k < K; ++k) {
    const int row = slot_row[(size_t)t * K + k];
    if (row < 0) continue;
    i32x4* dst = x_perm + (size_t)row * row_vecs;
#pragma unroll
    for (int j = 0; j < VEC_PER_THREAD; ++j) {
      int c = threadIdx.x + 256 * j;
      // non-temporal: streamed out now, not written back during the GEMM
      if (c < row_vecs) __builtin_nontemporal_store(v[j], dst + c);
    }
  }
}

// Rows longer than the register-resident path allows: copy through memory.
__global__ __launch_bounds__(256) void perm_gather_long(const i32x4* __restrict__ x,
                                                        int row_vecs, int K,
                                                        const int32_t* __restrict__ slot_row,
                                                        i32x4* __restrict__ x_perm) {
  const int t = blockIdx.x;
  const i32x4* src = x + (size_t)t * row_vecs;
  for (int k = 0; k < K; ++k) {
    const int row = slot_row[(size_t)t * K + k];
    if (row < 0) continue;
    i32x4* dst = x_perm + (size_t)row * row_vecs;
    for (int c = threadIdx.x; c < row_vecs; c += 256) __builtin_nontemporal_store(src[c], dst + c);
  }
}

inline size_t align256(size_t b) { return (b + 255) & ~(size_t)255; }

}  // namespace

size_t permute_ws_bytes(int T, int K, int n_ffn) {
  (void)K;
  const size_t nblk = (size_t)(T + kBlockTokens - 1) / kBlockTokens;
  return align256((size_t)n_ffn * nblk * 4) + align256((size_t)n_ffn * 4 + 4);
}

hipError_t launch_permute(const void* x, int dtype, const int32_t* idx, int T, int H, int K,
                          int n_ffn, int32_t* offsets, void* x_perm, int32_t* row_src,
                          int32_t* slot_row, void* ws, hipStream_t s) {
  const int nblk = (T + kBlockTokens - 1) / kBlockTokens;
  int32_t* cnt = (int32_t*)ws;
  int32_t* tot = (int32_t*)((char*)ws + align256((size_t)n_ffn * nblk * 4));
  const size_t lds = (size_t)(n_ffn > 0 ? n_ffn : 1) * sizeof(unsigned long long);
  if (nblk == 1 && n_ffn > 0) {
    MOE_LAUNCH("permute_small", s,
               perm_small<<<1, 1024, (size_t)n_ffn * 12, s>>>(idx, T, K, n_ffn, offsets, row_src,
                                                              slot_row));
  } else {
    if (n_ffn > 0) {
      MOE_LAUNCH("permute_hist", s,
                 perm_hist<<<nblk, kWave, lds, s>>>(idx, T, K, n_ffn, nblk, cnt));
      MOE_LAUNCH("permute_scan_blocks", s,
                 perm_scan_blocks<<<ceil_div(n_ffn, 4), 256, 0, s>>>(cnt, nblk, n_ffn, tot));
    }
    MOE_LAUNCH("permute_scan_experts", s,
               perm_scan_experts<<<1, 1024, 0, s>>>(tot, n_ffn, offsets));
    MOE_LAUNCH("permute_scatter", s,
               perm_scatter<<<nblk, kWave, lds, s>>>(idx, T, K, n_ffn, nblk, cnt, offsets,
                                                     row_src, slot_row));
  }
  if (!x_perm) return hipGetLastError();   // indices only: the GEMM gathers x rows itself
  const int esize = dtype == MOE_BF16 ? 2 : 4;
  const int row_vecs = (int)((size_t)H * esize / 16);
  if (row_vecs <= 256 * 4)
    MOE_LAUNCH("permute_gather", s,
               perm_gather<4><<<T, 256, 0, s>>>((const i32x4*)x, row_vecs, K, slot_row,
                                                (i32x4*)x_perm));
  else
    MOE_LAUNCH("permute_gather", s,
               perm_gather_long<<<T, 256, 0, s>>>((const i32x4*)x, row_vecs, K, slot_row,
                                                  (i32x4*)x_perm));
  return hipGetLastError();
}

}  // namespace moe
