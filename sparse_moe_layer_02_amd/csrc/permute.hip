// Dispatch on one GPU (LongCat-Flash Technical Report notes, Key claims
// [§2.2]: the dispatch half of dispatch/combine): every FFN selection (t, k)
// gets a row in an expert-major buffer; inside one expert, rows follow the
// token order.  The order must not depend on atomic arrival, so ranks are
// computed from bitmasks, in one kernel:
//   block b = tokens [64b, 64b+64) (1024 threads).
//   mask[e] (LDS, 64 bits) = OR of (1 << (t - 64b)) over its tokens t that
//     chose e.  A token chooses an expert at most once, so the rank of (t, e)
//     among the block's rows of e is popcount(mask[e] & bits below t - 64b).
//   before[e] = picks of e by tokens < 64b.  The block counts them itself
//     (an LDS histogram of the picks on the shorter side of its tokens: those
//     before it, or those after it, whence before[e] = counts[e] - after[e]
//     - popcount(mask[e])), so no other block's result is awaited and there
//     is no second launch.  Each block reads at most half of the T*K picks.
//   offsets = exclusive scan of counts over the FFN experts (every block
//     scans the n_ffn counts; block 0 writes them).
//   row(t, e) = offsets[e] + before[e] + rank.
// When a grouped copy is asked for, perm_gather then copies the x rows (one
// read of x[t] feeding all of its rows).
#include "moe_internal.h"

namespace moe {
namespace {

constexpr int kBlockTokens = 64;
constexpr int kPermThreads = 1024;
constexpr int kPermWaves = kPermThreads / kWave;

// Exclusive scan of v over the block's 1024 threads (fixed order); *total
// receives the sum.  Uses part[kPermWaves + 1] of LDS.
__device__ __forceinline__ int block_exclusive_scan(int v, int* part, int* total) {
  const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
  int incl = v;
#pragma unroll
  for (int off = 1; off < kWave; off <<= 1) {
    const int o = __shfl_up(incl, off);
    if (lane >= off) incl += o;
  }
  if (lane == kWave - 1) part[wave] = incl;
  __syncthreads();
  if (threadIdx.x == 0) {
    int run = 0;
    for (int w = 0; w < kPermWaves; ++w) {
      const int x = part[w];
      part[w] = run;
      run += x;
    }
    part[kPermWaves] = run;
  }
  __syncthreads();
  *total = part[kPermWaves];
  return part[wave] + incl - v;
}

__global__ __launch_bounds__(kPermThreads) void perm_fused(
    const int32_t* __restrict__ idx, const int32_t* __restrict__ counts, int T, int K, int n_ffn,
    int32_t* __restrict__ offsets, int32_t* __restrict__ row_src,
    int32_t* __restrict__ slot_row) {
  extern __shared__ unsigned long long mask[];        // [n_ffn]
  int* before = (int*)(mask + n_ffn);                  // [n_ffn]: side counts, then row bases
  __shared__ int part[kPermWaves + 1];
  const int tid = threadIdx.x;
  const int t0 = blockIdx.x * kBlockTokens, t1 = min(T, t0 + kBlockTokens);
  for (int e = tid; e < n_ffn; e += kPermThreads) {
    mask[e] = 0ull;
    before[e] = 0;
  }
  __syncthreads();
  // the block's own picks
  const int p0 = t0 * K, p1 = t1 * K;
  for (int i = p0 + tid; i < p1; i += kPermThreads) {
    const int e = idx[i];
    if ((unsigned)e < (unsigned)n_ffn) atomicOr(&mask[e], 1ull << (i / K - t0));
  }
  // the picks on the shorter side
  const bool lower = t0 <= T - t1;
  const int s0 = lower ? 0 : p1, s1 = lower ? p0 : T * K;
  auto count = [&](int e) {
    if ((unsigned)e < (unsigned)n_ffn) atomicAdd(&before[e], 1);
  };
  int s_vec = s0;
  if ((((uintptr_t)idx) & 15) == 0 && (s0 & 3) == 0) {
    // 16-byte loads, four in flight per thread
    const i32x4* v4 = (const i32x4*)idx;
    const int q0 = s0 >> 2, q1 = s1 >> 2;
    int q = q0 + tid;
    for (; q + 3 * kPermThreads < q1; q += 4 * kPermThreads) {
      i32x4 a[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) a[u] = v4[q + u * kPermThreads];
#pragma unroll
      for (int u = 0; u < 4; ++u)
#pragma unroll
        for (int j = 0; j < 4; ++j) count(a[u][j]);
    }
    for (; q < q1; q += kPermThreads) {
      const i32x4 a = v4[q];
#pragma unroll
      for (int j = 0; j < 4; ++j) count(a[j]);
    }
    s_vec = q1 << 2;
  }
  for (int i = s_vec + tid; i < s1; i += kPermThreads) count(idx[i]);
  __syncthreads();
  // offsets (a chunk of experts per thread) and the block's row bases
  const int per = (n_ffn + kPermThreads - 1) / kPermThreads;
  const int lo = min(n_ffn, tid * per), hi = min(n_ffn, lo + per);
  int sum = 0;
  for (int e = lo; e < hi; ++e) sum += counts[e];
  int total;
  int run = block_exclusive_scan(sum, part, &total);
  for (int e = lo; e < hi; ++e) {
    const int c = counts[e];
    if (blockIdx.x == 0) offsets[e] = run;
    before[e] = run + (lower ? before[e] : c - before[e] - __popcll(mask[e]));
    run += c;
  }
  if (blockIdx.x == 0 && tid == 0) offsets[n_ffn] = total;
  __syncthreads();
  // rows of the block's picks.  With counts as moe_route wrote them for idx,
  // every row is in [0, T*K); otherwise rows are clamped into that range, so
  // no write leaves the buffers (the grouping is then meaningless).
  const int cap = T * K;
  for (int i = p0 + tid; i < p1; i += kPermThreads) {
    const int e = idx[i];
    if ((unsigned)e < (unsigned)n_ffn) {
      const int l = i / K - t0;
      int row = before[e] + __popcll(mask[e] & ((1ull << l) - 1ull));
      row = min(max(row, 0), cap - 1);
      slot_row[i] = row;
      row_src[row] = i;
    } else {
      slot_row[i] = -1;   // an identity pick: no row
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

}  // namespace

hipError_t launch_permute(const void* x, int dtype, const int32_t* idx, const int32_t* counts,
                          int T, int H, int K, int n_ffn, int32_t* offsets, void* x_perm,
                          int32_t* row_src, int32_t* slot_row, hipStream_t s) {
  const unsigned nblk = ceil_div(T, kBlockTokens);
  const size_t lds = (size_t)(n_ffn > 0 ? n_ffn : 1) * 12;
  MOE_LAUNCH("permute", s,
             perm_fused<<<nblk, kPermThreads, lds, s>>>(idx, counts, T, K, n_ffn, offsets,
                                                         row_src, slot_row));
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
