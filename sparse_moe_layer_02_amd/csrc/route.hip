// Top-K routing with a selection bias (LongCat-Flash Technical Report notes,
// Key claims [§2.1, §2.1.1]): keys = fp32 logits + bias pick K experts from
// the pool of FFN and zero-computation experts; gates are the softmax of the
// unbiased logits at the picks; counts is the routing-frequency histogram.
//
// One wave64 per token.  Lane l holds experts e = l + 64*i (i < EPL).  Each
// key becomes a 32-bit word whose unsigned order is the key order (-0.0
// folded onto +0.0, NaN below -inf, 0 = absent), and a candidate is the
// 64-bit integer (key word, ~e), so that on equal keys the lower expert id is
// larger.  The K largest candidates are found by a threshold and a rank
// among the few candidates above it (select_token); K rounds of a wave max
// over every candidate remain for the cases the threshold cannot narrow.
// Wave reductions use DPP row shifts and row broadcasts (the result lands in
// lane 63 and is read out once) rather than LDS-routed shuffles.
// counts comes from a second kernel over the picks (route_hist), so that the
// top-K kernel's 4-token blocks do not each add a histogram to counts with
// global atomics (on a 96-expert pool that contention cost more than the
// selection itself).
#include "moe_internal.h"

namespace moe {
namespace {

constexpr int kRouteThreads = 256;
constexpr int kTokensPerBlock = 4;   // one token per wave: many waves in flight

__device__ __forceinline__ uint32_t key_order(float k) {
  if (k != k) return 1u;                    // NaN: above "taken", below every number
  if (k == 0.0f) k = 0.0f;                  // -0.0 == +0.0
  uint32_t b = __float_as_uint(k);
  return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}

// One DPP step of a max reduction: combine with the value of the lane the
// control selects; lanes with no source (or outside the row mask) take the
// identity `id`.
template <int CTRL, int ROW_MASK = 0xf>
__device__ __forceinline__ uint32_t dpp_u32(uint32_t v, uint32_t id) {
  return (uint32_t)__builtin_amdgcn_update_dpp((int)id, (int)v, CTRL, ROW_MASK, 0xf, false);
}

// Prefix-max within 16-lane rows (row_shr 1, 2, 4, 8), then row 0's and row
// 2's maxima into rows 1 and 3 (row_bcast 15), then rows 0-1 into rows 2-3
// (row_bcast 31): lane 63 holds the wave's maximum.
template <int CTRL, int ROW_MASK = 0xf>
__device__ __forceinline__ uint64_t dpp_max_step_u64(uint64_t v) {
  const uint32_t lo = dpp_u32<CTRL, ROW_MASK>((uint32_t)v, 0u);
  const uint32_t hi = dpp_u32<CTRL, ROW_MASK>((uint32_t)(v >> 32), 0u);
  const uint64_t o = ((uint64_t)hi << 32) | lo;
  return o > v ? o : v;
}

__device__ __forceinline__ uint64_t wave_max_u64(uint64_t v) {
  v = dpp_max_step_u64<0x111>(v);         // row_shr:1
  v = dpp_max_step_u64<0x112>(v);         // row_shr:2
  v = dpp_max_step_u64<0x114>(v);         // row_shr:4
  v = dpp_max_step_u64<0x118>(v);         // row_shr:8
  v = dpp_max_step_u64<0x142, 0xa>(v);    // row_bcast:15
  v = dpp_max_step_u64<0x143, 0xc>(v);    // row_bcast:31
  const uint32_t lo = __builtin_amdgcn_readlane((uint32_t)v, 63);
  const uint32_t hi = __builtin_amdgcn_readlane((uint32_t)(v >> 32), 63);
  return ((uint64_t)hi << 32) | lo;
}

template <int CTRL, int ROW_MASK = 0xf>
__device__ __forceinline__ float dpp_f32(float v, float id) {
  return __uint_as_float(dpp_u32<CTRL, ROW_MASK>(__float_as_uint(v), __float_as_uint(id)));
}

__device__ __forceinline__ float wave_max_f32(float v) {
  v = fmaxf(v, dpp_f32<0x111>(v, -INFINITY));
  v = fmaxf(v, dpp_f32<0x112>(v, -INFINITY));
  v = fmaxf(v, dpp_f32<0x114>(v, -INFINITY));
  v = fmaxf(v, dpp_f32<0x118>(v, -INFINITY));
  v = fmaxf(v, dpp_f32<0x142, 0xa>(v, -INFINITY));
  v = fmaxf(v, dpp_f32<0x143, 0xc>(v, -INFINITY));
  return __uint_as_float(__builtin_amdgcn_readlane(__float_as_uint(v), 63));
}

// Sum in a fixed order: prefix sums within rows, then across rows, read from
// lane 63 (bitwise reproducible run to run).
__device__ __forceinline__ float wave_sum_f32(float v) {
  v += dpp_f32<0x111>(v, 0.0f);
  v += dpp_f32<0x112>(v, 0.0f);
  v += dpp_f32<0x114>(v, 0.0f);
  v += dpp_f32<0x118>(v, 0.0f);
  v += dpp_f32<0x142, 0xa>(v, 0.0f);
  v += dpp_f32<0x143, 0xc>(v, 0.0f);
  return __uint_as_float(__builtin_amdgcn_readlane(__float_as_uint(v), 63));
}

// counts[e] = number of picks of expert e, after the top-K kernel (whose
// block 0 zeroes counts): each block counts 16 K picks in an LDS histogram
// and adds its nonzero bins to counts, a few global atomics per expert
// instead of one per 4-token block (integer counts are exact in any order).
constexpr int kHistThreads = 1024;
constexpr int kHistPer = 16;                       // picks per thread
constexpr int kHistChunk = kHistThreads * kHistPer;
__global__ __launch_bounds__(kHistThreads) void route_hist(const int32_t* __restrict__ idx,
                                                           long long n, int E,
                                                           int32_t* __restrict__ counts) {
  __shared__ int hist[1024];
  for (int e = threadIdx.x; e < E; e += kHistThreads) hist[e] = 0;
  __syncthreads();
  const long long i0 = (long long)blockIdx.x * kHistChunk + threadIdx.x;
  int v[kHistPer];
#pragma unroll
  for (int u = 0; u < kHistPer; ++u) {
    const long long i = i0 + (long long)u * kHistThreads;
    v[u] = i < n ? idx[i] : -1;
  }
#pragma unroll
  for (int u = 0; u < kHistPer; ++u)
    if (v[u] >= 0 && v[u] < E) atomicAdd(&hist[v[u]], 1);
  __syncthreads();
  for (int e = threadIdx.x; e < E; e += kHistThreads)
    if (hist[e]) atomicAdd(&counts[e], hist[e]);
}

__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
  v = max(v, dpp_u32<0x111>(v, 0u));         // row_shr:1
  v = max(v, dpp_u32<0x112>(v, 0u));         // row_shr:2
  v = max(v, dpp_u32<0x114>(v, 0u));         // row_shr:4
  v = max(v, dpp_u32<0x118>(v, 0u));         // row_shr:8
  v = max(v, dpp_u32<0x142, 0xa>(v, 0u));    // row_bcast:15
  v = max(v, dpp_u32<0x143, 0xc>(v, 0u));    // row_bcast:31
  return __builtin_amdgcn_readlane(v, 63);
}

// Lanes below this one holding a set bit of `bits` (a ballot).
__device__ __forceinline__ int lanes_below(uint64_t bits) {
  return __builtin_amdgcn_mbcnt_hi((uint32_t)(bits >> 32),
                                   __builtin_amdgcn_mbcnt_lo((uint32_t)bits, 0u));
}

// Selection of one token's K picks (one wave; lane l holds the key words
// kq[i] and logits lg[i] of experts l + 64 i).
//
// Fast path (K <= 64).  The K-th largest of the 64 lane maxima, theta, is a
// lower bound of the K-th largest key (the K largest lane maxima are K
// distinct keys >= theta), so every key of the top K -- ties at the K-th
// key included -- is >= theta.  theta comes from at most K rounds of a
// 32-bit wave max over one value per lane.  The candidates (keys >= theta,
// usually K plus a few) are compacted into LDS, and each is ranked by
// comparing its 64-bit (key word, ~e) against all of them: rank r < K is
// pick r.  The order is the rounds' order exactly (descending key, lower id
// first on equal keys), in a few hundred vector instructions per token
// instead of K rounds over every key.  More than 64 candidates (many keys
// equal at theta) take the rounds below.
template <int EPL>
__device__ __forceinline__ void select_token(const uint32_t (&kq0)[EPL], const float (&lg)[EPL],
                                             int E, int K, float mx, float den, int lane,
                                             uint64_t* cand, float* cand_lg, float* lrow,
                                             int32_t* __restrict__ idx_row,
                                             float* __restrict__ gate_row) {
  uint32_t kq[EPL];
  uint32_t lm = 0;
#pragma unroll
  for (int i = 0; i < EPL; ++i) {
    kq[i] = kq0[i];
    lm = max(lm, kq[i]);
  }
  if (K <= kWave) {
    // theta: the K-th largest lane maximum, counted with multiplicity.  At
    // least K lanes hold a key (K <= E and K <= 64), and every key word is
    // >= 1, so each round removes at least one lane and ends by round K.
    uint32_t theta = 1, v = lm;
    int seen = 0;
    for (int r = 0; r < K; ++r) {
      const uint32_t w = wave_max_u32(v);
      const uint64_t hit = __ballot(v == w);
      seen += __popcll(hit);
      theta = w;
      if (seen >= K) break;
      if (v == w) v = 0;
    }
    int c = 0;
#pragma unroll
    for (int i = 0; i < EPL; ++i) c += kq[i] >= theta ? 1 : 0;
    // exclusive prefix of c over the lanes (c <= 16: five bit planes)
    int pre = 0, M = 0;
#pragma unroll
    for (int b = 0; b < 5; ++b) {
      const uint64_t bits = __ballot((c >> b) & 1);
      pre += lanes_below(bits) << b;
      M += __popcll(bits) << b;
    }
    if (M <= kWave) {
#pragma unroll
      for (int i = 0; i < EPL; ++i)
        if (kq[i] >= theta) {
          cand[pre] = ((uint64_t)kq[i] << 32) | (uint32_t)(~(uint32_t)(lane + kWave * i));
          cand_lg[pre] = lg[i];
          ++pre;
        }
      wave_lds_sync();   // the wave's writes land before a lane reads another's
      if (lane < M) {
        const uint64_t mine = cand[lane];
        int rank = 0;
        for (int m = 0; m < M; ++m) rank += cand[m] > mine ? 1 : 0;
        if (rank < K) {
          idx_row[rank] = (int)(~(uint32_t)mine);
          gate_row[rank] = expf(cand_lg[lane] - mx) / den;
        }
      }
      wave_lds_sync();   // cand is rewritten for the wave's next token
      return;
    }
  }
  // Rounds: K times, the largest remaining 64-bit candidate of the wave.
  // The token's logits go to LDS for the gates; pick k stays in lane k % 64,
  // and every 64 picks (or at the last) the lanes write them at once.
#pragma unroll
  for (int i = 0; i < EPL; ++i)
    if (lane + kWave * i < E) lrow[lane + kWave * i] = lg[i];
  wave_lds_sync();
  int pick = 0;
  for (int k = 0; k < K; ++k) {
    // the lane's best: the largest key word, the lowest i among equal ones
    uint32_t bk = 0;
    int bi = 0;
#pragma unroll
    for (int i = 0; i < EPL; ++i)
      if (kq[i] > bk) {
        bk = kq[i];
        bi = i;
      }
    const uint64_t mine =
        bk ? ((uint64_t)bk << 32) | (uint32_t)(~(uint32_t)(lane + kWave * bi)) : 0ull;
    const uint64_t best = wave_max_u64(mine);
    const int e = (int)(~(uint32_t)best);
#pragma unroll
    for (int i = 0; i < EPL; ++i)
      if (lane + kWave * i == e) kq[i] = 0;
    if (lane == (k & (kWave - 1))) pick = e;
    if ((k & (kWave - 1)) == kWave - 1 || k == K - 1) {
      const int base = k & ~(kWave - 1);
      if (lane <= k - base) {
        idx_row[base + lane] = pick;
        gate_row[base + lane] = expf(lrow[pick] - mx) / den;
      }
    }
  }
  wave_lds_sync();
}

template <int EPL>
__global__ __launch_bounds__(kRouteThreads) void route_kernel(
    const float* __restrict__ logits, const float* __restrict__ bias, int T, int E, int K,
    int32_t* __restrict__ idx, float* __restrict__ gate, int32_t* __restrict__ counts,
    int32_t* __restrict__ status) {
  if (blockIdx.x == 0)   // the histogram kernel that follows accumulates into counts
    for (int e = threadIdx.x; e < E; e += kRouteThreads) counts[e] = 0;
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = threadIdx.x / kWave;
  constexpr int kWaves = kRouteThreads / kWave;
  __shared__ uint64_t cand[kWaves][kWave];
  __shared__ float cand_lg[kWaves][kWave];
  __shared__ float lrow[kWaves][kWave * EPL];   // the rounds' gates
  bool bad = false;
  const int t_end = min(T, (blockIdx.x + 1) * kTokensPerBlock);
  for (int t = blockIdx.x * kTokensPerBlock + wave; t < t_end; t += kWaves) {
    const float* lr = logits + (size_t)t * E;
    uint32_t kq[EPL];
    float lg[EPL];
    float mx = -INFINITY;
#pragma unroll
    for (int i = 0; i < EPL; ++i) {
      const int e = lane + kWave * i;
      if (e < E) {
        lg[i] = lr[e];
        const float key = lg[i] + bias[e];
        // -inf (a masked expert) is a valid key and logit; a NaN key or a
        // +inf logit leaves the selection or the softmax undefined
        bad |= (key != key) || (lg[i] == INFINITY);
        kq[i] = key_order(key);
        mx = fmaxf(mx, lg[i]);
      } else {
        lg[i] = -INFINITY;
        kq[i] = 0;
      }
    }
    // softmax statistics over the unbiased logits (fixed reduction order)
    mx = wave_max_f32(mx);
    bad |= mx == -INFINITY;   // every logit -inf: no softmax
    float part = 0.0f;
#pragma unroll
    for (int i = 0; i < EPL; ++i)
      if (lane + kWave * i < E) part += expf(lg[i] - mx);
    const float den = wave_sum_f32(part);
    select_token<EPL>(kq, lg, E, K, mx, den, lane, cand[wave], cand_lg[wave], lrow[wave],
                      idx + (size_t)t * K, gate + (size_t)t * K);
  }
  if (bad && status) *status = 1;
}

}  // namespace

hipError_t launch_route(const float* logits, const float* bias, int T, int E, int K,
                        int32_t* idx, float* gate, int32_t* counts, int32_t* status,
                        hipStream_t s) {
  const unsigned grid = ceil_div(T, kTokensPerBlock);
  const int epl = (E + kWave - 1) / kWave;
#define MOE_ROUTE(N)                                                                    \
  MOE_LAUNCH("route_topk", s,                                                          \
             route_kernel<N><<<grid, kRouteThreads, 0, s>>>(logits, bias, T, E, K, idx, \
                                                            gate, counts, status))
  if (epl <= 1) MOE_ROUTE(1);
  else if (epl <= 2) MOE_ROUTE(2);
  else if (epl <= 4) MOE_ROUTE(4);
  else if (epl <= 8) MOE_ROUTE(8);
  else if (epl <= 12) MOE_ROUTE(12);
  else MOE_ROUTE(16);
#undef MOE_ROUTE
  const long long picks = (long long)T * K;
  MOE_LAUNCH("route_hist", s,
             route_hist<<<ceil_div(picks, kHistChunk), kHistThreads, 0, s>>>(idx, picks, E,
                                                                             counts));
  return hipGetLastError();
}

}  // namespace moe
