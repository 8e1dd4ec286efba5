// Top-K routing with a selection bias (LongCat-Flash Technical Report notes,
// Key claims [§2.1, §2.1.1]): keys = fp32 logits + bias pick K experts from
// the pool of FFN and zero-computation experts; gates are the softmax of the
// unbiased logits at the picks; counts is the routing-frequency histogram.
//
// One wave64 per token.  Lane l holds experts e = l + 64*i (i < EPL).  Each
// candidate is packed into one 64-bit integer whose unsigned order is the
// selection order:
//   high 32 bits: the fp32 key mapped to an order-preserving integer
//                 (-0.0 folded onto +0.0; NaN below -inf),
//   low 32 bits : ~e, so that on equal keys the lower expert id is larger.
// Zero marks a taken (or absent) candidate.  K rounds of a lane-local max and
// a 6-step xor-shuffle max across the wave yield the picks in order.
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

__device__ __forceinline__ uint64_t wave_max_u64(uint64_t v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) {
    uint32_t lo = __shfl_xor((uint32_t)v, off);
    uint32_t hi = __shfl_xor((uint32_t)(v >> 32), off);
    uint64_t o = ((uint64_t)hi << 32) | lo;
    v = o > v ? o : v;
  }
  return v;
}

__device__ __forceinline__ float wave_max_f32(float v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v = fmaxf(v, __shfl_xor(v, off));
  return v;
}

__device__ __forceinline__ float wave_sum_f32(float v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off);
  return v;
}

__global__ void zero_i32(int32_t* p, int n) {
  int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = 0;
}

template <int EPL>
__global__ __launch_bounds__(kRouteThreads) void route_kernel(
    const float* __restrict__ logits, const float* __restrict__ bias, int T, int E, int K,
    int32_t* __restrict__ idx, float* __restrict__ gate, int32_t* __restrict__ counts,
    int32_t* __restrict__ status) {
  __shared__ int hist[EPL * kWave];
  for (int e = threadIdx.x; e < E; e += kRouteThreads) hist[e] = 0;
  __syncthreads();

  const int lane = threadIdx.x & (kWave - 1);
  const int wave = threadIdx.x / kWave;
  constexpr int kWaves = kRouteThreads / kWave;
  float bs[EPL];
#pragma unroll
  for (int i = 0; i < EPL; ++i) {
    int e = lane + kWave * i;
    bs[i] = e < E ? bias[e] : 0.0f;
  }
  bool bad = false;
  const int t_end = min(T, (blockIdx.x + 1) * kTokensPerBlock);
  for (int t = blockIdx.x * kTokensPerBlock + wave; t < t_end; t += kWaves) {
    const float* lr = logits + (size_t)t * E;
    float lg[EPL];
    uint64_t cand[EPL];
    float mx = -INFINITY;
#pragma unroll
    for (int i = 0; i < EPL; ++i) {
      int e = lane + kWave * i;
      if (e < E) {
        lg[i] = lr[e];
        float key = lg[i] + bs[i];
        bad |= (key != key) || !isfinite(lg[i]);
        cand[i] = ((uint64_t)key_order(key) << 32) | (uint32_t)(~(uint32_t)e);
        mx = fmaxf(mx, lg[i]);
      } else {
        lg[i] = -INFINITY;
        cand[i] = 0;
      }
    }
    // softmax statistics over the unbiased logits (fixed reduction order)
    mx = wave_max_f32(mx);
    float part = 0.0f;
#pragma unroll
    for (int i = 0; i < EPL; ++i)
      if (lane + kWave * i < E) part += expf(lg[i] - mx);
    const float den = wave_sum_f32(part);

    for (int k = 0; k < K; ++k) {
      uint64_t best = 0;
#pragma unroll
      for (int i = 0; i < EPL; ++i) best = cand[i] > best ? cand[i] : best;
      best = wave_max_u64(best);
      const int e = (int)(~(uint32_t)best);
      float mine = 0.0f;
#pragma unroll
      for (int i = 0; i < EPL; ++i)
        if (lane + kWave * i == e) {
          cand[i] = 0;
          mine = lg[i];
        }
      const float le = __shfl(mine, e & (kWave - 1));
      if (lane == 0) {
        idx[(size_t)t * K + k] = e;
        gate[(size_t)t * K + k] = expf(le - mx) / den;
        atomicAdd(&hist[e], 1);
      }
    }
  }
  if (bad && status) *status = 1;
  __syncthreads();
  for (int e = threadIdx.x; e < E; e += kRouteThreads)
    if (hist[e]) atomicAdd(&counts[e], hist[e]);
}

}  // namespace

hipError_t launch_route(const float* logits, const float* bias, int T, int E, int K,
                        int32_t* idx, float* gate, int32_t* counts, int32_t* status,
                        hipStream_t s) {
  MOE_LAUNCH("route_clear", s, zero_i32<<<ceil_div(E, 256), 256, 0, s>>>(counts, E));
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
  return hipGetLastError();
}

}  // namespace moe
