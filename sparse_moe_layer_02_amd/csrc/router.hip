// Router scores over the whole expert pool (LongCat-Flash Technical Report
// notes, Key claims [§2.1, §2.4]): logits[t][e] = sum_h x[t][h] * w_router[e][h],
// fp32 products and fp32 accumulation.
// LDS-tiled FMA kernel: 64 tokens x 64 experts per block, K step 16, each
// thread owns a 4x4 patch.  Any T, E, H.
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
  float acc[4][4] = {};
  for (int k0 = 0; k0 < H; k0 += kTK) {
    for (int i = threadIdx.x; i < kTM * kTK; i += kThreads) {
      const int r = i / kTK, k = i % kTK;
      As[k][r] = (m0 + r < T && k0 + k < H) ? ld_f32(x + (size_t)(m0 + r) * H + k0 + k) : 0.0f;
      Bs[k][r] = (n0 + r < E && k0 + k < H) ? w[(size_t)(n0 + r) * H + k0 + k] : 0.0f;
    }
    __syncthreads();
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

}  // namespace

hipError_t launch_router_logits(const void* x, int dtype, const float* w, int T, int H, int E,
                                float* logits, hipStream_t s) {
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
