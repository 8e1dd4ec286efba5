// Bias controller of the FFN experts' selection bias (LongCat-Flash Technical
// Report notes, Key claims [§2.1.1, §2.1.2] and Method: each FFN expert's bias
// is adjusted from token-routing frequency by a PID controller so that the
// average number of activated FFN experts per token holds a target; the
// zero-computation experts' biases are excluded from the update).
//
// Per FFN expert i, from the batch's routing counts (moe_route):
//   err_i       = target / n_ffn - counts[i] / T
//   integral_i += err_i
//   bias_i     += kp * err_i + ki * integral_i + kd * (err_i - prev_i)
//   prev_i      = err_i
// One thread per FFN expert, fp32 state owned by the caller.
#include "moe_internal.h"

namespace moe {
namespace {

__global__ __launch_bounds__(256) void bias_update_kernel(const int32_t* __restrict__ counts,
                                                          int T, int n_ffn, float target, float kp,
                                                          float ki, float kd,
                                                          float* __restrict__ bias,
                                                          float* __restrict__ integral,
                                                          float* __restrict__ prev) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= n_ffn) return;
  const float err = target / (float)n_ffn - (float)counts[i] / (float)T;
  const float acc = integral[i] + err;
  integral[i] = acc;
  bias[i] += kp * err + ki * acc + kd * (err - prev[i]);
  prev[i] = err;
}

}  // namespace

hipError_t launch_bias_update(const int32_t* counts, int T, int n_ffn, float target, float kp,
                              float ki, float kd, float* bias, float* integral, float* prev,
                              hipStream_t s) {
  MOE_LAUNCH("bias_update", s,
             bias_update_kernel<<<ceil_div(n_ffn, 256), 256, 0, s>>>(
                 counts, T, n_ffn, target, kp, ki, kd, bias, integral, prev));
  return hipGetLastError();
}

}  // namespace moe
