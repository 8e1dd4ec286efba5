// Identity experts and the combine step (LongCat-Flash Technical Report notes,
// Key claims [§2.1] identity "zero-computation" experts, [§2.2] combine,
// [§2.3.2 Eq. 8] the variance-compensation factor on FFN expert outputs).
// Both are HBM-bound row sweeps: one block per token with one 8-element piece
// per thread (H / 8 threads rounded up to whole waves, at most 1024, so a
// 6144-wide row is one pass of 768 threads: measured 6 % faster than four
// waves looping over the row), 16-byte vector loads, fp32 arithmetic, a fixed
// summation order (slot order) and no atomics, so results are bitwise
// reproducible.  Outputs are stored non-temporally: streamed to HBM as they
// are written rather than left dirty in the caches to be written back during
// the next kernel's reads (measured: ~0.15 ms less per layer over every
// kernel that writes rows).  The y_perm rows, each read once, are loaded
// non-temporally too: 188 -> 157 us on the 8192-token layer, 340 -> 318 us on
// the 16384-token one.
#include "moe_internal.h"

namespace moe {
namespace {

constexpr int kMaxThreads = 1024;
constexpr int kMaxK = 1024;
constexpr int kBatch = 8;

template <typename T> struct Vec8;
template <> struct Vec8<bf16> {
  static __device__ __forceinline__ void load(const bf16* p, float* o) {
    bf16x8 v = *(const bf16x8*)p;
#pragma unroll
    for (int i = 0; i < 8; ++i) o[i] = (float)v[i];
  }
  // a piece read once (a y_perm row), loaded non-temporally and converted
  // only where it is used
  using Raw = bf16x8;
  static __device__ __forceinline__ Raw load_raw(const bf16* p) {
    return __builtin_nontemporal_load((const Raw*)p);
  }
  static __device__ __forceinline__ void load_nt(const bf16* p, float* o) {
    const Raw v = load_raw(p);
#pragma unroll
    for (int i = 0; i < 8; ++i) o[i] = (float)v[i];
  }
  static __device__ __forceinline__ float at(const Raw& r, int i) { return (float)r[i]; }
  static __device__ __forceinline__ void store(bf16* p, const float* o) {
    bf16x8 v;
#pragma unroll
    for (int i = 0; i < 8; ++i) v[i] = (bf16)o[i];
    __builtin_nontemporal_store(v, (bf16x8*)p);
  }
};
template <> struct Vec8<float> {
  static __device__ __forceinline__ void load(const float* p, float* o) {
    f32x4 a = *(const f32x4*)p, b = *(const f32x4*)(p + 4);
#pragma unroll
    for (int i = 0; i < 4; ++i) { o[i] = a[i]; o[4 + i] = b[i]; }
  }
  struct Raw { f32x4 a, b; };
  static __device__ __forceinline__ Raw load_raw(const float* p) {
    return Raw{__builtin_nontemporal_load((const f32x4*)p),
               __builtin_nontemporal_load((const f32x4*)(p + 4))};
  }
  static __device__ __forceinline__ void load_nt(const float* p, float* o) {
    const Raw v = load_raw(p);
#pragma unroll
    for (int i = 0; i < 4; ++i) { o[i] = v.a[i]; o[4 + i] = v.b[i]; }
  }
  static __device__ __forceinline__ float at(const Raw& r, int i) { return i < 4 ? r.a[i] : r.b[i - 4]; }
  static __device__ __forceinline__ void store(float* p, const float* o) {
    f32x4 a, b;
#pragma unroll
    for (int i = 0; i < 4; ++i) { a[i] = o[i]; b[i] = o[4 + i]; }
    __builtin_nontemporal_store(a, (f32x4*)p);
    __builtin_nontemporal_store(b, (f32x4*)(p + 4));
  }
};

// combine_lanes: a row of H elements in blocks of at most kLaneThreads
// threads, one 8-element piece each (a 6144-wide row: two blocks of 384).
// Measured on the 8192-token layer: one 768-thread block per row 190 us,
// two of 384 185 us, three of 256 191 us.
constexpr int kLaneThreads = 384;
inline int lane_parts(int H) { return (H + 8 * kLaneThreads - 1) / (8 * kLaneThreads); }
inline int lane_threads(int H) {
  const int per = (H + 8 * lane_parts(H) - 1) / (8 * lane_parts(H));   // pieces per block
  return ((per + kWave - 1) / kWave) * kWave;
}

// Threads per block for a row of H elements: one 8-element piece each.
inline int row_threads(int H) {
  const int t = ((H + 8 * kWave - 1) / (8 * kWave)) * kWave;
  return t < kMaxThreads ? t : kMaxThreads;
}

// y_acc[t] = (sum of the gates of t's identity-expert slots) * x[t]
template <typename T>
__global__ __launch_bounds__(kMaxThreads) void zero_experts_kernel(
    const T* __restrict__ x, const int32_t* __restrict__ idx, const float* __restrict__ gate,
    int H, int K, int n_ffn, float* __restrict__ y_acc) {
  const int t = blockIdx.x;
  float gs = 0.0f;
  for (int k = 0; k < K; ++k)
    if (idx[(size_t)t * K + k] >= n_ffn) gs += gate[(size_t)t * K + k];
  const T* xr = x + (size_t)t * H;
  float* yr = y_acc + (size_t)t * H;
  for (int c = threadIdx.x * 8; c < H; c += blockDim.x * 8) {
    float v[8];
    Vec8<T>::load(xr + c, v);
#pragma unroll
    for (int i = 0; i < 8; ++i) v[i] *= gs;
    Vec8<float>::store(yr + c, v);
  }
}

// The token's slot list, read by wave 0 (64 slots per step, one lane each):
// the FFN slots' rows and weights (scale * gate), compacted in slot order into
// LDS, and the sum of the identity slots' gates (slot_row < 0), added in slot
// order on every lane -- the same fp32 order as zero_experts_kernel.
struct SlotList {
  int rows[kMaxK];
  float wts[kMaxK];
  int n;
  float identity_gate;
};

__device__ __forceinline__ void read_slots(SlotList& sl, const int32_t* __restrict__ slot_row,
                                           const float* __restrict__ gate, float scale, int K,
                                           int t) {
  const int lane = threadIdx.x;
  int n = 0;
  float gs = 0.0f;
  for (int k0 = 0; k0 < K; k0 += kWave) {
    const int k = k0 + lane;
    const bool in = k < K;
    const int r = in ? slot_row[(size_t)t * K + k] : 0;
    const float g = in ? gate[(size_t)t * K + k] : 0.0f;
    const bool ffn = in && r >= 0;
    const unsigned long long m = __ballot(ffn);
    if (ffn) {
      const int pos = n + __popcll(m & ((1ull << lane) - 1ull));
      sl.rows[pos] = r;
      sl.wts[pos] = scale * g;
    }
    n += __popcll(m);
    for (unsigned long long b = __ballot(in && r < 0); b; b &= b - 1ull)
      gs += __shfl(g, __ffsll((long long)b) - 1);
  }
  if (lane == 0) {
    sl.n = n;
    sl.identity_gate = gs;
  }
}

// y[t] = ident[t] + sum over FFN slots (in slot order) of (scale*gate) * y_perm[row]
//   IDENTITY = false: ident[t] = y_acc[t] (fp32, from zero_experts_kernel);
//   IDENTITY = true:  ident[t] = (sum of the identity slots' gates) * x[t],
//     computed here with the same fp32 operations, so the result is bitwise
//     that of the two kernels, without y_acc's 4H bytes written and read
//     per token.
template <typename T, bool IDENTITY>
__global__ __launch_bounds__(kMaxThreads) void combine_kernel(
    const T* __restrict__ y_perm, const int32_t* __restrict__ slot_row,
    const float* __restrict__ gate, float scale, const float* __restrict__ y_acc,
    const T* __restrict__ x, int H, int K, T* __restrict__ y) {
  __shared__ SlotList sl;
  const int t = blockIdx.x;
  if (threadIdx.x < kWave) read_slots(sl, slot_row, gate, scale, K, t);
  __syncthreads();
  const int n = sl.n;
  const float gs = sl.identity_gate;
  T* yr = y + (size_t)t * H;
  for (int c = threadIdx.x * 8; c < H; c += blockDim.x * 8) {
    float acc[8];
    if constexpr (IDENTITY) {
      Vec8<T>::load(x + (size_t)t * H + c, acc);
#pragma unroll
      for (int i = 0; i < 8; ++i) acc[i] *= gs;
    } else {
      Vec8<float>::load(y_acc + (size_t)t * H + c, acc);
    }
    // up to kBatch rows in flight per thread; accumulation stays in slot order
    for (int j0 = 0; j0 < n; j0 += kBatch) {
      float v[kBatch][8];
#pragma unroll
      for (int u = 0; u < kBatch; ++u)
        if (j0 + u < n) Vec8<T>::load_nt(y_perm + (size_t)sl.rows[j0 + u] * H + c, v[u]);
#pragma unroll
      for (int u = 0; u < kBatch; ++u) {
        if (j0 + u >= n) break;
        const float w = sl.wts[j0 + u];
#pragma unroll
        for (int i = 0; i < 8; ++i) acc[i] = fmaf(w, v[u][i], acc[i]);
      }
    }
    Vec8<T>::store(yr + c, acc);
  }
}

// The same sum for K <= KS <= 16 slots per token and rows of at most 8 x 1024
// elements, one 8-element piece per thread, a row split over lane_parts(H)
// blocks (block b: token b / parts, part b % parts).  Every wave reads the token's
// slots itself -- lane k loads slot k, and each value is then read out of its
// lane into a scalar register -- so no wave waits for another and there is no
// LDS list and no barrier (prefill: 195 -> 189 us; decode: 10.5 -> 8.0 us).
// Blocks that loop over several tokens, loading the next token's slots before
// the current token's rows, measured slower (202 us at 4 tokens per block,
// 208 us at 16): finer blocks balance better, and the slot latency was not
// what bounds the sweep.  Same fp32 operations in the same order as
// combine_kernel.
template <typename T, bool IDENTITY, int KS>
__global__ __launch_bounds__(kMaxThreads) void combine_lanes(
    const T* __restrict__ y_perm, const int32_t* __restrict__ slot_row,
    const float* __restrict__ gate, float scale, const float* __restrict__ y_acc,
    const T* __restrict__ x, int H, int K, int parts, T* __restrict__ y) {
  const int t = blockIdx.x / parts, part = blockIdx.x - t * parts;
  const int lane = threadIdx.x & (kWave - 1);
  int lrow = -1;      // lane k < K: slot k's row of y_perm (-1: identity expert)
  float lg = 0.0f;    // lane k < K: slot k's gate
  if (lane < K) {
    lrow = slot_row[(size_t)t * K + lane];
    lg = gate[(size_t)t * K + lane];
  }
  int row[KS];
  float g[KS];
#pragma unroll
  for (int k = 0; k < KS; ++k) {
    row[k] = __builtin_amdgcn_readlane(lrow, k);
    g[k] = __uint_as_float(__builtin_amdgcn_readlane(__float_as_uint(lg), k));
  }
  float gs = 0.0f;
#pragma unroll
  for (int k = 0; k < KS; ++k)
    if (k < K && row[k] < 0) gs += g[k];
  const int c0 = (part * blockDim.x + threadIdx.x) * 8;
  const int c = c0 < H ? c0 : H - 8;   // surplus lanes load a valid piece, store nothing
  float acc[8];
  if constexpr (IDENTITY) {
    Vec8<T>::load(x + (size_t)t * H + c, acc);
#pragma unroll
    for (int i = 0; i < 8; ++i) acc[i] *= gs;
  } else {
    Vec8<float>::load(y_acc + (size_t)t * H + c, acc);
  }
  typename Vec8<T>::Raw v[KS];
#pragma unroll
  for (int k = 0; k < KS; ++k)
    if (k < K && row[k] >= 0) v[k] = Vec8<T>::load_raw(y_perm + (size_t)row[k] * H + c);
#pragma unroll
  for (int k = 0; k < KS; ++k)
    if (k < K && row[k] >= 0) {
      const float w = scale * g[k];
#pragma unroll
      for (int i = 0; i < 8; ++i) acc[i] = fmaf(w, Vec8<T>::at(v[k], i), acc[i]);
    }
  if (c0 < H) Vec8<T>::store(y + (size_t)t * H + c, acc);
}

}  // namespace

hipError_t launch_zero_experts(const void* x, int dtype, const int32_t* idx, const float* gate,
                               int T, int H, int K, int n_ffn, float* y_acc, hipStream_t s) {
  if (dtype == MOE_BF16)
    MOE_LAUNCH("zero_experts", s,
               zero_experts_kernel<bf16><<<T, row_threads(H), 0, s>>>(
                   (const bf16*)x, idx, gate, H, K, n_ffn, y_acc));
  else
    MOE_LAUNCH("zero_experts", s,
               zero_experts_kernel<float><<<T, row_threads(H), 0, s>>>(
                   (const float*)x, idx, gate, H, K, n_ffn, y_acc));
  return hipGetLastError();
}

hipError_t launch_combine(const void* y_perm, int dtype, const int32_t* slot_row,
                          const float* gate, float scale, const float* y_acc, const void* x,
                          int T, int H, int K, void* y, hipStream_t s) {
#define MOE_STREAM(TY, ID, KS)                                                              \
  combine_lanes<TY, ID, KS><<<T * lane_parts(H), lane_threads(H), 0, s>>>(                  \
      (const TY*)y_perm, slot_row, gate, scale, y_acc, (const TY*)x, H, K, lane_parts(H),   \
      (TY*)y)
#define MOE_COMBINE(TY, ID)                                                                  \
  (H > 8 * kMaxThreads ? combine_kernel<TY, ID><<<T, row_threads(H), 0, s>>>(                \
                   (const TY*)y_perm, slot_row, gate, scale, y_acc, (const TY*)x, H, K, (TY*)y) \
   : K <= 4  ? MOE_STREAM(TY, ID, 4)                                                         \
   : K <= 8  ? MOE_STREAM(TY, ID, 8)                                                         \
   : K <= 12 ? MOE_STREAM(TY, ID, 12)                                                        \
   : K <= 16 ? MOE_STREAM(TY, ID, 16)                                                        \
             : combine_kernel<TY, ID><<<T, row_threads(H), 0, s>>>(                          \
                   (const TY*)y_perm, slot_row, gate, scale, y_acc, (const TY*)x, H, K, (TY*)y))
  if (dtype == MOE_BF16) {
    if (x) MOE_LAUNCH("combine_identity", s, MOE_COMBINE(bf16, true));
    else MOE_LAUNCH("combine", s, MOE_COMBINE(bf16, false));
  } else {
    if (x) MOE_LAUNCH("combine_identity", s, MOE_COMBINE(float, true));
    else MOE_LAUNCH("combine", s, MOE_COMBINE(float, false));
  }
#undef MOE_COMBINE
#undef MOE_STREAM
  return hipGetLastError();
}

}  // namespace moe
