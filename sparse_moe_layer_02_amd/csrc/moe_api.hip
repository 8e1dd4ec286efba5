// C-ABI entry points: host-side validation (no HIP call before it passes),
// then the kernels are enqueued on the caller's stream.  See
// include/moe_mi355x.h for the contract of each call.
#include "moe_internal.h"

using namespace moe;

namespace {

constexpr int kMaxE = 1024;      // route: one wave64 holds up to 16 keys per lane
constexpr int kMaxFfn = 4096;    // permute: 64-bit LDS mask per FFN expert
constexpr int kMaxKCombine = 1024;

inline bool dtype_ok(int d) { return d == MOE_F32 || d == MOE_BF16; }
inline bool aligned(const void* p, size_t a) { return ((uintptr_t)p % a) == 0; }
inline bool fits_i32(long long v) { return v >= 0 && v < (1ll << 31); }
inline bool finite(float v) { return v == v && v - v == 0.0f; }

inline moe_status launched(hipError_t e) { return e == hipSuccess ? MOE_OK : MOE_ERR_LAUNCH; }

}  // namespace

extern "C" {

const char* moe_status_string(int s) {
  switch (s) {
    case MOE_OK: return "ok";
    case MOE_ERR_NULL: return "null pointer";
    case MOE_ERR_SHAPE: return "unsupported shape";
    case MOE_ERR_DTYPE: return "unknown dtype";
    case MOE_ERR_ALIGN: return "misaligned pointer";
    case MOE_ERR_WORKSPACE: return "workspace too small";
    case MOE_ERR_LAUNCH: return "kernel launch failed";
    case MOE_ERR_TOO_LARGE: return "sizes exceed the fixed scratch";
    default: return "unknown status";
  }
}

moe_status moe_router_logits(const void* x, int x_dtype, const float* w_router, int T, int H,
                             int E, float* logits, void* stream) {
  if (!x || !w_router || !logits) return MOE_ERR_NULL;
  if (!dtype_ok(x_dtype)) return MOE_ERR_DTYPE;
  if (T < 1 || H < 1 || E < 1 || !fits_i32((long long)T * E)) return MOE_ERR_SHAPE;
  if (!aligned(x, x_dtype == MOE_BF16 ? 2 : 4) || !aligned(w_router, 4) || !aligned(logits, 4))
    return MOE_ERR_ALIGN;
  return launched(launch_router_logits(x, x_dtype, w_router, nullptr, T, H, E, logits,
                                       (hipStream_t)stream));
}

moe_status moe_router_split_weights(const float* w_router, int E, int H, void* w_planes,
                                    void* stream) {
  if (!w_router || !w_planes) return MOE_ERR_NULL;
  if (E < 1 || H < 1 || H % 8 || (long long)E * H > (1ll << 40)) return MOE_ERR_SHAPE;
  if (!aligned(w_router, 16) || !aligned(w_planes, 16)) return MOE_ERR_ALIGN;
  return launched(launch_router_split(w_router, E, H, w_planes, (hipStream_t)stream));
}

moe_status moe_router_logits_planes(const void* x, int x_dtype, const float* w_router,
                                    const void* w_planes, int T, int H, int E, float* logits,
                                    void* stream) {
  if (!x || !w_router || !logits) return MOE_ERR_NULL;
  if (!dtype_ok(x_dtype)) return MOE_ERR_DTYPE;
  if (T < 1 || H < 1 || E < 1 || !fits_i32((long long)T * E)) return MOE_ERR_SHAPE;
  if (w_planes && H % 8) return MOE_ERR_SHAPE;
  if (!aligned(x, x_dtype == MOE_BF16 ? 2 : 4) || !aligned(w_router, 4) || !aligned(logits, 4) ||
      !aligned(w_planes, 16))
    return MOE_ERR_ALIGN;
  return launched(launch_router_logits(x, x_dtype, w_router, w_planes, T, H, E, logits,
                                       (hipStream_t)stream));
}

moe_status moe_route(const float* logits, const float* bias, int T, int E, int K,
                     int32_t* topk_idx, float* topk_gate, int32_t* counts, int32_t* dev_status,
                     void* stream) {
  if (!logits || !bias || !topk_idx || !topk_gate || !counts) return MOE_ERR_NULL;
  if (T < 1 || E < 1 || E > kMaxE || K < 1 || K > E || !fits_i32((long long)T * K) ||
      !fits_i32((long long)T * E))
    return MOE_ERR_SHAPE;
  if (!aligned(logits, 4) || !aligned(bias, 4) || !aligned(topk_idx, 4) ||
      !aligned(topk_gate, 4) || !aligned(counts, 4) || !aligned(dev_status, 4))
    return MOE_ERR_ALIGN;
  return launched(launch_route(logits, bias, T, E, K, topk_idx, topk_gate, counts, dev_status,
                               (hipStream_t)stream));
}

moe_status moe_permute(const void* x, int dtype, const int32_t* topk_idx, const int32_t* counts,
                       int T, int H, int K, int n_ffn, int32_t* offsets, void* x_perm,
                       int32_t* row_src, int32_t* slot_row, void* stream) {
  if ((x_perm && !x) || !topk_idx || !counts || !offsets || !row_src || !slot_row)
    return MOE_ERR_NULL;
  if (!dtype_ok(dtype)) return MOE_ERR_DTYPE;
  if (T < 1 || H < 1 || H % 8 || K < 1 || n_ffn < 0 || n_ffn > kMaxFfn ||
      !fits_i32((long long)T * K))
    return MOE_ERR_SHAPE;
  if (!aligned(x, 16) || !aligned(x_perm, 16) || !aligned(topk_idx, 4) || !aligned(counts, 4) ||
      !aligned(offsets, 4) || !aligned(row_src, 4) || !aligned(slot_row, 4))
    return MOE_ERR_ALIGN;
  return launched(launch_permute(x, dtype, topk_idx, counts, T, H, K, n_ffn, offsets, x_perm,
                                 row_src, slot_row, (hipStream_t)stream));
}

size_t moe_expert_ffn_workspace_bytes(int rows_cap, int n_ffn, int I, int dtype) {
  if (rows_cap < 1 || n_ffn < 0 || I < 1 || !dtype_ok(dtype)) return 0;
  return ffn_ws_bytes(rows_cap, n_ffn, I, dtype);
}

namespace {
// The checks the expert-FFN entry points share; a is the activation source.
// check_ws = false: the workspace is the library's own (noalloc variant).
moe_status ffn_checks(const void* a, const int32_t* offsets, int rows_cap, int n_ffn, int H, int I,
                      const void* w13, const void* w2, int dtype, const void* y_perm,
                      const void* ws, size_t ws_bytes, bool check_ws = true) {
  if (!a || !offsets || (n_ffn != 0 && (!w13 || !w2)) || !y_perm || (check_ws && !ws))
    return MOE_ERR_NULL;
  if (!dtype_ok(dtype)) return MOE_ERR_DTYPE;
  if (rows_cap < 1 || n_ffn < 0 || n_ffn > kMaxFfn || H < 1 || I < 1) return MOE_ERR_SHAPE;
  if (dtype == MOE_BF16 && (H % 128 || I % 64)) return MOE_ERR_SHAPE;
  if (dtype == MOE_F32 && (long long)rows_cap / 32 + n_ffn + 8 > 65535) return MOE_ERR_SHAPE;
  const size_t al = dtype == MOE_BF16 ? 16 : 4;
  if (!aligned(a, al) || !aligned(w13, al) || !aligned(w2, al) || !aligned(y_perm, al) ||
      !aligned(offsets, 4) || !aligned(ws, 256))
    return MOE_ERR_ALIGN;
  if (check_ws && ws_bytes < ffn_ws_bytes(rows_cap, n_ffn, I, dtype)) return MOE_ERR_WORKSPACE;
  return MOE_OK;
}
}  // namespace

moe_status moe_expert_ffn(const void* x_perm, const int32_t* offsets, int rows_cap, int n_ffn,
                          int H, int I, const void* w13, const void* w2, int dtype, void* y_perm,
                          void* ws, size_t ws_bytes, void* stream) {
  const moe_status st =
      ffn_checks(x_perm, offsets, rows_cap, n_ffn, H, I, w13, w2, dtype, y_perm, ws, ws_bytes);
  if (st != MOE_OK || n_ffn == 0) return st;
  return launched(launch_expert_ffn(x_perm, nullptr, 1, 1, offsets, rows_cap, n_ffn, H, I, w13,
                                    w2, dtype, y_perm, ws, (hipStream_t)stream));
}

moe_status moe_expert_ffn_gather(const void* x, int T, int K, const int32_t* row_src,
                                 const int32_t* offsets, int rows_cap, int n_ffn, int H, int I,
                                 const void* w13, const void* w2, int dtype, void* y_perm,
                                 void* ws, size_t ws_bytes, void* stream) {
  if (!row_src) return MOE_ERR_NULL;
  const moe_status st =
      ffn_checks(x, offsets, rows_cap, n_ffn, H, I, w13, w2, dtype, y_perm, ws, ws_bytes);
  if (st != MOE_OK) return st;
  if (T < 1 || K < 1 || !fits_i32((long long)T * K)) return MOE_ERR_SHAPE;
  if (!aligned(row_src, 4)) return MOE_ERR_ALIGN;
  if (n_ffn == 0) return MOE_OK;
  return launched(launch_expert_ffn(x, row_src, K, T, offsets, rows_cap, n_ffn, H, I, w13, w2,
                                    dtype, y_perm, ws, (hipStream_t)stream));
}

moe_status moe_expert_ffn_gather_noalloc(const void* x, int T, int K, const int32_t* row_src,
                                         const int32_t* offsets, int rows_cap, int n_ffn, int H,
                                         int I, const void* w13, const void* w2, int dtype,
                                         void* y_perm, void* stream) {
  if (!row_src) return MOE_ERR_NULL;
  const moe_status st =
      ffn_checks(x, offsets, rows_cap, n_ffn, H, I, w13, w2, dtype, y_perm, nullptr, 0, false);
  if (st != MOE_OK) return st;
  if (T < 1 || K < 1 || !fits_i32((long long)T * K)) return MOE_ERR_SHAPE;
  if (!aligned(row_src, 4)) return MOE_ERR_ALIGN;
  if (ffn_ws_bytes(rows_cap, n_ffn, I, dtype) > MOE_EXPERT_FFN_NOALLOC_SCRATCH_BYTES)
    return MOE_ERR_TOO_LARGE;
  if (n_ffn == 0) return MOE_OK;
  void* ws = nullptr;
  if (noalloc_scratch(&ws) != hipSuccess) return MOE_ERR_LAUNCH;
  return launched(launch_expert_ffn(x, row_src, K, T, offsets, rows_cap, n_ffn, H, I, w13, w2,
                                    dtype, y_perm, ws, (hipStream_t)stream));
}

moe_status moe_zero_experts(const void* x, int dtype, const int32_t* topk_idx,
                            const float* topk_gate, int T, int H, int K, int n_ffn, float* y_acc,
                            void* stream) {
  if (!x || !topk_idx || !topk_gate || !y_acc) return MOE_ERR_NULL;
  if (!dtype_ok(dtype)) return MOE_ERR_DTYPE;
  if (T < 1 || H < 1 || H % 8 || K < 1 || n_ffn < 0 || !fits_i32((long long)T * K))
    return MOE_ERR_SHAPE;
  if (!aligned(x, 16) || !aligned(y_acc, 16) || !aligned(topk_idx, 4) || !aligned(topk_gate, 4))
    return MOE_ERR_ALIGN;
  return launched(launch_zero_experts(x, dtype, topk_idx, topk_gate, T, H, K, n_ffn, y_acc,
                                      (hipStream_t)stream));
}

moe_status moe_combine(const void* y_perm, int dtype, const int32_t* slot_row,
                       const float* topk_gate, float ffn_scale, const float* y_acc, int T, int H,
                       int K, void* y, void* stream) {
  if (!y_perm || !slot_row || !topk_gate || !y_acc || !y) return MOE_ERR_NULL;
  if (!dtype_ok(dtype)) return MOE_ERR_DTYPE;
  if (T < 1 || H < 1 || H % 8 || K < 1 || K > kMaxKCombine || !fits_i32((long long)T * K))
    return MOE_ERR_SHAPE;
  if (!aligned(y_perm, 16) || !aligned(y_acc, 16) || !aligned(y, 16) || !aligned(slot_row, 4) ||
      !aligned(topk_gate, 4))
    return MOE_ERR_ALIGN;
  return launched(launch_combine(y_perm, dtype, slot_row, topk_gate, ffn_scale, y_acc, nullptr,
                                 T, H, K, y, (hipStream_t)stream));
}

moe_status moe_combine_identity(const void* y_perm, const void* x, int dtype,
                                const int32_t* slot_row, const float* topk_gate, float ffn_scale,
                                int T, int H, int K, void* y, void* stream) {
  if (!y_perm || !x || !slot_row || !topk_gate || !y) return MOE_ERR_NULL;
  if (!dtype_ok(dtype)) return MOE_ERR_DTYPE;
  if (T < 1 || H < 1 || H % 8 || K < 1 || K > kMaxKCombine || !fits_i32((long long)T * K))
    return MOE_ERR_SHAPE;
  if (!aligned(y_perm, 16) || !aligned(x, 16) || !aligned(y, 16) || !aligned(slot_row, 4) ||
      !aligned(topk_gate, 4))
    return MOE_ERR_ALIGN;
  return launched(launch_combine(y_perm, dtype, slot_row, topk_gate, ffn_scale, nullptr, x, T, H,
                                 K, y, (hipStream_t)stream));
}

moe_status moe_bias_update(const int32_t* counts, int T, int n_ffn, float target, float kp,
                           float ki, float kd, float* bias, float* integral, float* prev_err,
                           void* stream) {
  if (!counts || !bias || !integral || !prev_err) return MOE_ERR_NULL;
  if (T < 1 || n_ffn < 1 || n_ffn > kMaxFfn || !finite(target) || !finite(kp) || !finite(ki) ||
      !finite(kd))
    return MOE_ERR_SHAPE;
  if (!aligned(counts, 4) || !aligned(bias, 4) || !aligned(integral, 4) || !aligned(prev_err, 4))
    return MOE_ERR_ALIGN;
  return launched(launch_bias_update(counts, T, n_ffn, target, kp, ki, kd, bias, integral,
                                     prev_err, (hipStream_t)stream));
}

// ------------------------------------------------------ one-call forward --
namespace {
struct ForwardWs {
  float* logits;
  int32_t* idx;
  float* gate;
  int32_t* counts;
  int32_t* offsets;
  int32_t* row_src;
  int32_t* slot_row;
  void* y_perm;
  void* ffn;
  size_t ffn_bytes;
  size_t total;
};

inline size_t al256(size_t b) { return (b + 255) & ~(size_t)255; }

// Parts of moe_forward's workspace, each 256-byte aligned, in this order.
ForwardWs forward_ws(char* base, int T, int H, int E, int n_ffn, int I, int K, int dtype) {
  const size_t rows = (size_t)T * K, es = dtype == MOE_BF16 ? 2 : 4;
  ForwardWs w{};
  size_t off = 0;
  auto take = [&](size_t bytes) {
    char* p = base ? base + off : nullptr;
    off += al256(bytes);
    return p;
  };
  w.logits = (float*)take((size_t)T * E * 4);
  w.idx = (int32_t*)take(rows * 4);
  w.gate = (float*)take(rows * 4);
  w.counts = (int32_t*)take((size_t)E * 4);
  w.offsets = (int32_t*)take(((size_t)n_ffn + 1) * 4);
  w.row_src = (int32_t*)take(rows * 4);
  w.slot_row = (int32_t*)take(rows * 4);
  w.y_perm = take(rows * H * es);
  w.ffn_bytes = n_ffn > 0 ? ffn_ws_bytes((int)rows, n_ffn, I, dtype) : 0;
  w.ffn = take(w.ffn_bytes);
  w.total = off;
  return w;
}

// Every check of the five calls moe_forward makes, before any of them.
moe_status forward_checks(const void* x, int dtype, const float* w_router, const void* w_planes,
                          const float* bias, const void* w13, const void* w2, int T, int H, int E,
                          int n_ffn, int I, int K, const void* y, const int32_t* dev_status,
                          const void* ws) {
  if (!x || !w_router || !bias || !y || !ws || (n_ffn > 0 && (!w13 || !w2))) return MOE_ERR_NULL;
  if (!dtype_ok(dtype)) return MOE_ERR_DTYPE;
  if (T < 1 || H < 1 || H % 8 || E < 1 || E > kMaxE || K < 1 || K > E || K > kMaxKCombine ||
      n_ffn < 0 || n_ffn > E || n_ffn > kMaxFfn || I < 1 || !fits_i32((long long)T * K) ||
      !fits_i32((long long)T * E))
    return MOE_ERR_SHAPE;
  if (dtype == MOE_BF16 && (H % 128 || I % 64)) return MOE_ERR_SHAPE;
  if (dtype == MOE_F32 && (long long)T * K / 32 + n_ffn + 8 > 65535) return MOE_ERR_SHAPE;
  const size_t al = dtype == MOE_BF16 ? 16 : 4;
  if (!aligned(x, 16) || !aligned(w_router, 4) || !aligned(w_planes, 16) || !aligned(bias, 4) ||
      !aligned(w13, al) || !aligned(w2, al) || !aligned(y, 16) || !aligned(dev_status, 4) ||
      !aligned(ws, 256))
    return MOE_ERR_ALIGN;
  return MOE_OK;
}
}  // namespace

size_t moe_forward_workspace_bytes(int T, int H, int E, int n_ffn, int I, int K, int dtype) {
  if (T < 1 || H < 1 || E < 1 || n_ffn < 0 || n_ffn > E || I < 1 || K < 1 || !dtype_ok(dtype) ||
      !fits_i32((long long)T * K) || !fits_i32((long long)T * E))
    return 0;
  return forward_ws(nullptr, T, H, E, n_ffn, I, K, dtype).total;
}

moe_status moe_forward(const void* x, int dtype, const float* w_router, const void* w_planes,
                       const float* bias, const void* w13, const void* w2, int T, int H, int E,
                       int n_ffn, int I, int K, float ffn_scale, void* y, int32_t* dev_status,
                       void* ws, size_t ws_bytes, void* stream) {
  const moe_status st = forward_checks(x, dtype, w_router, w_planes, bias, w13, w2, T, H, E,
                                       n_ffn, I, K, y, dev_status, ws);
  if (st != MOE_OK) return st;
  const ForwardWs w = forward_ws((char*)ws, T, H, E, n_ffn, I, K, dtype);
  if (ws_bytes < w.total) return MOE_ERR_WORKSPACE;
  const hipStream_t s = (hipStream_t)stream;
  hipError_t e = launch_router_logits(x, dtype, w_router, w_planes, T, H, E, w.logits, s);
  if (e == hipSuccess)
    e = launch_route(w.logits, bias, T, E, K, w.idx, w.gate, w.counts, dev_status, s);
  if (e == hipSuccess)
    e = launch_permute(x, dtype, w.idx, w.counts, T, H, K, n_ffn, w.offsets, nullptr, w.row_src,
                       w.slot_row, s);
  if (e == hipSuccess && n_ffn > 0)
    e = launch_expert_ffn(x, w.row_src, K, T, w.offsets, T * K, n_ffn, H, I, w13, w2, dtype,
                          w.y_perm, w.ffn, s);
  if (e == hipSuccess)
    e = launch_combine(w.y_perm, dtype, w.slot_row, w.gate, ffn_scale, nullptr, x, T, H, K, y, s);
  return launched(e);
}

size_t moe_router_similarity_workspace_bytes(int E, int H) {
  if (E < 1 || H < 1 || H % 4 || !fits_i32((long long)E * E)) return 0;
  return similarity_ws_bytes(E, H);
}

moe_status moe_router_similarity(const float* w_router, int E, int H, float* sim, float* mean,
                                 void* ws, size_t ws_bytes, void* stream) {
  if (!w_router || !sim || !mean || !ws) return MOE_ERR_NULL;
  if (E < 1 || H < 1 || H % 4 || !fits_i32((long long)E * E)) return MOE_ERR_SHAPE;
  if (!aligned(w_router, 16) || !aligned(sim, 4) || !aligned(mean, 4) || !aligned(ws, 256))
    return MOE_ERR_ALIGN;
  if (ws_bytes < similarity_ws_bytes(E, H)) return MOE_ERR_WORKSPACE;
  return launched(launch_router_similarity(w_router, E, H, sim, mean, ws, (hipStream_t)stream));
}

}  // extern "C"
