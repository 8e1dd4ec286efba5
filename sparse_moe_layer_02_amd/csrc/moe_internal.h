// Internal declarations shared by the HIP translation units of the library.
// Target: gfx950 (CDNA4), wave64.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "../../include/moe_mi355x.h"

namespace moe {

typedef __bf16 bf16;
typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4;
typedef __attribute__((__vector_size__(4 * sizeof(int)))) int i32x4;

constexpr int kWave = 64;

__device__ __forceinline__ float bf16_to_f32(bf16 v) { return (float)v; }
__device__ __forceinline__ bf16 f32_to_bf16(float v) { return (bf16)v; }  // RNE on gfx950

// Load/store one element of T as fp32.
template <typename T> __device__ __forceinline__ float ld_f32(const T* p);
template <> __device__ __forceinline__ float ld_f32<float>(const float* p) { return *p; }
template <> __device__ __forceinline__ float ld_f32<bf16>(const bf16* p) { return (float)*p; }
template <typename T> __device__ __forceinline__ void st_f32(T* p, float v);
template <> __device__ __forceinline__ void st_f32<float>(float* p, float v) { *p = v; }
template <> __device__ __forceinline__ void st_f32<bf16>(bf16* p, float v) { *p = (bf16)v; }

// s_waitcnt with only vmcnt constrained (gfx9 encoding: vmcnt[3:0] at bits
// 3:0 and vmcnt[5:4] at bits 15:14; expcnt and lgkmcnt left at their maximum).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 0xF) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}

// Workgroup barrier that does not drain outstanding global loads: LDS
// accesses of this wave complete first (lgkmcnt 0), the compiler may not move
// memory accesses across it, and loads into LDS that are still in flight stay
// in flight (their completion is awaited with wait_vmcnt).
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_s_waitcnt((0x3F & 0xF) | ((0x3F >> 4) << 14) | (0x7 << 4) | (0x0 << 8));
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// Order the LDS accesses of one wave across its lanes: this wave's LDS
// writes have completed (lgkmcnt 0) and the compiler moves no memory access
// across this point, so a lane may next read what another lane wrote.
__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_s_waitcnt((0x3F & 0xF) | ((0x3F >> 4) << 14) | (0x7 << 4) | (0x0 << 8));
  asm volatile("" ::: "memory");
  __builtin_amdgcn_wave_barrier();
  asm volatile("" ::: "memory");
}

inline unsigned ceil_div(size_t a, size_t b) { return (unsigned)((a + b - 1) / b); }

// ---- opt-in per-kernel event timing (profile.hip) --------------------------
int prof_begin(const char* name, hipStream_t s);   // -1 when timing is off
void prof_end(int token, hipStream_t s);
#define MOE_LAUNCH(name, stream, ...)                 \
  do {                                                \
    const int moe_tok_ = ::moe::prof_begin(name, stream); \
    __VA_ARGS__;                                      \
    ::moe::prof_end(moe_tok_, stream);                \
  } while (0)

// ---- launchers (each returns hipGetLastError() after enqueueing) ----------
// planes: the weights split by launch_router_split, or NULL (split in the kernel)
hipError_t launch_router_logits(const void* x, int dtype, const float* w, const void* planes,
                                int T, int H, int E, float* logits, hipStream_t s);
hipError_t launch_router_split(const float* w, int E, int H, void* planes, hipStream_t s);
hipError_t launch_route(const float* logits, const float* bias, int T, int E, int K,
                        int32_t* idx, float* gate, int32_t* counts, int32_t* status,
                        hipStream_t s);
hipError_t launch_permute(const void* x, int dtype, const int32_t* idx, const int32_t* counts,
                          int T, int H, int K, int n_ffn, int32_t* offsets, void* x_perm,
                          int32_t* row_src, int32_t* slot_row, hipStream_t s);
size_t ffn_ws_bytes(int rows_cap, int n_ffn, int I, int dtype);
// Device address, on the current device, of the fixed scratch array of
// moe_expert_ffn_gather_noalloc (MOE_EXPERT_FFN_NOALLOC_SCRATCH_BYTES).
hipError_t noalloc_scratch(void** addr);
// gather == nullptr: row r's activations are x_perm[r]; otherwise they are
// token row gather[r] / gK (clamped to [0, gT)) of x_perm, i.e. of x.
hipError_t launch_expert_ffn(const void* x_perm, const int32_t* gather, int gK, int gT,
                             const int32_t* offsets, int rows_cap, int n_ffn, int H, int I,
                             const void* w13, const void* w2, int dtype, void* y_perm, void* ws,
                             hipStream_t s);
hipError_t launch_zero_experts(const void* x, int dtype, const int32_t* idx, const float* gate,
                               int T, int H, int K, int n_ffn, float* y_acc, hipStream_t s);
// x == nullptr: the identity term is y_acc; otherwise it is computed from x
// and the identity slots' gates (slot_row < 0) and y_acc is not read.
hipError_t launch_combine(const void* y_perm, int dtype, const int32_t* slot_row,
                          const float* gate, float scale, const float* y_acc, const void* x,
                          int T, int H, int K, void* y, hipStream_t s);
hipError_t launch_bias_update(const int32_t* counts, int T, int n_ffn, float target, float kp,
                              float ki, float kd, float* bias, float* integral, float* prev,
                              hipStream_t s);
size_t similarity_ws_bytes(int E, int H);
hipError_t launch_router_similarity(const float* w, int E, int H, float* sim, float* mean,
                                    void* ws, hipStream_t s);

}  // namespace moe
