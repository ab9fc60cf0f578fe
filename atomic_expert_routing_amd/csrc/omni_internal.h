// Internal declarations shared by the libomni.so translation units (gfx950).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "omni.h"

namespace omni {

// ----------------------------------------------------------------- device helpers

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

// bf16 is the top half of an fp32 word: widening is exact.
__device__ __forceinline__ float bf16lo(unsigned int w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16hi(unsigned int w) { return __uint_as_float(w & 0xffff0000u); }

// 16 bytes -> 8 floats (bf16) ; the fp32 variant is 4 floats.
__device__ __forceinline__ void widen8(const u32x4 v, float* f) {
  f[0] = bf16lo(v.x); f[1] = bf16hi(v.x);
  f[2] = bf16lo(v.y); f[3] = bf16hi(v.y);
  f[4] = bf16lo(v.z); f[5] = bf16hi(v.z);
  f[6] = bf16lo(v.w); f[7] = bf16hi(v.w);
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  return v;
}

// Order-preserving map float -> uint32 (larger float -> larger uint).
__device__ __forceinline__ unsigned int float_ord(float f) {
  unsigned int b = __float_as_uint(f);
  return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}
__device__ __forceinline__ float ord_float(unsigned int u) {
  return __uint_as_float((u & 0x80000000u) ? (u & 0x7fffffffu) : ~u);
}

// ----------------------------------------------------------------- host launchers
// Each returns hipSuccess or the launch error; arguments are pre-validated.

// logits[L, Nr+Nc] (fp32) = x [L,d] . [Wr; Wc]^T
hipError_t launch_router_gemm(const void* x, const void* Wr, const void* Wc, int L, int d,
                              int Nr, int Nc, omni_dtype dt, float* logits, hipStream_t s);

// per token: LogSoftmax of both logit halves, implicit top-K, gate softmax
hipError_t launch_router_topk(const float* logits, int L, int Nr, int Nc, int K,
                              int32_t* idx, float* score, float* gate, hipStream_t s);
size_t router_topk_lds_bytes(int Nr, int Nc, int K);

struct SchedPlan {
  int M, G, ntiles, passes, digit_bits;
  size_t ws_bytes;
  // workspace carve (byte offsets)
  size_t off_keys_a, off_vals_a, off_keys_b, off_vals_b, off_hist, off_totals;
};
SchedPlan plan_schedule(int64_t L, int64_t K, int64_t N, int64_t B);
hipError_t launch_schedule(const int32_t* idx, int M, int B, int G, const SchedPlan& plan,
                           int32_t* perm, int32_t* group_off, void* ws, hipStream_t s);

// act[m] = gate[m] * SiLU(x[m/K] . W[idx[m]]) for m in schedule order
hipError_t launch_expert_act(const void* x, const void* W, const int32_t* idx, const float* gate,
                             const int32_t* perm, int L, int d, int K, omni_dtype dt,
                             float* act, hipStream_t s);
// y[t] = sum_k act[t*K+k] * V[idx[t*K+k]]
hipError_t launch_expert_out(const void* V, const int32_t* idx, const float* act, int L, int d,
                             int K, omni_dtype dt, float* y, hipStream_t s);

}  // namespace omni
