// Dynamic Expert Assembly on gfx950.
//
// OmniMoE digest (paper.rainbus.top), method paragraph, step 1: each atomic
// expert e is a pair of d-vectors (row e of W, row e of V) computing
// sigma(x w_e^T) v_e; step 3: every active group q computes
// O_q = (G_q . sigma(X_q W_q^T)) V_q over its scheduled tasks.
//
// The product is split in two passes so that y needs no atomics:
//   expert_act  walks the tasks in schedule order (groups of B consecutive
//               experts, tokens ascending inside a group) and computes the
//               gated activation a_m = g_m * SiLU(x_t . W[e_m]) of every task:
//               the (G_q . sigma(X_q W_q^T)) factor.  Consecutive tasks reuse
//               the same W rows (same group) and x rows (same token).
//   expert_out  y_t = sum_k a_{t,k} V[e_{t,k}]: the product with V_q, summed
//               per token in k order by the thread that owns y_t's columns.
// fp32 atomics on MI355X run at a few hundred G ops/s, far below what a
// scatter-add of every group's O_q rows into y would need; the owner-computes
// sum writes each y element exactly once and is deterministic.

#include "omni_internal.h"

namespace omni {
namespace {

constexpr int ACT_TPW = 16;  // tasks per wave in expert_act

template <bool BF16>
struct Vec;
template <>
struct Vec<true> {  // 8 bf16 per 16-byte load
  static constexpr int E = 8;
  __device__ static float dot(const u32x4 a, const u32x4 b) {
    float fa[8], fb[8];
    widen8(a, fa);
    widen8(b, fb);
    float s = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i) s = fmaf(fa[i], fb[i], s);
    return s;
  }
  __device__ static void axpy(float a, const u32x4 v, float* acc) {
    float f[8];
    widen8(v, f);
#pragma unroll
    for (int i = 0; i < 8; ++i) acc[i] = fmaf(a, f[i], acc[i]);
  }
};
template <>
struct Vec<false> {  // 4 fp32 per 16-byte load
  static constexpr int E = 4;
  __device__ static float dot(const u32x4 a, const u32x4 b) {
    float s = __uint_as_float(a.x) * __uint_as_float(b.x);
    s = fmaf(__uint_as_float(a.y), __uint_as_float(b.y), s);
    s = fmaf(__uint_as_float(a.z), __uint_as_float(b.z), s);
    return fmaf(__uint_as_float(a.w), __uint_as_float(b.w), s);
  }
  __device__ static void axpy(float a, const u32x4 v, float* acc) {
    acc[0] = fmaf(a, __uint_as_float(v.x), acc[0]);
    acc[1] = fmaf(a, __uint_as_float(v.y), acc[1]);
    acc[2] = fmaf(a, __uint_as_float(v.z), acc[2]);
    acc[3] = fmaf(a, __uint_as_float(v.w), acc[3]);
  }
};

__device__ __forceinline__ int readlane(int v, int l) { return __builtin_amdgcn_readlane(v, l); }
__device__ __forceinline__ float readlane(float v, int l) {
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), l));
}

// One wave per ACT_TPW consecutive scheduled tasks.  A row of d elements is
// NCH chunks of 64 lanes x 16 bytes; lane `lane` holds bytes [16*lane, +16)
// of each chunk.  The task metadata is fetched once per wave (one task per
// lane) and broadcast; the next task's W row (and x row, when the token
// changes) is in flight while the current one is reduced.
template <bool BF16, int NCH>
__global__ __launch_bounds__(256) void expert_act(const uint16_t* __restrict__ x_,
                                                  const uint16_t* __restrict__ W_,
                                                  const int32_t* __restrict__ idx,
                                                  const float* __restrict__ gate,
                                                  const int32_t* __restrict__ perm, int M, int d,
                                                  int K, float* __restrict__ act) {
  using V = Vec<BF16>;
  const int lane = threadIdx.x & 63;
  const int wave = blockIdx.x * 4 + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int p0 = wave * ACT_TPW;
  if (p0 >= M) return;
  const int n = min(ACT_TPW, M - p0);
  const size_t row_bytes = (size_t)d * (BF16 ? 2 : 4);
  const char* xb = (const char*)x_;
  const char* Wb = (const char*)W_;

  int my_m = 0, my_e = 0;
  float my_g = 0.f;
  if (lane < n) {
    my_m = perm[p0 + lane];
    my_e = idx[my_m];
    my_g = gate[my_m];
  }

  const int cbytes = lane * 16;  // byte offset inside a 1 KB chunk
  auto load_row = [&](const char* base, u32x4* r) {
#pragma unroll
    for (int c = 0; c < NCH; ++c) {
      const size_t o = (size_t)c * 1024 + cbytes;
      r[c] = o < row_bytes ? *(const u32x4*)(base + o) : u32x4{0u, 0u, 0u, 0u};
    }
  };

  u32x4 xc[NCH], xn[NCH], wc[NCH], wn[NCH];
  int t_cur = readlane(my_m, 0) / K;
  load_row(xb + (size_t)t_cur * row_bytes, xn);
  load_row(Wb + (size_t)readlane(my_e, 0) * row_bytes, wn);
  for (int i = 0; i < n; ++i) {
#pragma unroll
    for (int c = 0; c < NCH; ++c) {
      xc[c] = xn[c];
      wc[c] = wn[c];
    }
    const int m = readlane(my_m, i);
    const float g = readlane(my_g, i);
    if (i + 1 < n) {
      const int t_next = readlane(my_m, i + 1) / K;
      if (t_next != t_cur) load_row(xb + (size_t)t_next * row_bytes, xn);
      t_cur = t_next;
      load_row(Wb + (size_t)readlane(my_e, i + 1) * row_bytes, wn);
    }
    float part = 0.f;
#pragma unroll
    for (int c = 0; c < NCH; ++c) part += V::dot(xc[c], wc[c]);
    const float h = wave_sum(part);
    if (lane == 0) act[m] = g * (h / (1.f + expf(-h)));
  }
}

// One thread per (token, 16-byte column chunk).
template <bool BF16>
__global__ __launch_bounds__(256) void expert_out(const uint16_t* __restrict__ V_,
                                                  const int32_t* __restrict__ idx,
                                                  const float* __restrict__ act, int L, int d,
                                                  int K, float* __restrict__ y) {
  using V = Vec<BF16>;
  constexpr int E = V::E;
  const int upt = d / E;
  const long long u = (long long)blockIdx.x * blockDim.x + threadIdx.x;
  const int t = (int)(u / upt);
  if (t >= L) return;
  const int c = (int)(u - (long long)t * upt) * E;
  const size_t row_bytes = (size_t)d * (BF16 ? 2 : 4);
  const char* Vb = (const char*)V_ + (size_t)c * (BF16 ? 2 : 4);
  const int32_t* it = idx + (size_t)t * K;
  const float* at = act + (size_t)t * K;
  float acc[E];
#pragma unroll
  for (int i = 0; i < E; ++i) acc[i] = 0.f;
  int k = 0;
  for (; k + 8 <= K; k += 8) {
    int e[8];
    float a[8];
    u32x4 v[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      e[j] = it[k + j];
      a[j] = at[k + j];
    }
#pragma unroll
    for (int j = 0; j < 8; ++j) v[j] = *(const u32x4*)(Vb + (size_t)e[j] * row_bytes);
#pragma unroll
    for (int j = 0; j < 8; ++j) V::axpy(a[j], v[j], acc);
  }
  for (; k < K; ++k) V::axpy(at[k], *(const u32x4*)(Vb + (size_t)it[k] * row_bytes), acc);
  float* yo = y + (size_t)t * d + c;
#pragma unroll
  for (int i = 0; i < E; i += 4) *(f32x4*)(yo + i) = f32x4{acc[i], acc[i + 1], acc[i + 2], acc[i + 3]};
}

template <bool BF16>
hipError_t launch_act_t(const void* x, const void* W, const int32_t* idx, const float* gate,
                        const int32_t* perm, int M, int d, int K, float* act, hipStream_t s) {
  const size_t row_bytes = (size_t)d * (BF16 ? 2 : 4);
  const int nch = (int)((row_bytes + 1023) / 1024);
  const int waves = (M + ACT_TPW - 1) / ACT_TPW;
  const dim3 grid((waves + 3) / 4), block(256);
  const uint16_t* xp = (const uint16_t*)x;
  const uint16_t* wp = (const uint16_t*)W;
#define OMNI_ACT(N)                                                                          \
  case N:                                                                                    \
    hipLaunchKernelGGL((expert_act<BF16, N>), grid, block, 0, s, xp, wp, idx, gate, perm, M, \
                       d, K, act);                                                           \
    break;
  switch (nch) {
    OMNI_ACT(1) OMNI_ACT(2) OMNI_ACT(3) OMNI_ACT(4) OMNI_ACT(5) OMNI_ACT(6) OMNI_ACT(7)
    OMNI_ACT(8)
    default:
      return hipErrorInvalidValue;
  }
#undef OMNI_ACT
  return hipGetLastError();
}

}  // namespace

hipError_t launch_expert_act(const void* x, const void* W, const int32_t* idx, const float* gate,
                             const int32_t* perm, int L, int d, int K, omni_dtype dt, float* act,
                             hipStream_t s) {
  const int M = L * K;
  return dt == OMNI_BF16 ? launch_act_t<true>(x, W, idx, gate, perm, M, d, K, act, s)
                         : launch_act_t<false>(x, W, idx, gate, perm, M, d, K, act, s);
}

hipError_t launch_expert_out(const void* V, const int32_t* idx, const float* act, int L, int d,
                             int K, omni_dtype dt, float* y, hipStream_t s) {
  const int E = dt == OMNI_BF16 ? 8 : 4;
  const long long units = (long long)L * (d / E);
  const dim3 grid((unsigned)((units + 255) / 256)), block(256);
  if (dt == OMNI_BF16)
    hipLaunchKernelGGL(expert_out<true>, grid, block, 0, s, (const uint16_t*)V, idx, act, L, d, K,
                       y);
  else
    hipLaunchKernelGGL(expert_out<false>, grid, block, 0, s, (const uint16_t*)V, idx, act, L, d,
                       K, y);
  return hipGetLastError();
}

}  // namespace omni
