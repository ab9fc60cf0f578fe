// Dynamic Expert Assembly on gfx950.
//
// OmniMoE digest (paper.rainbus.top), method paragraph, step 1: atomic expert
// e is a pair of d-vectors (row e of W, row e of V) computing
// sigma(x w_e^T) v_e; step 3: each active group q computes
// O_q = (G_q . sigma(X_q W_q^T)) V_q over its scheduled tasks.
//
// The product runs as two passes so that y needs no atomics:
//   expert_act  walks the tasks in schedule order (groups of B consecutive
//               experts, tokens ascending inside a group) and computes every
//               task's gated activation a_m = g_m * SiLU(x_t . W[e_m]): the
//               (G_q . sigma(X_q W_q^T)) factor of the group product.
//   expert_out  y_t = sum_k a_{t,k} V[e_{t,k}]: the product with V_q, summed
//   (_w)        per token in k order by the lanes that own y_t's columns.
// fp32 atomics on MI355X sustain a few hundred G ops/s, far below what a
// scatter-add of every group's O_q rows into y would need (about 2 ms at
// 4096 tokens x 128 experts x d = 2048); the owner-computes sum writes each
// y element once and is deterministic.

#include "omni_internal.h"

namespace omni {
namespace {

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

// Non-temporal 16-byte load for V rows that are streamed once per task
// (measured 5% faster than plain loads in the output pass at uniform
// routing).
__device__ __forceinline__ u32x4 ld16_nt(const char* p) {
  return __builtin_nontemporal_load((const u32x4*)p);
}

__device__ __forceinline__ int uni(int v) { return __builtin_amdgcn_readfirstlane(v); }
__device__ __forceinline__ float uni(float v) {
  return __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(v)));
}

// ------------------------------------------------------------------ expert_act
// The 8 XCDs of an MI355X each have their own L2 and workgroup i runs on XCD
// i % 8.  The scheduled task stream is cut into chunks of ACT_CHUNK tasks;
// chunk c is visited by the 8 one-wave workgroups 8c .. 8c+7, and workgroup
// 8c+x takes the chunk's tasks whose token t has t % 8 == x.  Each XCD so
// reads the x rows of one eighth of the tokens, a set that stays resident
// in its L2, while the stream order inside the chunk (group, then token)
// is kept.  The wave's tasks are compacted into LDS; the W row of the next
// task is in flight while the current one is reduced (two row buffers).
// Measured on the 4096-token, 1.7M-expert workload: chunks of 8 to 32 tasks
// are equally fast and 128 is 10% slower; without the XCD split the x rows
// fall out of L2 and the pass is 15% slower; plain loads of W beat
// non-temporal ones (repeated experts of a group can hit in the caches).
constexpr int ACT_CHUNK = 32;
constexpr int XCDS = 8;

template <bool BF16, int NCH>
__global__ __launch_bounds__(64) void expert_act(const uint16_t* __restrict__ x_,
                                                 const uint16_t* __restrict__ W_,
                                                 const int32_t* __restrict__ idx,
                                                 const float* __restrict__ gate,
                                                 const int32_t* __restrict__ perm, int M, int d,
                                                 int K, float* __restrict__ act) {
  using V = Vec<BF16>;
  __shared__ int sm[ACT_CHUNK];
  __shared__ int se[ACT_CHUNK];
  __shared__ float sg[ACT_CHUNK];
  const int lane = threadIdx.x;
  const unsigned long long lt = (1ull << lane) - 1ull;
  const int chunk = blockIdx.x / XCDS, part = blockIdx.x % XCDS;
  const int p0 = chunk * ACT_CHUNK;
  const int n = min(ACT_CHUNK, M - p0);
  int cnt = 0;
  for (int h = 0; h < ACT_CHUNK; h += 64) {  // ACT_CHUNK <= 64: one pass
    const bool v = h + lane < n;
    const int m = v ? perm[p0 + h + lane] : 0;
    const bool mine = v && (m / K) % XCDS == part;
    const unsigned long long b = __ballot(mine);
    if (mine) {
      const int pos = cnt + __popcll(b & lt);
      sm[pos] = m;
      se[pos] = idx[m];
      sg[pos] = gate[m];
    }
    cnt += __popcll(b);
  }
  if (cnt == 0) return;
  __syncthreads();

  // a row is NCH chunks of 64 lanes x 16 bytes; lane l holds bytes [16l, 16l+16)
  const unsigned row_bytes = (unsigned)d * (BF16 ? 2u : 4u);
  const unsigned cb = lane * 16u;
  auto load_x = [&](int t, u32x4* r) {
    const char* base = (const char*)x_ + (size_t)t * row_bytes;
#pragma unroll
    for (int c = 0; c < NCH; ++c) {
      const unsigned o = c * 1024u + cb;
      r[c] = o < row_bytes ? *(const u32x4*)(base + o) : u32x4{0u, 0u, 0u, 0u};
    }
  };
  auto load_w = [&](int e, u32x4* r) {
    const char* base = (const char*)W_ + (size_t)e * row_bytes;
#pragma unroll
    for (int c = 0; c < NCH; ++c) {
      const unsigned o = c * 1024u + cb;
      r[c] = o < row_bytes ? *(const u32x4*)(base + o) : u32x4{0u, 0u, 0u, 0u};
    }
  };
  u32x4 xr[NCH], wa[NCH], wb[NCH];
  int t_cur = -1;
  auto step = [&](int i, const u32x4* w) {
    const int m = uni(sm[i]);
    const float g = uni(sg[i]);
    const int t = m / K;
    if (t != t_cur) {  // consecutive tasks of one token reuse its x row
      load_x(t, xr);
      t_cur = t;
    }
    float part_sum = 0.f;
#pragma unroll
    for (int c = 0; c < NCH; ++c) part_sum += V::dot(xr[c], w[c]);
    const float h = wave_sum(part_sum);
    if (lane == 0) act[m] = g * (h / (1.f + expf(-h)));
  };
  load_w(uni(se[0]), wa);
  for (int i = 0; i < cnt; i += 2) {
    if (i + 1 < cnt) load_w(uni(se[i + 1]), wb);
    step(i, wa);
    if (i + 1 < cnt) {
      if (i + 2 < cnt) load_w(uni(se[i + 2]), wa);
      step(i + 1, wb);
    }
  }
}

// ------------------------------------------------------------------ expert_out
// y_t = sum_k a_{t,k} V[e_{t,k}], each element summed over k in order, in
// one of two forms (the same y, bit for bit):
//
// expert_out_w (no token order): one wave per token, four tokens per
// workgroup.  Lane l holds bytes [1024 c + 16 l, +16) of the row for
// c < NCH, so each V row is read by one wave in NCH back-to-back 1 KB
// loads, non-temporally (each row is used once per task); 16 loads per lane
// are in flight.  Measured at 4096 tokens x 1.7M experts: 766 against 776 us
// for the assembly call with the per-token workgroups below.
//
// expert_out (with a token order): one workgroup per token: the token's K
// (expert, activation) pairs are staged in LDS once; each thread owns 16
// bytes of y's row and streams the K rows of V, OUT_UNROLL row loads in
// flight (kept together by a scheduling barrier).  The grid has
// 8 * ceil(L/8) slots and workgroup b (which runs on XCD b % 8) takes slot
// (b % 8) * ceil(L/8) + b / 8: each XCD walks its own contiguous eighth of
// the order, so tokens that the order puts together share that XCD's L2.
// Slots past L and entries outside [0, L) do nothing.  The order is there
// for routing whose tokens share experts, so the V rows are plain loads
// that the caches keep (16384 clustered tokens: 640 us against 1349 us
// non-temporal); this form is also 3% faster than one wave per token there.
constexpr int OUT_UNROLL = 16;
template <bool BF16>
__global__ __launch_bounds__(512) void expert_out(const uint16_t* __restrict__ V_,
                                                  const int32_t* __restrict__ idx,
                                                  const float* __restrict__ act,
                                                  const int32_t* __restrict__ order, int L, int d,
                                                  int K, float* __restrict__ y) {
  using V = Vec<BF16>;
  constexpr int E = V::E;
  __shared__ int se[OMNI_MAX_K];
  __shared__ float sa[OMNI_MAX_K];
  int t = blockIdx.x;
  if (order) {
    const int per = (L + 7) / 8;
    const int slot = (blockIdx.x % 8) * per + blockIdx.x / 8;
    if (slot >= L) return;
    t = order[slot];
    if ((unsigned)t >= (unsigned)L) return;
  }
  const int tid = threadIdx.x;
  for (int k = tid; k < K; k += blockDim.x) {
    se[k] = idx[(size_t)t * K + k];
    sa[k] = act[(size_t)t * K + k];
  }
  __syncthreads();
  const int c = tid * E;
  if (c >= d) return;
  const size_t row_bytes = (size_t)d * (BF16 ? 2 : 4);
  const unsigned cb = (unsigned)c * (BF16 ? 2u : 4u);
  const char* Vb = (const char*)V_;
  float acc[E];
#pragma unroll
  for (int i = 0; i < E; ++i) acc[i] = 0.f;
  int k = 0;
  for (; k + OUT_UNROLL <= K; k += OUT_UNROLL) {
    u32x4 v[OUT_UNROLL];
#pragma unroll
    for (int j = 0; j < OUT_UNROLL; ++j)
      v[j] = *(const u32x4*)(Vb + (size_t)uni(se[k + j]) * row_bytes + cb);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int j = 0; j < OUT_UNROLL; ++j) V::axpy(uni(sa[k + j]), v[j], acc);
  }
  for (; k < K; ++k)
    V::axpy(uni(sa[k]), *(const u32x4*)(Vb + (size_t)uni(se[k]) * row_bytes + cb), acc);
  float* yo = y + (size_t)t * d + c;
#pragma unroll
  for (int i = 0; i < E; i += 4) *(f32x4*)(yo + i) = f32x4{acc[i], acc[i + 1], acc[i + 2], acc[i + 3]};
}

template <bool BF16, int NCH>
__global__ __launch_bounds__(256) void expert_out_w(const uint16_t* __restrict__ V_,
                                                    const int32_t* __restrict__ idx,
                                                    const float* __restrict__ act, int L, int d,
                                                    int K, float* __restrict__ y) {
  using V = Vec<BF16>;
  constexpr int E = V::E;
  constexpr int U = NCH >= 16 ? 1 : 16 / NCH;
  __shared__ int se[4][OMNI_MAX_K];
  __shared__ float sa[4][OMNI_MAX_K];
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
  const int t = 4 * blockIdx.x + w;
  if (t >= L) return;  // whole wave; no workgroup barrier follows
  for (int k = lane; k < K; k += 64) {
    se[w][k] = idx[(size_t)t * K + k];
    sa[w][k] = act[(size_t)t * K + k];
  }
  wave_sync();
  const unsigned row_bytes = (unsigned)d * (BF16 ? 2u : 4u);
  const unsigned cb = lane * 16u;
  const char* Vb = (const char*)V_;
  float acc[NCH][E];
#pragma unroll
  for (int c = 0; c < NCH; ++c)
#pragma unroll
    for (int i = 0; i < E; ++i) acc[c][i] = 0.f;
  auto load_row = [&](int e, u32x4* r) {
    const char* base = Vb + (size_t)e * row_bytes;
#pragma unroll
    for (int c = 0; c < NCH; ++c) {
      const unsigned o = c * 1024u + cb;
      r[c] = o < row_bytes ? ld16_nt(base + o) : u32x4{0u, 0u, 0u, 0u};
    }
  };
  int k = 0;
  for (; k + U <= K; k += U) {
    u32x4 v[U][NCH];
#pragma unroll
    for (int j = 0; j < U; ++j) load_row(uni(se[w][k + j]), v[j]);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int j = 0; j < U; ++j) {
      const float a = uni(sa[w][k + j]);
#pragma unroll
      for (int c = 0; c < NCH; ++c) V::axpy(a, v[j][c], acc[c]);
    }
  }
  for (; k < K; ++k) {
    u32x4 v[NCH];
    load_row(uni(se[w][k]), v);
    const float a = uni(sa[w][k]);
#pragma unroll
    for (int c = 0; c < NCH; ++c) V::axpy(a, v[c], acc[c]);
  }
  float* yo = y + (size_t)t * d;
#pragma unroll
  for (int c = 0; c < NCH; ++c) {
    const unsigned o = c * 1024u + cb;  // byte offset in the input row
    if (o < row_bytes) {
      const int col = (int)(o / (BF16 ? 2u : 4u));
#pragma unroll
      for (int i = 0; i < E; i += 4)
        *(f32x4*)(yo + col + i) = f32x4{acc[c][i], acc[c][i + 1], acc[c][i + 2], acc[c][i + 3]};
    }
  }
}

// ------------------------------------------------------------------ token-centric baseline
// The execution order the pages compare against (makerbund section 5: the
// ablation that reverts expert-centric scheduling): each token fetches the
// rows of its own K experts, with no schedule.  One workgroup per token:
// wave w computes a_k = g_k * SiLU(x_t . W[e_k]) for k = w, w+4, ... (x_t held
// in registers, TC_ROWS W rows in flight), the K activations meet in LDS, and
// the V pass is the one of expert_out (one workgroup per token).
constexpr int TC_ROWS = 4;

template <bool BF16, int NCH>
__global__ __launch_bounds__(256) void expert_tc(const uint16_t* __restrict__ x_,
                                                 const uint16_t* __restrict__ W_,
                                                 const uint16_t* __restrict__ V_,
                                                 const int32_t* __restrict__ idx,
                                                 const float* __restrict__ gate, int d, int K,
                                                 float* __restrict__ y) {
  using V = Vec<BF16>;
  constexpr int E = V::E;
  __shared__ int se[OMNI_MAX_K];
  __shared__ float sa[OMNI_MAX_K];
  const int t = blockIdx.x, tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  for (int k = tid; k < K; k += 256) se[k] = idx[(size_t)t * K + k];
  __syncthreads();

  const unsigned row_bytes = (unsigned)d * (BF16 ? 2u : 4u);
  const unsigned cb = lane * 16u;
  u32x4 xr[NCH];
  {
    const char* base = (const char*)x_ + (size_t)t * row_bytes;
#pragma unroll
    for (int c = 0; c < NCH; ++c) {
      const unsigned o = c * 1024u + cb;
      xr[c] = o < row_bytes ? *(const u32x4*)(base + o) : u32x4{0u, 0u, 0u, 0u};
    }
  }
  // W pass: rows k = wave + 4*(r0 + q), TC_ROWS at a time
  for (int k0 = wave; k0 < K; k0 += 4 * TC_ROWS) {
    u32x4 w[TC_ROWS][NCH];
#pragma unroll
    for (int q = 0; q < TC_ROWS; ++q) {
      const int k = k0 + 4 * q;
      const char* base = (const char*)W_ + (size_t)uni(se[k < K ? k : k0]) * row_bytes;
#pragma unroll
      for (int c = 0; c < NCH; ++c) {
        const unsigned o = c * 1024u + cb;
        w[q][c] = (k < K && o < row_bytes) ? *(const u32x4*)(base + o) : u32x4{0u, 0u, 0u, 0u};
      }
    }
#pragma unroll
    for (int q = 0; q < TC_ROWS; ++q) {
      const int k = k0 + 4 * q;
      float part = 0.f;
#pragma unroll
      for (int c = 0; c < NCH; ++c) part += V::dot(xr[c], w[q][c]);
      const float h = wave_sum(part);
      if (lane == 0 && k < K) sa[k] = gate[(size_t)t * K + k] * (h / (1.f + expf(-h)));
    }
  }
  __syncthreads();
  // V pass: each thread owns 16 bytes of y's row
  for (int c0 = tid * E; c0 < d; c0 += 256 * E) {
    const unsigned ob = (unsigned)c0 * (BF16 ? 2u : 4u);
    float acc[E];
#pragma unroll
    for (int i = 0; i < E; ++i) acc[i] = 0.f;
    int k = 0;
    for (; k + OUT_UNROLL <= K; k += OUT_UNROLL) {
      u32x4 v[OUT_UNROLL];
#pragma unroll
      for (int j = 0; j < OUT_UNROLL; ++j)
        v[j] = ld16_nt((const char*)V_ + (size_t)uni(se[k + j]) * row_bytes + ob);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int j = 0; j < OUT_UNROLL; ++j) V::axpy(uni(sa[k + j]), v[j], acc);
    }
    for (; k < K; ++k)
      V::axpy(uni(sa[k]), ld16_nt((const char*)V_ + (size_t)uni(se[k]) * row_bytes + ob), acc);
    float* yo = y + (size_t)t * d + c0;
#pragma unroll
    for (int i = 0; i < E; i += 4) *(f32x4*)(yo + i) = f32x4{acc[i], acc[i + 1], acc[i + 2], acc[i + 3]};
  }
}

template <bool BF16>
hipError_t launch_tc_t(const void* x, const void* W, const void* V, const int32_t* idx,
                       const float* gate, int L, int d, int K, float* y, hipStream_t s) {
  const size_t row_bytes = (size_t)d * (BF16 ? 2 : 4);
  const int nch = (int)((row_bytes + 1023) / 1024);
  const uint16_t* xp = (const uint16_t*)x;
  const uint16_t* wp = (const uint16_t*)W;
  const uint16_t* vp = (const uint16_t*)V;
#define OMNI_TC(N)                                                                           \
  case N:                                                                                    \
    hipLaunchKernelGGL((expert_tc<BF16, N>), dim3(L), dim3(256), 0, s, xp, wp, vp, idx, gate, \
                       d, K, y);                                                             \
    break;
  switch (nch) {
    OMNI_TC(1) OMNI_TC(2) OMNI_TC(3) OMNI_TC(4) OMNI_TC(5) OMNI_TC(6) OMNI_TC(7) OMNI_TC(8)
    default:
      return hipErrorInvalidValue;  // d above the validated limit
  }
#undef OMNI_TC
  return hipGetLastError();
}

template <bool BF16>
hipError_t launch_act_t(const void* x, const void* W, const int32_t* idx, const float* gate,
                        const int32_t* perm, int M, int d, int K, float* act, hipStream_t s) {
  const size_t row_bytes = (size_t)d * (BF16 ? 2 : 4);
  const int nch = (int)((row_bytes + 1023) / 1024);
  const uint16_t* xp = (const uint16_t*)x;
  const uint16_t* wp = (const uint16_t*)W;
  const dim3 grid((unsigned)(((M + ACT_CHUNK - 1) / ACT_CHUNK) * XCDS)), block(64);
#define OMNI_ACT(N)                                                                          \
  case N:                                                                                    \
    hipLaunchKernelGGL((expert_act<BF16, N>), grid, block, 0, s, xp, wp, idx, gate, perm, M, \
                       d, K, act);                                                           \
    break;
  switch (nch) {
    OMNI_ACT(1) OMNI_ACT(2) OMNI_ACT(3) OMNI_ACT(4) OMNI_ACT(5) OMNI_ACT(6) OMNI_ACT(7)
    OMNI_ACT(8)
    default:
      return hipErrorInvalidValue;  // d above the validated limit
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

hipError_t launch_expert_tc(const void* x, const void* W, const void* V, const int32_t* idx,
                            const float* gate, int L, int d, int K, omni_dtype dt, float* y,
                            hipStream_t s) {
  return dt == OMNI_BF16 ? launch_tc_t<true>(x, W, V, idx, gate, L, d, K, y, s)
                         : launch_tc_t<false>(x, W, V, idx, gate, L, d, K, y, s);
}

hipError_t launch_expert_out(const void* V, const int32_t* idx, const float* act,
                             const int32_t* order, int L, int d, int K, omni_dtype dt, float* y,
                             hipStream_t s) {
  const bool bf = dt == OMNI_BF16;
  if (order) {
    const int threads = ((d / (bf ? 8 : 4) + 63) / 64) * 64;  // <= 512 for the supported d
    if (bf)
      hipLaunchKernelGGL((expert_out<true>), dim3(8 * ((L + 7) / 8)), dim3(threads), 0, s,
                         (const uint16_t*)V, idx, act, order, L, d, K, y);
    else
      hipLaunchKernelGGL((expert_out<false>), dim3(8 * ((L + 7) / 8)), dim3(threads), 0, s,
                         (const uint16_t*)V, idx, act, order, L, d, K, y);
    return hipGetLastError();
  }
  const int nch = (int)(((size_t)d * (bf ? 2 : 4) + 1023) / 1024);  // 1..8 for the supported d
  const dim3 grid((L + 3) / 4), block(256);
#define OMNI_OUT(BF, N)                                                                         \
  case N:                                                                                      \
    hipLaunchKernelGGL((expert_out_w<BF, N>), grid, block, 0, s, (const uint16_t*)V, idx, act, \
                       L, d, K, y);                                                            \
    break
#define OMNI_OUT_ALL(BF)                                                                        \
  switch (nch) {                                                                               \
    OMNI_OUT(BF, 1); OMNI_OUT(BF, 2); OMNI_OUT(BF, 3); OMNI_OUT(BF, 4);                         \
    OMNI_OUT(BF, 5); OMNI_OUT(BF, 6); OMNI_OUT(BF, 7); OMNI_OUT(BF, 8);                         \
    default: return hipErrorInvalidValue;                                                      \
  }
  if (bf) { OMNI_OUT_ALL(true) }
  else { OMNI_OUT_ALL(false) }
#undef OMNI_OUT_ALL
#undef OMNI_OUT
  return hipGetLastError();
}

}  // namespace omni
