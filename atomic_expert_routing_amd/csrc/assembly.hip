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

#include <algorithm>

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

// A buffer resource spanning one row of `bytes` bytes: its loads take the
// row's base from scalar registers, and a load past the row's end returns
// zero (the ragged last 1 KB chunk of a row needs no test).  Word 3 selects
// the 32-bit data format; a zero format would make every untyped load
// return zero.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t row_rsrc(const void* row, unsigned bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(row), 0, (int)bytes, 0x00020000);
}
// Cache policies of the buffer loads (the instruction's cache-policy field):
// plain, or non-temporal (streamed: the line is not kept for reuse).
constexpr int LD_PLAIN = 0, LD_NT = 2;

// Chunk c (1 KB) of a row through its buffer resource: lane l's 16 bytes at
// c * 1024 + 16 l.
template <int POLICY>
__device__ __forceinline__ u32x4 ld_row16(__amdgpu_buffer_rsrc_t r, unsigned off) {
  return __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, POLICY);
}

__device__ __forceinline__ int uni(int v) { return __builtin_amdgcn_readfirstlane(v); }
__device__ __forceinline__ float uni(float v) {
  return __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(v)));
}

// ------------------------------------------------------------------ expert_act
// The activation pass walks the schedule group by group.  act_plan cuts the
// sorted tasks into chunks along group boundaries: chunk c starts at the
// first group boundary in [c*ACT_CHUNK, (c+1)*ACT_CHUNK) (found from the
// group of that position, idx/B, and group_off), or at c*ACT_CHUNK when one
// group covers that whole window (a group larger than a chunk is split).
// A chunk so holds whole groups (1 to 2*ACT_CHUNK-1 tasks), and all tasks of
// one group and token class run in one wave, next to each other in time:
// a W row that several of them use is fetched once and served from the
// cache to the others.
//
// The 8 XCDs of an MI355X each have their own L2 and workgroup i runs on XCD
// i % 8.  Chunk c is visited by the 8 one-wave workgroups 8c .. 8c+7, and
// workgroup 8c+x takes the chunk's tasks whose token t has t % 8 == x.  Each
// XCD so reads the x rows of one eighth of the tokens, a set that stays
// resident in its L2, while the stream order inside the chunk (group, then
// token) is kept.  The wave's tasks are compacted into LDS; the W row of
// the next task is in flight while the current one is reduced (two row
// buffers).  Measured on the 4096-token, 1.7M-expert workload: chunks of 8
// to 32 tasks are equally fast and 128 is 10% slower; without the XCD split
// the x rows fall out of L2 and the pass is 15% slower.
// Both rows are buffer loads (scalar row base); the W rows are
// non-temporal, so the stream of W rows, each used by about one task, does
// not push the XCD's x rows out of L2.  Per-task call (act_plan, this pass,
// the output pass), against plain global loads: 815 -> 791 us at 4096
// tokens x 1.7M experts, 430 -> 418 us at 1M, 191 -> 172 us at 280,900
// (the same y bit for bit).
constexpr int ACT_CHUNK = 32;
constexpr int XCDS = 8;
constexpr int ACT_MAX_CHUNK_GROUPS = 16384;

__global__ __launch_bounds__(256) void act_plan(const int32_t* __restrict__ idx,
                                                const int32_t* __restrict__ perm,
                                                const int32_t* __restrict__ group_off, int M,
                                                int B, int G, int nchunks,
                                                int32_t* __restrict__ start,
                                                const int32_t* run_flag, int run_want) {
  if (gated_out(run_flag, run_want)) return;
  const int c = blockIdx.x * 256 + threadIdx.x;
  if (c > nchunks) return;
  const int p = c * ACT_CHUNK;
  int s = M;
  if (p < M) {
    // ids outside [0, N) break the precondition; clamping keeps the reads in bounds
    const int g = min(max(idx[perm[p]] / B, 0), G - 1);
    const int a = group_off[g];
    if (a == p) {
      s = p;
    } else {
      const int b = group_off[g + 1];
      s = (b > p && b < p + ACT_CHUNK) ? b : p;
    }
  }
  start[c] = s;
}

template <bool BF16, int NCH>
__global__ __launch_bounds__(64) void expert_act(const uint16_t* __restrict__ x_,
                                                 const uint16_t* __restrict__ W_,
                                                 const int32_t* __restrict__ idx,
                                                 const float* __restrict__ gate,
                                                 const int32_t* __restrict__ perm,
                                                 const int32_t* __restrict__ start, int nchunks,
                                                 int d, int K, float* __restrict__ act,
                                                 const int32_t* run_flag, int run_want) {
  using V = Vec<BF16>;
  __shared__ int sm[2 * ACT_CHUNK];
  __shared__ int se[2 * ACT_CHUNK];
  __shared__ float sg[2 * ACT_CHUNK];
  static_assert(2 * ACT_CHUNK <= 64, "one lane per task of a chunk");
  const int lane = threadIdx.x;
  const unsigned long long lt = (1ull << lane) - 1ull;
  const int part = blockIdx.x % XCDS;
  // the gate's words are read together with the first chunk's bounds (one
  // memory latency, not two, before the work starts)
  const int g_distinct = run_flag ? run_flag[1] : 0, g_sampled = run_flag ? run_flag[2] : 0;
  const unsigned row_bytes = (unsigned)d * (BF16 ? 2u : 4u);
  const unsigned cb = lane * 16u;
  auto load_x = [&](int t, u32x4* r) {
    const auto rs = row_rsrc((const char*)x_ + (size_t)t * row_bytes, row_bytes);
#pragma unroll
    for (int c = 0; c < NCH; ++c) r[c] = ld_row16<LD_PLAIN>(rs, c * 1024u + cb);
  };
  auto load_w = [&](int e, u32x4* r) {
    const auto rs = row_rsrc((const char*)W_ + (size_t)e * row_bytes, row_bytes);
#pragma unroll
    for (int c = 0; c < NCH; ++c) r[c] = ld_row16<LD_NT>(rs, c * 1024u + cb);
  };
  // grid-stride over the chunks: workgroup 8j + x takes chunks j, j + G, ...
  // (G = gridDim / 8) for token class x
  for (int chunk = blockIdx.x / XCDS; chunk < nchunks; chunk += gridDim.x / XCDS) {
    const int p0 = start[chunk];
    const int n = start[chunk + 1] - p0;  // 0 .. 2*ACT_CHUNK-1
    if (run_flag && auto_choice_of(g_distinct, g_sampled) != run_want) return;
    const bool v = lane < n;
    const int m = v ? perm[p0 + lane] : 0;
    const bool mine = v && (m / K) % XCDS == part;
    const unsigned long long b = __ballot(mine);
    const int cnt = __popcll(b);
    wave_sync();  // the previous chunk's reads of sm, se, sg are done
    if (mine) {
      const int pos = __popcll(b & lt);
      sm[pos] = m;
      se[pos] = idx[m];
      sg[pos] = gate[m];
    }
    if (cnt == 0) continue;
    wave_sync();

    u32x4 xr[NCH], wa[NCH], wb[NCH];
    int t_cur = -1;
    auto step = [&](int i, const u32x4* w) {
      const int mi = uni(sm[i]);
      const float g = uni(sg[i]);
      const int t = mi / K;
      if (t != t_cur) {  // consecutive tasks of one token reuse its x row
        load_x(t, xr);
        t_cur = t;
      }
      float part_sum = 0.f;
#pragma unroll
      for (int c = 0; c < NCH; ++c) part_sum += V::dot(xr[c], w[c]);
      const float h = wave_sum(part_sum);
      if (lane == 0) act[mi] = g * (h / (1.f + expf(-h)));
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
                                                  int K, float* __restrict__ y,
                                                  const int32_t* run_flag, int run_want) {
  if (gated_out(run_flag, run_want)) return;
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
                                                    int K, float* __restrict__ y,
                                                    const int32_t* run_flag, int run_want) {
  using V = Vec<BF16>;
  constexpr int E = V::E;
  constexpr int U = NCH >= 16 ? 1 : 16 / NCH;
  __shared__ int se[4][OMNI_MAX_K];
  __shared__ float sa[4][OMNI_MAX_K];
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
  const int t = 4 * blockIdx.x + w;
  if (t >= L) return;  // whole wave; no workgroup barrier follows
  // the gate's words are read beside the token's ids and activations
  const int g_distinct = run_flag ? run_flag[1] : 0, g_sampled = run_flag ? run_flag[2] : 0;
  for (int k = lane; k < K; k += 64) {
    se[w][k] = idx[(size_t)t * K + k];
    sa[w][k] = act[(size_t)t * K + k];
  }
  if (run_flag && auto_choice_of(g_distinct, g_sampled) != run_want) return;
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
// in registers, TC_ROWS W rows in flight, loaded as in expert_act: buffer
// loads, non-temporal), the K activations meet in LDS, and the V pass is the
// one of expert_out (one workgroup per token).
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
      // rows past K: an empty buffer, whose loads return zero
      const auto rs = row_rsrc((const char*)W_ + (size_t)uni(se[k < K ? k : k0]) * row_bytes,
                               k < K ? row_bytes : 0u);
#pragma unroll
      for (int c = 0; c < NCH; ++c) w[q][c] = ld_row16<LD_NT>(rs, c * 1024u + cb);
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
                        const int32_t* perm, const int32_t* group_off, int M, int d, int K, int B,
                        int G, float* act, int32_t* start, hipStream_t s, RunGate run) {
  const size_t row_bytes = (size_t)d * (BF16 ? 2 : 4);
  const int nch = (int)((row_bytes + 1023) / 1024);
  const uint16_t* xp = (const uint16_t*)x;
  const uint16_t* wp = (const uint16_t*)W;
  const int nchunks = (M + ACT_CHUNK - 1) / ACT_CHUNK;
  hipLaunchKernelGGL(act_plan, dim3((nchunks + 1 + 255) / 256), dim3(256), 0, s, idx, perm,
                     group_off, M, B, G, nchunks, start, run.flag, run.want);
  // at most ACT_MAX_CHUNK_GROUPS chunks run side by side, each group of 8
  // workgroups looping over chunks: a launch whose run gate is off then costs
  // a few microseconds, not one workgroup per 32 tasks
  const dim3 grid((unsigned)(std::min(nchunks, ACT_MAX_CHUNK_GROUPS) * XCDS)), block(64);
#define OMNI_ACT(N)                                                                          \
  case N:                                                                                    \
    hipLaunchKernelGGL((expert_act<BF16, N>), grid, block, 0, s, xp, wp, idx, gate, perm,    \
                       start, nchunks, d, K, act, run.flag, run.want);                       \
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

// ------------------------------------------------------------------ automatic choice
// The per-task passes read one W and one V row per task; the blocked form
// (blocked.hip) reads each row once per block of 64 tokens of the token
// order, at the price of dense MFMA tiles over the block's union of experts.
// The choice rests on how often the step's tasks repeat their experts, which
// only the device knows.  auto_mark takes a fixed sample of the tasks (all of
// them when there are at most AUTO_SAMPLE; else tasks i * 2654435761 mod M,
// distinct for distinct i) and counts the distinct experts among them, one
// bit per expert, the count of newly set bits adding up as it goes.
// The blocked form is taken when the sample holds each of its experts
// AUTO_REUSE times or more on average (auto_choice, which every kernel of
// both forms evaluates from the two counts; the form not chosen returns at
// once).  The two sorts (the schedule's, over the tasks, and the token order
// the blocked form follows) share one set of launches.  Measured: at 16384
// clustered tokens x K = 256 the blocked form takes 0.48 ms against 1.7 ms;
// on spread-out routing (1.2 to 1.6 tasks per expert) the per-task passes
// take 0.78 ms against 1.1 ms at 4096 tokens x 1.7M experts.
constexpr int AUTO_SAMPLE = 65536;

// gate[1] = 0 distinct experts so far, gate[2] = the sample size S
__global__ __launch_bounds__(256) void auto_clear(uint32_t* __restrict__ bits, int nwords,
                                                  int32_t* __restrict__ gate, int S) {
  for (int i = blockIdx.x * 256 + threadIdx.x; i < nwords; i += gridDim.x * 256) bits[i] = 0u;
  if (blockIdx.x == 0 && threadIdx.x == 0) {
    gate[1] = 0;
    gate[2] = S;
  }
}

// One sampled task per thread; the newly set bits are summed per workgroup
// and added to the count once per workgroup (1024 waves adding to the one
// counter serialised on it: 15.6 us for 65536 samples).
constexpr int AUTO_MARK_THREADS = 1024;
__global__ __launch_bounds__(AUTO_MARK_THREADS) void auto_mark(
    const int32_t* __restrict__ idx, int M, int N, int S, uint32_t* __restrict__ bits,
    int32_t* __restrict__ counter) {
  __shared__ int wsum[AUTO_MARK_THREADS / 64];
  const int i = blockIdx.x * AUTO_MARK_THREADS + threadIdx.x;
  int fresh = 0;
  if (i < S) {
    const int m = M <= S ? i : (int)(((uint64_t)i * 2654435761ull) % (uint64_t)M);
    const int e = idx[m];
    if ((unsigned)e < (unsigned)N) {
      const uint32_t bit = 1u << (e & 31);
      fresh = (atomicOr(&bits[e >> 5], bit) & bit) ? 0 : 1;
    }
  }
  fresh = wave_sum_i(fresh);
  if ((threadIdx.x & 63) == 0) wsum[threadIdx.x >> 6] = fresh;
  __syncthreads();
  if (threadIdx.x == 0) {
    int t = 0;
#pragma unroll
    for (int w = 0; w < AUTO_MARK_THREADS / 64; ++w) t += wsum[w];
    if (t) atomicAdd(counter, t);
  }
}

__global__ void set_i32(int32_t* __restrict__ p, int v) { p[0] = v; }

}  // namespace

int auto_sample_size(int64_t M) { return (int)std::min<int64_t>(M, AUTO_SAMPLE); }

hipError_t launch_auto_sample(const int32_t* idx, int M, int64_t N, uint32_t* bits, int32_t* gate,
                              hipStream_t s) {
  const int nwords = (int)((N + 31) / 32);
  const int S = auto_sample_size(M);
  hipLaunchKernelGGL(auto_clear, dim3((unsigned)std::min(512, (nwords + 255) / 256)), dim3(256),
                     0, s, bits, nwords, gate, S);
  hipLaunchKernelGGL(auto_mark, dim3((unsigned)((S + AUTO_MARK_THREADS - 1) / AUTO_MARK_THREADS)),
                     dim3(AUTO_MARK_THREADS), 0, s, idx, M, (int)N, S, bits, gate + 1);
  return hipGetLastError();
}

hipError_t launch_set_i32(int32_t* p, int v, hipStream_t s) {
  hipLaunchKernelGGL(set_i32, dim3(1), dim3(1), 0, s, p, v);
  return hipGetLastError();
}

int expert_act_chunks(int64_t M) { return (int)((M + ACT_CHUNK - 1) / ACT_CHUNK); }

hipError_t launch_expert_act(const void* x, const void* W, const int32_t* idx, const float* gate,
                             const int32_t* perm, const int32_t* group_off, int L, int d, int K,
                             int B, int G, omni_dtype dt, float* act, int32_t* start,
                             hipStream_t s, RunGate run) {
  const int M = L * K;
  return dt == OMNI_BF16
             ? launch_act_t<true>(x, W, idx, gate, perm, group_off, M, d, K, B, G, act, start, s,
                                  run)
             : launch_act_t<false>(x, W, idx, gate, perm, group_off, M, d, K, B, G, act, start, s,
                                   run);
}

hipError_t launch_expert_tc(const void* x, const void* W, const void* V, const int32_t* idx,
                            const float* gate, int L, int d, int K, omni_dtype dt, float* y,
                            hipStream_t s) {
  return dt == OMNI_BF16 ? launch_tc_t<true>(x, W, V, idx, gate, L, d, K, y, s)
                         : launch_tc_t<false>(x, W, V, idx, gate, L, d, K, y, s);
}

hipError_t launch_expert_out(const void* V, const int32_t* idx, const float* act,
                             const int32_t* order, int L, int d, int K, omni_dtype dt, float* y,
                             hipStream_t s, RunGate run) {
  const bool bf = dt == OMNI_BF16;
  if (order) {
    const int threads = ((d / (bf ? 8 : 4) + 63) / 64) * 64;  // <= 512 for the supported d
    if (bf)
      hipLaunchKernelGGL((expert_out<true>), dim3(8 * ((L + 7) / 8)), dim3(threads), 0, s,
                         (const uint16_t*)V, idx, act, order, L, d, K, y, run.flag, run.want);
    else
      hipLaunchKernelGGL((expert_out<false>), dim3(8 * ((L + 7) / 8)), dim3(threads), 0, s,
                         (const uint16_t*)V, idx, act, order, L, d, K, y, run.flag, run.want);
    return hipGetLastError();
  }
  const int nch = (int)(((size_t)d * (bf ? 2 : 4) + 1023) / 1024);  // 1..8 for the supported d
  const dim3 grid((L + 3) / 4), block(256);
#define OMNI_OUT(BF, N)                                                                         \
  case N:                                                                                      \
    hipLaunchKernelGGL((expert_out_w<BF, N>), grid, block, 0, s, (const uint16_t*)V, idx, act, \
                       L, d, K, y, run.flag, run.want);                                        \
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

namespace omni {

AutoPlan plan_expert_auto(int64_t L, int64_t d, int64_t N, int64_t K, int64_t B, omni_dtype dt) {
  auto a256 = [](size_t n) { return (n + 255) & ~(size_t)255; };
  AutoPlan p{};
  const int64_t M = L * K;
  p.G = (int)((N + B - 1) / B);
  p.sample = auto_sample_size(M);
  p.sched = plan_schedule(L, K, N, B);
  p.blocked_ok = dt == OMNI_BF16 && d % BLK_D_TILE == 0 && L <= INT32_MAX - BLK_TOKENS;
  size_t o = 0;
  p.off_flag = o;   o += 256;  // [1] distinct experts in the sample, [2] the sample size
  p.off_bits = o;   o += a256((size_t)((N + 31) / 32) * 4);
  const size_t base = o;
  // per-task passes: perm, group_off, then the schedule's sort buffers,
  // whose space the activations and chunk starts take over afterwards
  p.off_perm = base;
  p.off_goff = p.off_perm + a256((size_t)M * 4);
  p.off_act = p.off_goff + a256((size_t)(p.G + 1) * 4);
  p.off_start = p.off_act + a256((size_t)M * 4);
  const size_t per_task_end =
      p.off_act + std::max(p.sched.ws_bytes, a256((size_t)M * 4) +
                                                 a256(((size_t)expert_act_chunks(M) + 1) * 4));
  size_t end = per_task_end;
  if (p.blocked_ok) {  // blocked form: the token order, then its sort or the blocked workspace
    p.blk = plan_blocked(L, K, N);
    p.order_sort = plan_schedule(L, 1, N, B);
    p.off_order = base;
    p.off_blk = p.off_order + a256((size_t)L * 4);
    end = std::max(end, p.off_blk + std::max(p.blk.ws_bytes, p.order_sort.ws_bytes));
  }
  p.ws_bytes = end;
  return p;
}

hipError_t launch_expert_auto(const void* x, const void* W, const void* V, const int32_t* idx,
                              const float* gate, int L, int d, int64_t N, int K, int B,
                              omni_dtype dt, float* y, int32_t* chosen, const AutoPlan& p,
                              void* ws, hipStream_t s) {
  char* w = (char*)ws;
  const int M = L * K;
  int32_t* perm = (int32_t*)(w + p.off_perm);
  int32_t* goff = (int32_t*)(w + p.off_goff);
  float* act = (float*)(w + p.off_act);
  int32_t* start = (int32_t*)(w + p.off_start);
  hipError_t e;
  RunGate per_task{}, blocked{};
  int32_t* choice = nullptr;  // the run gate: [1] distinct experts, [2] sample size
  if (p.blocked_ok) {
    choice = (int32_t*)(w + p.off_flag);
    e = launch_auto_sample(idx, M, N, (uint32_t*)(w + p.off_bits), choice, s);
    if (e != hipSuccess) return e;
    per_task = RunGate{choice, 0};
    blocked = RunGate{choice, 1};
  }
  // the sort of the chosen form: the pages' schedule of the tasks for the
  // per-task passes, the token order for the blocked form (it also writes
  // `chosen`)
  const SortSpec tasks{idx, 1, M, B, p.sched, perm, w + p.off_act};
  const SortSpec tokens =
      p.blocked_ok ? token_order_spec(idx, L, K, N, B, (int32_t*)(w + p.off_order), w + p.off_blk)
                   : tasks;
  e = sort_dual(tasks, tokens, choice, chosen, s);
  if (e != hipSuccess) return e;
  // per-task passes: group offsets, then the two passes over the schedule
  e = launch_sched_offsets(p.sched, w + p.off_act, M, p.G, goff, s, per_task);
  if (e != hipSuccess) return e;
  e = launch_expert_act(x, W, idx, gate, perm, goff, L, d, K, B, p.G, dt, act, start, s,
                        per_task);
  if (e != hipSuccess) return e;
  e = launch_expert_out(V, idx, act, nullptr, L, d, K, dt, y, s, per_task);
  if (e != hipSuccess || !p.blocked_ok) return e;
  // blocked form: the dense products per block of the token order
  return launch_expert_blocked(x, W, V, idx, gate, (const int32_t*)(w + p.off_order), L, d, K,
                               y, p.blk, w + p.off_blk, s, blocked);
}

}  // namespace omni
