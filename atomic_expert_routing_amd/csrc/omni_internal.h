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

// ----------------------------------------------------------------- wave exchanges
// DPP (data-parallel primitives) move a value between lanes inside the VALU
// instead of through the LDS crossbar.  gfx9 encodings:
//   quad_perm [1,0,3,2] = 0xB1 (lane ^ 1), quad_perm [2,3,0,1] = 0x4E (lane ^ 2)
//   row_shl:n = 0x100+n (lane i reads i+n in its row of 16), row_shr:n = 0x110+n
//   row_ror:n = 0x120+n, row_mirror = 0x140, row_half_mirror = 0x141
//   row_bcast:15 = 0x142, row_bcast:31 = 0x143
template <int CTRL, int ROWS = 0xf, bool ZERO_OOB = false>
__device__ __forceinline__ int dpp(int v) {
  return __builtin_amdgcn_update_dpp(0, v, CTRL, ROWS, 0xf, ZERO_OOB);
}

// Value held by lane ^ J (J a power of two below 64).
template <int J>
__device__ __forceinline__ int xor_lane(int v) {
  if constexpr (J == 1) {
    return dpp<0xB1>(v);
  } else if constexpr (J == 2) {
    return dpp<0x4E>(v);
  } else if constexpr (J == 4 || J == 8) {
    const int from_below = dpp<0x110 + J>(v);  // lane i reads i - J
    const int from_above = dpp<0x100 + J>(v);  // lane i reads i + J
    return (threadIdx.x & J) ? from_below : from_above;
  } else if constexpr (J == 16) {
    return __builtin_amdgcn_ds_swizzle(v, 0x401F);  // bit mode: xor 16 within 32 lanes
  } else {
    return __shfl_xor(v, J, 64);
  }
}

__device__ __forceinline__ float fxor_lane1(float v) { return __int_as_float(dpp<0xB1>(__float_as_int(v))); }

// Reductions: xor 1 and xor 2 inside quads, then half-row and row mirrors
// leave every lane of a 16-lane row holding the row's result; the four rows
// are combined through scalar reads (so the result is wave-uniform).
#define OMNI_ROW_REDUCE(T, AS, FROM, OP)                        \
  v = OP(v, FROM(dpp<0xB1>(AS(v))));                            \
  v = OP(v, FROM(dpp<0x4E>(AS(v))));                            \
  v = OP(v, FROM(dpp<0x141>(AS(v))));                           \
  v = OP(v, FROM(dpp<0x140>(AS(v))));                           \
  const T r0 = FROM(__builtin_amdgcn_readlane(AS(v), 0));       \
  const T r1 = FROM(__builtin_amdgcn_readlane(AS(v), 16));      \
  const T r2 = FROM(__builtin_amdgcn_readlane(AS(v), 32));      \
  const T r3 = FROM(__builtin_amdgcn_readlane(AS(v), 48));      \
  return OP(OP(OP(r0, r1), r2), r3);

__device__ __forceinline__ float add_f(float a, float b) { return a + b; }
__device__ __forceinline__ int add_i(int a, int b) { return a + b; }
__device__ __forceinline__ int max_i(int a, int b) { return a > b ? a : b; }
__device__ __forceinline__ unsigned max_u(unsigned a, unsigned b) { return a > b ? a : b; }
__device__ __forceinline__ unsigned min_u(unsigned a, unsigned b) { return a < b ? a : b; }
__device__ __forceinline__ int f2i(float f) { return __float_as_int(f); }
__device__ __forceinline__ float i2f(int i) { return __int_as_float(i); }
__device__ __forceinline__ int u2i(unsigned u) { return (int)u; }
__device__ __forceinline__ unsigned i2u(int i) { return (unsigned)i; }
__device__ __forceinline__ int id_i(int i) { return i; }

__device__ __forceinline__ float wave_sum(float v) { OMNI_ROW_REDUCE(float, f2i, i2f, add_f) }
__device__ __forceinline__ float wave_max(float v) { OMNI_ROW_REDUCE(float, f2i, i2f, fmaxf) }
__device__ __forceinline__ int wave_max_i(int v) { OMNI_ROW_REDUCE(int, id_i, id_i, max_i) }
__device__ __forceinline__ int wave_sum_i(int v) { OMNI_ROW_REDUCE(int, id_i, id_i, add_i) }
__device__ __forceinline__ unsigned wave_umax(unsigned v) { OMNI_ROW_REDUCE(unsigned, u2i, i2u, max_u) }
__device__ __forceinline__ unsigned wave_umin(unsigned v) { OMNI_ROW_REDUCE(unsigned, u2i, i2u, min_u) }
#undef OMNI_ROW_REDUCE

// Orders one wave's LDS accesses where the wave works alone on its data
// (several waves with separate LDS slices share a workgroup), so no
// workgroup barrier is needed.
__device__ __forceinline__ void wave_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// Inclusive prefix sum over the 64 lanes: row_shr steps inside each row of
// 16 (lanes below the shift add 0), then row broadcasts of lane 15 into
// rows 1 and 3 and of lane 31 into rows 2 and 3.
__device__ __forceinline__ int wave_incl_scan(int v) {
  v += dpp<0x111, 0xf, true>(v);
  v += dpp<0x112, 0xf, true>(v);
  v += dpp<0x114, 0xf, true>(v);
  v += dpp<0x118, 0xf, true>(v);
  v += dpp<0x142, 0xa>(v);
  v += dpp<0x143, 0xc>(v);
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

// ----------------------------------------------------------------- run gates
// The expert assembly picks its form on the device from a sample of the
// routing: gate[1] distinct experts among gate[2] sampled tasks (both set by
// earlier kernels of the same call); the blocked form when each sampled
// expert is used AUTO_REUSE times or more on average.  Every kernel of either
// form reads the two words and computes the choice itself, so the host never
// waits for it and no launch is spent on deciding.
constexpr int AUTO_REUSE = 2;
__device__ __forceinline__ int auto_choice_of(int distinct, int sampled) {
  distinct = __builtin_amdgcn_readfirstlane(distinct);
  sampled = __builtin_amdgcn_readfirstlane(sampled);
  return (int64_t)sampled >= (int64_t)AUTO_REUSE * distinct ? 1 : 0;
}
__device__ __forceinline__ int auto_choice(const int32_t* gate) {
  return auto_choice_of(gate[1], gate[2]);
}
// A launch that may be skipped on the device: the kernel returns at once
// unless the choice read from `flag` equals want (flag == nullptr: always
// runs).
struct RunGate {
  const int32_t* flag = nullptr;
  int want = 0;
};
__device__ __forceinline__ bool gated_out(const int32_t* flag, int want) {
  return flag && auto_choice(flag) != want;
}

// ----------------------------------------------------------------- host launchers
// Each returns hipSuccess or the launch error; arguments are pre-validated.

// k-tile depth of the pipelined MFMA product: its Kd must be a multiple
constexpr int GEMM_KTILE = 64;

// C[M, N] (+)= A[M, Kd] . B[N, Kd]^T on MFMA (bf16 in, fp32 out); B rows
// n >= n_split come from B1 (row n - n_split), C rows m >= m_split go to C1.
// Kd must be a multiple of 64.
hipError_t launch_gemm_bt_bf16(const void* A, const void* B0, const void* B1, int n_split, int M,
                               int N, int Kd, float* C0, float* C1, int m_split, int ldc,
                               bool accumulate, hipStream_t s);

// out[M, F] (bf16) = SiLU(A Wg^T) * (A Wu^T), A [M, Kd], Wg and Wu [F, Kd] bf16;
// F % 16 == 0, Kd % GEMM_KTILE == 0
hipError_t launch_gemm_swiglu_bf16(const void* A, const void* Wg, const void* Wu, int M, int F,
                                   int Kd, uint16_t* out, hipStream_t s);

// fp32 VALU product C[m, n] (+)= sum_k A[m*sam + k*sak] * B[n*sbn + k*sbk]
hipError_t gemm_f32(const float* A, long sam, long sak, const float* B, long sbn, long sbk, int M,
                    int N, int Kd, float* C, int ldc, bool accumulate, hipStream_t s);

// y (+)= SiLU(x Wg^T) * (x Wu^T) Wd^T; ws per shared_mlp_ws_bytes
size_t shared_mlp_ws_bytes(int64_t L, int64_t F, omni_dtype dt);
hipError_t launch_shared_mlp(const void* x, const void* Wg, const void* Wu, const void* Wd, int L,
                             int d, int F, omni_dtype dt, float* y, bool accumulate, void* ws,
                             hipStream_t s);

// logits[L, Nr+Nc] (fp32) = x [L,d] . [Wr; Wc]^T
hipError_t launch_router_gemm(const void* x, const void* Wr, const void* Wc, int L, int d,
                              int Nr, int Nc, omni_dtype dt, float* logits, hipStream_t s);

// per token: LogSoftmax of both logit halves, implicit top-K, gate softmax
hipError_t launch_router_topk(const float* logits, int L, int Nr, int Nc, int K,
                              int32_t* idx, float* score, float* gate, hipStream_t s);
size_t router_topk_lds_bytes(int Nr, int Nc, int K);

struct SchedPlan {
  int M, G, rounds, ntiles, passes, digit_bits;  // a tile is rounds x 256 elements
  size_t ws_bytes;
  // workspace carve (byte offsets)
  size_t off_keys_a, off_vals_a, off_keys_b, off_vals_b, off_hist, off_totals;
};
SchedPlan plan_schedule(int64_t L, int64_t K, int64_t N, int64_t B);
// The sorted group ids left in the workspace by the last launch_schedule.
const int32_t* schedule_sorted_keys(const SchedPlan& plan, const void* ws);
// (with a gate: only when the device's choice equals run.want)
hipError_t launch_schedule(const int32_t* idx, int M, int B, int G, const SchedPlan& plan,
                           int32_t* perm, int32_t* group_off, void* ws, hipStream_t s,
                           RunGate run = {});
// One stable sort of the elements p < M by idx[p * stride] / B, planned by
// plan, indices in sorted order to vals_last, buffers in ws.
struct SortSpec {
  const int32_t* idx;
  int stride, M, B;
  SchedPlan plan;
  int32_t* vals_last;
  void* ws;
};
// Runs sort a, or with a gate the sort the device's choice selects (b for the
// blocked form), in one set of launches; both must have the same digit split
// (plan_schedule with the same N and B).  chosen (optional) receives the
// choice (0 without a gate).
hipError_t sort_dual(const SortSpec& a, const SortSpec& b, const int32_t* gate, int32_t* chosen,
                     hipStream_t s);
// One sort, run only when the device's choice equals run.want (always
// without a gate); chosen (optional) receives the choice.
hipError_t sort_gated(const SortSpec& a, RunGate run, int32_t* chosen, hipStream_t s);
// group_off from the sorted keys a sort with `plan` left in ws
hipError_t launch_sched_offsets(const SchedPlan& plan, const void* ws, int M, int G,
                                int32_t* group_off, hipStream_t s, RunGate run = {});
// order[0..M) = 0..M-1 stably sorted by keys[i] in [0, key_bound); workspace
// plan_schedule(M, 1, key_bound, 1).ws_bytes
hipError_t launch_sort_keys(const int32_t* keys, int M, int64_t key_bound, int32_t* order,
                            void* ws, hipStream_t s, RunGate run = {});
// order[0..L) = the tokens stably sorted by idx[t*K] / B (the group of each
// token's first expert); uses the schedule's workspace (plan_schedule(L, K, ..)
// covers it)
SortSpec token_order_spec(const int32_t* idx, int L, int K, int64_t N, int B, int32_t* order,
                          void* ws);
hipError_t launch_token_order(const int32_t* idx, int L, int K, int64_t N, int B,
                              int32_t* order, void* ws, hipStream_t s, RunGate run = {},
                              int32_t* chosen = nullptr);

// act[m] = gate[m] * SiLU(x[m/K] . W[idx[m]]) for m in schedule order, in
// chunks along the group boundaries of group_off (B experts per group, G
// groups); start [expert_act_chunks(L*K) + 1] int32 is workspace
int expert_act_chunks(int64_t M);
hipError_t launch_expert_act(const void* x, const void* W, const int32_t* idx, const float* gate,
                             const int32_t* perm, const int32_t* group_off, int L, int d, int K,
                             int B, int G, omni_dtype dt, float* act, int32_t* start,
                             hipStream_t s, RunGate run = {});
// token-centric baseline: y[t] = sum_k gate * SiLU(x_t . W[e]) * V[e], one token per workgroup
hipError_t launch_expert_tc(const void* x, const void* W, const void* V, const int32_t* idx,
                            const float* gate, int L, int d, int K, omni_dtype dt, float* y,
                            hipStream_t s);
// y[t] = sum_k act[t*K+k] * V[idx[t*K+k]]; tokens visited in `order` (a
// permutation of [0, L), XCD x taking its x-th eighth) or, if null, by id
hipError_t launch_expert_out(const void* V, const int32_t* idx, const float* act,
                             const int32_t* order, int L, int d, int K, omni_dtype dt, float* y,
                             hipStream_t s, RunGate run = {});

// ----------------------------------------------------------------- blocked assembly
constexpr int BLK_TOKENS = 64;       // tokens per block (consecutive entries of the order)
constexpr int BLK_UNION_TILE = 128;  // union columns per tile
constexpr int BLK_D_TILE = 256;      // y columns per output tile (d must be a multiple)
constexpr int BLK_BWD_MAX_L = 524288;  // tokens of the backward's LDS bitmap (128 KB)
struct BlockedPlan {
  int nb, ucap, sort_keys;  // blocks, union capacity per block, LDS sort size
  size_t off_U, off_nU, off_toff, off_G, off_Ahi, off_Alo, ws_bytes;
};
BlockedPlan plan_blocked(int64_t L, int64_t K, int64_t N);
// y[t] for every t of `order` (a permutation of [0, L)), by dense products over
// each block of 64 consecutive order entries and the union of their experts
hipError_t launch_expert_blocked(const void* x, const void* W, const void* V, const int32_t* idx,
                                 const float* gate, const int32_t* order, int L, int d, int K,
                                 float* y, const BlockedPlan& p, void* ws, hipStream_t s,
                                 RunGate run = {});

// The schedule and the per-task passes, or the token order and the blocked
// assembly, chosen on the device from a sample of the routing (see
// assembly.hip); ws per plan_expert_auto.
struct AutoPlan {
  BlockedPlan blk;
  SchedPlan sched, order_sort;
  bool blocked_ok;  // bf16, d a multiple of BLK_D_TILE, L small enough
  int G, sample;    // groups; tasks the choice samples
  size_t off_flag, off_bits, off_perm, off_goff, off_act, off_start, off_order, off_blk;
  size_t ws_bytes;
};
AutoPlan plan_expert_auto(int64_t L, int64_t d, int64_t N, int64_t K, int64_t B, omni_dtype dt);
// the device's choice of form: gate[1] = distinct experts among a fixed
// sample of the tasks (auto_sample_size(M) of them), gate[2] = the sample
// size; bits [ceil(N/32)] uint32 is workspace
int auto_sample_size(int64_t M);
hipError_t launch_auto_sample(const int32_t* idx, int M, int64_t N, uint32_t* bits, int32_t* gate,
                              hipStream_t s);
hipError_t launch_set_i32(int32_t* p, int v, hipStream_t s);
hipError_t launch_expert_auto(const void* x, const void* W, const void* V, const int32_t* idx,
                              const float* gate, int L, int d, int64_t N, int K, int B,
                              omni_dtype dt, float* y, int32_t* chosen, const AutoPlan& p,
                              void* ws, hipStream_t s);

// ----------------------------------------------------------------- measurement aid
// sink needs gather_probe_blocks(n) * 256 floats
int gather_probe_blocks(int64_t n);
hipError_t launch_gather_probe(const void* A, int64_t nA, const int32_t* rows, int64_t n,
                               int row_bytes, float* sink, hipStream_t s);

// ----------------------------------------------------------------- dense router
constexpr int DENSE_ROUTER_CHUNK = 65536;  // experts per logits chunk
struct DenseRouterPlan {
  int chunk, nchunks;
  size_t off_logits, off_state, off_part, ws_bytes;
};
DenseRouterPlan plan_dense_router(int64_t L, int64_t N, int64_t K);
hipError_t launch_dense_router(const void* x, const void* Wn, int L, int d, int N, int K,
                               omni_dtype dt, int32_t* idx, float* score, float* gate,
                               const DenseRouterPlan& p, void* ws, hipStream_t s);

// ----------------------------------------------------------------- backward
struct BwdPlan {
  int M, U_max, ntiles, Lq;
  SchedPlan sched, rsort;  // the sort of the tasks by expert; of the used experts for the rows
  size_t off_dh, off_ga, off_perm, off_eoff, off_seg, off_cnt, off_sched, ws_bytes;
  size_t off_rkey, off_rord, off_goff, off_rec;
};
BwdPlan plan_expert_backward(int64_t L, int64_t d, int64_t N, int64_t K);
// the tasks sorted by expert (the plan's perm), the used experts (uniq,
// n_uniq) and each one's first position in the sorted tasks (the plan's seg,
// seg[n_uniq] = L*K)
hipError_t launch_expert_segments(const int32_t* idx, int N, int32_t* uniq, int32_t* n_uniq,
                                  const BwdPlan& p, void* ws, hipStream_t s);
// the used experts' dW / dV rows from the per-task terms dh, ga and the
// sort by expert (launch_expert_segments) that the plan's workspace already
// holds (the last step of the backward)
hipError_t launch_expert_grad_rows(const void* x, const float* dy, int d, int K, omni_dtype dt,
                                   const int32_t* n_uniq, omni_dtype grad_dt, void* dW_rows,
                                   void* dV_rows, const BwdPlan& p, void* ws, hipStream_t s,
                                   RunGate run = {});
// the per-token pass of the per-task backward: dx, dgate and the per-task
// terms dh, ga (into the plan's workspace); reads n_uniq from the segments
hipError_t launch_expert_bwd_token(const void* x, const void* W, const void* V,
                                   const int32_t* idx, const float* gate, const float* dy, int L,
                                   int d, int K, omni_dtype dt, float* dx, float* dgate,
                                   const int32_t* n_uniq, const BwdPlan& p, void* ws,
                                   hipStream_t s, RunGate run = {});
// dx (expert part, overwritten), dgate, used experts and their dW / dV rows
hipError_t launch_expert_backward(const void* x, const void* W, const void* V, const int32_t* idx,
                                  const float* gate, const float* dy, int L, int d, int N, int K,
                                  omni_dtype dt, float* dx, float* dgate, int32_t* uniq,
                                  int32_t* n_uniq, omni_dtype grad_dt, void* dW_rows,
                                  void* dV_rows, const BwdPlan& p, void* ws, hipStream_t s);

// the blocked form of the backward: dgate, the per-task terms and dx by
// dense products over the forward's token blocks, then the rows as above
struct BlockedBwdPlan {
  BlockedPlan blk;
  BwdPlan bwd;
  SchedPlan ksort;  // the sort of the used experts by their first token position
  int ucap_e, smax;  // used-expert capacity, expert-set capacity
  size_t off_blk, off_kmap, off_dyh, off_dyl, off_bwd;
  size_t off_pos, off_key, off_eord, off_ksort, off_ns, off_stoff, off_T, off_dht, off_gat;
  size_t set_elems, ws_bytes;  // dense set-tile capacity (elements per matrix and term)
};
BlockedBwdPlan plan_expert_backward_blocked(int64_t L, int64_t d, int64_t N, int64_t K);
hipError_t launch_expert_backward_blocked(const void* x, const void* W, const void* V,
                                          const int32_t* idx, const float* gate, const float* dy,
                                          const int32_t* order, int L, int d, int N, int K,
                                          float* dx, float* dgate, int32_t* uniq, int32_t* n_uniq,
                                          omni_dtype grad_dt, void* dW_rows, void* dV_rows,
                                          const BlockedBwdPlan& p, void* ws, hipStream_t s,
                                          RunGate run = {}, bool segments_done = false);

// the backward in the form the device picks by the forward's rule: the
// per-task passes, or the blocked form over the token order (tokens sorted
// by their first expert); both share the sort of the tasks by expert
struct AutoBwdPlan {
  BlockedBwdPlan blk;  // with blocked_ok; its per-task plan blk.bwd serves both forms
  BwdPlan bwd;         // without: the per-task backward alone
  SchedPlan order_sort;
  bool blocked_ok;
  size_t off_flag, off_bits, off_order, off_osort, off_main, ws_bytes;
};
AutoBwdPlan plan_expert_backward_auto(int64_t L, int64_t d, int64_t N, int64_t K, omni_dtype dt);
hipError_t launch_expert_backward_auto(const void* x, const void* W, const void* V,
                                       const int32_t* idx, const float* gate, const float* dy,
                                       int L, int d, int N, int K, omni_dtype dt, float* dx,
                                       float* dgate, int32_t* uniq, int32_t* n_uniq,
                                       omni_dtype grad_dt, void* dW_rows, void* dV_rows,
                                       int32_t* chosen, const AutoBwdPlan& p, void* ws,
                                       hipStream_t s);

struct RouterBwdPlan {
  int Ntot_p, L_p;
  size_t off_ds_hi, off_ds_lo, off_dsT_hi, off_dsT_lo, off_xT, off_wT, off_ds, ws_bytes;
};
RouterBwdPlan plan_router_backward(int64_t L, int64_t d, int64_t Nr, int64_t Nc, omni_dtype dt);
// dx += router part; dWr, dWc overwritten
hipError_t launch_router_backward(const void* x, const void* Wr, const void* Wc,
                                  const int32_t* idx, const float* gate, const float* dgate,
                                  int L, int d, int Nr, int Nc, int K, omni_dtype dt, float* dx,
                                  float* dWr, float* dWc, const RouterBwdPlan& p, void* ws,
                                  hipStream_t s);

}  // namespace omni
