// C ABI of libomni.so: host-side validation, workspace carving and launches.
// Every check runs before the first launch, so a rejected call enqueues
// nothing and leaves every output untouched.

#include <cstdarg>
#include <cstdio>
#include <mutex>

#include "omni_internal.h"

namespace {

thread_local char g_err[512] = "";

omni_status fail(omni_status s, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof g_err, fmt, ap);
  va_end(ap);
  return s;
}

omni_status ok() {
  g_err[0] = '\0';
  return OMNI_OK;
}

omni_status hip_status(hipError_t e, const char* what) {
  if (e == hipSuccess) return ok();
  return fail(OMNI_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

constexpr int64_t I32_LIMIT = 2147483647;

size_t align256(size_t n) { return (n + 255) & ~(size_t)255; }

// Group size as the kernels take it: every B >= N puts all N experts in
// group 0, exactly as B = N does, so B is clamped to N (which fits an int).
int group_size(int64_t B, int64_t N) { return (int)(B < N ? B : N); }

omni_status check_dtype_d(omni_dtype dt, int64_t d) {
  if (dt != OMNI_F32 && dt != OMNI_BF16) return fail(OMNI_ERR_INVALID_ARG, "unknown dtype %d", (int)dt);
  if (d <= 0) return fail(OMNI_ERR_INVALID_ARG, "d must be positive (got %lld)", (long long)d);
  if (d % 8) return fail(OMNI_ERR_UNSUPPORTED, "d must be a multiple of 8 (got %lld)", (long long)d);
  const int64_t dmax = dt == OMNI_BF16 ? OMNI_MAX_D_BF16 : OMNI_MAX_D_F32;
  if (d > dmax) return fail(OMNI_ERR_UNSUPPORTED, "d = %lld exceeds %lld", (long long)d, (long long)dmax);
  return OMNI_OK;
}

omni_status check_tasks(int64_t L, int64_t K) {
  if (L <= 0 || K <= 0)
    return fail(OMNI_ERR_INVALID_ARG, "L and K must be positive (L=%lld K=%lld)", (long long)L, (long long)K);
  if (L > I32_LIMIT / K)
    return fail(OMNI_ERR_UNSUPPORTED, "L*K = %lld tasks exceeds 2^31-1", (long long)(L * K));
  return OMNI_OK;
}

omni_status router_ws(int64_t L, int64_t d, int64_t Nr, int64_t Nc, int64_t K, omni_dtype dt, size_t* out) {
  omni_status s;
  if ((s = check_dtype_d(dt, d)) != OMNI_OK) return s;
  if ((s = check_tasks(L, K)) != OMNI_OK) return s;
  if (Nr <= 0 || Nc <= 0)
    return fail(OMNI_ERR_INVALID_ARG, "N_r and N_c must be positive (%lld, %lld)", (long long)Nr, (long long)Nc);
  if (Nr > OMNI_MAX_GRID_SIDE || Nc > OMNI_MAX_GRID_SIDE)
    return fail(OMNI_ERR_UNSUPPORTED, "grid side above %d (N_r=%lld N_c=%lld)", OMNI_MAX_GRID_SIDE,
                (long long)Nr, (long long)Nc);
  if (K > Nr * Nc)
    return fail(OMNI_ERR_INVALID_ARG, "K = %lld exceeds N_r*N_c = %lld", (long long)K, (long long)(Nr * Nc));
  if (K > OMNI_MAX_K) return fail(OMNI_ERR_UNSUPPORTED, "K = %lld exceeds %d", (long long)K, OMNI_MAX_K);
  if (L > I32_LIMIT / (Nr + Nc)) return fail(OMNI_ERR_UNSUPPORTED, "L*(N_r+N_c) exceeds 2^31-1");
  *out = align256((size_t)L * (size_t)(Nr + Nc) * 4);
  return OMNI_OK;
}

omni_status schedule_ws(int64_t L, int64_t K, int64_t N, int64_t B, size_t* out) {
  omni_status s;
  if ((s = check_tasks(L, K)) != OMNI_OK) return s;
  if (N <= 0 || B <= 0)
    return fail(OMNI_ERR_INVALID_ARG, "N and B must be positive (N=%lld B=%lld)", (long long)N, (long long)B);
  if (N > I32_LIMIT) return fail(OMNI_ERR_UNSUPPORTED, "N = %lld exceeds 2^31-1", (long long)N);
  if (B > I32_LIMIT)
    return fail(OMNI_ERR_UNSUPPORTED, "B = %lld exceeds 2^31-1 (any B >= N gives one group)",
                (long long)B);
  *out = omni::plan_schedule(L, K, N, group_size(B, N)).ws_bytes;
  return OMNI_OK;
}

omni_status expert_ws(int64_t L, int64_t d, int64_t N, int64_t K, omni_dtype dt, size_t* out) {
  omni_status s;
  if ((s = check_dtype_d(dt, d)) != OMNI_OK) return s;
  if ((s = check_tasks(L, K)) != OMNI_OK) return s;
  if (K > OMNI_MAX_K) return fail(OMNI_ERR_UNSUPPORTED, "K = %lld exceeds %d", (long long)K, OMNI_MAX_K);
  if (N <= 0) return fail(OMNI_ERR_INVALID_ARG, "N must be positive (got %lld)", (long long)N);
  if (N > I32_LIMIT) return fail(OMNI_ERR_UNSUPPORTED, "N = %lld exceeds 2^31-1", (long long)N);
  *out = align256((size_t)L * (size_t)K * 4);
  return OMNI_OK;
}

// omni_expert_forward: the activations [L*K] fp32, then the activation
// pass's chunk starts [ceil(L*K / chunk) + 1] int32
omni_status expert_fwd_ws(int64_t L, int64_t d, int64_t N, int64_t K, int64_t B, omni_dtype dt,
                          size_t* out) {
  omni_status s;
  if ((s = expert_ws(L, d, N, K, dt, out)) != OMNI_OK) return s;
  if (B <= 0) return fail(OMNI_ERR_INVALID_ARG, "B must be positive (got %lld)", (long long)B);
  if (B > I32_LIMIT)
    return fail(OMNI_ERR_UNSUPPORTED, "B = %lld exceeds 2^31-1 (any B >= N gives one group)",
                (long long)B);
  *out = align256((size_t)L * (size_t)K * 4) +
         align256(((size_t)omni::expert_act_chunks(L * K) + 1) * 4);
  return OMNI_OK;
}

omni_status expert_auto_ws(int64_t L, int64_t d, int64_t N, int64_t K, int64_t B, omni_dtype dt,
                           size_t* out) {
  omni_status s;
  if ((s = expert_fwd_ws(L, d, N, K, B, dt, out)) != OMNI_OK) return s;
  if ((s = schedule_ws(L, K, N, B, out)) != OMNI_OK) return s;
  *out = omni::plan_expert_auto(L, d, N, K, group_size(B, N), dt).ws_bytes;
  return OMNI_OK;
}

omni_status expert_bwd_ws(int64_t L, int64_t d, int64_t N, int64_t K, omni_dtype dt, size_t* out) {
  omni_status s;
  if ((s = expert_ws(L, d, N, K, dt, out)) != OMNI_OK) return s;
  if (L > I32_LIMIT - 8)  // the row pass keys tokens by 8 * ceil(L / 8) + 1 values
    return fail(OMNI_ERR_UNSUPPORTED, "L = %lld exceeds 2^31-9", (long long)L);
  *out = omni::plan_expert_backward(L, d, N, K).ws_bytes;
  return OMNI_OK;
}

omni_status auto_bwd_ws(int64_t L, int64_t d, int64_t N, int64_t K, omni_dtype dt, size_t* out) {
  omni_status s;
  if ((s = expert_bwd_ws(L, d, N, K, dt, out)) != OMNI_OK) return s;
  *out = omni::plan_expert_backward_auto(L, d, N, K, dt).ws_bytes;
  return OMNI_OK;
}

omni_status router_bwd_ws(int64_t L, int64_t d, int64_t Nr, int64_t Nc, int64_t K, omni_dtype dt,
                          size_t* out) {
  omni_status s;
  if ((s = router_ws(L, d, Nr, Nc, K, dt, out)) != OMNI_OK) return s;
  *out = omni::plan_router_backward(L, d, Nr, Nc, dt).ws_bytes;
  return OMNI_OK;
}

omni_status mlp_ws(int64_t L, int64_t d, int64_t F, omni_dtype dt, size_t* out) {
  omni_status s;
  if ((s = check_dtype_d(dt, d)) != OMNI_OK) return s;
  if (L <= 0 || F <= 0)
    return fail(OMNI_ERR_INVALID_ARG, "L and d_ff must be positive (L=%lld d_ff=%lld)", (long long)L,
                (long long)F);
  if (L > I32_LIMIT / F || L > I32_LIMIT / d)
    return fail(OMNI_ERR_UNSUPPORTED, "L*d_ff or L*d exceeds 2^31-1");
  if (dt == OMNI_BF16 && (d % omni::GEMM_KTILE || F % omni::GEMM_KTILE))
    return fail(OMNI_ERR_UNSUPPORTED, "bf16 shared MLP needs d and d_ff multiples of %d (d=%lld d_ff=%lld)",
                omni::GEMM_KTILE, (long long)d, (long long)F);
  *out = omni::shared_mlp_ws_bytes(L, F, dt);
  return OMNI_OK;
}

omni_status dense_router_ws(int64_t L, int64_t d, int64_t N, int64_t K, omni_dtype dt, size_t* out) {
  omni_status s;
  if ((s = check_dtype_d(dt, d)) != OMNI_OK) return s;
  if ((s = check_tasks(L, K)) != OMNI_OK) return s;
  if (N <= 0) return fail(OMNI_ERR_INVALID_ARG, "N must be positive (got %lld)", (long long)N);
  if (N > I32_LIMIT) return fail(OMNI_ERR_UNSUPPORTED, "N = %lld exceeds 2^31-1", (long long)N);
  if (K > N) return fail(OMNI_ERR_INVALID_ARG, "K = %lld exceeds N = %lld", (long long)K, (long long)N);
  if (K > OMNI_MAX_K) return fail(OMNI_ERR_UNSUPPORTED, "K = %lld exceeds %d", (long long)K, OMNI_MAX_K);
  if (dt == OMNI_BF16 && d % omni::GEMM_KTILE)
    return fail(OMNI_ERR_UNSUPPORTED, "bf16 dense router needs d %% %d == 0 (d=%lld)", omni::GEMM_KTILE,
                (long long)d);
  const omni::DenseRouterPlan p = omni::plan_dense_router(L, N, K);
  if ((int64_t)p.nchunks * K > I32_LIMIT / L)
    return fail(OMNI_ERR_UNSUPPORTED, "L * candidates exceeds 2^31-1");
  *out = p.ws_bytes;
  return OMNI_OK;
}

omni_status blocked_ws(int64_t L, int64_t d, int64_t N, int64_t K, omni_dtype dt, size_t* out) {
  omni_status s;
  if ((s = expert_ws(L, d, N, K, dt, out)) != OMNI_OK) return s;
  if (dt != OMNI_BF16)
    return fail(OMNI_ERR_UNSUPPORTED, "the blocked assembly takes bf16 inputs only (MFMA products)");
  if (d % omni::BLK_D_TILE)
    return fail(OMNI_ERR_UNSUPPORTED, "the blocked assembly needs d %% %d == 0 (d=%lld)",
                omni::BLK_D_TILE, (long long)d);
  if (L > I32_LIMIT - omni::BLK_TOKENS)
    return fail(OMNI_ERR_UNSUPPORTED, "L = %lld too large for the blocked assembly", (long long)L);
  *out = omni::plan_blocked(L, K, N).ws_bytes;
  return OMNI_OK;
}

omni_status blocked_bwd_ws(int64_t L, int64_t d, int64_t N, int64_t K, omni_dtype dt, size_t* out) {
  omni_status s;
  if ((s = blocked_ws(L, d, N, K, dt, out)) != OMNI_OK) return s;
  if (L > omni::BLK_BWD_MAX_L)
    return fail(OMNI_ERR_UNSUPPORTED, "the blocked backward takes L <= %d (L=%lld)",
                omni::BLK_BWD_MAX_L, (long long)L);
  *out = omni::plan_expert_backward_blocked(L, d, N, K).ws_bytes;
  return OMNI_OK;
}

omni_status check_ws(const void* ws, size_t have, size_t need) {
  if (have < need)
    return fail(OMNI_ERR_WORKSPACE, "workspace of %zu bytes, %zu needed", have, need);
  if (need && !ws) return fail(OMNI_ERR_INVALID_ARG, "workspace pointer is NULL");
  if ((uintptr_t)ws % 256) return fail(OMNI_ERR_INVALID_ARG, "workspace is not 256-byte aligned");
  return OMNI_OK;
}

bool aligned16(const void* p) { return ((uintptr_t)p & 15) == 0; }

// omni_schedule's checks apart from the workspace; *need = its workspace size
omni_status schedule_args(const int32_t* idx, int64_t L, int64_t K, int64_t N, int64_t B,
                          const int32_t* perm, const int32_t* group_off,
                          const int32_t* token_order, size_t* need) {
  omni_status s = schedule_ws(L, K, N, B, need);
  if (s != OMNI_OK) return s;
  if (!idx) return fail(OMNI_ERR_INVALID_ARG, "omni_schedule: NULL idx");
  if (!perm != !group_off)
    return fail(OMNI_ERR_INVALID_ARG, "omni_schedule: perm and group_off go together");
  if (!perm && !token_order) return fail(OMNI_ERR_INVALID_ARG, "omni_schedule: no output");
  if (token_order && L > I32_LIMIT - 7)
    return fail(OMNI_ERR_UNSUPPORTED, "token order needs L <= 2^31-8 (L=%lld)", (long long)L);
  return OMNI_OK;
}

// The schedule's launches on validated arguments; ws holds the sort buffers.
omni_status schedule_launch(const int32_t* idx, int64_t L, int64_t K, int64_t N, int64_t B,
                            int32_t* perm, int32_t* group_off, int32_t* token_order, void* ws,
                            hipStream_t st) {
  hipError_t e = hipSuccess;
  const int Bi = group_size(B, N);
  if (perm) {
    const omni::SchedPlan plan = omni::plan_schedule(L, K, N, Bi);
    e = omni::launch_schedule(idx, plan.M, Bi, plan.G, plan, perm, group_off, ws, st);
    if (e != hipSuccess) return hip_status(e, "schedule launch");
  }
  if (!token_order) return ok();
  e = omni::launch_token_order(idx, (int)L, (int)K, N, Bi, token_order, ws, st);
  return hip_status(e, "token order launch");
}

// ----------------------------------------------------------------- allocation-free schedule
// omni_schedule_noalloc keeps the sort buffers in this fixed device array
// instead of a caller workspace.  The code object gives every GPU it is
// loaded on its own copy, held until the process ends.  In host code the
// name `scratch` is only a host-side stand-in: the device address of a GPU's
// copy comes from hipGetSymbolAddress (looked up once per device, with that
// device current) and only that address is handed to kernels.
static __device__ __align__(256) unsigned char scratch[OMNI_SCHEDULE_NOALLOC_MAX_WS];

constexpr int MAX_DEVICES = 64;
std::mutex g_scratch_mu;
void* g_scratch_addr[MAX_DEVICES] = {};

// Device address of `scratch` on the device that runs `st`.
omni_status scratch_address(hipStream_t st, void** out) {
  int dev = -1, cur = -1;
  hipError_t e = hipGetDevice(&cur);
  if (e != hipSuccess) return hip_status(e, "omni_schedule_noalloc: hipGetDevice");
  dev = cur;
  if (st) {
    e = hipStreamGetDevice(st, &dev);
    if (e != hipSuccess) return hip_status(e, "omni_schedule_noalloc: hipStreamGetDevice");
  }
  if (dev < 0 || dev >= MAX_DEVICES)
    return fail(OMNI_ERR_UNSUPPORTED, "omni_schedule_noalloc: device %d beyond %d", dev, MAX_DEVICES);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_addr[dev]) {
    if (dev != cur && (e = hipSetDevice(dev)) != hipSuccess)
      return hip_status(e, "omni_schedule_noalloc: hipSetDevice");
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (dev != cur) {
      const hipError_t r = hipSetDevice(cur);
      if (e == hipSuccess) e = r;
    }
    if (e != hipSuccess) return hip_status(e, "omni_schedule_noalloc: hipGetSymbolAddress");
    if (!p || (uintptr_t)p % 256)
      return fail(OMNI_ERR_HIP, "omni_schedule_noalloc: scratch address %p unusable", p);
    g_scratch_addr[dev] = p;
  }
  *out = g_scratch_addr[dev];
  return OMNI_OK;
}

}  // namespace

extern "C" {

omni_status omni_router(const void* x, const void* Wr, const void* Wc, int64_t L, int64_t d,
                        int64_t Nr, int64_t Nc, int64_t K, omni_dtype dt, int32_t* idx,
                        float* score, float* gate, void* ws, size_t ws_bytes, void* stream) {
  size_t need = 0;
  omni_status s = router_ws(L, d, Nr, Nc, K, dt, &need);
  if (s != OMNI_OK) return s;
  if (!x || !Wr || !Wc || !idx || !score || !gate)
    return fail(OMNI_ERR_INVALID_ARG, "omni_router: NULL array pointer");
  if (!aligned16(x) || !aligned16(Wr) || !aligned16(Wc))
    return fail(OMNI_ERR_INVALID_ARG, "omni_router: x, Wr and Wc must be 16-byte aligned");
  if ((s = check_ws(ws, ws_bytes, need)) != OMNI_OK) return s;
  hipStream_t st = (hipStream_t)stream;
  float* logits = (float*)ws;
  hipError_t e = omni::launch_router_gemm(x, Wr, Wc, (int)L, (int)d, (int)Nr, (int)Nc, dt, logits, st);
  if (e != hipSuccess) return hip_status(e, "router projection launch");
  e = omni::launch_router_topk(logits, (int)L, (int)Nr, (int)Nc, (int)K, idx, score, gate, st);
  return hip_status(e, "router top-K launch");
}

omni_status omni_schedule(const int32_t* idx, int64_t L, int64_t K, int64_t N, int64_t B,
                          int32_t* perm, int32_t* group_off, int32_t* token_order, void* ws,
                          size_t ws_bytes, void* stream) {
  size_t need = 0;
  omni_status s = schedule_args(idx, L, K, N, B, perm, group_off, token_order, &need);
  if (s != OMNI_OK) return s;
  if ((s = check_ws(ws, ws_bytes, need)) != OMNI_OK) return s;
  return schedule_launch(idx, L, K, N, B, perm, group_off, token_order, ws, (hipStream_t)stream);
}

omni_status omni_schedule_noalloc(const int32_t* idx, int64_t L, int64_t K, int64_t N, int64_t B,
                                  int32_t* perm, int32_t* group_off, int32_t* token_order,
                                  void* stream) {
  size_t need = 0;
  omni_status s = schedule_args(idx, L, K, N, B, perm, group_off, token_order, &need);
  if (s != OMNI_OK) return s;
  if (need > (size_t)OMNI_SCHEDULE_NOALLOC_MAX_WS)
    return fail(OMNI_ERR_UNSUPPORTED,
                "omni_schedule_noalloc: these sizes need %zu bytes of scratch, above the fixed "
                "%zu (use omni_schedule with a workspace)",
                need, (size_t)OMNI_SCHEDULE_NOALLOC_MAX_WS);
  hipStream_t st = (hipStream_t)stream;
  void* ws = nullptr;
  if ((s = scratch_address(st, &ws)) != OMNI_OK) return s;
  return schedule_launch(idx, L, K, N, B, perm, group_off, token_order, ws, st);
}

omni_status omni_expert_forward(const void* x, const void* W, const void* V, const int32_t* idx,
                                const float* gate, const int32_t* perm, const int32_t* group_off,
                                const int32_t* token_order, int64_t L, int64_t d, int64_t N,
                                int64_t K, int64_t B, omni_dtype dt, float* y, void* ws,
                                size_t ws_bytes, void* stream) {
  size_t need = 0;
  omni_status s = expert_fwd_ws(L, d, N, K, B, dt, &need);
  if (s != OMNI_OK) return s;
  if (!x || !W || !V || !idx || !gate || !perm || !group_off || !y)
    return fail(OMNI_ERR_INVALID_ARG, "omni_expert_forward: NULL array pointer");
  if (token_order && L > I32_LIMIT - 7)
    return fail(OMNI_ERR_UNSUPPORTED, "token order needs L <= 2^31-8 (L=%lld)", (long long)L);
  if (!aligned16(x) || !aligned16(W) || !aligned16(V) || !aligned16(y))
    return fail(OMNI_ERR_INVALID_ARG, "omni_expert_forward: x, W, V and y must be 16-byte aligned");
  if ((s = check_ws(ws, ws_bytes, need)) != OMNI_OK) return s;
  hipStream_t st = (hipStream_t)stream;
  const int Bi = group_size(B, N);
  const int G = (int)((N + Bi - 1) / Bi);
  float* act = (float*)ws;
  int32_t* start = (int32_t*)((char*)ws + align256((size_t)L * (size_t)K * 4));
  hipError_t e = omni::launch_expert_act(x, W, idx, gate, perm, group_off, (int)L, (int)d, (int)K,
                                         Bi, G, dt, act, start, st);
  if (e != hipSuccess) return hip_status(e, "expert activation launch");
  e = omni::launch_expert_out(V, idx, act, token_order, (int)L, (int)d, (int)K, dt, y, st);
  return hip_status(e, "expert output launch");
}

omni_status omni_expert_forward_auto(const void* x, const void* W, const void* V,
                                     const int32_t* idx, const float* gate, int64_t L, int64_t d,
                                     int64_t N, int64_t K, int64_t B, omni_dtype dt, float* y,
                                     int32_t* chosen, void* ws, size_t ws_bytes, void* stream) {
  size_t need = 0;
  omni_status s = expert_auto_ws(L, d, N, K, B, dt, &need);
  if (s != OMNI_OK) return s;
  if (!x || !W || !V || !idx || !gate || !y)
    return fail(OMNI_ERR_INVALID_ARG, "omni_expert_forward_auto: NULL array pointer");
  if (!aligned16(x) || !aligned16(W) || !aligned16(V) || !aligned16(y))
    return fail(OMNI_ERR_INVALID_ARG,
                "omni_expert_forward_auto: x, W, V and y must be 16-byte aligned");
  if ((s = check_ws(ws, ws_bytes, need)) != OMNI_OK) return s;
  const int Bi = group_size(B, N);
  const omni::AutoPlan plan = omni::plan_expert_auto(L, d, N, K, Bi, dt);
  hipError_t e = omni::launch_expert_auto(x, W, V, idx, gate, (int)L, (int)d, N, (int)K, Bi, dt,
                                          y, chosen, plan, ws, (hipStream_t)stream);
  return hip_status(e, "automatic assembly launch");
}

omni_status omni_expert_forward_blocked(const void* x, const void* W, const void* V,
                                        const int32_t* idx, const float* gate,
                                        const int32_t* token_order, int64_t L, int64_t d,
                                        int64_t N, int64_t K, omni_dtype dt, float* y, void* ws,
                                        size_t ws_bytes, void* stream) {
  size_t need = 0;
  omni_status s = blocked_ws(L, d, N, K, dt, &need);
  if (s != OMNI_OK) return s;
  if (!x || !W || !V || !idx || !gate || !token_order || !y)
    return fail(OMNI_ERR_INVALID_ARG, "omni_expert_forward_blocked: NULL array pointer");
  if (!aligned16(x) || !aligned16(W) || !aligned16(V) || !aligned16(y))
    return fail(OMNI_ERR_INVALID_ARG,
                "omni_expert_forward_blocked: x, W, V and y must be 16-byte aligned");
  if ((s = check_ws(ws, ws_bytes, need)) != OMNI_OK) return s;
  const omni::BlockedPlan plan = omni::plan_blocked(L, K, N);
  hipError_t e = omni::launch_expert_blocked(x, W, V, idx, gate, token_order, (int)L, (int)d,
                                             (int)K, y, plan, ws, (hipStream_t)stream);
  return hip_status(e, "blocked assembly launch");
}

omni_status omni_expert_forward_token_centric(const void* x, const void* W, const void* V,
                                              const int32_t* idx, const float* gate, int64_t L,
                                              int64_t d, int64_t N, int64_t K, omni_dtype dt,
                                              float* y, void* stream) {
  size_t need = 0;
  omni_status s = expert_ws(L, d, N, K, dt, &need);  // same size rules; no workspace used
  if (s != OMNI_OK) return s;
  if (!x || !W || !V || !idx || !gate || !y)
    return fail(OMNI_ERR_INVALID_ARG, "omni_expert_forward_token_centric: NULL array pointer");
  if (!aligned16(x) || !aligned16(W) || !aligned16(V) || !aligned16(y))
    return fail(OMNI_ERR_INVALID_ARG,
                "omni_expert_forward_token_centric: x, W, V and y must be 16-byte aligned");
  hipError_t e = omni::launch_expert_tc(x, W, V, idx, gate, (int)L, (int)d, (int)K, dt, y,
                                        (hipStream_t)stream);
  return hip_status(e, "token-centric expert launch");
}

omni_status omni_expert_backward(const void* x, const void* W, const void* V, const int32_t* idx,
                                 const float* gate, const float* dy, int64_t L, int64_t d,
                                 int64_t N, int64_t K, omni_dtype dt, float* dx, float* dgate,
                                 int32_t* uniq, int32_t* n_uniq, omni_dtype grad_dt,
                                 void* dW_rows, void* dV_rows, void* ws, size_t ws_bytes,
                                 void* stream) {
  size_t need = 0;
  omni_status s = expert_bwd_ws(L, d, N, K, dt, &need);
  if (s != OMNI_OK) return s;
  if (!x || !W || !V || !idx || !gate || !dy || !dx || !dgate || !uniq || !n_uniq || !dW_rows ||
      !dV_rows)
    return fail(OMNI_ERR_INVALID_ARG, "omni_expert_backward: NULL array pointer");
  if (!aligned16(x) || !aligned16(W) || !aligned16(V) || !aligned16(dy) || !aligned16(dx) ||
      !aligned16(dW_rows) || !aligned16(dV_rows))
    return fail(OMNI_ERR_INVALID_ARG,
                "omni_expert_backward: x, W, V, dy, dx, dW_rows and dV_rows must be 16-byte aligned");
  if (grad_dt != OMNI_F32 && grad_dt != OMNI_BF16)
    return fail(OMNI_ERR_INVALID_ARG, "omni_expert_backward: unknown grad_dt %d", (int)grad_dt);
  if ((s = check_ws(ws, ws_bytes, need)) != OMNI_OK) return s;
  const omni::BwdPlan plan = omni::plan_expert_backward(L, d, N, K);
  hipError_t e = omni::launch_expert_backward(x, W, V, idx, gate, dy, (int)L, (int)d, (int)N,
                                              (int)K, dt, dx, dgate, uniq, n_uniq, grad_dt,
                                              dW_rows, dV_rows, plan, ws, (hipStream_t)stream);
  return hip_status(e, "expert backward launch");
}

omni_status omni_expert_backward_blocked(const void* x, const void* W, const void* V,
                                         const int32_t* idx, const float* gate, const float* dy,
                                         const int32_t* token_order, int64_t L, int64_t d,
                                         int64_t N, int64_t K, omni_dtype dt, float* dx,
                                         float* dgate, int32_t* uniq, int32_t* n_uniq,
                                         omni_dtype grad_dt, void* dW_rows, void* dV_rows,
                                         void* ws, size_t ws_bytes, void* stream) {
  size_t need = 0;
  omni_status s = blocked_bwd_ws(L, d, N, K, dt, &need);
  if (s != OMNI_OK) return s;
  if (!x || !W || !V || !idx || !gate || !dy || !token_order || !dx || !dgate || !uniq ||
      !n_uniq || !dW_rows || !dV_rows)
    return fail(OMNI_ERR_INVALID_ARG, "omni_expert_backward_blocked: NULL array pointer");
  if (!aligned16(x) || !aligned16(W) || !aligned16(V) || !aligned16(dy) || !aligned16(dx) ||
      !aligned16(dW_rows) || !aligned16(dV_rows))
    return fail(OMNI_ERR_INVALID_ARG,
                "omni_expert_backward_blocked: x, W, V, dy, dx, dW_rows and dV_rows must be "
                "16-byte aligned");
  if (grad_dt != OMNI_F32 && grad_dt != OMNI_BF16)
    return fail(OMNI_ERR_INVALID_ARG, "omni_expert_backward_blocked: unknown grad_dt %d",
                (int)grad_dt);
  if ((s = check_ws(ws, ws_bytes, need)) != OMNI_OK) return s;
  const omni::BlockedBwdPlan plan = omni::plan_expert_backward_blocked(L, d, N, K);
  hipError_t e = omni::launch_expert_backward_blocked(
      x, W, V, idx, gate, dy, token_order, (int)L, (int)d, (int)N, (int)K, dx, dgate, uniq, n_uniq,
      grad_dt, dW_rows, dV_rows, plan, ws, (hipStream_t)stream);
  return hip_status(e, "blocked expert backward launch");
}

omni_status omni_expert_backward_auto(const void* x, const void* W, const void* V,
                                      const int32_t* idx, const float* gate, const float* dy,
                                      int64_t L, int64_t d, int64_t N, int64_t K, omni_dtype dt,
                                      float* dx, float* dgate, int32_t* uniq, int32_t* n_uniq,
                                      omni_dtype grad_dt, void* dW_rows, void* dV_rows,
                                      int32_t* chosen, void* ws, size_t ws_bytes, void* stream) {
  size_t need = 0;
  omni_status s = auto_bwd_ws(L, d, N, K, dt, &need);
  if (s != OMNI_OK) return s;
  if (!x || !W || !V || !idx || !gate || !dy || !dx || !dgate || !uniq || !n_uniq || !dW_rows ||
      !dV_rows)
    return fail(OMNI_ERR_INVALID_ARG, "omni_expert_backward_auto: NULL array pointer");
  if (!aligned16(x) || !aligned16(W) || !aligned16(V) || !aligned16(dy) || !aligned16(dx) ||
      !aligned16(dW_rows) || !aligned16(dV_rows))
    return fail(OMNI_ERR_INVALID_ARG,
                "omni_expert_backward_auto: x, W, V, dy, dx, dW_rows and dV_rows must be 16-byte "
                "aligned");
  if (grad_dt != OMNI_F32 && grad_dt != OMNI_BF16)
    return fail(OMNI_ERR_INVALID_ARG, "omni_expert_backward_auto: unknown grad_dt %d",
                (int)grad_dt);
  if ((s = check_ws(ws, ws_bytes, need)) != OMNI_OK) return s;
  const omni::AutoBwdPlan plan = omni::plan_expert_backward_auto(L, d, N, K, dt);
  hipError_t e = omni::launch_expert_backward_auto(
      x, W, V, idx, gate, dy, (int)L, (int)d, (int)N, (int)K, dt, dx, dgate, uniq, n_uniq,
      grad_dt, dW_rows, dV_rows, chosen, plan, ws, (hipStream_t)stream);
  return hip_status(e, "automatic expert backward launch");
}

omni_status omni_router_backward(const void* x, const void* Wr, const void* Wc,
                                 const int32_t* idx, const float* gate, const float* dgate,
                                 int64_t L, int64_t d, int64_t Nr, int64_t Nc, int64_t K,
                                 omni_dtype dt, float* dx, float* dWr, float* dWc, void* ws,
                                 size_t ws_bytes, void* stream) {
  size_t need = 0;
  omni_status s = router_bwd_ws(L, d, Nr, Nc, K, dt, &need);
  if (s != OMNI_OK) return s;
  if (!x || !Wr || !Wc || !idx || !gate || !dgate || !dx || !dWr || !dWc)
    return fail(OMNI_ERR_INVALID_ARG, "omni_router_backward: NULL array pointer");
  if (!aligned16(x) || !aligned16(Wr) || !aligned16(Wc) || !aligned16(dx))
    return fail(OMNI_ERR_INVALID_ARG, "omni_router_backward: x, Wr, Wc and dx must be 16-byte aligned");
  if ((s = check_ws(ws, ws_bytes, need)) != OMNI_OK) return s;
  const omni::RouterBwdPlan plan = omni::plan_router_backward(L, d, Nr, Nc, dt);
  hipError_t e = omni::launch_router_backward(x, Wr, Wc, idx, gate, dgate, (int)L, (int)d, (int)Nr,
                                              (int)Nc, (int)K, dt, dx, dWr, dWc, plan, ws,
                                              (hipStream_t)stream);
  return hip_status(e, "router backward launch");
}

omni_status omni_shared_mlp(const void* x, const void* Wg, const void* Wu, const void* Wd, int64_t L,
                            int64_t d, int64_t d_ff, omni_dtype dt, float* y, int accumulate,
                            void* ws, size_t ws_bytes, void* stream) {
  size_t need = 0;
  omni_status s = mlp_ws(L, d, d_ff, dt, &need);
  if (s != OMNI_OK) return s;
  if (!x || !Wg || !Wu || !Wd || !y) return fail(OMNI_ERR_INVALID_ARG, "omni_shared_mlp: NULL array pointer");
  if (!aligned16(x) || !aligned16(Wg) || !aligned16(Wu) || !aligned16(Wd) || !aligned16(y))
    return fail(OMNI_ERR_INVALID_ARG, "omni_shared_mlp: x, Wg, Wu, Wd and y must be 16-byte aligned");
  if ((s = check_ws(ws, ws_bytes, need)) != OMNI_OK) return s;
  hipError_t e = omni::launch_shared_mlp(x, Wg, Wu, Wd, (int)L, (int)d, (int)d_ff, dt, y,
                                         accumulate != 0, ws, (hipStream_t)stream);
  return hip_status(e, "shared MLP launch");
}

omni_status omni_dense_router(const void* x, const void* Wn, int64_t L, int64_t d, int64_t N,
                              int64_t K, omni_dtype dt, int32_t* idx, float* score, float* gate,
                              void* ws, size_t ws_bytes, void* stream) {
  size_t need = 0;
  omni_status s = dense_router_ws(L, d, N, K, dt, &need);
  if (s != OMNI_OK) return s;
  if (!x || !Wn || !idx || !score || !gate)
    return fail(OMNI_ERR_INVALID_ARG, "omni_dense_router: NULL array pointer");
  if (!aligned16(x) || !aligned16(Wn))
    return fail(OMNI_ERR_INVALID_ARG, "omni_dense_router: x and Wn must be 16-byte aligned");
  if ((s = check_ws(ws, ws_bytes, need)) != OMNI_OK) return s;
  const omni::DenseRouterPlan plan = omni::plan_dense_router(L, N, K);
  hipError_t e = omni::launch_dense_router(x, Wn, (int)L, (int)d, (int)N, (int)K, dt, idx, score,
                                           gate, plan, ws, (hipStream_t)stream);
  return hip_status(e, "dense router launch");
}

omni_status omni_gather_probe(const void* A, int64_t n_rows_A, int64_t row_bytes,
                              const int32_t* rows, int64_t n, float* sink, size_t sink_floats,
                              void* stream) {
  if (!A || !rows || !sink) return fail(OMNI_ERR_INVALID_ARG, "omni_gather_probe: NULL pointer");
  if (!aligned16(A)) return fail(OMNI_ERR_INVALID_ARG, "omni_gather_probe: A must be 16-byte aligned");
  if (n <= 0 || n_rows_A <= 0)
    return fail(OMNI_ERR_INVALID_ARG, "omni_gather_probe: n and n_rows_A must be positive");
  if (row_bytes < 16 || row_bytes > 65536 || row_bytes % 16)
    return fail(OMNI_ERR_UNSUPPORTED, "omni_gather_probe: row_bytes %lld not a multiple of 16 "
                "in [16, 65536]", (long long)row_bytes);
  const size_t need = (size_t)omni::gather_probe_blocks(n) * 256;
  if (sink_floats < need)
    return fail(OMNI_ERR_WORKSPACE, "omni_gather_probe: sink of %zu floats, %zu needed",
                sink_floats, need);
  hipError_t e = omni::launch_gather_probe(A, n_rows_A, rows, n, (int)row_bytes, sink,
                                           (hipStream_t)stream);
  return hip_status(e, "gather probe launch");
}

omni_status omni_workspace_bytes(omni_op op, int64_t L, int64_t d, int64_t Nr, int64_t Nc,
                                 int64_t K, int64_t N, int64_t B, omni_dtype dt, size_t* out) {
  if (!out) return fail(OMNI_ERR_INVALID_ARG, "omni_workspace_bytes: out is NULL");
  size_t need = 0;
  omni_status s;
  switch (op) {
    case OMNI_OP_ROUTER: s = router_ws(L, d, Nr, Nc, K, dt, &need); break;
    case OMNI_OP_SCHEDULE: s = schedule_ws(L, K, N, B, &need); break;
    case OMNI_OP_EXPERT_FORWARD: s = expert_fwd_ws(L, d, N, K, B, dt, &need); break;
    case OMNI_OP_EXPERT_BACKWARD: s = expert_bwd_ws(L, d, N, K, dt, &need); break;
    case OMNI_OP_ROUTER_BACKWARD: s = router_bwd_ws(L, d, Nr, Nc, K, dt, &need); break;
    case OMNI_OP_SHARED_MLP: s = mlp_ws(L, d, N, dt, &need); break;
    case OMNI_OP_DENSE_ROUTER: s = dense_router_ws(L, d, N, K, dt, &need); break;
    case OMNI_OP_EXPERT_FORWARD_BLOCKED: s = blocked_ws(L, d, N, K, dt, &need); break;
    case OMNI_OP_EXPERT_BACKWARD_BLOCKED: s = blocked_bwd_ws(L, d, N, K, dt, &need); break;
    case OMNI_OP_EXPERT_FORWARD_AUTO: s = expert_auto_ws(L, d, N, K, B, dt, &need); break;
    case OMNI_OP_EXPERT_BACKWARD_AUTO: s = auto_bwd_ws(L, d, N, K, dt, &need); break;
    default: return fail(OMNI_ERR_INVALID_ARG, "unknown op %d", (int)op);
  }
  if (s != OMNI_OK) return s;
  *out = need;
  return ok();
}

const char* omni_status_string(omni_status s) {
  switch (s) {
    case OMNI_OK: return "ok";
    case OMNI_ERR_INVALID_ARG: return "invalid argument";
    case OMNI_ERR_UNSUPPORTED: return "unsupported size or dtype";
    case OMNI_ERR_WORKSPACE: return "workspace too small";
    case OMNI_ERR_HIP: return "HIP runtime error";
  }
  return "unknown status";
}

const char* omni_last_error(void) { return g_err; }

int omni_abi_version(void) { return OMNI_ABI_VERSION; }

}  // extern "C"
