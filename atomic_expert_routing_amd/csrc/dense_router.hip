// Dense (fully connected) router on gfx950: the ablation that replaces the
// Cartesian Product Router (makerbund article, section 五: a conventional
// fully connected router over all N experts).
//
//   s = x Wn^T over all N experts (Wn [N, d]), p = LogSoftmax(s) over N,
//   top-K under (p desc, n asc), gate = softmax over the K selected scores.
//
// The experts are processed in chunks of DENSE_ROUTER_CHUNK.  For each chunk
// an MFMA (or, for fp32 inputs, VALU) product writes the chunk's logits
// [L, nc]; dense_chunk then updates, per token, a running top K (64-bit keys:
// the order-preserving image of the logit, then the complemented id, so ties
// go to the smaller id) and the chunk's (max, sum of exp(s - max)).  Only
// logits above the token's current K-th key can enter, so one pass per chunk
// usually suffices; when too many pass (the first chunk, or rising logits)
// the chunk's own exact top K comes from an MSD radix select.  dense_finish
// combines the partial sums into the LogSoftmax constant and writes ids,
// scores and gates sorted by (score desc, id asc).

#include "omni_internal.h"

namespace omni {
namespace {

constexpr int DR_THREADS = 256;
constexpr int DR_CAP = 2048;  // LDS buffer of boundary-bucket keys / survivors
static_assert(DR_CAP >= OMNI_MAX_K && (DR_CAP & (DR_CAP - 1)) == 0,
              "the merge pads DR_CAP + OMNI_MAX_K keys to at most 2 * DR_CAP");
constexpr int DR_BINS = 2048;

typedef unsigned long long u64;

// (value, id) -> 64-bit key: larger value first, then smaller id
__device__ __forceinline__ u64 dr_key(unsigned ord, unsigned id) {
  return ((u64)ord << 32) | (u64)(~id);
}

// Exclusive prefix over the block (thread order) and the block total.
__device__ int dr_block_excl(int v, int* red, int* total) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int inc = wave_incl_scan(v);
  __syncthreads();
  if (lane == 63) red[w] = inc;
  __syncthreads();
  int before = 0, all = 0;
#pragma unroll
  for (int i = 0; i < DR_THREADS / 64; ++i) {
    before += i < w ? red[i] : 0;
    all += red[i];
  }
  *total = all;
  return before + inc - v;
}

// Bitonic sort of n (a power of two) keys in LDS, descending.
__device__ void dr_sort_desc(u64* a, int n) {
  for (int k = 2; k <= n; k <<= 1)
    for (int j = k >> 1; j > 0; j >>= 1) {
      __syncthreads();
      for (int i = threadIdx.x; i < n; i += DR_THREADS) {
        const int p = i ^ j;
        if (p > i) {
          const u64 x = a[i], y = a[p];
          const bool desc = (i & k) == 0;
          if (desc ? x < y : x > y) {
            a[i] = y;
            a[p] = x;
          }
        }
      }
    }
  __syncthreads();
}

// Exact top-K keys of row[0..n) (ids id0 + i), by an MSD radix select over
// the 64-bit keys: level 0 is an 11-bit histogram of the key's top bits,
// further digits refine the boundary bucket while it holds more than DR_CAP
// keys, then one pass collects the keys above the bucket into sel and the
// bucket into buf, which is sorted exactly.  Leaves min(K, n) keys in sel
// (unsorted) and returns their number.  Whole-workgroup call.
__device__ int dr_radix_topk(const float* row, int n, int id0, int K, int* hist, u64* buf,
                             u64* sel, int* red, int* sh) {
  const int tid = threadIdx.x;
  auto key_of = [&](int i) -> u64 { return dr_key(float_ord(row[i]), (unsigned)(id0 + i)); };
  for (int b = tid; b < DR_BINS; b += DR_THREADS) hist[b] = 0;
  __syncthreads();
  for (int i = tid; i < n; i += DR_THREADS) atomicAdd(&hist[float_ord(row[i]) >> 21], 1);
  __syncthreads();
  u64 prefix = 0;  // key bits above `shift`
  int shift = 53, width = 11, above = 0, cnt_b = 0;
  bool all = false;  // fewer than K keys: take them all
  for (;;) {
    const int nb = 1 << width;
    const int per = (nb + DR_THREADS - 1) / DR_THREADS;
    int local = 0;
    for (int q = 0; q < per; ++q) {
      const int b = tid * per + q;
      local += b < nb ? hist[b] : 0;
    }
    int total;
    const int ex = dr_block_excl(local, red, &total);
    const int from_me = total - ex;  // keys in bins >= tid * per
    const int need = K - above;
    if (tid == 0) sh[0] = -1;
    __syncthreads();
    if (from_me >= need && from_me - local < need) {
      int run = from_me - local;
      for (int q = per - 1; q >= 0; --q) {
        const int b = tid * per + q;
        const int c = b < nb ? hist[b] : 0;
        if (run + c >= need) {
          sh[0] = b;
          sh[1] = run;
          break;
        }
        run += c;
      }
    }
    __syncthreads();
    if (sh[0] < 0) {
      all = true;
      break;
    }
    const int bucket = sh[0];
    above += sh[1];
    cnt_b = hist[bucket];
    prefix = (prefix << width) | (u64)bucket;
    if (cnt_b <= DR_CAP || shift == 0) break;
    const int nshift = shift >= 11 ? shift - 11 : 0;
    const int nwidth = shift - nshift;
    __syncthreads();  // every thread has read hist[bucket]
    for (int b = tid; b < DR_BINS; b += DR_THREADS) hist[b] = 0;
    __syncthreads();
    for (int i = tid; i < n; i += DR_THREADS) {
      const u64 k = key_of(i);
      if ((k >> shift) == prefix)
        atomicAdd(&hist[(int)((k >> nshift) & ((1ull << nwidth) - 1ull))], 1);
    }
    __syncthreads();
    shift = nshift;
    width = nwidth;
  }
  if (tid == 0) {
    sh[2] = 0;
    sh[3] = 0;
  }
  __syncthreads();
  for (int i = tid; i < n; i += DR_THREADS) {
    const u64 k = key_of(i);
    const u64 top = k >> shift;
    if (all || top > prefix) {
      sel[atomicAdd(&sh[2], 1)] = k;
    } else if (top == prefix) {
      buf[atomicAdd(&sh[3], 1)] = k;
    }
  }
  __syncthreads();
  const int nsel = sh[2];
  if (all) return nsel;
  int nb = 1;
  while (nb < cnt_b) nb <<= 1;
  for (int i = cnt_b + tid; i < nb; i += DR_THREADS) buf[i] = 0ull;
  dr_sort_desc(buf, nb);
  for (int i = tid; i < K - nsel; i += DR_THREADS) sel[nsel + i] = buf[i];
  __syncthreads();
  return K;
}

// One chunk of experts for every token (one workgroup per token).  state[t]
// holds the token's K best keys so far, sorted descending (slot 0: none).
// One pass over the chunk's logits (16-byte loads) accumulates the chunk's
// (max, sum exp(v - max)) into part[t * nparts + slot] and collects the keys
// above the token's current K-th key; if more than DR_CAP pass (always on
// the first chunk), the chunk's own top K is taken by dr_radix_topk instead.
// The survivors and the old state are merged, sorted, and the first K kept.
__global__ __launch_bounds__(DR_THREADS) void dense_chunk(const float* __restrict__ vals, int n,
                                                          int ld, int id0, int K, int slot,
                                                          int nparts, u64* __restrict__ state,
                                                          float2* __restrict__ part) {
  __shared__ int hist[DR_BINS];
  // survivors (<= DR_CAP) + the old state (<= OMNI_MAX_K), padded to a power
  // of two for the sort
  __shared__ u64 buf[2 * DR_CAP];
  __shared__ u64 sel[OMNI_MAX_K];
  __shared__ int red[DR_THREADS / 64];
  __shared__ float redf[2 * (DR_THREADS / 64)];
  __shared__ int sh[4];
  const int t = blockIdx.x, tid = threadIdx.x;
  const float* row = vals + (size_t)t * ld;
  u64* st = state + (size_t)t * K;
  const u64 T = slot == 0 ? 0ull : st[K - 1];  // keys must exceed the K-th best so far
  if (tid == 0) sh[2] = 0;
  __syncthreads();
  float m = -INFINITY, se = 0.f;
  auto visit = [&](float v, int i) {
    if (v > m) {
      se = se * expf(m - v) + 1.f;
      m = v;
    } else {
      se += expf(v - m);
    }
    const u64 k = dr_key(float_ord(v), (unsigned)(id0 + i));
    if (k > T) {
      const int p = atomicAdd(&sh[2], 1);
      if (p < DR_CAP) buf[p] = k;
    }
  };
  const bool vec = ((ld & 3) == 0) && ((((uintptr_t)vals) & 15) == 0);
  int i0 = 0;
  if (vec) {
    for (int i = 4 * tid; i + 3 < n; i += 4 * DR_THREADS) {
      const f32x4 f = *(const f32x4*)(row + i);
      visit(f[0], i);
      visit(f[1], i + 1);
      visit(f[2], i + 2);
      visit(f[3], i + 3);
    }
    i0 = n & ~3;
  }
  for (int i = i0 + tid; i < n; i += DR_THREADS) visit(row[i], i);
  {
    const float wm = wave_max(m);
    float sw = (m == -INFINITY) ? 0.f : se * expf(m - wm);
    sw = wave_sum(sw);
    const int w = tid >> 6;
    if ((tid & 63) == 0) {
      redf[2 * w] = wm;
      redf[2 * w + 1] = sw;
    }
  }
  __syncthreads();
  int nnew = sh[2];
  if (nnew > DR_CAP) {  // too many survivors: the chunk's exact top K
    nnew = dr_radix_topk(row, n, id0, K, hist, buf, sel, red, sh);
    for (int i = tid; i < nnew; i += DR_THREADS) buf[i] = sel[i];
    __syncthreads();
  }
  // merge with the previous state, keep the best K (sorted)
  const int nold = slot == 0 ? 0 : K;
  for (int i = tid; i < nold; i += DR_THREADS) buf[nnew + i] = st[i];
  const int tot = nnew + nold;
  int nb = 1;
  while (nb < tot) nb <<= 1;
  for (int i = tot + tid; i < nb; i += DR_THREADS) buf[i] = 0ull;
  dr_sort_desc(buf, nb);
  for (int i = tid; i < K; i += DR_THREADS) st[i] = i < tot ? buf[i] : 0ull;
  if (tid == 0) {
    float M = -INFINITY;
    for (int w = 0; w < DR_THREADS / 64; ++w) M = fmaxf(M, redf[2 * w]);
    float S = 0.f;
    for (int w = 0; w < DR_THREADS / 64; ++w)
      if (redf[2 * w] > -INFINITY) S += redf[2 * w + 1] * expf(redf[2 * w] - M);
    part[(size_t)t * nparts + slot] = make_float2(M, S);
  }
}

// lse from the chunk partials; ids, scores p = s - lse and gates (softmax
// over the K selected) from the final state (already sorted).
__global__ __launch_bounds__(DR_THREADS) void dense_finish(const u64* __restrict__ state,
                                                           const float2* __restrict__ part,
                                                           int nparts, int K,
                                                           int32_t* __restrict__ idx_out,
                                                           float* __restrict__ score_out,
                                                           float* __restrict__ gate_out) {
  __shared__ float redf[3];
  const int t = blockIdx.x, tid = threadIdx.x;
  const u64* st = state + (size_t)t * K;
  if (tid == 0) {
    float M = -INFINITY;
    for (int c = 0; c < nparts; ++c) M = fmaxf(M, part[(size_t)t * nparts + c].x);
    float S = 0.f;
    for (int c = 0; c < nparts; ++c) {
      const float2 pc = part[(size_t)t * nparts + c];
      if (pc.x > -INFINITY) S += pc.y * expf(pc.x - M);
    }
    const float top = ord_float((unsigned)(st[0] >> 32));
    float z = 0.f;
    for (int k = 0; k < K; ++k) z += expf(ord_float((unsigned)(st[k] >> 32)) - top);
    redf[0] = M + logf(S);
    redf[1] = z;
    redf[2] = top;
  }
  __syncthreads();
  const float lse = redf[0], z = redf[1], top = redf[2];
  for (int k = tid; k < K; k += DR_THREADS) {
    const u64 key = st[k];
    const float v = ord_float((unsigned)(key >> 32));
    idx_out[(size_t)t * K + k] = (int32_t)(~(unsigned)key);
    score_out[(size_t)t * K + k] = v - lse;
    gate_out[(size_t)t * K + k] = expf(v - top) / z;
  }
}

}  // namespace

DenseRouterPlan plan_dense_router(int64_t L, int64_t N, int64_t K) {
  DenseRouterPlan p{};
  p.chunk = (int)(N < DENSE_ROUTER_CHUNK ? N : DENSE_ROUTER_CHUNK);
  p.nchunks = (int)((N + p.chunk - 1) / p.chunk);
  size_t o = 0;
  auto take = [&](size_t bytes) {
    const size_t at = o;
    o += (bytes + 255) & ~(size_t)255;
    return at;
  };
  p.off_logits = take((size_t)L * p.chunk * 4);
  p.off_state = take((size_t)L * K * 8);
  p.off_part = take((size_t)L * p.nchunks * 8);
  p.ws_bytes = o;
  return p;
}

hipError_t launch_dense_router(const void* x, const void* Wn, int L, int d, int N, int K,
                               omni_dtype dt, int32_t* idx, float* score, float* gate,
                               const DenseRouterPlan& p, void* ws, hipStream_t s) {
  char* w = (char*)ws;
  float* logits = (float*)(w + p.off_logits);
  u64* state = (u64*)(w + p.off_state);
  float2* part = (float2*)(w + p.off_part);
  hipError_t e;
  for (int c = 0; c < p.nchunks; ++c) {
    const int c0 = c * p.chunk;
    const int nc = N - c0 < p.chunk ? N - c0 : p.chunk;
    if (dt == OMNI_BF16) {
      const uint16_t* Wc = (const uint16_t*)Wn + (size_t)c0 * d;
      if ((e = launch_gemm_bt_bf16(x, Wc, Wc, nc, L, nc, d, logits, logits, L, nc, false, s)))
        return e;
    } else {
      const float* Wc = (const float*)Wn + (size_t)c0 * d;
      if ((e = gemm_f32((const float*)x, d, 1, Wc, d, 1, L, nc, d, logits, nc, false, s))) return e;
    }
    hipLaunchKernelGGL(dense_chunk, dim3(L), dim3(DR_THREADS), 0, s, logits, nc, nc, c0, K, c,
                       p.nchunks, state, part);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  hipLaunchKernelGGL(dense_finish, dim3(L), dim3(DR_THREADS), 0, s, state, part, p.nchunks, K,
                     idx, score, gate);
  return hipGetLastError();
}

}  // namespace omni
