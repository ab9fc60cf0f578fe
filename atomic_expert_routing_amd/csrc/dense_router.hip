// Dense (fully connected) router on gfx950: the ablation that replaces the
// Cartesian Product Router (makerbund article, section 五: a conventional
// fully connected router over all N experts).
//
//   s = x Wn^T over all N experts (Wn [N, d]), p = LogSoftmax(s) over N,
//   top-K under (p desc, n asc), gate = softmax over the K selected scores.
//
// The experts are processed in chunks of DENSE_ROUTER_CHUNK.  For each chunk an MFMA
// (or, for fp32 inputs, VALU) product writes the chunk's logits [L, nc];
// dense_select then picks, per token, the chunk's K largest logits (ties to
// the smaller expert id) and the chunk's (max, sum of exp(s - max)).  Every
// global top-K element is in its chunk's top K, so a final dense_select over
// the L x (chunks x K) candidates gives the global top K; it also combines
// the partial sums into the LogSoftmax constant and writes ids, scores and
// gates sorted by (score desc, id asc).
//
// dense_select is an MSD radix select over 64-bit keys (the order-preserving
// image of the value, then the complemented id): an 11-bit histogram pass
// (with the online max / sum of exp in chunk mode), refined by further
// digits only while the boundary bucket is larger than the LDS buffer; then
// one pass collects everything above the boundary bucket and the bucket
// itself, which is sorted exactly in LDS.

#include "omni_internal.h"

namespace omni {
namespace {

constexpr int DR_THREADS = 256;
constexpr int DR_CAP = 2048;  // LDS buffer of boundary-bucket keys
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

// CHUNK: vals = this chunk's logits (ids id0 + i); writes K candidate
// (value, id) pairs (unsorted; padded with -inf when n < K) and the chunk's
// (max, sum exp(v - max)) to part[t * nparts + slot].
// FINAL: vals/ids = the token's candidates from every chunk; combines the
// nparts partials into lse and writes idx, score = v - lse and gate =
// softmax over the selected, sorted by (score desc, id asc).
// Selection runs on the 64-bit keys (value order, then smaller id), which are
// distinct, so refining the boundary bucket always ends with at most DR_CAP
// keys in it.
template <bool FINAL>
__global__ __launch_bounds__(DR_THREADS) void dense_select(
    const float* __restrict__ vals, const int32_t* __restrict__ ids, int n, int ld, int id0,
    int K, int nparts, int slot, float* __restrict__ cand_v, int32_t* __restrict__ cand_i,
    int cand_ld, float2* __restrict__ part, int32_t* __restrict__ idx_out,
    float* __restrict__ score_out, float* __restrict__ gate_out) {
  __shared__ int hist[DR_BINS];
  __shared__ u64 buf[DR_CAP];
  __shared__ u64 sel[OMNI_MAX_K];
  __shared__ int red[DR_THREADS / 64];
  __shared__ float redf[2 * (DR_THREADS / 64)];
  __shared__ int s_nsel, s_nbuf, s_bucket, s_above;
  const int t = blockIdx.x, tid = threadIdx.x;
  const float* row = vals + (size_t)t * ld;
  const int32_t* irow = FINAL ? ids + (size_t)t * ld : nullptr;
  auto key_of = [&](int i) -> u64 {
    const unsigned id = FINAL ? (unsigned)irow[i] : (unsigned)(id0 + i);
    return dr_key(float_ord(row[i]), id);
  };

  // ---- level 0: 11-bit histogram of key bits 63..53 (+ online max and sum
  //      of exp in chunk mode)
  for (int b = tid; b < DR_BINS; b += DR_THREADS) hist[b] = 0;
  __syncthreads();
  float m = -INFINITY, se = 0.f;
  for (int i = tid; i < n; i += DR_THREADS) {
    const float v = row[i];
    atomicAdd(&hist[float_ord(v) >> 21], 1);
    if constexpr (!FINAL) {
      if (v > m) {
        se = se * expf(m - v) + 1.f;
        m = v;
      } else {
        se += expf(v - m);
      }
    }
  }
  if constexpr (!FINAL) {
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

  // ---- boundary bucket: count(keys in higher buckets) < K - above <= count(>= it);
  //      refine with the next digit while the bucket overflows the buffer
  u64 prefix = 0;  // key bits above `shift`
  int shift = 53, width = 11, above = 0, cnt_b = 0;
  bool all = false;  // fewer than K keys in total: take them all
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
    if (tid == 0) s_bucket = -1;
    __syncthreads();
    if (from_me >= need && from_me - local < need) {
      int run = from_me - local;
      for (int q = per - 1; q >= 0; --q) {
        const int b = tid * per + q;
        const int c = b < nb ? hist[b] : 0;
        if (run + c >= need) {
          s_bucket = b;
          s_above = run;
          break;
        }
        run += c;
      }
    }
    __syncthreads();
    if (s_bucket < 0) {
      all = true;
      break;
    }
    const int bucket = s_bucket;
    above += s_above;
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
      if ((k >> shift) == prefix) atomicAdd(&hist[(int)((k >> nshift) & ((1ull << nwidth) - 1ull))], 1);
    }
    __syncthreads();
    shift = nshift;
    width = nwidth;
  }

  // ---- collect: keys above the boundary bucket into sel, the bucket into buf
  if (tid == 0) {
    s_nsel = 0;
    s_nbuf = 0;
  }
  __syncthreads();
  for (int i = tid; i < n; i += DR_THREADS) {
    const u64 k = key_of(i);
    const u64 top = k >> shift;
    if (all || top > prefix) {
      sel[atomicAdd(&s_nsel, 1)] = k;
    } else if (top == prefix) {
      buf[atomicAdd(&s_nbuf, 1)] = k;
    }
  }
  __syncthreads();
  int nsel = s_nsel;
  if (!all) {
    const int need = K - nsel;
    int nb = 1;
    while (nb < cnt_b) nb <<= 1;
    for (int i = cnt_b + tid; i < nb; i += DR_THREADS) buf[i] = 0ull;
    dr_sort_desc(buf, nb);
    for (int i = tid; i < need; i += DR_THREADS) sel[nsel + i] = buf[i];
    nsel = K;
  }
  __syncthreads();

  if constexpr (!FINAL) {
    for (int i = tid; i < K; i += DR_THREADS) {
      const u64 k = i < nsel ? sel[i] : 0ull;
      cand_v[(size_t)t * cand_ld + i] = i < nsel ? ord_float((unsigned)(k >> 32)) : -INFINITY;
      cand_i[(size_t)t * cand_ld + i] = i < nsel ? (int32_t)(~(unsigned)k) : 0;
    }
    if (tid == 0) {
      float M = -INFINITY;
      for (int w = 0; w < DR_THREADS / 64; ++w) M = fmaxf(M, redf[2 * w]);
      float S = 0.f;
      for (int w = 0; w < DR_THREADS / 64; ++w)
        if (redf[2 * w] > -INFINITY) S += redf[2 * w + 1] * expf(redf[2 * w] - M);
      part[(size_t)t * nparts + slot] = make_float2(M, S);
    }
  } else {
    int nk = 1;
    while (nk < K) nk <<= 1;
    for (int i = tid; i < nk; i += DR_THREADS) buf[i] = i < K ? sel[i] : 0ull;
    dr_sort_desc(buf, nk);
    if (tid == 0) {
      float M = -INFINITY;
      for (int c = 0; c < nparts; ++c) M = fmaxf(M, part[(size_t)t * nparts + c].x);
      float S = 0.f;
      for (int c = 0; c < nparts; ++c) {
        const float2 pc = part[(size_t)t * nparts + c];
        if (pc.x > -INFINITY) S += pc.y * expf(pc.x - M);
      }
      const float top = ord_float((unsigned)(buf[0] >> 32));
      float z = 0.f;
      for (int k = 0; k < K; ++k) z += expf(ord_float((unsigned)(buf[k] >> 32)) - top);
      redf[0] = M + logf(S);
      redf[1] = z;
      redf[2] = top;
    }
    __syncthreads();
    const float lse = redf[0], z = redf[1], top = redf[2];
    for (int k = tid; k < K; k += DR_THREADS) {
      const u64 key = buf[k];
      const float v = ord_float((unsigned)(key >> 32));
      idx_out[(size_t)t * K + k] = (int32_t)(~(unsigned)key);
      score_out[(size_t)t * K + k] = v - lse;
      gate_out[(size_t)t * K + k] = expf(v - top) / z;
    }
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
  p.off_cand_v = take((size_t)L * p.nchunks * K * 4);
  p.off_cand_i = take((size_t)L * p.nchunks * K * 4);
  p.off_part = take((size_t)L * p.nchunks * 8);
  p.ws_bytes = o;
  return p;
}

hipError_t launch_dense_router(const void* x, const void* Wn, int L, int d, int N, int K,
                               omni_dtype dt, int32_t* idx, float* score, float* gate,
                               const DenseRouterPlan& p, void* ws, hipStream_t s) {
  char* w = (char*)ws;
  float* logits = (float*)(w + p.off_logits);
  float* cand_v = (float*)(w + p.off_cand_v);
  int32_t* cand_i = (int32_t*)(w + p.off_cand_i);
  float2* part = (float2*)(w + p.off_part);
  const int cand_ld = p.nchunks * K;
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
    // chunk c's candidates go to columns [c*K, c*K + K) of the candidate rows;
    // its partial sums to part[t * nchunks + c]
    hipLaunchKernelGGL(dense_select<false>, dim3(L), dim3(DR_THREADS), 0, s, logits,
                       (const int32_t*)nullptr, nc, nc, c0, K, p.nchunks, c,
                       cand_v + (size_t)c * K, cand_i + (size_t)c * K, cand_ld, part,
                       (int32_t*)nullptr, (float*)nullptr, (float*)nullptr);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  hipLaunchKernelGGL(dense_select<true>, dim3(L), dim3(DR_THREADS), 0, s, cand_v, cand_i, cand_ld,
                     cand_ld, 0, K, p.nchunks, 0, (float*)nullptr, (int32_t*)nullptr, 0, part,
                     idx, score, gate);
  return hipGetLastError();
}

}  // namespace omni
