// Backward pass of the routed branch on gfx950.
//
// The forward (OmniMoE digest, paper.rainbus.top, method paragraph, steps 1-3)
// computes per token y_t = sum_k g_k SiLU(x_t . W[e_k]) V[e_k] with
// g = softmax(S), S_k = p_r[i_k] + p_c[j_k], p = LogSoftmax(x W_r^T | x W_c^T).
// For an upstream gradient dy this file computes, per task (t, k, e):
//   h = x_t . W[e], a = SiLU(h), u = V[e] . dy_t
//   dgate = a u,  dh = g u SiLU'(h),  ga = g a
//   dx_t += dh W[e],  dW[e] += dh x_t,  dV[e] += ga dy_t
// and for the router dS = g (dgate - sum_k g_k dgate_k), scattered into the
// raw row / column logit gradients ds, then dW_r|c = ds^T x, dx += ds W_r|c.
// The LogSoftmax Jacobian adds -softmax(s) * sum(dp) to ds, and sum(dp) over
// a token's row logits equals sum_k dS_k, which is exactly zero (the softmax
// Jacobian's rows sum to zero); that term is therefore not formed.
//
// Kernels (the same expert-centric organisation as the forward), in launch
// order:
//   seg_count/scan/write  the tasks sorted by expert id (the schedule with
//                      groups of one expert) are cut into per-expert
//                      segments: list of used experts and segment starts.
//   expert_bwd_token   one workgroup per token (the grid strides over the
//                      tokens beyond 8192): its K (W, V) rows give h and u;
//                      dgate, dh, ga per task and the token-owned dx_t.
//   row_keys, a radix sort, row_recs
//                      the used experts ordered for the row pass: by the
//                      XCD class t % 8 of their first task's token t, then
//                      by t, dealt out so that workgroup b (on XCD b % 8)
//                      mostly takes an expert of class b % 8.
//   expert_bwd_rows    one workgroup per used expert (the grid strides over
//                      them beyond 32768): dW and dV rows summed
//                      over the expert's tasks in (token, k) order, written
//                      once, no atomics (each row has one owner).
//   router_bwd_ds      one workgroup per token: dS and the token's ds row
//                      (row logits then column logits), each entry summed in
//                      k order.
//   transpose_bf16 + the MFMA product of the forward router (bf16 ds split
//                      into a high and a low bf16 part, fp32 accumulation),
//                      or gemm_f32_strided for fp32 inputs.

#include <algorithm>

#include "omni_internal.h"

namespace omni {
namespace {

__device__ __forceinline__ int uni(int v) { return __builtin_amdgcn_readfirstlane(v); }
__device__ __forceinline__ float uni(float v) {
  return __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(v)));
}

// Round-to-nearest-even fp32 -> bf16 bits (finite inputs).
__device__ __forceinline__ unsigned bf16_rne(float f) {
  const unsigned u = __float_as_uint(f);
  return (u + 0x7fffu + ((u >> 16) & 1u)) >> 16;
}

// A 16-byte chunk of an input row holds E elements (8 bf16 or 4 fp32); the
// matching fp32 chunk of dy is E floats.
template <bool BF16>
struct Chunk {
  static constexpr int E = BF16 ? 8 : 4;
  __device__ static void widen(const u32x4 v, float* f) {
    if constexpr (BF16) {
      widen8(v, f);
    } else {
      f[0] = __uint_as_float(v.x); f[1] = __uint_as_float(v.y);
      f[2] = __uint_as_float(v.z); f[3] = __uint_as_float(v.w);
    }
  }
};

__device__ __forceinline__ float silu_grad(float h, float sg) { return sg * (1.f + h * (1.f - sg)); }

// ------------------------------------------------------------------ expert_bwd_token
// 256 threads per token.  Lane l of every wave holds chunks l + 64j of x_t
// and dy_t; wave w takes tasks k = w, w+4, ..., two (W, V) row pairs in
// flight.  dx_t is summed per wave in registers, then over the 4 waves in
// LDS in wave order.
constexpr int BWD_WAVES = 4;
// Grid bounds of the per-task kernels, which stride over their tokens or
// used experts: the workgroups of the form not chosen by the automatic
// backward only read the choice and leave, and their dispatch costs time in
// proportion to their number.
constexpr int BWD_TOKEN_GRID = 8192;
constexpr int BWD_ROWS_GRID = 32768;  // a multiple of 8

template <bool BF16, int NCH>
__global__ __launch_bounds__(256) void expert_bwd_token(
    const uint16_t* __restrict__ x_, const uint16_t* __restrict__ W_, const uint16_t* __restrict__ V_,
    const int32_t* __restrict__ idx, const float* __restrict__ gate, const float* __restrict__ dy,
    const int32_t* __restrict__ n_uniq, int L, int d, int K, float* __restrict__ dx,
    float* __restrict__ dgate, float* __restrict__ dh_out, float* __restrict__ ga_out,
    const int32_t* run_flag, int run_want) {
  if (gated_out(run_flag, run_want)) return;
  using C = Chunk<BF16>;
  constexpr int E = C::E;
  extern __shared__ __attribute__((aligned(16))) float red[];  // [BWD_WAVES][d]
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = uni(tid >> 6);
  const unsigned row_bytes = (unsigned)d * (BF16 ? 2u : 4u);
  const int nchunk = (int)(row_bytes / 16);

  // workgroup b takes tokens b, b + grid, ... (one each up to the grid bound)
  for (int t = blockIdx.x; t < L; t += gridDim.x) {
    float xr[NCH][E], dyr[NCH][E], acc[NCH][E];
#pragma unroll
    for (int j = 0; j < NCH; ++j) {
      const int c = lane + 64 * j;
      const bool in = c < nchunk;
      u32x4 v = in ? *(const u32x4*)((const char*)x_ + (size_t)t * row_bytes + c * 16u)
                   : u32x4{0u, 0u, 0u, 0u};
      C::widen(v, xr[j]);
      const float* dyp = dy + (size_t)t * d + c * E;
#pragma unroll
      for (int q = 0; q < E; q += 4) {
        const f32x4 f = in ? *(const f32x4*)(dyp + q) : f32x4{0.f, 0.f, 0.f, 0.f};
        dyr[j][q] = f[0]; dyr[j][q + 1] = f[1]; dyr[j][q + 2] = f[2]; dyr[j][q + 3] = f[3];
      }
#pragma unroll
      for (int q = 0; q < E; ++q) acc[j][q] = 0.f;
    }

    // Rows used by fewer than two tasks on average (used experts, counted by
    // the sort that ran before this kernel, above half the task count) are
    // loaded non-temporally: 4096 tokens x 1.7M experts (1.17 tasks per used
    // expert) 2.46 -> 2.38 ms for the whole call.  With reuse the plain loads
    // let repeated rows hit the caches (16384 clustered tokens, 167 tasks per
    // expert: 11.6 ms plain against 13.5 ms non-temporal).
    const bool stream_rows = 2ll * n_uniq[0] > (long long)L * K;
    auto load_rows = [&](int k, u32x4* w, u32x4* v) {
      const bool live = k < K;
      const int e = live ? uni(idx[(size_t)t * K + k]) : 0;
      const char* wb = (const char*)W_ + (size_t)e * row_bytes;
      const char* vb = (const char*)V_ + (size_t)e * row_bytes;
      if (stream_rows) {
#pragma unroll
        for (int j = 0; j < NCH; ++j) {
          const int c = lane + 64 * j;
          const bool in = live && c < nchunk;
          w[j] = in ? __builtin_nontemporal_load((const u32x4*)(wb + c * 16u)) : u32x4{0u, 0u, 0u, 0u};
          v[j] = in ? __builtin_nontemporal_load((const u32x4*)(vb + c * 16u)) : u32x4{0u, 0u, 0u, 0u};
        }
      } else {
#pragma unroll
        for (int j = 0; j < NCH; ++j) {
          const int c = lane + 64 * j;
          const bool in = live && c < nchunk;
          w[j] = in ? *(const u32x4*)(wb + c * 16u) : u32x4{0u, 0u, 0u, 0u};
          v[j] = in ? *(const u32x4*)(vb + c * 16u) : u32x4{0u, 0u, 0u, 0u};
        }
      }
    };
    auto task = [&](int k, const u32x4* w, const u32x4* v) {
      float wf[NCH][E];
      float ph = 0.f, pu = 0.f;
#pragma unroll
      for (int j = 0; j < NCH; ++j) {
        float vf[E];
        C::widen(w[j], wf[j]);
        C::widen(v[j], vf);
#pragma unroll
        for (int q = 0; q < E; ++q) {
          ph = fmaf(xr[j][q], wf[j][q], ph);
          pu = fmaf(dyr[j][q], vf[q], pu);
        }
      }
      const float h = wave_sum(ph), u = wave_sum(pu);
      const size_t m = (size_t)t * K + k;
      const float g = uni(gate[m]);
      const float sg = 1.f / (1.f + expf(-h));
      const float a = h * sg;
      const float dh = g * u * silu_grad(h, sg);
#pragma unroll
      for (int j = 0; j < NCH; ++j)
#pragma unroll
        for (int q = 0; q < E; ++q) acc[j][q] = fmaf(dh, wf[j][q], acc[j][q]);
      if (lane == 0) {
        dgate[m] = a * u;
        dh_out[m] = dh;
        ga_out[m] = g * a;
      }
    };
    u32x4 wa[NCH], va[NCH], wb[NCH], vb[NCH];
    load_rows(wave, wa, va);
    for (int k = wave; k < K; k += 2 * BWD_WAVES) {
      load_rows(k + BWD_WAVES, wb, vb);
      task(k, wa, va);
      if (k + BWD_WAVES < K) {
        load_rows(k + 2 * BWD_WAVES, wa, va);
        task(k + BWD_WAVES, wb, vb);
      }
    }
    // dx_t: per-wave partial sums meet in LDS, added in wave order
#pragma unroll
    for (int j = 0; j < NCH; ++j) {
      const int c = lane + 64 * j;
      if (c < nchunk)
#pragma unroll
        for (int q = 0; q < E; ++q) red[wave * d + c * E + q] = acc[j][q];
    }
    __syncthreads();
    for (int col = tid * 4; col < d; col += 256 * 4) {
      f32x4 s = *(const f32x4*)(red + col);
#pragma unroll
      for (int w = 1; w < BWD_WAVES; ++w) {
        const f32x4 o = *(const f32x4*)(red + w * d + col);
        s[0] += o[0]; s[1] += o[1]; s[2] += o[2]; s[3] += o[3];
      }
      *(f32x4*)(dx + (size_t)t * d + col) = s;
    }
    __syncthreads();  // red is written again for the next token
  }
}

// ------------------------------------------------------------------ per-expert segments
// keys[p] (ascending expert ids of the sorted tasks) -> uniq[r] = r-th distinct
// expert, seg_start[r] = its first position, seg_start[U] = M, n_uniq = U.
constexpr int SEG_THREADS = 256, SEG_PER = 16, SEG_TILE = SEG_THREADS * SEG_PER;

__device__ __forceinline__ bool seg_head(const int32_t* keys, int p, int M) {
  return p < M && (p == 0 || keys[p] != keys[p - 1]);
}

// Exclusive scan of v over the 256 threads of a workgroup; *total = sum.
__device__ int block_excl_scan(int v, int* total) {
  __shared__ int wsum[SEG_THREADS / 64];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int inc = wave_incl_scan(v);
  if (lane == 63) wsum[wave] = inc;
  __syncthreads();
  int before = 0, all = 0;
#pragma unroll
  for (int w = 0; w < SEG_THREADS / 64; ++w) {
    before += w < wave ? wsum[w] : 0;
    all += wsum[w];
  }
  __syncthreads();
  *total = all;
  return before + inc - v;
}

__global__ __launch_bounds__(SEG_THREADS) void seg_count(const int32_t* __restrict__ keys, int M,
                                                         int* __restrict__ cnt) {
  const int p0 = blockIdx.x * SEG_TILE + threadIdx.x * SEG_PER;
  int c = 0;
  for (int i = 0; i < SEG_PER; ++i) c += seg_head(keys, p0 + i, M);
  int total;
  block_excl_scan(c, &total);
  if (threadIdx.x == 0) cnt[blockIdx.x] = total;
}

// One workgroup: exclusive scan of the tile counts in place.
__global__ __launch_bounds__(SEG_THREADS) void seg_scan(int* __restrict__ cnt, int ntiles, int M,
                                                        int32_t* __restrict__ n_uniq,
                                                        int32_t* __restrict__ seg_start) {
  int carry = 0;
  for (int base = 0; base < ntiles; base += SEG_THREADS) {
    const int i = base + threadIdx.x;
    const int v = i < ntiles ? cnt[i] : 0;
    int total;
    const int ex = block_excl_scan(v, &total);
    if (i < ntiles) cnt[i] = carry + ex;
    carry += total;
  }
  if (threadIdx.x == 0) {
    n_uniq[0] = carry;
    seg_start[carry] = M;
  }
}

__global__ __launch_bounds__(SEG_THREADS) void seg_write(const int32_t* __restrict__ keys, int M,
                                                         const int* __restrict__ base,
                                                         int32_t* __restrict__ uniq,
                                                         int32_t* __restrict__ seg_start) {
  const int p0 = blockIdx.x * SEG_TILE + threadIdx.x * SEG_PER;
  int c = 0;
  for (int i = 0; i < SEG_PER; ++i) c += seg_head(keys, p0 + i, M);
  int total;
  int r = base[blockIdx.x] + block_excl_scan(c, &total);
  for (int i = 0; i < SEG_PER; ++i) {
    const int p = p0 + i;
    if (seg_head(keys, p, M)) {
      uniq[r] = keys[p];
      seg_start[r] = p;
      ++r;
    }
  }
}

// ------------------------------------------------------------------ the row order
// The row pass reads, per task, the x and dy rows of the task's token; most
// used experts have one task.  Workgroup b runs on XCD b % 8, whose L2 is its
// own, so the used experts are dealt out by the token t of their first task:
// class t % 8 goes to XCD t % 8, which then reads the x and dy rows of one
// eighth of the tokens, and inside a class by ascending t, so that the
// experts of one token run close together in time.
//
// key[u] = (t % 8) * Lq + t / 8 for used expert u (Lq = ceil(L / 8)), 8 * Lq
// for the slots past n_uniq.
__global__ __launch_bounds__(256) void row_keys(const int32_t* __restrict__ perm,
                                                const int32_t* __restrict__ seg,
                                                const int32_t* __restrict__ n_uniq, int K, int Lq,
                                                int U, int32_t* __restrict__ key,
                                                const int32_t* run_flag, int run_want) {
  if (gated_out(run_flag, run_want)) return;
  const int n = *n_uniq;
  for (int u = blockIdx.x * 256 + threadIdx.x; u < U; u += gridDim.x * 256) {
    int k = 8 * Lq;
    if (u < n) {
      const int t = perm[seg[u]] / K;
      k = (t & 7) * Lq + (t >> 3);
    }
    key[u] = k;
  }
}

// With rord = the used experts sorted by key and goff its key offsets, class
// x is rord[goff[x Lq] .. goff[(x+1) Lq]).  With m the smallest class size,
// workgroup b < 8m takes entry b / 8 of class b % 8; the classes' remaining
// entries follow, class by class, from b = 8m.  rec[b] = {u, seg[u],
// seg[u + 1], perm[seg[u]]}: the row, its task range and its first task, so
// that the row pass starts its data loads at once.
__global__ __launch_bounds__(256) void row_recs(const int32_t* __restrict__ rord,
                                                const int32_t* __restrict__ goff,
                                                const int32_t* __restrict__ seg,
                                                const int32_t* __restrict__ perm,
                                                const int32_t* __restrict__ n_uniq, int Lq,
                                                int4* __restrict__ rec, const int32_t* run_flag,
                                                int run_want) {
  if (gated_out(run_flag, run_want)) return;
  __shared__ int off[9];
  if (threadIdx.x < 9) off[threadIdx.x] = goff[threadIdx.x * Lq];
  __syncthreads();
  const int n = *n_uniq;
  int m = n;
#pragma unroll
  for (int x = 0; x < 8; ++x) m = min(m, off[x + 1] - off[x]);
  for (int b = blockIdx.x * 256 + threadIdx.x; b < n; b += gridDim.x * 256) {
    int q;
    if (b < 8 * m) {
      q = off[b & 7] + (b >> 3);
    } else {
      int k = b - 8 * m, x = 0;
      for (; x < 7; ++x) {  // the extras of classes 0..x-1 come first
        const int extra = off[x + 1] - off[x] - m;
        if (k < extra) break;
        k -= extra;
      }
      q = off[x] + m + k;
    }
    const int u = rord[q];
    const int s0 = seg[u];
    rec[b] = int4{u, s0, seg[u + 1], perm[s0]};
  }
}

// ------------------------------------------------------------------ expert_bwd_rows
// One workgroup per used expert r (row uniq[r]); thread i owns 16 bytes of
// the input row (E columns) of both gradients.  The segment's tasks are
// visited in sorted order (token, then k), the next task's x and dy chunks
// in flight while the current one is accumulated; the rows are written once
// at the end (fp32, or bf16 rounded to nearest even), so every row has one
// owner and no atomics are needed.  (Measured at 4096 tokens x 1.7M experts:
// workgroups that each walk a run of 32 experts with a deeper prefetch were
// slower, 1.96 ms against 1.70 ms: a wave's row stores then sit between its
// loads, and gfx9's single vector-memory counter makes the loads wait for
// them.)
// The rows are stored non-temporally, so that the x and dy rows the next
// segments read stay in L2 (bf16 rows: whole call 2.10 -> 1.93 ms at 4096
// tokens x 1.7M experts).
template <bool OUT_BF16, int E>
__device__ __forceinline__ void store_row_chunk(void* rows, size_t r, int d, int c,
                                                const float* v) {
  if constexpr (OUT_BF16) {
    uint16_t* o = (uint16_t*)rows + r * d + c * E;
#pragma unroll
    for (int q = 0; q + 8 <= E; q += 8) {
      u32x4 w;
      w.x = bf16_rne(v[q]) | (bf16_rne(v[q + 1]) << 16);
      w.y = bf16_rne(v[q + 2]) | (bf16_rne(v[q + 3]) << 16);
      w.z = bf16_rne(v[q + 4]) | (bf16_rne(v[q + 5]) << 16);
      w.w = bf16_rne(v[q + 6]) | (bf16_rne(v[q + 7]) << 16);
      __builtin_nontemporal_store(w, (u32x4*)(o + q));
    }
    if constexpr (E % 8 == 4) {  // fp32 inputs (E = 4): 8 bytes of bf16
      const int q = E - 4;
      uint2 w{bf16_rne(v[q]) | (bf16_rne(v[q + 1]) << 16), bf16_rne(v[q + 2]) | (bf16_rne(v[q + 3]) << 16)};
      *(uint2*)(o + q) = w;
    }
  } else if (E == 8 && d % 512 == 0) {
    // fp32 rows from bf16 inputs: a wave's 64 chunks are 2 KB of the row.
    // Lanes exchange halves so that each of the two stores writes 1 KB
    // contiguously (lane l: floats 4l.. of the wave's first or second KB),
    // then store non-temporally; without the exchange a store instruction
    // covers every other 16 bytes, and non-temporal stores of such half
    // lines made the call 1.5x slower.
    const int lane = threadIdx.x & 63;
    float* o = (float*)rows + r * d + (c - lane) * E;
#pragma unroll
    for (int half = 0; half < 2; ++half) {
      const int src = 32 * half + (lane >> 1);
      f32x4 w;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float lo = __shfl(v[i], src, 64), hi = __shfl(v[4 + i], src, 64);
        w[i] = (lane & 1) ? hi : lo;
      }
      __builtin_nontemporal_store(w, (f32x4*)(o + 256 * half + 4 * lane));
    }
  } else {
    float* o = (float*)rows + r * d + c * E;
#pragma unroll
    for (int q = 0; q < E; q += 4) *(f32x4*)(o + q) = f32x4{v[q], v[q + 1], v[q + 2], v[q + 3]};
  }
}

template <bool BF16, bool OUT_BF16>
__global__ __launch_bounds__(512) void expert_bwd_rows(
    const uint16_t* __restrict__ x_, const float* __restrict__ dy, const int32_t* __restrict__ perm,
    const int4* __restrict__ rec, const int32_t* __restrict__ n_uniq,
    const float* __restrict__ dh, const float* __restrict__ ga, int d, int K,
    void* __restrict__ dW_rows, void* __restrict__ dV_rows, const int32_t* run_flag,
    int run_want) {
  if (gated_out(run_flag, run_want)) return;
  using C = Chunk<BF16>;
  constexpr int E = C::E;
  const int c = threadIdx.x;
  const unsigned row_bytes = (unsigned)d * (BF16 ? 2u : 4u);
  if (c * 16u >= row_bytes) return;  // no barrier below
  // Workgroup b takes used experts b, b + grid, ...  The first record is
  // loaded beside the count (slot blockIdx.x exists: the grid is at most the
  // used-expert bound, the length of rec); slots past n_uniq are never used.
  const int n = n_uniq[0];
  int4 rc = rec[blockIdx.x];
  for (int b = blockIdx.x; b < n; b += gridDim.x) {
    if (b != (int)blockIdx.x) rc = rec[b];
    const int r = uni(rc.x), s0 = uni(rc.y), s1 = uni(rc.z), m0 = uni(rc.w);
    float aw[E], av[E];
#pragma unroll
    for (int q = 0; q < E; ++q) aw[q] = av[q] = 0.f;
    auto load = [&](int p, u32x4& xv, f32x4* dv, float& sdh, float& sga) {
      const int m = p == s0 ? m0 : uni(perm[p]);
      const int t = m / K;
      sdh = uni(dh[m]);
      sga = uni(ga[m]);
      xv = *(const u32x4*)((const char*)x_ + (size_t)t * row_bytes + c * 16u);
      const float* dyp = dy + (size_t)t * d + c * E;
#pragma unroll
      for (int q = 0; q < E / 4; ++q) dv[q] = *(const f32x4*)(dyp + 4 * q);
    };
    u32x4 xa, xb;
    f32x4 da[E / 4], db[E / 4];
    float ha, gaa, hb, gab;
    auto accum = [&](const u32x4 xv, const f32x4* dv, float sdh, float sga) {
      float xf[E];
      C::widen(xv, xf);
#pragma unroll
      for (int q = 0; q < E; ++q) {
        aw[q] = fmaf(sdh, xf[q], aw[q]);
        av[q] = fmaf(sga, dv[q / 4][q % 4], av[q]);
      }
    };
    load(s0, xa, da, ha, gaa);
    for (int p = s0; p < s1; p += 2) {
      if (p + 1 < s1) load(p + 1, xb, db, hb, gab);
      accum(xa, da, ha, gaa);
      if (p + 1 < s1) {
        if (p + 2 < s1) load(p + 2, xa, da, ha, gaa);
        accum(xb, db, hb, gab);
      }
    }
    store_row_chunk<OUT_BF16, E>(dW_rows, (size_t)r, d, c, aw);
    store_row_chunk<OUT_BF16, E>(dV_rows, (size_t)r, d, c, av);
  }
}

// ------------------------------------------------------------------ router_bwd_ds
// One workgroup per token.  dS_k = g_k (dgate_k - sum_j g_j dgate_j); entry n
// of the token's logit-gradient row (rows 0..Nr-1, then columns) is the sum
// of dS_k over the tasks that select it, taken in k order by the thread of
// the first such task.  Written as fp32, or as bf16 high + low parts
// (v = hi + lo to about 2^-16 relative) padded with zeros to ld columns.
template <bool SPLIT>
__global__ __launch_bounds__(256) void router_bwd_ds(const int32_t* __restrict__ idx,
                                                     const float* __restrict__ gate,
                                                     const float* __restrict__ dgate, int K,
                                                     int Nr, int Nc, int ld,
                                                     float* __restrict__ ds,
                                                     uint16_t* __restrict__ ds_hi,
                                                     uint16_t* __restrict__ ds_lo) {
  extern __shared__ float row[];  // [ld]
  __shared__ float sdS[OMNI_MAX_K];
  __shared__ int srow[OMNI_MAX_K], scol[OMNI_MAX_K];
  __shared__ float wpart[4];
  const int t = blockIdx.x, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  float part = 0.f;
  for (int k = tid; k < K; k += 256) {
    const size_t m = (size_t)t * K + k;
    part += gate[m] * dgate[m];
  }
  part = wave_sum(part);
  if (lane == 0) wpart[wave] = part;
  for (int n = tid; n < ld; n += 256) row[n] = 0.f;
  __syncthreads();
  const float gdg = wpart[0] + wpart[1] + wpart[2] + wpart[3];
  for (int k = tid; k < K; k += 256) {
    const size_t m = (size_t)t * K + k;
    const int e = idx[m];
    sdS[k] = gate[m] * (dgate[m] - gdg);
    srow[k] = e / Nc;
    scol[k] = e % Nc;
  }
  __syncthreads();
  for (int k = tid; k < K; k += 256) {
    const int i = srow[k], j = scol[k];
    bool first_r = true, first_c = true;
    float sr = 0.f, sc = 0.f;
    for (int q = 0; q < K; ++q) {
      if (srow[q] == i) {
        first_r &= q >= k;
        sr += sdS[q];
      }
      if (scol[q] == j) {
        first_c &= q >= k;
        sc += sdS[q];
      }
    }
    if (first_r) row[i] = sr;
    if (first_c) row[Nr + j] = sc;
  }
  __syncthreads();
  if constexpr (SPLIT) {
    for (int n = 2 * tid; n < ld; n += 512) {  // ld is even
      const float v0 = row[n], v1 = row[n + 1];
      const unsigned h0 = bf16_rne(v0), h1 = bf16_rne(v1);
      const unsigned l0 = bf16_rne(v0 - __uint_as_float(h0 << 16));
      const unsigned l1 = bf16_rne(v1 - __uint_as_float(h1 << 16));
      *(unsigned*)(ds_hi + (size_t)t * ld + n) = h0 | (h1 << 16);
      *(unsigned*)(ds_lo + (size_t)t * ld + n) = l0 | (l1 << 16);
    }
  } else {
    for (int n = tid; n < ld; n += 256) ds[(size_t)t * ld + n] = row[n];
  }
}

// ------------------------------------------------------------------ transpose
// out[c * ldo + off + r] = r < R ? in[r * ldi + c] : 0, for c < Cn, r < Rspan
// (bf16).  64 x 64 tiles through LDS; a thread moves 16-byte chunks (8
// elements) in both directions where the chunk is whole and aligned, single
// elements at the ragged edges.  (2-byte accesses throughout ran the five
// transposes of the router backward at about 1.9 TB/s.)
constexpr int TP = 72;  // LDS row pitch in elements: 144 bytes, 16-byte aligned rows

__global__ __launch_bounds__(256) void transpose_bf16(const uint16_t* __restrict__ in, int R,
                                                      int Cn, int ldi, int Rspan,
                                                      uint16_t* __restrict__ out, int ldo,
                                                      int off) {
  __shared__ __attribute__((aligned(16))) uint16_t tile[64 * TP];
  const int c0 = blockIdx.x * 64, r0 = blockIdx.y * 64;
  const int ch = threadIdx.x & 7, row = threadIdx.x >> 3;  // chunk 0..7, row 0..31
  const bool in_vec = (ldi & 7) == 0 && ((uintptr_t)in & 15) == 0;
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int i = row + 32 * j, r = r0 + i, c = c0 + 8 * ch;
    u32x4 v{0u, 0u, 0u, 0u};
    if (r < R) {
      const uint16_t* src = in + (size_t)r * ldi + c;
      if (in_vec && c + 8 <= Cn) {
        v = *(const u32x4*)src;
      } else {
        uint16_t e[8];
#pragma unroll
        for (int q = 0; q < 8; ++q) e[q] = c + q < Cn ? src[q] : (uint16_t)0;
        v.x = e[0] | ((unsigned)e[1] << 16);
        v.y = e[2] | ((unsigned)e[3] << 16);
        v.z = e[4] | ((unsigned)e[5] << 16);
        v.w = e[6] | ((unsigned)e[7] << 16);
      }
    }
    *(u32x4*)(tile + i * TP + 8 * ch) = v;
  }
  __syncthreads();
  const bool out_vec = ((ldo | off) & 7) == 0 && ((uintptr_t)out & 15) == 0;
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int i = row + 32 * j, c = c0 + i, r = r0 + 8 * ch;  // out row c, elements r .. r+7
    if (c >= Cn) continue;
    uint16_t e[8];
#pragma unroll
    for (int q = 0; q < 8; ++q) e[q] = tile[(8 * ch + q) * TP + i];
    uint16_t* dst = out + (size_t)c * ldo + off + r;
    if (out_vec && r + 8 <= Rspan) {
      *(u32x4*)dst = u32x4{e[0] | ((unsigned)e[1] << 16), e[2] | ((unsigned)e[3] << 16),
                           e[4] | ((unsigned)e[5] << 16), e[6] | ((unsigned)e[7] << 16)};
    } else {
#pragma unroll
      for (int q = 0; q < 8; ++q)
        if (r + q < Rspan) dst[q] = e[q];
    }
  }
}

template <bool BF16>
hipError_t launch_bwd_token_t(const void* x, const void* W, const void* V, const int32_t* idx,
                              const float* gate, const float* dy, const int32_t* n_uniq, int L,
                              int d, int K, float* dx, float* dgate, float* dh, float* ga,
                              hipStream_t s, RunGate run) {
  const int nch = (int)(((size_t)d * (BF16 ? 2 : 4) / 16 + 63) / 64);
  const size_t lds = (size_t)BWD_WAVES * d * 4;
  const uint16_t *xp = (const uint16_t*)x, *wp = (const uint16_t*)W, *vp = (const uint16_t*)V;
  const dim3 grid((unsigned)std::min(L, BWD_TOKEN_GRID));
#define OMNI_BT(N)                                                                            \
  case N:                                                                                     \
    hipLaunchKernelGGL((expert_bwd_token<BF16, N>), grid, dim3(256), lds, s, xp, wp, vp, idx,  \
                       gate, dy, n_uniq, L, d, K, dx, dgate, dh, ga, run.flag, run.want);     \
    break;
  switch (nch) {
    OMNI_BT(1) OMNI_BT(2) OMNI_BT(3) OMNI_BT(4) OMNI_BT(5) OMNI_BT(6) OMNI_BT(7) OMNI_BT(8)
    default:
      return hipErrorInvalidValue;  // d above the validated limit
  }
#undef OMNI_BT
  return hipGetLastError();
}

}  // namespace

// ------------------------------------------------------------------ host entry points

BwdPlan plan_expert_backward(int64_t L, int64_t d, int64_t N, int64_t K) {
  BwdPlan p{};
  p.M = (int)(L * K);
  p.U_max = (int)(N < L * K ? N : L * K);
  p.sched = plan_schedule(L, K, N, 1);
  p.ntiles = (p.M + SEG_TILE - 1) / SEG_TILE;
  size_t o = 0;
  auto take = [&](size_t bytes) {
    const size_t at = o;
    o += (bytes + 255) & ~(size_t)255;
    return at;
  };
  p.off_dh = take((size_t)p.M * 4);
  p.off_ga = take((size_t)p.M * 4);
  p.off_perm = take((size_t)p.M * 4);
  p.off_eoff = take((size_t)(N + 1) * 4);
  p.off_seg = take((size_t)(p.M + 1) * 4);
  p.off_cnt = take((size_t)p.ntiles * 4);
  // the row order: keys, the sorted experts, key offsets, one record per row
  p.Lq = (int)((L + 7) / 8);
  p.rsort = plan_schedule(p.U_max, 1, 8ll * p.Lq + 1, 1);
  p.off_rkey = take((size_t)p.U_max * 4);
  p.off_rord = take((size_t)p.U_max * 4);
  p.off_goff = take((size_t)(8 * p.Lq + 2) * 4);
  p.off_rec = take((size_t)p.U_max * 16);
  // the expert sort's workspace is free again when the row order is sorted
  p.off_sched = take(std::max(p.sched.ws_bytes, p.rsort.ws_bytes));
  p.ws_bytes = o;
  (void)d;
  return p;
}

hipError_t launch_expert_backward(const void* x, const void* W, const void* V, const int32_t* idx,
                                  const float* gate, const float* dy, int L, int d, int N, int K,
                                  omni_dtype dt, float* dx, float* dgate, int32_t* uniq,
                                  int32_t* n_uniq, omni_dtype grad_dt, void* dW_rows,
                                  void* dV_rows, const BwdPlan& p, void* ws, hipStream_t s) {
  // the sort by expert first: the per-token pass reads the used-expert count
  hipError_t e = launch_expert_segments(idx, N, uniq, n_uniq, p, ws, s);
  if (e != hipSuccess) return e;
  e = launch_expert_bwd_token(x, W, V, idx, gate, dy, L, d, K, dt, dx, dgate, n_uniq, p, ws, s);
  if (e != hipSuccess) return e;
  return launch_expert_grad_rows(x, dy, d, K, dt, n_uniq, grad_dt, dW_rows, dV_rows, p, ws, s);
}

hipError_t launch_expert_bwd_token(const void* x, const void* W, const void* V,
                                   const int32_t* idx, const float* gate, const float* dy, int L,
                                   int d, int K, omni_dtype dt, float* dx, float* dgate,
                                   const int32_t* n_uniq, const BwdPlan& p, void* ws,
                                   hipStream_t s, RunGate run) {
  char* w = (char*)ws;
  float* dh = (float*)(w + p.off_dh);
  float* ga = (float*)(w + p.off_ga);
  return dt == OMNI_BF16
             ? launch_bwd_token_t<true>(x, W, V, idx, gate, dy, n_uniq, L, d, K, dx, dgate, dh, ga,
                                        s, run)
             : launch_bwd_token_t<false>(x, W, V, idx, gate, dy, n_uniq, L, d, K, dx, dgate, dh, ga,
                                         s, run);
}

hipError_t launch_expert_segments(const int32_t* idx, int N, int32_t* uniq, int32_t* n_uniq,
                                  const BwdPlan& p, void* ws, hipStream_t s) {
  char* w = (char*)ws;
  int32_t* perm = (int32_t*)(w + p.off_perm);
  int32_t* eoff = (int32_t*)(w + p.off_eoff);
  int32_t* seg = (int32_t*)(w + p.off_seg);
  int* cnt = (int*)(w + p.off_cnt);
  void* sws = w + p.off_sched;
  // tasks sorted by expert id: the schedule with groups of one expert
  hipError_t e = launch_schedule(idx, p.M, 1, N, p.sched, perm, eoff, sws, s);
  if (e != hipSuccess) return e;
  const int32_t* keys = schedule_sorted_keys(p.sched, sws);
  hipLaunchKernelGGL(seg_count, dim3(p.ntiles), dim3(SEG_THREADS), 0, s, keys, p.M, cnt);
  hipLaunchKernelGGL(seg_scan, dim3(1), dim3(SEG_THREADS), 0, s, cnt, p.ntiles, p.M, n_uniq, seg);
  hipLaunchKernelGGL(seg_write, dim3(p.ntiles), dim3(SEG_THREADS), 0, s, keys, p.M, cnt, uniq, seg);
  return hipGetLastError();
}

hipError_t launch_expert_grad_rows(const void* x, const float* dy, int d, int K, omni_dtype dt,
                                   const int32_t* n_uniq, omni_dtype grad_dt, void* dW_rows,
                                   void* dV_rows, const BwdPlan& p, void* ws, hipStream_t s,
                                   RunGate run) {
  char* w = (char*)ws;
  float* dh = (float*)(w + p.off_dh);
  float* ga = (float*)(w + p.off_ga);
  const int32_t* perm = (const int32_t*)(w + p.off_perm);
  const int32_t* seg = (const int32_t*)(w + p.off_seg);
  int32_t* rkey = (int32_t*)(w + p.off_rkey);
  int32_t* rord = (int32_t*)(w + p.off_rord);
  int32_t* goff = (int32_t*)(w + p.off_goff);
  int4* rec = (int4*)(w + p.off_rec);
  const unsigned ogrid = (unsigned)std::min(2048, (p.U_max + 255) / 256);
  hipLaunchKernelGGL(row_keys, dim3(ogrid), dim3(256), 0, s, perm, seg, n_uniq, K, p.Lq, p.U_max,
                     rkey, run.flag, run.want);
  hipError_t e = launch_schedule(rkey, p.U_max, 1, 8 * p.Lq + 1, p.rsort, rord, goff,
                                 w + p.off_sched, s, run);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(row_recs, dim3(ogrid), dim3(256), 0, s, rord, goff, seg, perm, n_uniq, p.Lq,
                     rec, run.flag, run.want);
  const bool bf = dt == OMNI_BF16;
  const int E = bf ? 8 : 4;
  const int threads = ((d / E + 63) / 64) * 64;  // <= 512 for the supported d
  // a bounded grid (a multiple of 8, so that slot b keeps its XCD b % 8 in
  // every round): with the blocked form chosen, these workgroups only read
  // the choice and leave, and one per possible used expert (1.7M on the
  // skewed workload) took 0.4 ms just to dispatch
  const dim3 grid((unsigned)std::min(p.U_max, BWD_ROWS_GRID));
  const bool obf = grad_dt == OMNI_BF16;
#define OMNI_ROWS(IB, OB)                                                                        \
  hipLaunchKernelGGL((expert_bwd_rows<IB, OB>), grid, dim3(threads), 0, s, (const uint16_t*)x, dy, \
                     perm, rec, n_uniq, dh, ga, d, K, dW_rows, dV_rows, run.flag, run.want)
  if (bf && obf) OMNI_ROWS(true, true);
  else if (bf) OMNI_ROWS(true, false);
  else if (obf) OMNI_ROWS(false, true);
  else OMNI_ROWS(false, false);
#undef OMNI_ROWS
  return hipGetLastError();
}

RouterBwdPlan plan_router_backward(int64_t L, int64_t d, int64_t Nr, int64_t Nc, omni_dtype dt) {
  RouterBwdPlan p{};
  const int Ntot = (int)(Nr + Nc);
  p.Ntot_p = (Ntot + 63) / 64 * 64;
  p.L_p = (int)((L + 63) / 64 * 64);
  size_t o = 0;
  auto take = [&](size_t bytes) {
    const size_t at = o;
    o += (bytes + 255) & ~(size_t)255;
    return at;
  };
  if (dt == OMNI_BF16) {
    p.off_ds_hi = take((size_t)L * p.Ntot_p * 2);
    p.off_ds_lo = take((size_t)L * p.Ntot_p * 2);
    p.off_dsT_hi = take((size_t)Ntot * p.L_p * 2);
    p.off_dsT_lo = take((size_t)Ntot * p.L_p * 2);
    p.off_xT = take((size_t)d * p.L_p * 2);
    p.off_wT = take((size_t)d * p.Ntot_p * 2);
  } else {
    p.off_ds = take((size_t)L * Ntot * 4);
  }
  p.ws_bytes = o;
  return p;
}

hipError_t launch_router_backward(const void* x, const void* Wr, const void* Wc,
                                  const int32_t* idx, const float* gate, const float* dgate,
                                  int L, int d, int Nr, int Nc, int K, omni_dtype dt, float* dx,
                                  float* dWr, float* dWc, const RouterBwdPlan& p, void* ws,
                                  hipStream_t s) {
  char* w = (char*)ws;
  const int Ntot = Nr + Nc;
  hipError_t e;
  if (dt == OMNI_BF16) {
    uint16_t* ds_hi = (uint16_t*)(w + p.off_ds_hi);
    uint16_t* ds_lo = (uint16_t*)(w + p.off_ds_lo);
    uint16_t* dsT_hi = (uint16_t*)(w + p.off_dsT_hi);
    uint16_t* dsT_lo = (uint16_t*)(w + p.off_dsT_lo);
    uint16_t* xT = (uint16_t*)(w + p.off_xT);
    uint16_t* wT = (uint16_t*)(w + p.off_wT);
    hipLaunchKernelGGL(router_bwd_ds<true>, dim3(L), dim3(256), (size_t)p.Ntot_p * 4, s, idx, gate,
                       dgate, K, Nr, Nc, p.Ntot_p, (float*)nullptr, ds_hi, ds_lo);
    const dim3 tb(256);
    // dsT [Ntot, L_p], xT [d, L_p], W_rc^T [d, Ntot_p] (zero padded)
    hipLaunchKernelGGL(transpose_bf16, dim3((Ntot + 63) / 64, p.L_p / 64), tb, 0, s, ds_hi, L, Ntot,
                       p.Ntot_p, p.L_p, dsT_hi, p.L_p, 0);
    hipLaunchKernelGGL(transpose_bf16, dim3((Ntot + 63) / 64, p.L_p / 64), tb, 0, s, ds_lo, L, Ntot,
                       p.Ntot_p, p.L_p, dsT_lo, p.L_p, 0);
    hipLaunchKernelGGL(transpose_bf16, dim3((d + 63) / 64, p.L_p / 64), tb, 0, s,
                       (const uint16_t*)x, L, d, d, p.L_p, xT, p.L_p, 0);
    hipLaunchKernelGGL(transpose_bf16, dim3((d + 63) / 64, (Nr + 63) / 64), tb, 0, s,
                       (const uint16_t*)Wr, Nr, d, d, Nr, wT, p.Ntot_p, 0);
    hipLaunchKernelGGL(transpose_bf16, dim3((d + 63) / 64, (p.Ntot_p - Nr + 63) / 64), tb, 0, s,
                       (const uint16_t*)Wc, Nc, d, d, p.Ntot_p - Nr, wT, p.Ntot_p, Nr);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    // dW_r | dW_c = ds^T x : [Ntot, d], rows split at Nr
    if ((e = launch_gemm_bt_bf16(dsT_hi, xT, xT, d, Ntot, d, p.L_p, dWr, dWc, Nr, d, false, s)))
      return e;
    if ((e = launch_gemm_bt_bf16(dsT_lo, xT, xT, d, Ntot, d, p.L_p, dWr, dWc, Nr, d, true, s)))
      return e;
    // dx += ds W_rc : [L, d]
    if ((e = launch_gemm_bt_bf16(ds_hi, wT, wT, d, L, d, p.Ntot_p, dx, dx, L, d, true, s))) return e;
    return launch_gemm_bt_bf16(ds_lo, wT, wT, d, L, d, p.Ntot_p, dx, dx, L, d, true, s);
  }
  float* ds = (float*)(w + p.off_ds);
  hipLaunchKernelGGL(router_bwd_ds<false>, dim3(L), dim3(256), (size_t)Ntot * 4, s, idx, gate,
                     dgate, K, Nr, Nc, Ntot, ds, (uint16_t*)nullptr, (uint16_t*)nullptr);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  const float* xf = (const float*)x;
  // dW_r[i, j] = sum_t ds[t, i] x[t, j]; likewise dW_c from columns Nr..
  if ((e = gemm_f32(ds, 1, Ntot, xf, 1, d, Nr, d, L, dWr, d, false, s))) return e;
  if ((e = gemm_f32(ds + Nr, 1, Ntot, xf, 1, d, Nc, d, L, dWc, d, false, s))) return e;
  // dx[t, j] += sum_i ds[t, i] W_r[i, j] + sum_j' ds[t, Nr + j'] W_c[j', j]
  if ((e = gemm_f32(ds, Ntot, 1, (const float*)Wr, 1, d, L, d, Nr, dx, d, true, s))) return e;
  return gemm_f32(ds + Nr, Ntot, 1, (const float*)Wc, 1, d, L, d, Nc, dx, d, true, s);
}

}  // namespace omni
