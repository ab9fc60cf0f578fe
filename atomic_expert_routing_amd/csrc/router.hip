// Cartesian Product Router on gfx950.
//
// OmniMoE digest (paper.rainbus.top), method paragraph, step 2: row and column
// logits s_r = x W_r, s_c = x W_c, LogSoftmax to p_r and p_c, scores
// S_ij = p_r[i] + p_c[j] on the implicit N_r x N_c grid, global top-K.
//
// Two kernels:
//   router_gemm_*    logits[L, N_r+N_c] = x . [W_r; W_c]^T   (bf16: MFMA)
//   router_topk      one workgroup per token: LogSoftmax, row/column
//                    pre-selection, K x K candidate merge, gate softmax.

#include "omni_internal.h"

namespace omni {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

// ------------------------------------------------------------------ bf16 GEMM
// 128 x 128 output tile per 256-thread workgroup; each of the 4 waves owns a
// 64 x 64 quadrant computed with v_mfma_f32_16x16x32_bf16 (4 x 4 MFMA tiles).
// Both operands are K-contiguous in HBM (x rows and W_r/W_c rows), so the
// tiles are staged row-wise in LDS with a 16-byte pad per row and each lane
// reads its 8-element k-slice with one 16-byte LDS load.
constexpr int GBM = 128, GBN = 128, GBK = 64, GPAD = 8, GLD = GBK + GPAD;

__global__ __launch_bounds__(256) void router_gemm_bf16(const uint16_t* __restrict__ x,
                                                        const uint16_t* __restrict__ Wr,
                                                        const uint16_t* __restrict__ Wc, int L,
                                                        int d, int Nr, int Nc,
                                                        float* __restrict__ C) {
  __shared__ __attribute__((aligned(16))) uint16_t As[GBM * GLD];
  __shared__ __attribute__((aligned(16))) uint16_t Bs[GBN * GLD];
  const int Ntot = Nr + Nc;
  const int tile_m = blockIdx.y * GBM, tile_n = blockIdx.x * GBN;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int wm = (wave >> 1) * 64, wn = (wave & 1) * 64;

  f32x4 acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  // Per thread: 4 16-byte chunks of the A tile and 4 of the B tile.
  // chunk c = tid + 256*i covers row c/8, columns (c%8)*8 .. +8 of the k-tile.
  const uint16_t* arow[4];
  const uint16_t* brow[4];
  bool aok[4], bok[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int c = tid + 256 * i, r = c >> 3;
    const int gm = tile_m + r, gn = tile_n + r;
    aok[i] = gm < L;
    bok[i] = gn < Ntot;
    arow[i] = x + (size_t)(aok[i] ? gm : 0) * d;
    brow[i] = gn < Nr ? Wr + (size_t)gn * d : Wc + (size_t)(bok[i] ? gn - Nr : 0) * d;
  }
  const int kc = (tid & 7) * 8;
  u32x4 ra[4], rb[4];
  auto gload = [&](int k0) {
    const int k = k0 + kc;
    const bool kin = k < d;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      ra[i] = (aok[i] && kin) ? *(const u32x4*)(arow[i] + k) : u32x4{0u, 0u, 0u, 0u};
      rb[i] = (bok[i] && kin) ? *(const u32x4*)(brow[i] + k) : u32x4{0u, 0u, 0u, 0u};
    }
  };
  auto sstore = [&]() {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = (tid + 256 * i) >> 3;
      *(u32x4*)(As + r * GLD + kc) = ra[i];
      *(u32x4*)(Bs + r * GLD + kc) = rb[i];
    }
  };

  const int nk = (d + GBK - 1) / GBK;
  gload(0);
  sstore();
  __syncthreads();
  for (int kt = 0; kt < nk; ++kt) {
    if (kt + 1 < nk) gload((kt + 1) * GBK);
#pragma unroll
    for (int ks = 0; ks < GBK / 32; ++ks) {
      const int kk = ks * 32 + (lane >> 4) * 8;
      bf16x8 af[4], bfr[4];
#pragma unroll
      for (int i = 0; i < 4; ++i)
        af[i] = *(const bf16x8*)(As + (wm + i * 16 + (lane & 15)) * GLD + kk);
#pragma unroll
      for (int j = 0; j < 4; ++j)
        bfr[j] = *(const bf16x8*)(Bs + (wn + j * 16 + (lane & 15)) * GLD + kk);
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[i], bfr[j], acc[i][j], 0, 0, 0);
    }
    __syncthreads();
    if (kt + 1 < nk) {
      sstore();
      __syncthreads();
    }
  }
  // D layout of the 16x16 MFMA tile: lane l holds rows 4*(l/16) + r, column l%16.
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int col = tile_n + wn + j * 16 + (lane & 15);
      if (col >= Ntot) continue;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int row = tile_m + wm + i * 16 + (lane >> 4) * 4 + r;
        if (row < L) C[(size_t)row * Ntot + col] = acc[i][j][r];
      }
    }
}

// ------------------------------------------------------------------ fp32 GEMM
// fp32 inputs: plain LDS-tiled VALU GEMM, 64 x 64 tile, 4 x 4 outputs/thread.
constexpr int FBM = 64, FBN = 64, FBK = 16;

__global__ __launch_bounds__(256) void router_gemm_f32(const float* __restrict__ x,
                                                       const float* __restrict__ Wr,
                                                       const float* __restrict__ Wc, int L,
                                                       int d, int Nr, int Nc,
                                                       float* __restrict__ C) {
  __shared__ float As[FBM][FBK + 1];
  __shared__ float Bs[FBN][FBK + 1];
  const int Ntot = Nr + Nc;
  const int tile_m = blockIdx.y * FBM, tile_n = blockIdx.x * FBN;
  const int tid = threadIdx.x, ty = tid >> 4, tx = tid & 15;
  float acc[4][4] = {};
  for (int k0 = 0; k0 < d; k0 += FBK) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int c = tid + 256 * i, r = c >> 4, k = k0 + (c & 15);
      const int gm = tile_m + r, gn = tile_n + r;
      As[r][c & 15] = (gm < L && k < d) ? x[(size_t)gm * d + k] : 0.f;
      float b = 0.f;
      if (gn < Ntot && k < d) b = gn < Nr ? Wr[(size_t)gn * d + k] : Wc[(size_t)(gn - Nr) * d + k];
      Bs[r][c & 15] = b;
    }
    __syncthreads();
#pragma unroll
    for (int k = 0; k < FBK; ++k) {
      float a[4], b[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) a[i] = As[ty * 4 + i][k];
#pragma unroll
      for (int j = 0; j < 4; ++j) b[j] = Bs[tx * 4 + j][k];
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = fmaf(a[i], b[j], acc[i][j]);
    }
    __syncthreads();
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int row = tile_m + ty * 4 + i;
    if (row >= L) continue;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int col = tile_n + tx * 4 + j;
      if (col < Ntot) C[(size_t)row * Ntot + col] = acc[i][j];
    }
  }
}

// ------------------------------------------------------------------ top-K
// Sort keys are 64-bit: high word = order-preserving image of the fp32 value,
// low word = bitwise-not of the index.  Sorting keys in descending order
// therefore orders by (value desc, index asc); 0 pads sort last.
__device__ __forceinline__ unsigned long long make_key(float v, unsigned int i) {
  return ((unsigned long long)float_ord(v) << 32) | (unsigned long long)(~i);
}
__device__ __forceinline__ float key_val(unsigned long long k) { return ord_float((unsigned int)(k >> 32)); }
__device__ __forceinline__ unsigned int key_idx(unsigned long long k) { return ~(unsigned int)k; }

// One bitonic compare-exchange stage over a power-of-two array (descending).
__device__ __forceinline__ void bitonic_stage(unsigned long long* a, int n, int k, int j) {
  for (int p = threadIdx.x; p < (n >> 1); p += blockDim.x) {
    const int lo = 2 * p - (p & (j - 1));
    const int hi = lo + j;
    const bool desc = (lo & k) == 0;
    const unsigned long long u = a[lo], v = a[hi];
    if (desc ? (u < v) : (u > v)) {
      a[lo] = v;
      a[hi] = u;
    }
  }
}

// Sort two independent power-of-two arrays with shared barriers.
__device__ void bitonic_sort2(unsigned long long* a, int na, unsigned long long* b, int nb) {
  const int n = na > nb ? na : nb;
  for (int k = 2; k <= n; k <<= 1)
    for (int j = k >> 1; j > 0; j >>= 1) {
      if (k <= na) bitonic_stage(a, na, k, j);
      if (b && k <= nb) bitonic_stage(b, nb, k, j);
      __syncthreads();
    }
}

__device__ float block_reduce(float v, bool is_max, float* red) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, nw = blockDim.x >> 6;
  v = is_max ? wave_max(v) : wave_sum(v);
  __syncthreads();
  if (lane == 0) red[wave] = v;
  __syncthreads();
  float r = red[0];
  for (int w = 1; w < nw; ++w) r = is_max ? fmaxf(r, red[w]) : r + red[w];
  return r;
}

__host__ __device__ inline int pow2_at_least(int n) {
  int p = 1;
  while (p < n) p <<= 1;
  return p;
}

// Number of rank pairs (a, b), a < Kr, b < Kc, with (a+1)(b+1) <= K.
__host__ __device__ inline int pair_count(int K, int Kr, int Kc) {
  int P = 0;
  for (int a = 0; a < Kr; ++a) {
    const int c = K / (a + 1);
    P += c < Kc ? c : Kc;
  }
  return P;
}

__global__ __launch_bounds__(256) void router_topk(const float* __restrict__ logits, int Nr,
                                                   int Nc, int K, int nr2, int nc2, int np2,
                                                   int32_t* __restrict__ idx,
                                                   float* __restrict__ score,
                                                   float* __restrict__ gate) {
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  unsigned long long* kr = (unsigned long long*)smem;  // [nr2] rows
  unsigned long long* kc = kr + nr2;                    // [nc2] columns
  unsigned long long* cand = kc + nc2;                  // [np2] candidates
  int* off = (int*)(cand + np2);                        // [OMNI_MAX_K + 1]
  __shared__ float red[16];

  const int t = blockIdx.x, tid = threadIdx.x;
  const float* sr = logits + (size_t)t * (Nr + Nc);
  const float* sc = sr + Nr;

  // LogSoftmax: p = s - (max + log sum exp(s - max)), rows and columns.
  float mr = -INFINITY, mc = -INFINITY;
  for (int i = tid; i < Nr; i += blockDim.x) mr = fmaxf(mr, sr[i]);
  for (int j = tid; j < Nc; j += blockDim.x) mc = fmaxf(mc, sc[j]);
  mr = block_reduce(mr, true, red);
  mc = block_reduce(mc, true, red + 8);
  float er = 0.f, ec = 0.f;
  for (int i = tid; i < Nr; i += blockDim.x) er += expf(sr[i] - mr);
  for (int j = tid; j < Nc; j += blockDim.x) ec += expf(sc[j] - mc);
  er = block_reduce(er, false, red);
  ec = block_reduce(ec, false, red + 8);
  const float lse_r = mr + logf(er), lse_c = mc + logf(ec);

  for (int i = tid; i < nr2; i += blockDim.x) kr[i] = i < Nr ? make_key(sr[i] - lse_r, i) : 0ull;
  for (int j = tid; j < nc2; j += blockDim.x) kc[j] = j < Nc ? make_key(sc[j] - lse_c, j) : 0ull;
  __syncthreads();
  bitonic_sort2(kr, nr2, kc, nc2);

  // Candidate rank pairs: row rank a keeps the first min(Kc, K/(a+1)) columns.
  const int Kr = K < Nr ? K : Nr, Kc = K < Nc ? K : Nc;
  if (tid < 64) {
    // wave 0: exclusive scan of the per-row counts (Kr <= 512 -> 8 per lane)
    const int per = (Kr + 63) / 64;
    const int a0 = tid * per;
    int loc = 0;
    for (int a = a0; a < a0 + per && a < Kr; ++a) {
      const int c = K / (a + 1);
      loc += c < Kc ? c : Kc;
    }
    int inc = loc;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int v = __shfl_up(inc, o, 64);
      if (tid >= o) inc += v;
    }
    int run = inc - loc;
    for (int a = a0; a < a0 + per && a < Kr; ++a) {
      off[a] = run;
      const int c = K / (a + 1);
      run += c < Kc ? c : Kc;
    }
    if (tid == 63) off[Kr] = inc;
  }
  __syncthreads();
  const int P = off[Kr];
  for (int a = tid; a < Kr; a += blockDim.x) {
    const unsigned long long rk = kr[a];
    const float pr = key_val(rk);
    const unsigned int i = key_idx(rk);
    const int base = off[a], cnt = off[a + 1] - base;
    for (int b = 0; b < cnt; ++b) {
      const unsigned long long ck = kc[b];
      cand[base + b] = make_key(pr + key_val(ck), i * (unsigned int)Nc + key_idx(ck));
    }
  }
  for (int c = P + tid; c < np2; c += blockDim.x) cand[c] = 0ull;
  __syncthreads();
  bitonic_sort2(cand, np2, nullptr, 0);

  // Gate: softmax over the K selected scores (cand[0] holds the largest).
  const float s0 = key_val(cand[0]);
  float es = 0.f;
  for (int k = tid; k < K; k += blockDim.x) es += expf(key_val(cand[k]) - s0);
  es = block_reduce(es, false, red);
  const float inv = 1.f / es;
  for (int k = tid; k < K; k += blockDim.x) {
    const unsigned long long ck = cand[k];
    const float s = key_val(ck);
    idx[(size_t)t * K + k] = (int32_t)key_idx(ck);
    score[(size_t)t * K + k] = s;
    gate[(size_t)t * K + k] = expf(s - s0) * inv;
  }
}

}  // namespace

hipError_t launch_router_gemm(const void* x, const void* Wr, const void* Wc, int L, int d,
                              int Nr, int Nc, omni_dtype dt, float* logits, hipStream_t s) {
  const int Ntot = Nr + Nc;
  if (dt == OMNI_BF16) {
    dim3 grid((Ntot + GBN - 1) / GBN, (L + GBM - 1) / GBM);
    hipLaunchKernelGGL(router_gemm_bf16, grid, dim3(256), 0, s, (const uint16_t*)x,
                       (const uint16_t*)Wr, (const uint16_t*)Wc, L, d, Nr, Nc, logits);
  } else {
    dim3 grid((Ntot + FBN - 1) / FBN, (L + FBM - 1) / FBM);
    hipLaunchKernelGGL(router_gemm_f32, grid, dim3(256), 0, s, (const float*)x,
                       (const float*)Wr, (const float*)Wc, L, d, Nr, Nc, logits);
  }
  return hipGetLastError();
}

size_t router_topk_lds_bytes(int Nr, int Nc, int K) {
  const int Kr = K < Nr ? K : Nr, Kc = K < Nc ? K : Nc;
  const int np2 = pow2_at_least(pair_count(K, Kr, Kc));
  return (size_t)(pow2_at_least(Nr) + pow2_at_least(Nc) + np2) * 8 + (OMNI_MAX_K + 1) * 4;
}

hipError_t launch_router_topk(const float* logits, int L, int Nr, int Nc, int K, int32_t* idx,
                              float* score, float* gate, hipStream_t s) {
  const int Kr = K < Nr ? K : Nr, Kc = K < Nc ? K : Nc;
  const int nr2 = pow2_at_least(Nr), nc2 = pow2_at_least(Nc);
  const int np2 = pow2_at_least(pair_count(K, Kr, Kc));
  const size_t lds = router_topk_lds_bytes(Nr, Nc, K);
  if (lds > 64 * 1024) {
    // beyond the default 64 KB of dynamic LDS: ask for exactly what is needed
    hipError_t e = hipFuncSetAttribute((const void*)router_topk,
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL(router_topk, dim3(L), dim3(256), lds, s, logits, Nr, Nc, K, nr2, nc2, np2,
                     idx, score, gate);
  return hipGetLastError();
}

}  // namespace omni
