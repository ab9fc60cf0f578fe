// Cartesian Product Router on gfx950.
//
// OmniMoE digest (paper.rainbus.top), method paragraph, step 2: row and column
// logits s_r = x W_r, s_c = x W_c, LogSoftmax to p_r and p_c, scores
// S_ij = p_r[i] + p_c[j] on the implicit N_r x N_c grid, global top-K.
//
// Kernels:
//   the logits logits[L, N_r+N_c] = x . [W_r; W_c]^T: bf16 on the pipelined
//                    MFMA product of gemm.hip when d % 64 == 0, else
//                    router_gemm_bf16 (register-staged MFMA); fp32 on VALU
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

typedef unsigned long long u64;
// LDS pointers of the top-K: typed in the LDS address space, so that every
// access is a DS instruction on an LDS offset whatever the compiler inlines
// (through a generic pointer it may fold a constant part of an index into
// the instruction offset and leave a base below the LDS window, which the
// hardware faults on).
typedef __attribute__((address_space(3))) u64 lds_u64;
typedef __attribute__((address_space(3))) int lds_int;

// Number of rank pairs (a, b), a < Kr, b < Kc, with (a+1)(b+1) <= K.
inline int pair_count(int K, int Kr, int Kc) {
  int P = 0;
  for (int a = 0; a < Kr; ++a) {
    const int c = K / (a + 1);
    P += c < Kc ? c : Kc;
  }
  return P;
}

// The top-K runs one wave (64 lanes) per token, one wave per workgroup, so
// every synchronisation is inside a wave: no workgroup barriers gate the
// steps.  Element i of a row / column vector lives in register v = i / 64
// of lane i % 64.

// Digit search of one radix pass: hist[0..256) counts the keys that match
// the current prefix by their digit.  Returns the largest digit d whose
// suffix count sum_{d' >= d} hist[d'] reaches `need`, with that bucket's
// size (*hd) and the count strictly above it (*above).  Lane l reads bins
// 4l .. 4l+3.
__device__ __forceinline__ int find_digit(const lds_int* hist, int need, int* hd, int* above) {
  const int lane = threadIdx.x & 63;
  const int h0 = hist[4 * lane], h1 = hist[4 * lane + 1];
  const int h2 = hist[4 * lane + 2], h3 = hist[4 * lane + 3];
  const int sl = h0 + h1 + h2 + h3;
  const int pre = wave_incl_scan(sl);                              // lanes 0..lane
  const int incl = __builtin_amdgcn_readlane(pre, 63) - pre + sl;  // lanes lane..63
  const int s3 = incl - sl + h3, s2 = s3 + h2, s1 = s2 + h1, s0 = s1 + h0;
  int best = -1;
  if (s0 >= need) best = 4 * lane;
  if (s1 >= need) best = 4 * lane + 1;
  if (s2 >= need) best = 4 * lane + 2;
  if (s3 >= need) best = 4 * lane + 3;
  best = wave_max_i(best);
  const int q = best & 3;
  const int hq = q == 0 ? h0 : q == 1 ? h1 : q == 2 ? h2 : h3;
  const int sq = q == 0 ? s0 : q == 1 ? s1 : q == 2 ? s2 : s3;
  *hd = __shfl(hq, best >> 2, 64);
  *above = __shfl(sq, best >> 2, 64) - *hd;
  return best;
}

__device__ __forceinline__ void zero_hist(lds_int* hist) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int q = 0; q < 4; ++q) hist[4 * lane + q] = 0;
}

// Select the R largest of n unique 64-bit keys in LDS; the R keys are
// written to out[0..R) in input order.
__device__ void select_top_lds(const lds_u64* keys, int n, int R, lds_int* hist, lds_u64* out) {
  const int lane = threadIdx.x & 63;
  const u64 lt = (1ull << lane) - 1ull;
  u64 prefix = 0, pmask = 0;
  int need = R;
  bool done = R >= n;
  if (!done) {
    unsigned mx = 0, mn = 0xffffffffu;  // range of the high (score) word
    for (int i = lane; i < n; i += 64) {
      const unsigned h = (unsigned)(keys[i] >> 32);
      mx = max(mx, h);
      mn = min(mn, h);
    }
    mx = wave_umax(mx);
    mn = wave_umin(mn);
    const unsigned diff = mx ^ mn;
    const int pass0 = diff ? __clz(diff) / 8 : 4;
    pmask = pass0 ? ~0ull << (64 - 8 * pass0) : 0ull;
    prefix = ((u64)mx << 32) & pmask;
    for (int pass = pass0; pass < 8 && !done; ++pass) {
      const int shift = 56 - 8 * pass;
      zero_hist(hist);
      wave_sync();
      for (int i = lane; i < n; i += 64) {
        const u64 k = keys[i];
        if ((k & pmask) == prefix)
          __hip_atomic_fetch_add(&hist[(int)((k >> shift) & 255)], 1, __ATOMIC_RELAXED,
                                 __HIP_MEMORY_SCOPE_WORKGROUP);
      }
      wave_sync();
      int hd, above;
      const int dig = find_digit(hist, need, &hd, &above);
      wave_sync();
      prefix |= (u64)dig << shift;
      pmask |= 0xffull << shift;
      need -= above;
      done = hd == need || shift == 0;
    }
  }
  int base = 0;
  for (int i0 = 0; i0 < n; i0 += 64) {
    const int i = i0 + lane;
    const u64 k = i < n ? keys[i] : 0ull;
    const bool sel = i < n && (k & pmask) >= prefix;
    const u64 bs = __ballot(sel);
    const int pos = base + __popcll(bs & lt);
    if (sel && pos < R) out[pos] = k;  // exactly R keys qualify
    base += __popcll(bs);
  }
}

// Select the R largest of n register-resident values under (value desc,
// index asc); val[v] holds element v*64 + lane, and 0 pads the lanes past n
// (every real value is nonzero).  The R-th largest value T is found by a
// bitwise search below the leading bits all values share: a bit is kept
// when at least R values are >= the candidate threshold, and the search
// stops as soon as exactly R qualify.  Counting is one compare per register
// plus a scalar popcount of the wave's ballot (measured faster than
// per-lane counts with a wave reduction, and than finishing on a compacted
// subset).  Values equal to T are taken by smallest index.  The R keys are
// written to out[0..R) in index order.
template <int VPL>
__device__ void select_top_regs(const unsigned (&val)[VPL], int n, int R, lds_u64* out) {
  const int lane = threadIdx.x & 63;
  const u64 lt = (1ull << lane) - 1ull;
  auto count_ge = [&](unsigned thr) {  // thr > 0, so padding never counts
    int c = 0;
#pragma unroll
    for (int v = 0; v < VPL; ++v) c += __popcll(__ballot(val[v] >= thr));
    return c;
  };
  unsigned T = 1;  // R >= n: every value (all are >= 1) is taken
  int need = R;    // values equal to T still to take, by index
  if (R < n) {
    unsigned mx = 0, mn = 0xffffffffu;
#pragma unroll
    for (int v = 0; v < VPL; ++v) {
      mx = max(mx, val[v]);
      mn = min(mn, v * 64 + lane < n ? val[v] : 0xffffffffu);
    }
    mx = wave_umax(mx);
    mn = wave_umin(mn);
    const unsigned diff = mx ^ mn;
    T = mx;  // all values equal: take the first R by index
    if (diff != 0) {
      const int hb = 31 - __clz(diff);
      T = mx & ~((2u << hb) - 1u);  // shared prefix, lower bits zero: count(>= T) = n
      for (int bit = hb; bit >= 0; --bit) {
        const unsigned cand = T | (1u << bit);
        const int c = count_ge(cand);
        if (c >= R) {
          T = cand;
          if (c == R) break;
        }
      }
    }
    need = R - (T == 0xffffffffu ? 0 : count_ge(T + 1u));
  }
  int base = 0, ties = 0;
#pragma unroll
  for (int v = 0; v < VPL; ++v) {
    const int i = v * 64 + lane;
    const bool eq = val[v] == T;
    const u64 be = __ballot(eq);
    const bool sel = val[v] > T || (eq && ties + __popcll(be & lt) < need);
    ties += __popcll(be);
    const u64 bs = __ballot(sel);
    const int pos = base + __popcll(bs & lt);
    if (sel && pos < R) out[pos] = ((u64)val[v] << 32) | (u64)(~(unsigned)i);
    base += __popcll(bs);
  }
}

// 64-bit wave max / min: the high words first, then the low words of the
// lanes that hold the extreme high word.
__device__ __forceinline__ u64 wave_umax64(u64 v) {
  const unsigned hi = wave_umax((unsigned)(v >> 32));
  const unsigned lo = wave_umax((unsigned)(v >> 32) == hi ? (unsigned)v : 0u);
  return ((u64)hi << 32) | lo;
}
__device__ __forceinline__ u64 wave_umin64(u64 v) {
  const unsigned hi = wave_umin((unsigned)(v >> 32));
  const unsigned lo = wave_umin((unsigned)(v >> 32) == hi ? (unsigned)v : 0xffffffffu);
  return ((u64)hi << 32) | lo;
}

// Select the R largest of n unique nonzero 64-bit keys held in registers
// (Q per lane, in any arrangement; 0 pads the unused slots).  The
// R-th largest key T is found bit by bit below the leading bits all keys
// share, keeping count(>= T) >= R and stopping as soon as exactly R keys
// qualify; being unique, exactly R keys are >= the final T.  They are
// written to out[0..R) (in slot order v, then lane).  Always inlined so that
// `out` stays a known LDS pointer (DS instructions, no generic addressing).
template <int Q>
__device__ __attribute__((always_inline)) void select_top_keys(const u64 (&key)[Q], int n, int R,
                                                               lds_u64* out) {
  const int lane = threadIdx.x & 63;
  const u64 lt = (1ull << lane) - 1ull;
  u64 T = 1;  // R >= n: every key is taken
  if (R < n) {
    u64 mx = 0, mn = ~0ull;
#pragma unroll
    for (int v = 0; v < Q; ++v) {
      mx = key[v] > mx ? key[v] : mx;
      const u64 k = key[v] != 0ull ? key[v] : ~0ull;  // 0 pads
      mn = k < mn ? k : mn;
    }
    mx = wave_umax64(mx);
    mn = wave_umin64(mn);
    const int hb = 63 - __clzll(mx ^ mn);  // n > R >= 1 unique keys: mx != mn
    T = hb == 63 ? 0ull : mx & ~((2ull << hb) - 1ull);  // shared prefix, lower bits 0
    for (int bit = hb; bit >= 0; --bit) {
      const u64 cand = T | (1ull << bit);
      int c = 0;
#pragma unroll
      for (int v = 0; v < Q; ++v) c += __popcll(__ballot(key[v] >= cand));
      if (c >= R) {
        T = cand;
        if (c == R) break;
      }
    }
  }
  int base = 0;
#pragma unroll
  for (int v = 0; v < Q; ++v) {
    const bool sel = key[v] >= T && key[v] != 0ull;
    const u64 bs = __ballot(sel);
    const int pos = base + __popcll(bs & lt);
    if (sel && pos < R) out[pos] = key[v];  // exactly R keys qualify
    base += __popcll(bs);
  }
}

// The rank-pair candidates as registers, then their top K into fs.  Lane l
// holds candidates c = l*Q .. l*Q + Q-1 (a contiguous run of the row-major
// rank-pair order): one binary search over the row offsets finds the row of
// its first candidate, and the run advances through the rows by arithmetic
// (row a has min(K_c, floor(K/(a+1))) candidates, at least one), so only
// the row and column keys are read from LDS.  Always inlined: rs, cs and
// off must stay known LDS pointers.  Through a generic pointer the compiler
// may fold a constant part of an index into the instruction offset and
// leave a base below the LDS window, which the hardware faults on.
template <int Q>
__device__ __attribute__((always_inline)) void select_cands_regs(const lds_u64* rs,
                                                                 const lds_u64* cs,
                                                                 const lds_int* off, int Kr,
                                                                 int P, int Kc, int Nc, int K,
                                                                 lds_u64* fs) {
  const int lane = threadIdx.x & 63;
  const int c0 = lane * Q;
  int a = 0;
  if (c0 < P) {
    int hi = Kr - 1;
    while (a < hi) {
      const int mid = (a + hi + 1) >> 1;
      if (off[mid] <= c0) a = mid;
      else hi = mid - 1;
    }
  }
  int cur = c0 < P ? off[a] : 0;  // first candidate of row a
  auto row_count = [&](int r) {   // min(K_c, floor(K / (r + 1))), exact for K < 2^20
    int q = (int)((float)K * __builtin_amdgcn_rcpf((float)(r + 1)));
    q += (q + 1) * (r + 1) <= K;
    q -= q * (r + 1) > K;
    return min(Kc, q);
  };
  int nxt = cur + row_count(a);
  int ra[Q], cb[Q];
#pragma unroll
  for (int v = 0; v < Q; ++v) {
    const int c = c0 + v;
    if (c == nxt && c < P) {  // rows hold at least one candidate: one step at a time
      ++a;
      cur = nxt;
      nxt += row_count(a);
    }
    ra[v] = a;
    cb[v] = c - cur;
  }
  u64 cand[Q];
#pragma unroll
  for (int v = 0; v < Q; ++v) {
    cand[v] = 0ull;
    if (c0 + v < P) {
      const u64 rk = rs[ra[v]], ck = cs[cb[v]];
      cand[v] = make_key(key_val(rk) + key_val(ck), key_idx(rk) * (unsigned)Nc + key_idx(ck));
    }
  }
  select_top_keys<Q>(cand, P, K, fs);
}

__device__ __forceinline__ u64 xor_lane64(u64 v, int j) {
  const int lo = (int)(unsigned)v, hi = (int)(unsigned)(v >> 32);
  int a, b;
  switch (j) {  // j is a compile-time constant after unrolling
    case 1: a = xor_lane<1>(lo); b = xor_lane<1>(hi); break;
    case 2: a = xor_lane<2>(lo); b = xor_lane<2>(hi); break;
    case 4: a = xor_lane<4>(lo); b = xor_lane<4>(hi); break;
    case 8: a = xor_lane<8>(lo); b = xor_lane<8>(hi); break;
    case 16: a = xor_lane<16>(lo); b = xor_lane<16>(hi); break;
    default: a = xor_lane<32>(lo); b = xor_lane<32>(hi); break;
  }
  return ((u64)(unsigned)b << 32) | (u64)(unsigned)a;
}

// Bitonic sort (descending) of 64*V keys held by one wave: element
// e = lane*V + v lives in register k[v] of lane `lane`.  With each lane
// holding V consecutive elements, the exchanges at distances below V stay
// inside a lane (compare and swap two registers) and the others cross lanes
// at distance j / V: the 15 shortest-distance stages of a 256-key sort need
// no lane exchange, and only 3 use the slower swizzle / permute forms
// (measured at K = 256 over 16384 tokens: the row and column sorts 72 -> 63
// us and the final sort with the gates 39 -> 33 us against the lane-minor
// layout, element v*64 + lane).
template <int V>
__device__ void wave_sort_desc(u64 (&k)[V]) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int size = 2; size <= 64 * V; size <<= 1) {
#pragma unroll
    for (int j = size >> 1; j > 0; j >>= 1) {
      if (j < V) {
#pragma unroll
        for (int v = 0; v < V; ++v) {
          if (v & j) continue;
          const bool desc = (((lane * V + v) & size) == 0);
          const u64 a = k[v], b = k[v | j];
          const bool sw = desc ? (a < b) : (a > b);
          k[v] = sw ? b : a;
          k[v | j] = sw ? a : b;
        }
      } else {
        const int jl = j / V;  // partner lane: lane ^ jl, same register
#pragma unroll
        for (int v = 0; v < V; ++v) {
          const bool desc = (((lane * V + v) & size) == 0);
          const u64 o = xor_lane64(k[v], jl);
          const bool lower = (lane & jl) == 0;
          const bool keep_max = lower == desc;
          k[v] = keep_max ? (k[v] > o ? k[v] : o) : (k[v] < o ? k[v] : o);
        }
      }
    }
  }
}

// Sort arr[0..n) (n <= 512) in place, descending.
template <int V>
__device__ void wave_sort_lds_t(lds_u64* arr, int n) {
  const int lane = threadIdx.x & 63;
  u64 k[V];
#pragma unroll
  for (int v = 0; v < V; ++v) k[v] = lane * V + v < n ? arr[lane * V + v] : 0ull;
  wave_sort_desc<V>(k);
#pragma unroll
  for (int v = 0; v < V; ++v)
    if (lane * V + v < n) arr[lane * V + v] = k[v];
}

__device__ void wave_sort_lds(lds_u64* arr, int n) {
  if (n <= 64) wave_sort_lds_t<1>(arr, n);
  else if (n <= 128) wave_sort_lds_t<2>(arr, n);
  else if (n <= 256) wave_sort_lds_t<4>(arr, n);
  else wave_sort_lds_t<8>(arr, n);
}

// Order the K selected candidates, softmax gate, write the token's outputs.
template <int V>
__device__ void emit_topk(const lds_u64* fs, int K, int32_t* idx, float* score, float* gate) {
  const int lane = threadIdx.x & 63;
  u64 k[V];
#pragma unroll
  for (int v = 0; v < V; ++v) k[v] = lane * V + v < K ? fs[lane * V + v] : 0ull;
  wave_sort_desc<V>(k);
  const float s0 = key_val(__shfl(k[0], 0, 64));  // largest score
  float es = 0.f;
  float ev[V];
#pragma unroll
  for (int v = 0; v < V; ++v) {
    ev[v] = lane * V + v < K ? __expf(key_val(k[v]) - s0) : 0.f;
    es += ev[v];
  }
  const float inv = 1.f / wave_sum(es);
#pragma unroll
  for (int v = 0; v < V; ++v) {
    const int e = lane * V + v;  // the element's rank
    if (e < K) {
      idx[e] = (int32_t)key_idx(k[v]);
      score[e] = key_val(k[v]);
      gate[e] = ev[v] * inv;
    }
  }
}

struct TopkLayout {
  int Kr, Kc, P;
  int regq;  // registers per lane holding the candidates, 0: candidates in LDS
  size_t o_rs, o_cs, o_cand, o_fs, o_hist, o_off, bytes;
};

inline TopkLayout topk_layout(int Nr, int Nc, int K) {
  TopkLayout l;
  l.Kr = K < Nr ? K : Nr;
  l.Kc = K < Nc ? K : Nc;
  l.P = pair_count(K, l.Kr, l.Kc);
  // register candidates only in the kernels for grid sides up to 24*64
  // (their row values leave room for them)
  const int q = (l.P + 63) / 64;
  l.regq = (Nr > 24 * 64 || Nc > 24 * 64) ? 0
         : q <= 1 ? 1 : q <= 2 ? 2 : q <= 4 ? 4 : q <= 8 ? 8 : q <= 12 ? 12 : q <= 16 ? 16
         : q <= 24 ? 24 : 0;
  size_t o = 0;
  l.o_rs = o; o += (size_t)l.Kr * 8;
  l.o_cs = o; o += (size_t)l.Kc * 8;
  l.o_cand = o; o += l.regq ? 0 : (size_t)l.P * 8;
  l.o_fs = o; o += (size_t)K * 8;
  l.o_hist = o; o += l.regq ? 0 : 256 * 4;
  l.o_off = o; o += (size_t)(l.Kr + 1) * 4;
  l.bytes = (o + 15) & ~(size_t)15;  // slices of several tokens stay 16-byte aligned
  return l;
}

// Load one logit vector (n <= 64*VPL) and turn it into LogSoftmax values,
// p = s - (max + log sum exp(s - max)), kept as order-preserving words.
template <int VPL>
__device__ __forceinline__ void log_softmax_ord(const float* s, int n, unsigned (&val)[VPL]) {
  const int lane = threadIdx.x & 63;
  float f[VPL];
  float m = -INFINITY;
#pragma unroll
  for (int v = 0; v < VPL; ++v) {
    f[v] = v * 64 + lane < n ? s[v * 64 + lane] : -INFINITY;
    m = fmaxf(m, f[v]);
  }
  m = wave_max(m);
  float e = 0.f;
#pragma unroll
  for (int v = 0; v < VPL; ++v) e += v * 64 + lane < n ? __expf(f[v] - m) : 0.f;
  const float lse = m + logf(wave_sum(e));
#pragma unroll
  for (int v = 0; v < VPL; ++v) val[v] = v * 64 + lane < n ? float_ord(f[v] - lse) : 0u;
}

// One wave per token.
//  1. LogSoftmax of the row and column logits.
//  2. Row pre-selection: the first min(K, N_r) rows under (p_r desc, i asc);
//     columns likewise.  A cell outside these rows or columns has at least
//     K cells before it under (S desc, n asc), so the top K lies inside.
//  3. Candidates: row rank a (0-based) is paired with the first
//     min(K_c, K/(a+1)) columns: a cell at ranks (a, b) has at least
//     (a+1)(b+1) - 1 cells before it, so (a+1)(b+1) <= K is necessary.
//  4. Top K of the candidates under (S desc, n asc); gate = softmax of S.
//     At most 24*64 candidates (K up to about 270) are held in registers,
//     24 per lane, which keeps the LDS slice of a token at 3K keys and lets
//     five tokens share each SIMD; more are staged in LDS.
// Several tokens share a workgroup (one wave each, each with its own LDS
// slice): one-wave workgroups leave most wave slots of a CU empty.
template <int VPL>
__global__ __launch_bounds__(256) void router_topk(const float* __restrict__ logits, int L, int Nr,
                                                   int Nc, int K, const TopkLayout lay, int wpg,
                                                   int32_t* __restrict__ idx,
                                                   float* __restrict__ score,
                                                   float* __restrict__ gate) {
  extern __shared__ __attribute__((aligned(16))) unsigned char smem_all[];
  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  unsigned char* smem = smem_all + (size_t)wv * lay.bytes;
  lds_u64* rs = (lds_u64*)(smem + lay.o_rs);
  lds_u64* cs = (lds_u64*)(smem + lay.o_cs);
  lds_u64* cand = (lds_u64*)(smem + lay.o_cand);
  lds_u64* fs = (lds_u64*)(smem + lay.o_fs);
  lds_int* hist = (lds_int*)(smem + lay.o_hist);
  lds_int* off = (lds_int*)(smem + lay.o_off);
  const int t = blockIdx.x * wpg + wv, lane = threadIdx.x & 63;
  if (t >= L) return;  // whole wave leaves; no workgroup barrier follows
  const float* sr = logits + (size_t)t * (Nr + Nc);

  // 1-2. rows, then columns
  {
    unsigned val[VPL];
    log_softmax_ord<VPL>(sr, Nr, val);
    select_top_regs<VPL>(val, Nr, lay.Kr, rs);
    log_softmax_ord<VPL>(sr + Nr, Nc, val);
    wave_sync();
    select_top_regs<VPL>(val, Nc, lay.Kc, cs);
  }
  wave_sync();
  wave_sort_lds(rs, lay.Kr);
  wave_sort_lds(cs, lay.Kc);
  {
    // exclusive scan of the per-row candidate counts (K_r <= 512)
    const int per = (lay.Kr + 63) / 64;
    const int a0 = lane * per;
    int loc = 0;
    for (int a = a0; a < a0 + per && a < lay.Kr; ++a) loc += min(lay.Kc, K / (a + 1));
    const int inc = wave_incl_scan(loc);
    int run = inc - loc;
    for (int a = a0; a < a0 + per && a < lay.Kr; ++a) {
      off[a] = run;
      run += min(lay.Kc, K / (a + 1));
    }
    if (lane == 63) off[lay.Kr] = inc;
  }
  wave_sync();

  // 3-4. candidate c belongs to the row rank a with off[a] <= c < off[a+1];
  // their top K goes to fs.  Up to 24*64 candidates stay in registers
  // (bit search by ballots); more are staged in LDS (radix select).
  switch (VPL <= 24 ? lay.regq : 0) {
    case 1: select_cands_regs<1>(rs, cs, off, lay.Kr, lay.P, lay.Kc, Nc, K, fs); break;
    case 2: select_cands_regs<2>(rs, cs, off, lay.Kr, lay.P, lay.Kc, Nc, K, fs); break;
    case 4: select_cands_regs<4>(rs, cs, off, lay.Kr, lay.P, lay.Kc, Nc, K, fs); break;
    case 8: select_cands_regs<8>(rs, cs, off, lay.Kr, lay.P, lay.Kc, Nc, K, fs); break;
    case 12: select_cands_regs<12>(rs, cs, off, lay.Kr, lay.P, lay.Kc, Nc, K, fs); break;
    case 16: select_cands_regs<16>(rs, cs, off, lay.Kr, lay.P, lay.Kc, Nc, K, fs); break;
    case 24: select_cands_regs<24>(rs, cs, off, lay.Kr, lay.P, lay.Kc, Nc, K, fs); break;
    default: {
      for (int c = lane; c < lay.P; c += 64) {
        int lo = 0, hi = lay.Kr - 1;
        while (lo < hi) {
          const int mid = (lo + hi + 1) >> 1;
          if (off[mid] <= c) lo = mid;
          else hi = mid - 1;
        }
        const u64 rk = rs[lo], ck = cs[c - off[lo]];
        cand[c] = make_key(key_val(rk) + key_val(ck), key_idx(rk) * (unsigned)Nc + key_idx(ck));
      }
      wave_sync();
      select_top_lds(cand, lay.P, K, hist, fs);
    }
  }
  wave_sync();
  int32_t* io = idx + (size_t)t * K;
  float* so = score + (size_t)t * K;
  float* go = gate + (size_t)t * K;
  if (K <= 64) emit_topk<1>(fs, K, io, so, go);
  else if (K <= 128) emit_topk<2>(fs, K, io, so, go);
  else if (K <= 256) emit_topk<4>(fs, K, io, so, go);
  else emit_topk<8>(fs, K, io, so, go);
}

}  // namespace

hipError_t launch_router_gemm(const void* x, const void* Wr, const void* Wc, int L, int d,
                              int Nr, int Nc, omni_dtype dt, float* logits, hipStream_t s) {
  const int Ntot = Nr + Nc;
  if (dt == OMNI_BF16 && d % GEMM_KTILE == 0) {
    return launch_gemm_bt_bf16(x, Wr, Wc, Nr, L, Ntot, d, logits, logits, L, Ntot, false, s);
  } else if (dt == OMNI_BF16) {  // d not a multiple of BK: zero-filled partial k-tile
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

size_t router_topk_lds_bytes(int Nr, int Nc, int K) { return topk_layout(Nr, Nc, K).bytes; }


// Two waves per token: waves 2j (rows) and 2j + 1 (columns) of a workgroup
// run LogSoftmax, pre-selection and key sort of their half side by side;
// after one barrier the row wave takes the candidates, their selection and
// the final sort.  Register-candidate form only, for the shapes instantiated
// in the launcher (the others keep one wave per token).  A token's chain of
// dependent steps loses one half's LogSoftmax, search and sort; the
// instructions are the same, so it pays where the SIMDs are not full: the router call (projection and
// top-K) at 4096 tokens 124.4 -> 121.2 us at 1.7M experts and 86.9 -> 83.5 us
// at 1M, 61.4 -> 60.5 us at 280,900, 460 -> 460 us at 16384 tokens x K = 256;
// the same ids, scores and gates.
template <int VPL, int Q>
__global__ __launch_bounds__(256) void router_topk_pair(const float* __restrict__ logits, int L,
                                                        int Nr, int Nc, int K, const TopkLayout lay,
                                                        int32_t* __restrict__ idx,
                                                        float* __restrict__ score,
                                                        float* __restrict__ gate) {
  extern __shared__ __attribute__((aligned(16))) unsigned char smem_all[];
  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int slot = wv >> 1, role = wv & 1;
  unsigned char* smem = smem_all + (size_t)slot * lay.bytes;
  lds_u64* rs = (lds_u64*)(smem + lay.o_rs);
  lds_u64* cs = (lds_u64*)(smem + lay.o_cs);
  lds_u64* fs = (lds_u64*)(smem + lay.o_fs);
  lds_int* off = (lds_int*)(smem + lay.o_off);
  const int t = blockIdx.x * 2 + slot, lane = threadIdx.x & 63;
  const bool live = t < L;
  if (live) {
    const float* src = logits + (size_t)t * (Nr + Nc) + (role ? Nr : 0);
    const int n = role ? Nc : Nr;
    const int R = role ? lay.Kc : lay.Kr;
    lds_u64* out = role ? cs : rs;
    unsigned val[VPL];
    log_softmax_ord<VPL>(src, n, val);
    select_top_regs<VPL>(val, n, R, out);
    wave_sync();
    wave_sort_lds(out, R);
  }
  __syncthreads();  // every wave of the workgroup reaches it once
  if (!live || role) return;
  {
    const int per = (lay.Kr + 63) / 64;
    const int a0 = lane * per;
    int loc = 0;
    for (int a = a0; a < a0 + per && a < lay.Kr; ++a) loc += min(lay.Kc, K / (a + 1));
    const int inc = wave_incl_scan(loc);
    int run = inc - loc;
    for (int a = a0; a < a0 + per && a < lay.Kr; ++a) {
      off[a] = run;
      run += min(lay.Kc, K / (a + 1));
    }
    if (lane == 63) off[lay.Kr] = inc;
  }
  wave_sync();
  select_cands_regs<Q>(rs, cs, off, lay.Kr, lay.P, lay.Kc, Nc, K, fs);
  wave_sync();
  int32_t* io = idx + (size_t)t * K;
  float* so = score + (size_t)t * K;
  float* go = gate + (size_t)t * K;
  if (K <= 64) emit_topk<1>(fs, K, io, so, go);
  else if (K <= 128) emit_topk<2>(fs, K, io, so, go);
  else if (K <= 256) emit_topk<4>(fs, K, io, so, go);
  else emit_topk<8>(fs, K, io, so, go);
}

hipError_t launch_router_topk(const float* logits, int L, int Nr, int Nc, int K, int32_t* idx,
                              float* score, float* gate, hipStream_t s) {
  const TopkLayout lay = topk_layout(Nr, Nc, K);
  const int need = (max(Nr, Nc) + 63) / 64;  // values per lane
  // per token 3K keys (rows, columns, the selected K) and the row offsets,
  // plus the candidates (at most K*(1 + H(K)) keys) when they do not fit in
  // registers: under 42 KB for K <= 512; up to four tokens share a
  // workgroup within the default 64 KB of dynamic LDS
  const size_t lds = lay.bytes;
  const int wpg = lds * 4 <= 65536 ? 4 : lds * 2 <= 65536 ? 2 : 1;
  if (lay.regq && need <= 24 && lds * 2 <= 65536) {
#define OMNI_TOPK_PAIR(V, QQ)                                                                   \
    if (need <= V && lay.regq == QQ) {                                                          \
      hipLaunchKernelGGL((router_topk_pair<V, QQ>), dim3((L + 1) / 2), dim3(256), lds * 2, s,    \
                         logits, L, Nr, Nc, K, lay, idx, score, gate);                          \
      return hipGetLastError();                                                                 \
    }
    OMNI_TOPK_PAIR(9, 8) OMNI_TOPK_PAIR(9, 12) OMNI_TOPK_PAIR(16, 12) OMNI_TOPK_PAIR(16, 24)
    OMNI_TOPK_PAIR(21, 12) OMNI_TOPK_PAIR(21, 24)
#undef OMNI_TOPK_PAIR
  }
#define OMNI_TOPK(V)                                                                           \
  if (need <= V) {                                                                             \
    hipLaunchKernelGGL(router_topk<V>, dim3((L + wpg - 1) / wpg), dim3(64 * wpg), lds * wpg, s, \
                       logits, L, Nr, Nc, K, lay, wpg, idx, score, gate);                     \
    return hipGetLastError();                                                                  \
  }
  OMNI_TOPK(1) OMNI_TOPK(2) OMNI_TOPK(4) OMNI_TOPK(8) OMNI_TOPK(9) OMNI_TOPK(12) OMNI_TOPK(16)
  OMNI_TOPK(21) OMNI_TOPK(24)
  OMNI_TOPK(32) OMNI_TOPK(48) OMNI_TOPK(64)
#undef OMNI_TOPK
  return hipErrorInvalidValue;  // N_r, N_c above 4096 are rejected before launch
}

}  // namespace omni
