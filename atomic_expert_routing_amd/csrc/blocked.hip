// Blocked expert assembly on gfx950: the dense form of the assembly for
// routing where many tokens share their experts.
//
// The assembly is O_q = (G_q . sigma(X_q W_q^T)) V_q per group of experts
// (OmniMoE digest, paper.rainbus.top, method paragraph, step 3; gist.science
// resume section 2.1), evaluated here with the grouping turned around: the
// tokens are cut into blocks of BLK_TOKENS consecutive entries of a token
// order (the schedule's order puts tokens that lead with the same experts
// together), and block b's group is the union U_b of the experts its tokens
// use.  With X_b the block's token rows and G_b[r][c] the gate of token r for
// expert U_b[c] (no task: the product is masked to zero),
//
//   y[t_r] = sum_c (G_b . SiLU(X_b W[U_b]^T))[r][c] V[U_b[c]]
//
// which is the definition y_t = sum_k g_tk SiLU(x_t . w_e) v_e with each
// token's K terms found among the block's columns.  Both products are dense
// MFMA tiles: each weight row of the union is read once per block and used
// by every token of the block, and y's rows are written by the block that
// owns them (no atomics, deterministic).  Kernels, in stream order:
//
//   blk_union  per block: the union (LDS bitonic sort of the block's ids,
//              then unique) and each task's column in it
//   blk_plan   one workgroup: prefix sums of the blocks' column tiles
//   blk_gates  per block: the dense gate tile G_b (no-task entries marked)
//   blk_act    A_b = G_b . SiLU(X_b W[U_b]^T), 64 x 128 MFMA tiles,
//              written as two bf16 terms hi + lo (about 16 significant bits)
//   blk_out    y_b = (A_hi + A_lo) V[U_b], 64 x 256 MFMA tiles; the V rows
//              pass through LDS, where the k-major operand is read transposed

#include <algorithm>
#include <climits>

#include "mfma_pipe.h"

namespace omni {
namespace {

constexpr int BT = BLK_TOKENS;               // tokens per block (MFMA tile rows)
constexpr int UPAD = BLK_UNION_TILE;         // union padded to whole column tiles
constexpr int TILE_ELEMS = BT * UPAD;        // G / A elements per column tile
constexpr unsigned NOTASK = 0xffffffffu;     // G entry of a pair that is no task

// Token of slot s of the order, or -1 past L or for an entry outside [0, L).
__device__ __forceinline__ int slot_token(const int32_t* __restrict__ order, int s, int L) {
  if (s >= L) return -1;
  const int t = order[s];
  return (unsigned)t < (unsigned)L ? t : -1;
}

// ------------------------------------------------------------------ blk_union
// One 1024-thread workgroup per block; P = 1024 * E >= BLK_TOKENS * K keys in
// LDS (padding and empty rows hold INT_MAX, above every expert id).
template <int E>
__global__ __launch_bounds__(1024) void blk_union(const int32_t* __restrict__ idx,
                                                  const int32_t* __restrict__ order, int L, int K,
                                                  int ucap, int32_t* __restrict__ U,
                                                  int32_t* __restrict__ nU,
                                                  int32_t* __restrict__ colmap) {
  extern __shared__ int keys[];
  __shared__ int wtot[16];
  constexpr int P = 1024 * E;
  const int b = blockIdx.x, tid = threadIdx.x;
  const int nt = BT * K;
  for (int i = tid; i < P; i += 1024) {
    int key = INT_MAX;
    if (i < nt) {
      const int r = i / K;
      const int t = slot_token(order, b * BT + r, L);
      if (t >= 0) key = idx[(size_t)t * K + (i - r * K)];
    }
    keys[i] = key;
  }
  __syncthreads();
  // bitonic sort, ascending
  for (int size = 2; size <= P; size <<= 1) {
    for (int stride = size >> 1; stride > 0; stride >>= 1) {
      for (int p = tid; p < P / 2; p += 1024) {
        const int i = 2 * p - (p & (stride - 1)), j = i + stride;
        const int a = keys[i], c = keys[j];
        if ((a > c) == ((i & size) == 0)) {
          keys[i] = c;
          keys[j] = a;
        }
      }
      __syncthreads();
    }
  }
  // unique: thread tid owns the sorted positions [tid*E, tid*E + E)
  int v[E];
  unsigned long long first = 0;
  int cnt = 0;
#pragma unroll
  for (int q = 0; q < E; ++q) {
    const int i = tid * E + q;
    v[q] = keys[i];
    const bool f = v[q] != INT_MAX && (i == 0 || keys[i - 1] != v[q]);
    first |= (unsigned long long)f << q;
    cnt += f;
  }
  const int inc = wave_incl_scan(cnt);
  if ((tid & 63) == 63) wtot[tid >> 6] = inc;
  __syncthreads();  // every key has been read: the front of the array is free
  int pos = inc - cnt, n = 0;
#pragma unroll
  for (int w = 0; w < 16; ++w) {
    pos += w < (tid >> 6) ? wtot[w] : 0;
    n += wtot[w];
  }
#pragma unroll
  for (int q = 0; q < E; ++q)
    if ((first >> q) & 1) keys[pos++] = v[q];
  __syncthreads();
  // n >= 1 when the block holds a token; a block with none gets an empty
  // union of one padding column (id 0), all of whose gates are masked
  const int npad = max(1, (n + UPAD - 1) / UPAD) * UPAD;
  int32_t* Ub = U + (size_t)b * ucap;
  for (int c = tid; c < npad; c += 1024) Ub[c] = n ? keys[min(c, n - 1)] : 0;
  if (tid == 0) nU[b] = n;
  for (int i = tid; i < nt; i += 1024) {
    const int r = i / K;
    const int t = slot_token(order, b * BT + r, L);
    if (t < 0) continue;
    const int e = idx[(size_t)t * K + (i - r * K)];
    int lo = 0, hi = n - 1;  // e is in the union: find its position
    while (lo < hi) {
      const int mid = (lo + hi) >> 1;
      if (keys[mid] < e) lo = mid + 1;
      else hi = mid;
    }
    colmap[(size_t)b * nt + i] = lo;
  }
}

// ------------------------------------------------------------------ blk_plan
// toff[b] = column tiles of the blocks before b (toff[nb] = all tiles): block
// b's G and A tiles start at element toff[b] * TILE_ELEMS.
__global__ __launch_bounds__(1024) void blk_plan(const int32_t* __restrict__ nU, int nb,
                                                 int32_t* __restrict__ toff) {
  __shared__ int wtot[16];
  const int tid = threadIdx.x;
  int carry = 0;
  for (int base = 0; base < nb; base += 1024) {
    const int b = base + tid;
    const int tiles = b < nb ? max(1, (nU[b] + UPAD - 1) / UPAD) : 0;
    const int inc = wave_incl_scan(tiles);
    if ((tid & 63) == 63) wtot[tid >> 6] = inc;
    __syncthreads();
    int off = inc - tiles, tot = 0;
#pragma unroll
    for (int w = 0; w < 16; ++w) {
      off += w < (tid >> 6) ? wtot[w] : 0;
      tot += wtot[w];
    }
    if (b < nb) toff[b] = carry + off;
    carry += tot;
    __syncthreads();
  }
  if (tid == 0) toff[nb] = carry;
}

// ------------------------------------------------------------------ blk_gates
__global__ __launch_bounds__(256) void blk_gates(const float* __restrict__ gate,
                                                 const int32_t* __restrict__ order,
                                                 const int32_t* __restrict__ colmap,
                                                 const int32_t* __restrict__ toff, int L, int K,
                                                 float* __restrict__ G) {
  const int b = blockIdx.x, tid = threadIdx.x;
  const int tiles = toff[b + 1] - toff[b];
  const int npad = tiles * UPAD;
  uint32_t* Gb = (uint32_t*)G + (size_t)toff[b] * TILE_ELEMS;
  const int n4 = tiles * (TILE_ELEMS / 4);
  for (int i = tid; i < n4; i += 256) ((u32x4*)Gb)[i] = u32x4{NOTASK, NOTASK, NOTASK, NOTASK};
  __syncthreads();  // the fill is complete before the gates land on it
  const int nt = BT * K;
  for (int i = tid; i < nt; i += 256) {
    const int r = i / K;
    const int t = slot_token(order, b * BT + r, L);
    if (t < 0) continue;
    Gb[r * npad + colmap[(size_t)b * nt + i]] = __float_as_uint(gate[(size_t)t * K + (i - r * K)]);
  }
}

// Block of column tile T: toff[b] <= T < toff[b+1] (toff strictly increasing).
__device__ __forceinline__ int tile_block(const int32_t* __restrict__ toff, int nb, int T) {
  int lo = 0, hi = nb - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (toff[mid] <= T) lo = mid;
    else hi = mid - 1;
  }
  return lo;
}

// ------------------------------------------------------------------ blk_act
// Persistent: workgroup w takes column tiles w, w + grid, ...  A tile is the
// block's 64 token rows x 128 union rows, k-tiles of 64 streamed through two
// LDS stages by direct loads (as in gemm_bt_bf16_pipe); 4 waves of 64 x 32.
constexpr int K1_BK = 64, K1_S = 2;
constexpr int K1_MI = 4, K1_NJ = 2, K1_WAVES = 4;
constexpr int K1_ROWB = 2 * K1_BK;               // 128 bytes per LDS row
constexpr int K1_TILEA = BT * K1_ROWB;           // 8 KB
constexpr int K1_TILEB = UPAD * K1_ROWB;         // 16 KB
constexpr int K1_STAGE = K1_TILEA + K1_TILEB;
constexpr int K1_LPWA = K1_TILEA / 1024 / K1_WAVES;  // 2 loads per wave per k-tile
constexpr int K1_LPWB = K1_TILEB / 1024 / K1_WAVES;  // 4
constexpr int K1_CPR = K1_ROWB / 16;                 // 8 chunks per row
constexpr int K1_RPI = 64 / K1_CPR;                  // 8 rows per load instruction
static_assert(BT == 16 * K1_MI && UPAD == 16 * K1_NJ * K1_WAVES, "tile shape");

__device__ __forceinline__ uint16_t bf16_rne(float f) {
  return __builtin_bit_cast(uint16_t, (__bf16)f);
}

__global__ __launch_bounds__(256) void blk_act(const uint16_t* __restrict__ x,
                                               const uint16_t* __restrict__ W,
                                               const int32_t* __restrict__ order,
                                               const int32_t* __restrict__ U,
                                               const int32_t* __restrict__ toff,
                                               const float* __restrict__ G, int L, int d, int nb,
                                               int ucap, uint16_t* __restrict__ Ahi,
                                               uint16_t* __restrict__ Alo) {
  extern __shared__ __attribute__((aligned(16))) unsigned char sm1[];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int total = toff[nb];
  const int nk = d / K1_BK;
  for (int T = blockIdx.x; T < total; T += gridDim.x) {
    const int b = tile_block(toff, nb, T);
    const int j = T - toff[b];
    const int npad = (toff[b + 1] - toff[b]) * UPAD;
    const int32_t* Ub = U + (size_t)b * ucap + j * UPAD;
    const uint16_t* asrc[K1_LPWA];
    const uint16_t* bsrc[K1_LPWB];
#pragma unroll
    for (int q = 0; q < K1_LPWA; ++q) {
      const int r = (wave * K1_LPWA + q) * K1_RPI + lane / K1_CPR;
      const int chunk = (lane % K1_CPR) ^ chunk_swz<K1_BK>(r);
      const int t = slot_token(order, b * BT + r, L);
      asrc[q] = x + (size_t)(t < 0 ? 0 : t) * d + chunk * 8;  // empty rows: any row, masked
    }
#pragma unroll
    for (int q = 0; q < K1_LPWB; ++q) {
      const int r = (wave * K1_LPWB + q) * K1_RPI + lane / K1_CPR;
      const int chunk = (lane % K1_CPR) ^ chunk_swz<K1_BK>(r);
      bsrc[q] = W + (size_t)Ub[r] * d + chunk * 8;
    }
    auto issue = [&](int kt) {
      unsigned char* st = sm1 + (kt % K1_S) * K1_STAGE;
      const int k0 = kt * K1_BK;
#pragma unroll
      for (int q = 0; q < K1_LPWA; ++q)
        __builtin_amdgcn_global_load_lds((const void*)(asrc[q] + k0),
                                         (lds_void*)(st + (wave * K1_LPWA + q) * 1024), 16, 0, 0);
#pragma unroll
      for (int q = 0; q < K1_LPWB; ++q)
        __builtin_amdgcn_global_load_lds(
            (const void*)(bsrc[q] + k0),
            (lds_void*)(st + K1_TILEA + (wave * K1_LPWB + q) * 1024), 16, 0, 0);
    };
    f32x4 acc[K1_MI][K1_NJ];
#pragma unroll
    for (int i = 0; i < K1_MI; ++i)
#pragma unroll
      for (int q = 0; q < K1_NJ; ++q) acc[i][q] = f32x4{0.f, 0.f, 0.f, 0.f};
    const int wn = wave * 16 * K1_NJ;
    auto load_frags = [&](const unsigned char* st, int ks, bf16x8* af, bf16x8* bfr) {
      const int kc = ks * 4 + (lane >> 4);
#pragma unroll
      for (int i = 0; i < K1_MI; ++i) {
        const int r = i * 16 + (lane & 15);
        af[i] = *(const bf16x8*)(st + r * K1_ROWB + ((kc ^ chunk_swz<K1_BK>(r)) << 4));
      }
#pragma unroll
      for (int q = 0; q < K1_NJ; ++q) {
        const int r = wn + q * 16 + (lane & 15);
        bfr[q] = *(const bf16x8*)(st + K1_TILEA + r * K1_ROWB + ((kc ^ chunk_swz<K1_BK>(r)) << 4));
      }
    };
    issue(0);
    for (int kt = 0; kt < nk; ++kt) {
      wait_vm_imm<0>();   // tile kt landed (for this wave's loads) ...
      block_sync_lds();   // ... and for every wave; tile kt-1's stage is free
      if (kt + 1 < nk) issue(kt + 1);
      const unsigned char* st = sm1 + (kt % K1_S) * K1_STAGE;
      bf16x8 af[2][K1_MI], bfr[2][K1_NJ];
      load_frags(st, 0, af[0], bfr[0]);
#pragma unroll
      for (int ks = 0; ks < K1_BK / 32; ++ks) {
        if (ks + 1 < K1_BK / 32) load_frags(st, ks + 1, af[(ks + 1) & 1], bfr[(ks + 1) & 1]);
#pragma unroll
        for (int i = 0; i < K1_MI; ++i)
#pragma unroll
          for (int q = 0; q < K1_NJ; ++q)
            acc[i][q] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[ks & 1][i], bfr[ks & 1][q],
                                                                acc[i][q], 0, 0, 0);
      }
    }
    // epilogue: a = g * SiLU(h) where (r, c) is a task, else 0; a = hi + lo
    const size_t go = (size_t)toff[b] * TILE_ELEMS;
    const uint32_t* Gb = (const uint32_t*)G + go;
#pragma unroll
    for (int i = 0; i < K1_MI; ++i)
#pragma unroll
      for (int q = 0; q < K1_NJ; ++q)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int r = i * 16 + 4 * (lane >> 4) + e;
          const int c = j * UPAD + wn + q * 16 + (lane & 15);
          const size_t o = (size_t)r * npad + c;
          const uint32_t gb = Gb[o];
          const float h = acc[i][q][e];
          const float a = gb == NOTASK ? 0.f : __uint_as_float(gb) * (h / (1.f + expf(-h)));
          const uint16_t hi = bf16_rne(a);
          Ahi[go + o] = hi;
          Alo[go + o] = bf16_rne(a - __uint_as_float((uint32_t)hi << 16));
        }
    block_sync_lds();  // every wave is done with the stages before the next tile refills them
  }
}

// ------------------------------------------------------------------ blk_out
// Workgroup (b, jt): y rows of block b, columns [256 jt, 256 jt + 256); 4
// waves of 64 x 64.  Per k-tile of 32 union rows, the V slice (32 x 256 bf16)
// lands in LDS row-major by direct loads, 16-byte chunk g of row R in slot
// g ^ ((R >> 3) & 3); the B operand (8 consecutive rows of one column per
// lane) is gathered with 2-byte LDS reads, which the slot rotation spreads
// over distinct banks.  The A fragments (hi and lo) come straight from
// global memory.  Double-buffered with a full wait per k-tile.
constexpr int K2_COLS = BLK_D_TILE, K2_KT = 32, K2_ROWB = 2 * K2_COLS;  // 512-byte LDS rows
constexpr int K2_STAGE = K2_KT * K2_ROWB;                      // 16 KB

__global__ __launch_bounds__(256) void blk_out(const uint16_t* __restrict__ V,
                                               const int32_t* __restrict__ order,
                                               const int32_t* __restrict__ U,
                                               const int32_t* __restrict__ toff,
                                               const uint16_t* __restrict__ Ahi,
                                               const uint16_t* __restrict__ Alo, int L, int d,
                                               int ucap, float* __restrict__ y) {
  extern __shared__ __attribute__((aligned(16))) unsigned char sm2[];
  const int tiles_y = d / K2_COLS;
  const int b = blockIdx.x / tiles_y, c0 = (blockIdx.x % tiles_y) * K2_COLS;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int npad = (toff[b + 1] - toff[b]) * UPAD;
  const int nk = npad / K2_KT;
  const size_t go = (size_t)toff[b] * TILE_ELEMS;
  const uint16_t* Ah = Ahi + go;
  const uint16_t* Al = Alo + go;
  const int32_t* Ub = U + (size_t)b * ucap;
  // V loads: wave w, load q covers LDS rows 2(4w+q) and 2(4w+q)+1
  int rowv[4], slotg[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    rowv[q] = 2 * (4 * wave + q) + (lane >> 5);
    slotg[q] = (lane & 31) ^ ((rowv[q] >> 3) & 3);  // global chunk held by this lane's slot
  }
  auto load_ids = [&](int kt, int* e) {
#pragma unroll
    for (int q = 0; q < 4; ++q) e[q] = Ub[kt * K2_KT + rowv[q]];
  };
  auto issue_v = [&](int kt, const int* e) {
    unsigned char* st = sm2 + (kt & 1) * K2_STAGE;
#pragma unroll
    for (int q = 0; q < 4; ++q)
      __builtin_amdgcn_global_load_lds((const void*)(V + (size_t)e[q] * d + c0 + slotg[q] * 8),
                                       (lds_void*)(st + (4 * wave + q) * 1024), 16, 0, 0);
  };
  auto load_a = [&](int kt, bf16x8* ah, bf16x8* al) {
    const int k = kt * K2_KT + 8 * (lane >> 4);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const size_t o = (size_t)(i * 16 + (lane & 15)) * npad + k;
      ah[i] = *(const bf16x8*)(Ah + o);
      al[i] = *(const bf16x8*)(Al + o);
    }
  };
  f32x4 acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int q = 0; q < 4; ++q) acc[i][q] = f32x4{0.f, 0.f, 0.f, 0.f};
  int ecur[4], enext[4];
  bf16x8 ah0[4], al0[4], ah1[4], al1[4];
  load_ids(0, ecur);
  issue_v(0, ecur);
  load_a(0, ah0, al0);
  if (nk > 1) load_ids(1, enext);
  const int kq = lane >> 4;  // k rows 8 kq .. 8 kq + 7 of a fragment
  // one k-tile: wait for it, start the next one's loads, multiply; the two
  // register buffers of A alternate between calls (fixed at compile time)
  auto step = [&](int kt, const bf16x8* ah, const bf16x8* al, bf16x8* ah_n, bf16x8* al_n) {
    wait_vm_imm<0>();
    block_sync_lds();
    if (kt + 1 < nk) {
      issue_v(kt + 1, enext);
      load_a(kt + 1, ah_n, al_n);
      if (kt + 2 < nk) load_ids(kt + 2, enext);
    }
    const unsigned char* st = sm2 + (kt & 1) * K2_STAGE;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int col = wave * 64 + q * 16 + (lane & 15);
      const unsigned char* p = st + (((col >> 3) ^ kq) << 4) + ((col & 7) << 1);
      bf16x8 vb;
#pragma unroll
      for (int e = 0; e < 8; ++e)
        vb[e] = __builtin_bit_cast(__bf16, *(const uint16_t*)(p + (8 * kq + e) * K2_ROWB));
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        acc[i][q] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ah[i], vb, acc[i][q], 0, 0, 0);
        acc[i][q] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(al[i], vb, acc[i][q], 0, 0, 0);
      }
    }
  };
  for (int kt = 0; kt < nk; kt += 2) {
    step(kt, ah0, al0, ah1, al1);
    if (kt + 1 < nk) step(kt + 1, ah1, al1, ah0, al0);
  }
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int r = i * 16 + 4 * (lane >> 4) + e;
      const int t = slot_token(order, b * BT + r, L);
      if (t < 0) continue;
      float* yr = y + (size_t)t * d + c0 + wave * 64 + (lane & 15);
#pragma unroll
      for (int q = 0; q < 4; ++q) yr[q * 16] = acc[i][q][e];
    }
}

constexpr int MI355X_CUS = 256;
constexpr int K1_WG_PER_CU = 3;  // 48 KB of LDS each

}  // namespace

BlockedPlan plan_blocked(int64_t L, int64_t K, int64_t N) {
  BlockedPlan p{};
  p.nb = (int)((L + BT - 1) / BT);
  const int64_t nt = BT * K;
  p.ucap = (int)(((std::min<int64_t>(nt, N) + UPAD - 1) / UPAD) * UPAD);
  int P = 1024;
  while (P < nt) P <<= 1;
  p.sort_keys = P;
  auto a256 = [](size_t n) { return (n + 255) & ~(size_t)255; };
  size_t o = 0;
  p.off_U = o;      o += a256((size_t)p.nb * p.ucap * 4);
  p.off_nU = o;     o += a256((size_t)p.nb * 4);
  p.off_col = o;    o += a256((size_t)p.nb * nt * 4);
  p.off_toff = o;   o += a256((size_t)(p.nb + 1) * 4);
  const size_t elems = (size_t)p.nb * BT * p.ucap;  // every block at its largest union
  p.off_G = o;      o += a256(elems * 4);
  p.off_Ahi = o;    o += a256(elems * 2);
  p.off_Alo = o;    o += a256(elems * 2);
  p.ws_bytes = o;
  return p;
}

hipError_t launch_expert_blocked(const void* x, const void* W, const void* V, const int32_t* idx,
                                 const float* gate, const int32_t* order, int L, int d, int K,
                                 float* y, const BlockedPlan& p, void* ws, hipStream_t s) {
  char* w = (char*)ws;
  int32_t* U = (int32_t*)(w + p.off_U);
  int32_t* nU = (int32_t*)(w + p.off_nU);
  int32_t* col = (int32_t*)(w + p.off_col);
  int32_t* toff = (int32_t*)(w + p.off_toff);
  float* G = (float*)(w + p.off_G);
  uint16_t* Ahi = (uint16_t*)(w + p.off_Ahi);
  uint16_t* Alo = (uint16_t*)(w + p.off_Alo);
  const size_t lds_u = (size_t)p.sort_keys * 4;
  switch (p.sort_keys / 1024) {
#define OMNI_BLK_UNION(E)                                                                     \
  case E:                                                                                     \
    hipLaunchKernelGGL(blk_union<E>, dim3(p.nb), dim3(1024), lds_u, s, idx, order, L, K,    \
                       p.ucap, U, nU, col);                                                   \
    break;
    OMNI_BLK_UNION(1) OMNI_BLK_UNION(2) OMNI_BLK_UNION(4) OMNI_BLK_UNION(8) OMNI_BLK_UNION(16)
    OMNI_BLK_UNION(32)
#undef OMNI_BLK_UNION
    default:
      return hipErrorInvalidValue;  // K above the validated limit
  }
  hipLaunchKernelGGL(blk_plan, dim3(1), dim3(1024), 0, s, nU, p.nb, toff);
  hipLaunchKernelGGL(blk_gates, dim3(p.nb), dim3(256), 0, s, gate, order, col, toff, L, K, G);
  const int max_tiles = p.nb * (p.ucap / UPAD);
  const int k1_grid = std::min(max_tiles, MI355X_CUS * K1_WG_PER_CU);
  hipLaunchKernelGGL(blk_act, dim3(k1_grid), dim3(256), K1_S * K1_STAGE, s,
                     (const uint16_t*)x, (const uint16_t*)W, order, U, toff, G, L, d, p.nb, p.ucap,
                     Ahi, Alo);
  hipLaunchKernelGGL(blk_out, dim3(p.nb * (d / K2_COLS)), dim3(256), 2 * K2_STAGE, s,
                     (const uint16_t*)V, order, U, toff, Ahi, Alo, L, d, p.ucap, y);
  return hipGetLastError();
}

}  // namespace omni
