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
//              then unique) and the dense gate tile G_b, no-task entries
//              marked, each task's gate at its id's position in the union
//   blk_plan   one workgroup: prefix sums of the blocks' column tiles
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
constexpr unsigned NOTASK = 0xffffffffu;     // G entry of a pair that is no task

// Token of slot s of the order, or -1 past L or for an entry outside [0, L).
__device__ __forceinline__ int slot_token(const int32_t* __restrict__ order, int s, int L) {
  if (s >= L) return -1;
  const int t = order[s];
  return (unsigned)t < (unsigned)L ? t : -1;
}

// ------------------------------------------------------------------ blk_union
// Bitonic sort (ascending) of P = 1024 * E keys, thread t holding positions
// [tE, tE + E) in v.  Compare-exchange partners at stride s sit in the same
// thread for s < E (registers), in lane ^ (s / E) of the same wave for
// E <= s < 64 E (lane exchanges, no barrier), and in another wave only for
// s >= 64 E (through LDS, two barriers).
// Compare-exchange of positions q and q ^ st (q < q ^ st), ascending if up.
template <int E>
__device__ __forceinline__ void cas(int (&v)[E], int q, int j, bool up) {
  const int a = v[q], c = v[j];
  const bool sw = (a > c) == up;
  v[q] = sw ? c : a;
  v[j] = sw ? a : c;
}

// Network sizes 2 .. E, all inside the thread: runs of E sorted, run t
// ascending when bit E of its first position is clear.
template <int E>
__device__ __forceinline__ void sort_runs(int (&v)[E], int tid) {
#pragma unroll
  for (int size = 2; size <= E; size <<= 1)
#pragma unroll
    for (int st = size >> 1; st > 0; st >>= 1)
#pragma unroll
      for (int q = 0; q < E; ++q)
        if ((q ^ st) > q) cas<E>(v, q, q ^ st, ((tid * E + q) & size) == 0);
}

// Strides E/2 .. 1 of a network size above E (one direction per thread).
template <int E>
__device__ __forceinline__ void merge_in_thread(int (&v)[E], bool up) {
#pragma unroll
  for (int st = E >> 1; st > 0; st >>= 1)
#pragma unroll
    for (int q = 0; q < E; ++q)
      if ((q ^ st) > q) cas<E>(v, q, q ^ st, up);
}

// Stride D * E: each position's partner is the same position of lane ^ D.
template <int E, int D>
__device__ __forceinline__ void exchange_lanes(int (&v)[E], bool up, int lane) {
  const bool lower = (lane & D) == 0;
#pragma unroll
  for (int q = 0; q < E; ++q) {
    const int o = xor_lane<D>(v[q]);
    v[q] = (lower == up) ? min(v[q], o) : max(v[q], o);
  }
}

// LDS word of sorted position i: one pad word after every E positions, so
// that the 64 lanes' runs (E words apart otherwise) fall in distinct banks.
template <int E>
__device__ __forceinline__ int padded(int i) {
  return i + i / E;
}

template <int E>
__device__ void bitonic_sort(int* keys, int (&v)[E], int tid) {
  constexpr int P = 1024 * E;
  const int lane = tid & 63;
  sort_runs<E>(v, tid);
  for (int size = 2 * E; size <= P; size <<= 1) {
    const bool up = ((tid * E) & size) == 0;
    for (int st = size >> 1; st >= 64 * E; st >>= 1) {  // across waves
#pragma unroll
      for (int q = 0; q < E; ++q) keys[padded<E>(tid * E + q)] = v[q];
      __syncthreads();
      const bool lower = ((tid * E) & st) == 0;
#pragma unroll
      for (int q = 0; q < E; ++q) {
        const int o = keys[padded<E>((tid * E + q) ^ st)];
        v[q] = (lower == up) ? min(v[q], o) : max(v[q], o);
      }
      __syncthreads();
    }
    for (int st = min(size >> 1, 32 * E); st >= E; st >>= 1) {  // inside the wave
      switch (st / E) {
        case 1: exchange_lanes<E, 1>(v, up, lane); break;
        case 2: exchange_lanes<E, 2>(v, up, lane); break;
        case 4: exchange_lanes<E, 4>(v, up, lane); break;
        case 8: exchange_lanes<E, 8>(v, up, lane); break;
        case 16: exchange_lanes<E, 16>(v, up, lane); break;
        default: exchange_lanes<E, 32>(v, up, lane); break;
      }
    }
    merge_in_thread<E>(v, up);
  }
}

// One 1024-thread workgroup per block; P = 1024 * E >= BLK_TOKENS * K keys
// (padding and empty rows hold INT_MAX, above every expert id); LDS holds
// P + 1024 words.
template <int E>
__global__ __launch_bounds__(1024) void blk_union(const int32_t* __restrict__ idx,
                                                  const float* __restrict__ gate,
                                                  const int32_t* __restrict__ order, int L, int K,
                                                  int ucap, int32_t* __restrict__ U,
                                                  int32_t* __restrict__ nU, float* __restrict__ G) {
  extern __shared__ int keys[];
  __shared__ int wtot[16];
  const int b = blockIdx.x, tid = threadIdx.x;
  const int nt = BT * K;
  // up to 16 positions per thread, the ids and gates stay in registers for
  // the scatter at the end (beyond, they are read again)
  constexpr bool KEEP = E <= 16;
  int v[E], id0[KEEP ? E : 1];
  float g0[KEEP ? E : 1];
#pragma unroll
  for (int q = 0; q < E; ++q) {
    const int i = tid * E + q;
    int key = INT_MAX;
    float g = 0.f;
    if (i < nt) {
      const int r = i / K;
      const int t = slot_token(order, b * BT + r, L);
      if (t >= 0) {
        key = idx[(size_t)t * K + (i - r * K)];
        if constexpr (KEEP) g = gate[(size_t)t * K + (i - r * K)];
      }
    }
    v[q] = key;
    if constexpr (KEEP) {
      id0[q] = key;
      g0[q] = g;
    }
  }
  bitonic_sort<E>(keys, v, tid);
  // unique: thread tid owns the sorted positions [tid*E, tid*E + E); the
  // position before its first is the previous thread's last
  if (tid < 1023) keys[padded<E>(tid * E + E - 1)] = v[E - 1];
  __syncthreads();
  unsigned long long first = 0;
  int cnt = 0;
#pragma unroll
  for (int q = 0; q < E; ++q) {
    const int prev = q ? v[q - 1] : (tid ? keys[padded<E>(tid * E - 1)] : -1);
    const bool f = v[q] != INT_MAX && v[q] != prev;
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
  // the gate tile G_b [64][npad]: every entry marked "no task", then each
  // task's gate at (its row, its id's position in the union)
  uint32_t* Gb = (uint32_t*)G + (size_t)b * BT * ucap;
  const int n4 = BT * npad / 4;
  for (int i = tid; i < n4; i += 1024) ((u32x4*)Gb)[i] = u32x4{NOTASK, NOTASK, NOTASK, NOTASK};
  __syncthreads();  // the fill is complete before the gates land on it
  auto position = [&](int e) {  // e is in the union: its index there
    int lo = 0, hi = n - 1;
    while (lo < hi) {
      const int mid = (lo + hi) >> 1;
      if (keys[mid] < e) lo = mid + 1;
      else hi = mid;
    }
    return lo;
  };
  if constexpr (KEEP) {
    // the E searches of this thread advance together (their LDS reads
    // overlap): base converges on the last union entry below the id
    int base[E];
#pragma unroll
    for (int q = 0; q < E; ++q) base[q] = 0;
    for (int len = n; len > 1;) {
      const int half = len >> 1;
#pragma unroll
      for (int q = 0; q < E; ++q) base[q] += keys[base[q] + half] < id0[q] ? half : 0;
      len -= half;
    }
#pragma unroll
    for (int q = 0; q < E; ++q) {
      if (id0[q] == INT_MAX) continue;  // padding or an empty row
      const int c = base[q] + (keys[base[q]] < id0[q]);
      Gb[((tid * E + q) / K) * npad + c] = __float_as_uint(g0[q]);
    }
  } else {
    for (int i = tid; i < nt; i += 1024) {
      const int r = i / K;
      const int t = slot_token(order, b * BT + r, L);
      if (t < 0) continue;
      const size_t m = (size_t)t * K + (i - r * K);
      Gb[r * npad + position(idx[m])] = __float_as_uint(gate[m]);
    }
  }
}

// ------------------------------------------------------------------ blk_plan
// toff[b] = column tiles of the blocks before b (toff[nb] = all tiles, the
// work list of blk_act); block b has toff[b+1] - toff[b] tiles.
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
// Persistent, over the column tiles of all blocks.  A tile is the
// block's 64 token rows x 128 union rows, k-tiles of 64 streamed through a
// 3-stage LDS ring by direct loads (as in gemm_bt_bf16_pipe); 4 waves of
// 64 x 32.
constexpr int K1_BK = 64, K1_S = 3;
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
  // XCD x (the workgroups b with b % 8 == x) takes the x-th eighth of the
  // tile list, which is in block order: a block's tiles, and the next blocks
  // of the same token cluster, share that XCD's L2 (x rows, W rows)
  const int xcd = blockIdx.x % 8, per = gridDim.x / 8;  // grid is a multiple of 8
  const int t_end = (int)((int64_t)total * (xcd + 1) / 8);
  for (int T = (int)((int64_t)total * xcd / 8) + (int)blockIdx.x / 8; T < t_end; T += per) {
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
    for (int kt = 0; kt < K1_S - 1 && kt < nk; ++kt) issue(kt);
    for (int kt = 0; kt < nk; ++kt) {
      // tile kt landed for this wave (the loads of at most S-2 later tiles may
      // still fly); after the barrier it has for every wave, and tile kt-1's
      // stage is free for tile kt+S-1
      wait_vm_tiles<K1_LPWA + K1_LPWB, K1_S - 2>(min(K1_S - 2, nk - 1 - kt));
      block_sync_lds();
      if (kt + K1_S - 1 < nk) issue(kt + K1_S - 1);
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
    const size_t go = (size_t)b * BT * ucap;  // block b's G and A tiles
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
// waves of 64 x 64.  A k-tile is 32 union rows: the V slice (32 x 256 bf16,
// row-major, 16-byte chunk g of row R in slot g ^ ((R >> 3) & 3)) and the A_hi
// and A_lo tiles (64 x 32 bf16 each) go to LDS by direct loads, through a
// 3-stage ring.  The B operand (8 consecutive rows of one column per lane)
// is gathered with 2-byte LDS reads, which the slot rotation spreads over
// distinct banks.  The union ids that address a tile's V rows are read by
// scalar loads two tiles ahead, so the vector-load counter only ever holds
// tile loads and the waits can leave the next tile in flight.
constexpr int K2_COLS = BLK_D_TILE, K2_KT = 32, K2_ROWB = 2 * K2_COLS;  // 512-byte V rows
constexpr int K2_VT = K2_KT * K2_ROWB;           // 16 KB V slice
constexpr int K2_AT = BT * K2_KT * 2;            // 4 KB per A term
constexpr int K2_STAGE = K2_VT + 2 * K2_AT;      // 24 KB
constexpr int K2_S = 3;
constexpr int K2_TILE_OPS = 6;  // vector loads per wave and k-tile: 4 of V, 1 each of A_hi, A_lo

__global__ __launch_bounds__(256) void blk_out(const uint16_t* __restrict__ V,
                                               const int32_t* __restrict__ order,
                                               const int32_t* __restrict__ U,
                                               const int32_t* __restrict__ toff,
                                               const uint16_t* __restrict__ Ahi,
                                               const uint16_t* __restrict__ Alo, int L, int d,
                                               int ucap, float* __restrict__ y) {
  extern __shared__ __attribute__((aligned(16))) unsigned char sm2[];
  const int tiles_y = d / K2_COLS;
  // workgroup (b, jt) = b * tiles_y + jt runs on XCD (b * tiles_y + jt) % 8:
  // at d = 2048 each XCD takes one column slice of every block, in block
  // order, so consecutive blocks of a token cluster share its V slice rows
  // (measured faster than giving each XCD a contiguous range of blocks,
  // whose union sizes differ)
  const int b = blockIdx.x / tiles_y, c0 = (blockIdx.x % tiles_y) * K2_COLS;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int npad = (toff[b + 1] - toff[b]) * UPAD;
  const int nk = npad / K2_KT;
  const size_t go = (size_t)b * BT * ucap;  // block b's A tiles
  // V loads: wave w, load q covers LDS rows 8w + 2q and 8w + 2q + 1 (lanes
  // 0-31 and 32-63), i.e. union rows 8w .. 8w+7 of the tile
  const int32_t* Uw = U + (size_t)b * ucap + 8 * wave;
  const int half = lane >> 5;
  int slotg[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) slotg[q] = (lane & 31) ^ (((8 * wave + 2 * q + half) >> 3) & 3);
  // A loads: wave w covers rows 16w .. 16w+15 of each term (64-byte rows)
  const size_t aoff = go + (size_t)(16 * wave + (lane >> 2)) * npad + (lane & 3) * 8;
  const uint16_t* ah_src = Ahi + aoff;
  const uint16_t* al_src = Alo + aoff;
  auto load_ids = [&](int kt, int* e) {
#pragma unroll
    for (int j = 0; j < 8; ++j) e[j] = Uw[kt * K2_KT + j];
  };
  auto issue = [&](int kt, const int* e) {
    unsigned char* st = sm2 + (kt % K2_S) * K2_STAGE;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int id = half ? e[2 * q + 1] : e[2 * q];
      __builtin_amdgcn_global_load_lds((const void*)(V + (size_t)id * d + c0 + slotg[q] * 8),
                                       (lds_void*)(st + (4 * wave + q) * 1024), 16, 0, 0);
    }
    __builtin_amdgcn_global_load_lds((const void*)(ah_src + kt * K2_KT),
                                     (lds_void*)(st + K2_VT + wave * 1024), 16, 0, 0);
    __builtin_amdgcn_global_load_lds((const void*)(al_src + kt * K2_KT),
                                     (lds_void*)(st + K2_VT + K2_AT + wave * 1024), 16, 0, 0);
  };
  f32x4 acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int q = 0; q < 4; ++q) acc[i][q] = f32x4{0.f, 0.f, 0.f, 0.f};
  // ids of even and odd k-tiles, read two tiles before the tile is issued
  int e0[8], e1[8];
  load_ids(0, e0);
  if (nk > 1) load_ids(1, e1);
  issue(0, e0);
  if (nk > 1) issue(1, e1);
  if (nk > 2) load_ids(2, e0);
  if (nk > 3) load_ids(3, e1);
  const int kq = lane >> 4;  // k rows 8 kq .. 8 kq + 7 of a fragment
  auto step = [&](int kt, int* e) {  // e: the id set of tile kt+2 (then of kt+4)
    // tile kt landed for this wave (only tile kt+1's loads may still fly) ...
    wait_vm_tiles<K2_TILE_OPS, 1>(kt + 1 < nk);
    block_sync_lds();  // ... and for every wave; tile kt-1's stage is free
    if (kt + 2 < nk) {
      issue(kt + 2, e);
      if (kt + 4 < nk) load_ids(kt + 4, e);
    }
    const unsigned char* st = sm2 + (kt % K2_S) * K2_STAGE;
    bf16x8 ah[4], al[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int o = (i * 16 + (lane & 15)) * 64 + kq * 16;
      ah[i] = *(const bf16x8*)(st + K2_VT + o);
      al[i] = *(const bf16x8*)(st + K2_VT + K2_AT + o);
    }
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
    step(kt, e0);
    if (kt + 1 < nk) step(kt + 1, e1);
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
constexpr int K1_WG_PER_CU = 2;  // 72 KB of LDS each

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
  int32_t* toff = (int32_t*)(w + p.off_toff);
  float* G = (float*)(w + p.off_G);
  uint16_t* Ahi = (uint16_t*)(w + p.off_Ahi);
  uint16_t* Alo = (uint16_t*)(w + p.off_Alo);
  const size_t lds_u = (size_t)(p.sort_keys + 1024) * 4;  // keys and one pad word per thread
  switch (p.sort_keys / 1024) {
#define OMNI_BLK_UNION(E)                                                                     \
  case E:                                                                                     \
    hipLaunchKernelGGL(blk_union<E>, dim3(p.nb), dim3(1024), lds_u, s, idx, gate, order, L, \
                       K, p.ucap, U, nU, G);                                                  \
    break;
    OMNI_BLK_UNION(1) OMNI_BLK_UNION(2) OMNI_BLK_UNION(4) OMNI_BLK_UNION(8) OMNI_BLK_UNION(16)
    OMNI_BLK_UNION(32)
#undef OMNI_BLK_UNION
    default:
      return hipErrorInvalidValue;  // K above the validated limit
  }
  hipLaunchKernelGGL(blk_plan, dim3(1), dim3(1024), 0, s, nU, p.nb, toff);
  const int max_tiles = p.nb * (p.ucap / UPAD);
  const int k1_grid = 8 * std::min((max_tiles + 7) / 8, MI355X_CUS * K1_WG_PER_CU / 8);
  hipLaunchKernelGGL(blk_act, dim3(k1_grid), dim3(256), K1_S * K1_STAGE, s,
                     (const uint16_t*)x, (const uint16_t*)W, order, U, toff, G, L, d, p.nb, p.ucap,
                     Ahi, Alo);
  hipLaunchKernelGGL(blk_out, dim3(p.nb * (d / K2_COLS)), dim3(256), K2_S * K2_STAGE, s,
                     (const uint16_t*)V, order, U, toff, Ahi, Alo, L, d, p.ucap, y);
  return hipGetLastError();
}

}  // namespace omni
