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
//
// The backward (the chain rule of the same definition) reuses them:
//   blk_union  also records each task's slot k at its (row, column)
//   split_bf16 dy = dy_hi + dy_lo
//   blk_act    (backward mode) H = X_b W[U_b]^T and D = dy_b V[U_b]^T in one
//              pipeline; per task dgate = D SiLU(h), dh = g D SiLU'(h),
//              g SiLU(h); the dense dH tile
//   blk_out    dx_b = dH W[U_b]
// and for the dW, dV rows groups the used experts into sets of 64 (experts
// of one token cluster together), with each set's token union:
//   inv_order, set_keys, a radix sort   the order of the used experts
//   set_union, set_plan, set_union      the unions and dense tiles DhT, GaT
//   blk_out    (set form) dW rows = DhT X[T_s], dV rows = GaT dy[T_s]

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

// Compare-exchange of positions q and j = q ^ st (q < j), ascending if up.
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

// The same sort for E <= 16 with the cross-wave stages replaced by merges:
// each wave sorts its 64 E keys with the network above (its last merge
// ascending in every wave), then four merge-path rounds through LDS turn the
// 16 sorted runs into 8, 4, 2 and 1: thread tid writes outputs tid*E ..
// tid*E + E-1 of its merged run, after a binary search on the run pair's
// diagonal for how many of the outputs before its first come from the left
// run (ties go to the left run).  A round costs one pass of LDS reads and
// writes where the network spends one to four LDS exchanges and ten
// register stages.  Measured on the skewed workload (16384 tokens, K = 256):
// the blocked forward 509 -> 491 us, the same union bit for bit.
// keys holds two buffers of P padded words; the result lands in the first
// (the round count is even), in the layout bitonic_sort leaves, and v ends
// holding positions tid*E .. tid*E + E-1.
template <int E>
__device__ void merge_sort(int* keys, int (&v)[E], int tid) {
  constexpr int P = 1024 * E;
  constexpr int PW = P + P / E;
  static_assert(E <= 16, "two padded buffers of 1024 * E words must fit the LDS");
  const int lane = tid & 63;
  sort_runs<E>(v, tid);
  for (int size = 2 * E; size <= 64 * E; size <<= 1) {
    const bool up = size == 64 * E || ((tid * E) & size) == 0;
    for (int st = min(size >> 1, 32 * E); st >= E; st >>= 1) {
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
  int* src = keys;
  int* dst = keys + PW;
#pragma unroll
  for (int q = 0; q < E; ++q) src[padded<E>(tid * E + q)] = v[q];
  __syncthreads();
  for (int len = 64 * E; len < P; len <<= 1) {
    const int o0 = (tid * E) & (2 * len - 1);  // first output's offset in the merged run
    const int base = tid * E - o0;             // the left run; the right one follows it
    int lo = max(0, o0 - len), hi = min(o0, len);
    while (lo < hi) {
      const int mid = (lo + hi) >> 1;
      if (src[padded<E>(base + mid)] <= src[padded<E>(base + len + o0 - 1 - mid)]) lo = mid + 1;
      else hi = mid;
    }
    int i = lo, j = o0 - lo;
    int x = src[padded<E>(base + min(i, len - 1))];
    int y = src[padded<E>(base + len + min(j, len - 1))];
#pragma unroll
    for (int q = 0; q < E; ++q) {
      const bool ta = j >= len || (i < len && x <= y);
      dst[padded<E>(tid * E + q)] = ta ? x : y;
      i += ta;
      j += !ta;
      const int nv = src[padded<E>(ta ? base + min(i, len - 1) : base + len + min(j, len - 1))];
      x = ta ? nv : x;
      y = ta ? y : nv;
    }
    __syncthreads();
    int* t = src;
    src = dst;
    dst = t;
  }
#pragma unroll
  for (int q = 0; q < E; ++q) v[q] = keys[padded<E>(tid * E + q)];
}

// One 1024-thread workgroup per block; P = 1024 * E >= BLK_TOKENS * K keys
// (padding and empty rows hold INT_MAX, above every expert id); LDS holds
// P + 1024 words, twice that for the merge sort (E <= 16).
template <int E>
__global__ __launch_bounds__(1024) void blk_union(const int32_t* __restrict__ idx,
                                                  const float* __restrict__ gate,
                                                  const int32_t* __restrict__ order, int L, int K,
                                                  int ucap, int32_t* __restrict__ U,
                                                  int32_t* __restrict__ nU, float* __restrict__ G,
                                                  int32_t* __restrict__ kmap,
                                                  const int32_t* run_flag, int run_want) {
  if (gated_out(run_flag, run_want)) return;
  extern __shared__ __attribute__((aligned(16))) int keys[];
  __shared__ int wtot[16];
  const int b = blockIdx.x, tid = threadIdx.x;
  const int nt = BT * K;
  // up to 16 positions per thread, the ids and gates stay in registers for
  // the scatter at the end (beyond, they are read again)
  constexpr bool KEEP = E <= 16;
  int v[E], id0[KEEP ? E : 1];
  float g0[KEEP ? E : 1];
  // row r = i / K and slot k = i % K of position i = tid*E + q: one division
  // per thread, then one step per position (a software division per
  // position, repeated in each pass of the scatter below, was a quarter of
  // the kernel's code; 4 us of 485 on the skewed workload's blocked
  // forward); kept as (r << 16) | k for the scatter (r < 2^15)
  int rk[KEEP ? E : 1];
  {
    int r = (tid * E) / K, k = tid * E - r * K;
#pragma unroll
    for (int q = 0; q < E; ++q) {
      const int i = tid * E + q;
      int key = INT_MAX;
      float g = 0.f;
      if (i < nt) {
        const int t = slot_token(order, b * BT + r, L);
        if (t >= 0) {
          key = idx[(size_t)t * K + k];
          if constexpr (KEEP) g = gate[(size_t)t * K + k];
        }
      }
      v[q] = key;
      if constexpr (KEEP) {
        id0[q] = key;
        g0[q] = g;
        rk[q] = (r << 16) | k;
      }
      if (++k == K) {
        k = 0;
        ++r;
      }
    }
  }
  if constexpr (E <= 16) merge_sort<E>(keys, v, tid);
  else bitonic_sort<E>(keys, v, tid);
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
  // task's gate at (its row, its id's position in the union); the slot map
  // (when asked for) holds each task's k at the same place and is read only
  // where the gate tile holds a task.  With room for 8 or more tile rows
  // (of both) in the LDS of the sort, the rows are assembled there and
  // stored whole; otherwise the gate tile is filled in place and the entries
  // are stored one by one (4-byte stores to scattered lines).
  uint32_t* Gb = (uint32_t*)G + (size_t)b * BT * ucap;
  int32_t* Kb = kmap ? kmap + (size_t)b * BT * ucap : nullptr;
  constexpr int LDS_WORDS = 1024 * E + 1024;
  const int row_words = kmap ? 2 * npad : npad;
  const int rows_per_pass = min(BT, LDS_WORDS / row_words);
  const bool staged = KEEP && rows_per_pass >= 8;
  if (!staged) {
    const int n4 = BT * npad / 4;
    for (int i = tid; i < n4; i += 1024) ((u32x4*)Gb)[i] = u32x4{NOTASK, NOTASK, NOTASK, NOTASK};
  }
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
    if (staged) {
      int col[E];
#pragma unroll
      for (int q = 0; q < E; ++q) col[q] = base[q] + (keys[base[q]] < id0[q]);
      uint32_t* stage = (uint32_t*)keys;                 // gate rows
      uint32_t* kstage = stage + rows_per_pass * npad;   // slot rows (with kmap)
      for (int r0 = 0; r0 < BT; r0 += rows_per_pass) {
        const int rows = min(rows_per_pass, BT - r0);
        __syncthreads();  // the union searches, or the previous pass's stores, are done
        for (int i = tid; i < rows * npad; i += 1024) {
          stage[i] = NOTASK;
          if (kmap) kstage[i] = 0u;
        }
        __syncthreads();
#pragma unroll
        for (int q = 0; q < E; ++q) {
          const int r = rk[q] >> 16;
          if (id0[q] != INT_MAX && r >= r0 && r < r0 + rows) {
            stage[(r - r0) * npad + col[q]] = __float_as_uint(g0[q]);
            if (kmap) kstage[(r - r0) * npad + col[q]] = (uint32_t)(rk[q] & 0xffff);
          }
        }
        __syncthreads();
        u32x4* dst = (u32x4*)(Gb + (size_t)r0 * npad);
        for (int i = tid; i < rows * npad / 4; i += 1024) dst[i] = ((const u32x4*)stage)[i];
        if (kmap) {
          u32x4* kdst = (u32x4*)(Kb + (size_t)r0 * npad);
          for (int i = tid; i < rows * npad / 4; i += 1024) kdst[i] = ((const u32x4*)kstage)[i];
        }
      }
      return;
    }
#pragma unroll
    for (int q = 0; q < E; ++q) {
      if (id0[q] == INT_MAX) continue;  // padding or an empty row
      const int c = base[q] + (keys[base[q]] < id0[q]);
      const int r = rk[q] >> 16;
      Gb[r * npad + c] = __float_as_uint(g0[q]);
      if (kmap) kmap[(size_t)b * BT * ucap + r * npad + c] = rk[q] & 0xffff;
    }
  } else {
    for (int i = tid; i < nt; i += 1024) {
      const int r = i / K;
      const int t = slot_token(order, b * BT + r, L);
      if (t < 0) continue;
      const size_t m = (size_t)t * K + (i - r * K);
      const int c = position(idx[m]);
      Gb[r * npad + c] = __float_as_uint(gate[m]);
      if (kmap) kmap[(size_t)b * BT * ucap + r * npad + c] = i - r * K;
    }
  }
}

// ------------------------------------------------------------------ blk_plan
// toff[b] = column tiles of the blocks before b (toff[nb] = all tiles, the
// work list of blk_act); block b has toff[b+1] - toff[b] tiles.
__global__ __launch_bounds__(1024) void blk_plan(const int32_t* __restrict__ nU, int nb,
                                                 int32_t* __restrict__ toff,
                                                 const int32_t* run_flag, int run_want) {
  if (gated_out(run_flag, run_want)) return;
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

__device__ __forceinline__ float sigmoid(float h) { return 1.f / (1.f + expf(-h)); }

// MODE BLK_FWD: one product, H = X_b W[U_b]^T; the epilogue writes
// A = G . SiLU(H) as hi + lo bf16 tiles.
// MODE BLK_BWD: three products through the same pipeline, H = X_b W[U_b]^T
// and D = dy_b V[U_b]^T with dy_b = dy_hi + dy_lo (two bf16 terms); at each
// task (t, k) the epilogue writes, with g its gate, s = SiLU(h) and
// s' = sig(h) (1 + h (1 - sig(h))):
//   dgate[t,k] = D s,   dh[t,k] = g D s',   ga[t,k] = g s
// and the dense tile dH = (task ? g D s' : 0) as hi + lo bf16 (for dx = dH W).
constexpr int BLK_FWD = 0, BLK_BWD = 1;

template <int MODE>
__global__ __launch_bounds__(256) void blk_act(const uint16_t* __restrict__ x,
                                               const uint16_t* __restrict__ W,
                                               const uint16_t* __restrict__ dyh,
                                               const uint16_t* __restrict__ dyl,
                                               const uint16_t* __restrict__ V,
                                               const int32_t* __restrict__ order,
                                               const int32_t* __restrict__ U,
                                               const int32_t* __restrict__ toff,
                                               const float* __restrict__ G,
                                               const int32_t* __restrict__ kmap, int L, int d,
                                               int K, int nb, int ucap,
                                               uint16_t* __restrict__ Ahi,
                                               uint16_t* __restrict__ Alo,
                                               float* __restrict__ dgate, float* __restrict__ dh,
                                               float* __restrict__ ga,
                                               const int32_t* run_flag, int run_want) {
  if (gated_out(run_flag, run_want)) return;
  extern __shared__ __attribute__((aligned(16))) unsigned char sm1[];
  constexpr int PHASES = MODE == BLK_FWD ? 1 : 3;
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
    size_t aro[K1_LPWA], bro[K1_LPWB];  // element offsets of this lane's 16-byte chunks
#pragma unroll
    for (int q = 0; q < K1_LPWA; ++q) {
      const int r = (wave * K1_LPWA + q) * K1_RPI + lane / K1_CPR;
      const int chunk = (lane % K1_CPR) ^ chunk_swz<K1_BK>(r);
      const int t = slot_token(order, b * BT + r, L);
      aro[q] = (size_t)(t < 0 ? 0 : t) * d + chunk * 8;  // empty rows: any row, masked
    }
#pragma unroll
    for (int q = 0; q < K1_LPWB; ++q) {
      const int r = (wave * K1_LPWB + q) * K1_RPI + lane / K1_CPR;
      const int chunk = (lane % K1_CPR) ^ chunk_swz<K1_BK>(r);
      bro[q] = (size_t)Ub[r] * d + chunk * 8;
    }
    // k-tile kk of the concatenated products: phase kk / nk, depth kk % nk
    auto issue = [&](int kk) {
      unsigned char* st = sm1 + (kk % K1_S) * K1_STAGE;
      const int ph = kk / nk, k0 = (kk - ph * nk) * K1_BK;
      const uint16_t* A = ph == 0 ? x : (ph == 1 ? dyh : dyl);
      const uint16_t* B = ph == 0 ? W : V;
#pragma unroll
      for (int q = 0; q < K1_LPWA; ++q)
        __builtin_amdgcn_global_load_lds((const void*)(A + aro[q] + k0),
                                         (lds_void*)(st + (wave * K1_LPWA + q) * 1024), 16, 0, 0);
#pragma unroll
      for (int q = 0; q < K1_LPWB; ++q)
        __builtin_amdgcn_global_load_lds(
            (const void*)(B + bro[q] + k0),
            (lds_void*)(st + K1_TILEA + (wave * K1_LPWB + q) * 1024), 16, 0, 0);
    };
    // acc: H, then (backward) D; hs keeps H once the D phases begin
    f32x4 acc[K1_MI][K1_NJ], hs[MODE == BLK_BWD ? K1_MI : 1][K1_NJ];
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
    auto multiply = [&](const unsigned char* st, f32x4 (&c)[K1_MI][K1_NJ]) {
      bf16x8 af[2][K1_MI], bfr[2][K1_NJ];
      load_frags(st, 0, af[0], bfr[0]);
#pragma unroll
      for (int ks = 0; ks < K1_BK / 32; ++ks) {
        if (ks + 1 < K1_BK / 32) load_frags(st, ks + 1, af[(ks + 1) & 1], bfr[(ks + 1) & 1]);
#pragma unroll
        for (int i = 0; i < K1_MI; ++i)
#pragma unroll
          for (int q = 0; q < K1_NJ; ++q)
            c[i][q] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[ks & 1][i], bfr[ks & 1][q],
                                                              c[i][q], 0, 0, 0);
      }
    };
    const int nkk = PHASES * nk;
    for (int kk = 0; kk < K1_S - 1 && kk < nkk; ++kk) issue(kk);
    for (int kk = 0; kk < nkk; ++kk) {
      // tile kk landed for this wave (the loads of at most S-2 later tiles may
      // still fly); after the barrier it has for every wave, and tile kk-1's
      // stage is free for tile kk+S-1
      wait_vm_tiles<K1_LPWA + K1_LPWB, K1_S - 2>(min(K1_S - 2, nkk - 1 - kk));
      block_sync_lds();
      if (kk + K1_S - 1 < nkk) issue(kk + K1_S - 1);
      const unsigned char* st = sm1 + (kk % K1_S) * K1_STAGE;
      if constexpr (MODE == BLK_BWD) {
        if (kk == nk) {  // H is complete: keep it, accumulate D from zero
#pragma unroll
          for (int i = 0; i < K1_MI; ++i)
#pragma unroll
            for (int q = 0; q < K1_NJ; ++q) {
              hs[i][q] = acc[i][q];
              acc[i][q] = f32x4{0.f, 0.f, 0.f, 0.f};
            }
        }
      }
      multiply(st, acc);
    }
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
          float a = 0.f;
          if constexpr (MODE == BLK_FWD) {
            const float h = acc[i][q][e];
            if (gb != NOTASK) a = __uint_as_float(gb) * (h * sigmoid(h));
          } else if (gb != NOTASK) {
            const float h = hs[i][q][e];
            const float g = __uint_as_float(gb), D = acc[i][q][e], sg = sigmoid(h);
            const float sl = h * sg, slp = sg * (1.f + h * (1.f - sg));
            a = g * D * slp;  // dh
            const size_t m = (size_t)order[b * BT + r] * K + kmap[go + o];
            dgate[m] = D * sl;
            dh[m] = a;
            ga[m] = g * sl;
          }
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
// row-major, 16-byte chunk g of row R in slot g ^ (2 ((R >> 3) & 3))) and the
// A_hi and A_lo tiles (64 x 32 bf16 each) go to LDS by direct loads, through
// a 3-stage ring.  The B operand (8 consecutive rows of one column per lane)
// is gathered with 2-byte LDS reads: lane group kq = lane / 16 reads rows
// 8 kq .. 8 kq + 7, all rows fall on the same banks (512 bytes apart), and
// the rotation puts the four groups' 16 columns in eight distinct 16-byte
// slots.  Rotating by ((R >> 3) & 3) gave groups 0 and 1 (and 2 and 3) the
// same two slots; the counters on the skewed workload fell from 20 M to
// 6.7 M bank-conflict cycles per call (the rest: two lanes reading the two
// halves of one 4-byte word), the blocked forward 490 -> 487 us.  Gathering
// the operand with two LDS transpose reads (ds_read_b64_tr_b16) per fragment
// instead, over a layout whose rotation also spreads the four rows a group
// reads, was slower (487 -> 515 us) with the same y.  The union ids that address a tile's V rows are read by
// scalar loads two tiles ahead, so the vector-load counter only ever holds
// tile loads and the waits can leave the next tile in flight.
constexpr int K2_COLS = BLK_D_TILE, K2_KT = 32, K2_ROWB = 2 * K2_COLS;  // 512-byte V rows
constexpr int K2_VT = K2_KT * K2_ROWB;           // 16 KB V slice
constexpr int K2_AT = BT * K2_KT * 2;            // 4 KB per A term
constexpr int K2_STAGE = K2_VT + 2 * K2_AT;      // 24 KB
constexpr int K2_S = 3;
// SETS false: workgroup (b, jt) as above; A and U at fixed per-block offsets
// (b * 64 * ucap, b * ucap); output row r of block b is token order[64 b + r].
// SETS true (the expert-set products of the backward): persistent over the
// items (set b, column tile jt) of the *nrows / 64 sets; A, U and the k-tile
// count come from the compact tile prefix toff; output row r of set b is row
// order[64 b + r] of y (an expert's rank among the used experts).
// NB = 2 takes the B rows as two bf16 terms (hi, lo): the products are
// A_hi B_hi + A_lo B_hi + A_hi B_lo.  OUT_BF16 writes y rounded to bf16.
template <bool SETS, int NB, bool OUT_BF16>
__global__ __launch_bounds__(256) void blk_out(const uint16_t* __restrict__ V,
                                               const uint16_t* __restrict__ V2,
                                               const int32_t* __restrict__ order,
                                               const int32_t* __restrict__ nrows,
                                               const int32_t* __restrict__ U,
                                               const int32_t* __restrict__ toff,
                                               const uint16_t* __restrict__ Ahi,
                                               const uint16_t* __restrict__ Alo, int L, int d,
                                               int ucap, void* __restrict__ y_,
                                               const int32_t* run_flag, int run_want) {
  if (gated_out(run_flag, run_want)) return;
  extern __shared__ __attribute__((aligned(16))) unsigned char sm2[];
  constexpr int STAGE = NB * K2_VT + 2 * K2_AT;
  constexpr int OPS = 4 * NB + 2;  // vector loads per wave and k-tile
  const int tiles_y = d / K2_COLS;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int half = lane >> 5, kq = lane >> 4;
  int slotg[4];
#pragma unroll
  for (int q = 0; q < 4; ++q)
    slotg[q] = (lane & 31) ^ ((((8 * wave + 2 * q + half) >> 3) & 3) << 1);
  const int rows = SETS ? *nrows : L;
  auto item = [&](int b, int c0) {
    const int ntile = SETS ? toff[b + 1] - toff[b] : 0;
    const int npad = SETS ? ntile * UPAD : (toff[b + 1] - toff[b]) * UPAD;
    const int nk = npad / K2_KT;
    const size_t go = SETS ? (size_t)toff[b] * BT * UPAD : (size_t)b * BT * ucap;
    // V loads: wave w, load q covers LDS rows 8w + 2q and 8w + 2q + 1 (lanes
    // 0-31 and 32-63), i.e. union rows 8w .. 8w+7 of the tile
    const int32_t* Uw = U + (SETS ? (size_t)toff[b] * UPAD : (size_t)b * ucap) + 8 * wave;
    // A loads: wave w covers rows 16w .. 16w+15 of each term (64-byte rows)
    const size_t aoff = go + (size_t)(16 * wave + (lane >> 2)) * npad + (lane & 3) * 8;
    auto load_ids = [&](int kt, int* e) {
#pragma unroll
      for (int j = 0; j < 8; ++j) e[j] = Uw[kt * K2_KT + j];
    };
    auto issue = [&](int kt, const int* e) {
      unsigned char* st = sm2 + (kt % K2_S) * STAGE;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const size_t ro = (size_t)(half ? e[2 * q + 1] : e[2 * q]) * d + c0 + slotg[q] * 8;
        __builtin_amdgcn_global_load_lds((const void*)(V + ro),
                                         (lds_void*)(st + (4 * wave + q) * 1024), 16, 0, 0);
        if constexpr (NB == 2)
          __builtin_amdgcn_global_load_lds((const void*)(V2 + ro),
                                           (lds_void*)(st + K2_VT + (4 * wave + q) * 1024), 16,
                                           0, 0);
      }
      __builtin_amdgcn_global_load_lds((const void*)(Ahi + aoff + kt * K2_KT),
                                       (lds_void*)(st + NB * K2_VT + wave * 1024), 16, 0, 0);
      __builtin_amdgcn_global_load_lds((const void*)(Alo + aoff + kt * K2_KT),
                                       (lds_void*)(st + NB * K2_VT + K2_AT + wave * 1024), 16, 0,
                                       0);
    };
    f32x4 acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int q = 0; q < 4; ++q) acc[i][q] = f32x4{0.f, 0.f, 0.f, 0.f};
    // ids of even and odd k-tiles, read two tiles before the tile is issued
    int e0[8], e1[8];
    if (nk > 0) load_ids(0, e0);
    if (nk > 1) load_ids(1, e1);
    if (nk > 0) issue(0, e0);
    if (nk > 1) issue(1, e1);
    if (nk > 2) load_ids(2, e0);
    if (nk > 3) load_ids(3, e1);
    auto vfrag = [&](const unsigned char* p) {
      bf16x8 vb;
#pragma unroll
      for (int e = 0; e < 8; ++e)
        vb[e] = __builtin_bit_cast(__bf16, *(const uint16_t*)(p + (8 * kq + e) * K2_ROWB));
      return vb;
    };
    auto step = [&](int kt, int* e) {  // e: the id set of tile kt+2 (then of kt+4)
      // tile kt landed for this wave (only tile kt+1's loads may still fly) ...
      wait_vm_tiles<OPS, 1>(kt + 1 < nk);
      block_sync_lds();  // ... and for every wave; tile kt-1's stage is free
      if (kt + 2 < nk) {
        issue(kt + 2, e);
        if (kt + 4 < nk) load_ids(kt + 4, e);
      }
      const unsigned char* st = sm2 + (kt % K2_S) * STAGE;
      bf16x8 ah[4], al[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int o = (i * 16 + (lane & 15)) * 64 + kq * 16;
        ah[i] = *(const bf16x8*)(st + NB * K2_VT + o);
        al[i] = *(const bf16x8*)(st + NB * K2_VT + K2_AT + o);
      }
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int col = wave * 64 + q * 16 + (lane & 15);
        const unsigned char* p = st + (((col >> 3) ^ (kq << 1)) << 4) + ((col & 7) << 1);
        const bf16x8 vb = vfrag(p);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          acc[i][q] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ah[i], vb, acc[i][q], 0, 0, 0);
          acc[i][q] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(al[i], vb, acc[i][q], 0, 0, 0);
        }
        if constexpr (NB == 2) {
          const bf16x8 vl = vfrag(p + K2_VT);
#pragma unroll
          for (int i = 0; i < 4; ++i)
            acc[i][q] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ah[i], vl, acc[i][q], 0, 0, 0);
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
        int t;
        if constexpr (SETS) t = b * BT + r < rows ? order[b * BT + r] : -1;
        else t = slot_token(order, b * BT + r, L);
        if (t < 0) continue;
        const size_t o = (size_t)t * d + c0 + wave * 64 + (lane & 15);
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          if constexpr (OUT_BF16) ((uint16_t*)y_)[o + q * 16] = bf16_rne(acc[i][q][e]);
          else ((float*)y_)[o + q * 16] = acc[i][q][e];
        }
      }
  };
  if constexpr (!SETS) {
    // workgroup (b, jt) = b * tiles_y + jt runs on XCD (b * tiles_y + jt) % 8:
    // at d = 2048 each XCD takes one column slice of every block, in block
    // order, so consecutive blocks of a token cluster share its V slice rows
    // (measured faster than giving each XCD a contiguous range of blocks,
    // whose union sizes differ)
    item(blockIdx.x / tiles_y, (blockIdx.x % tiles_y) * K2_COLS);
  } else {
    const int items = (rows + BT - 1) / BT * tiles_y;
    for (int it = blockIdx.x; it < items; it += gridDim.x) {
      item(it / tiles_y, (it % tiles_y) * K2_COLS);
      block_sync_lds();  // every wave is done with the stages before the next item refills them
    }
  }
}

// ------------------------------------------------------------------ expert sets
// The backward's dW and dV rows as dense products over sets of 64 used
// experts: the experts are ordered by the first position, in the token order,
// of a token that uses them (experts of one token cluster come together), set
// s is experts 64 s .. 64 s + 63 of that order, T_s the union of their
// tokens (ascending), and with DhT_s [64 x |T_s|] holding dh of each task
// (zero elsewhere) and GaT_s likewise g SiLU(h):
//   dW rows of set s = DhT_s X[T_s],   dV rows = GaT_s dy[T_s]
// (blk_out in its set form).  Each expert belongs to one set, so every row
// is written once, by the workgroup that sums it.

// pos[order[s]] = s
__global__ __launch_bounds__(256) void inv_order(const int32_t* __restrict__ order, int L,
                                                 int32_t* __restrict__ pos,
                                                 const int32_t* run_flag, int run_want) {
  if (gated_out(run_flag, run_want)) return;
  for (int s = blockIdx.x * 256 + threadIdx.x; s < L; s += gridDim.x * 256) {
    const int t = order[s];
    if ((unsigned)t < (unsigned)L) pos[t] = s;
  }
}

// key[u] = the smallest pos of a token of used expert u (u < n_uniq), L for
// the capacity slots past n_uniq; one wave per expert
__global__ __launch_bounds__(256) void set_keys(const int32_t* __restrict__ perm,
                                                const int32_t* __restrict__ seg,
                                                const int32_t* __restrict__ n_uniq,
                                                const int32_t* __restrict__ pos, int K, int L,
                                                int ucap_e, int32_t* __restrict__ key,
                                                const int32_t* run_flag, int run_want) {
  if (gated_out(run_flag, run_want)) return;
  const int n = *n_uniq, lane = threadIdx.x & 63;
  const int nw = gridDim.x * 4;
  for (int u = blockIdx.x * 4 + (threadIdx.x >> 6); u < ucap_e; u += nw) {
    unsigned m = (unsigned)L;
    if (u < n) {
      for (int i = seg[u] + lane; i < seg[u + 1]; i += 64)
        m = min(m, min((unsigned)pos[perm[i] / K], (unsigned)L));
      m = wave_umin(m);
    }
    if (lane == 0) key[u] = (int)m;
  }
}

// Per set: the token union by an LDS bitmap over [0, L) and the exclusive
// prefix of its word popcounts (a token's rank in the union).  COUNT writes
// the union size; otherwise the union (padded with token 0 up to whole
// 128-entry tiles) and the dense tiles DhT, GaT as hi + lo bf16.
template <bool COUNT>
__global__ __launch_bounds__(1024) void set_union(
    const int32_t* __restrict__ eord, const int32_t* __restrict__ n_uniq,
    const int32_t* __restrict__ perm, const int32_t* __restrict__ seg, int K, int L,
    const int32_t* __restrict__ stoff, const float* __restrict__ dh, const float* __restrict__ ga,
    int32_t* __restrict__ nS, int32_t* __restrict__ T, uint16_t* __restrict__ dht_hi,
    uint16_t* __restrict__ dht_lo, uint16_t* __restrict__ gat_hi, uint16_t* __restrict__ gat_lo,
    const int32_t* run_flag, int run_want) {
  if (gated_out(run_flag, run_want)) return;
  extern __shared__ unsigned bm[];  // W bitmap words, then their prefix
  __shared__ int wtot[16];
  const int W = (L + 31) / 32;
  unsigned* pre = bm + W;
  const int n = *n_uniq, nsets = (n + BT - 1) / BT;
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int cw = (W + 1023) / 1024;  // prefix: thread tid owns words [tid cw, tid cw + cw)
  for (int si = blockIdx.x; si < nsets; si += gridDim.x) {
    for (int i = tid; i < W; i += 1024) bm[i] = 0u;
    __syncthreads();
    for (int r = wv; r < BT && si * BT + r < n; r += 16) {  // wave: experts r, r + 16, ...
      const int u = eord[si * BT + r];
      for (int i = seg[u] + lane; i < seg[u + 1]; i += 64) {
        const int t = perm[i] / K;
        atomicOr(&bm[t >> 5], 1u << (t & 31));
      }
    }
    __syncthreads();
    int loc = 0;
    for (int w = tid * cw; w < min(W, tid * cw + cw); ++w) loc += __popc(bm[w]);
    const int inc = wave_incl_scan(loc);
    if (lane == 63) wtot[wv] = inc;
    __syncthreads();
    int run = inc - loc, ns = 0;
#pragma unroll
    for (int w = 0; w < 16; ++w) {
      run += w < wv ? wtot[w] : 0;
      ns += wtot[w];
    }
    for (int w = tid * cw; w < min(W, tid * cw + cw); ++w) {
      pre[w] = run;
      run += __popc(bm[w]);
    }
    if constexpr (COUNT) {
      if (tid == 0) nS[si] = ns;
      __syncthreads();  // wtot and the bitmap are reused by the next set
      continue;
    }
    __syncthreads();
    const int npad = (stoff[si + 1] - stoff[si]) * UPAD;
    int32_t* Ts = T + (size_t)stoff[si] * UPAD;
    for (int w = tid; w < W; w += 1024) {
      unsigned bits = bm[w];
      int r0 = pre[w];
      while (bits) {
        Ts[r0++] = w * 32 + __builtin_ctz(bits);
        bits &= bits - 1u;
      }
    }
    for (int c = ns + tid; c < npad; c += 1024) Ts[c] = 0;
    const size_t go = (size_t)stoff[si] * BT * UPAD;
    const int n8 = BT * npad / 8;
    const u32x4 z = u32x4{0u, 0u, 0u, 0u};
    for (int i = tid; i < n8; i += 1024) {
      ((u32x4*)(dht_hi + go))[i] = z;
      ((u32x4*)(dht_lo + go))[i] = z;
      ((u32x4*)(gat_hi + go))[i] = z;
      ((u32x4*)(gat_lo + go))[i] = z;
    }
    __syncthreads();  // the fill is complete before the tasks land on it
    for (int r = wv; r < BT && si * BT + r < n; r += 16) {
      const int u = eord[si * BT + r];
      for (int i = seg[u] + lane; i < seg[u + 1]; i += 64) {
        const int m = perm[i], t = m / K;
        const int c = pre[t >> 5] + __popc(bm[t >> 5] & ((1u << (t & 31)) - 1u));
        const size_t o = go + (size_t)r * npad + c;
        const float a = dh[m], g = ga[m];
        const uint16_t ah = bf16_rne(a), gh = bf16_rne(g);
        dht_hi[o] = ah;
        dht_lo[o] = bf16_rne(a - __uint_as_float((uint32_t)ah << 16));
        gat_hi[o] = gh;
        gat_lo[o] = bf16_rne(g - __uint_as_float((uint32_t)gh << 16));
      }
    }
    __syncthreads();  // the bitmap is cleared for the next set only after every use
  }
}

// stoff[s] = column tiles of the sets before s, for the ceil(n_uniq / 64)
// sets (the capacity slots past them have none); stoff[smax] = all tiles
__global__ __launch_bounds__(1024) void set_plan(const int32_t* __restrict__ nS,
                                                 const int32_t* __restrict__ n_uniq, int smax,
                                                 int32_t* __restrict__ stoff,
                                                 const int32_t* run_flag, int run_want) {
  if (gated_out(run_flag, run_want)) return;
  __shared__ int wtot[16];
  const int tid = threadIdx.x;
  const int nsets = (*n_uniq + BT - 1) / BT;
  int carry = 0;
  for (int base = 0; base < smax; base += 1024) {
    const int si = base + tid;
    const int tiles = si < nsets ? max(1, (nS[si] + UPAD - 1) / UPAD) : 0;
    const int inc = wave_incl_scan(tiles);
    if ((tid & 63) == 63) wtot[tid >> 6] = inc;
    __syncthreads();
    int off = inc - tiles, tot = 0;
#pragma unroll
    for (int w = 0; w < 16; ++w) {
      off += w < (tid >> 6) ? wtot[w] : 0;
      tot += wtot[w];
    }
    if (si < smax) stoff[si] = carry + off;
    carry += tot;
    __syncthreads();
  }
  if (tid == 0) stoff[smax] = carry;
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

namespace {

// blk_union (with the task-slot map when kmap is not null) and blk_plan
hipError_t launch_union_plan(const int32_t* idx, const float* gate, const int32_t* order, int L,
                             int K, const BlockedPlan& p, void* ws, int32_t* kmap, hipStream_t s,
                             RunGate run = {}) {
  char* w = (char*)ws;
  int32_t* U = (int32_t*)(w + p.off_U);
  int32_t* nU = (int32_t*)(w + p.off_nU);
  int32_t* toff = (int32_t*)(w + p.off_toff);
  float* G = (float*)(w + p.off_G);
  // keys and one pad word per thread; two such buffers for the merge sort
  const size_t lds_u = (size_t)(p.sort_keys + 1024) * 4 * (p.sort_keys <= 16 * 1024 ? 2 : 1);
  switch (p.sort_keys / 1024) {
#define OMNI_BLK_UNION(E)                                                                     \
  case E:                                                                                     \
    hipLaunchKernelGGL(blk_union<E>, dim3(p.nb), dim3(1024), lds_u, s, idx, gate, order, L, \
                       K, p.ucap, U, nU, G, kmap, run.flag, run.want);                        \
    break;
    OMNI_BLK_UNION(1) OMNI_BLK_UNION(2) OMNI_BLK_UNION(4) OMNI_BLK_UNION(8) OMNI_BLK_UNION(16)
    OMNI_BLK_UNION(32)
#undef OMNI_BLK_UNION
    default:
      return hipErrorInvalidValue;  // K above the validated limit
  }
  hipLaunchKernelGGL(blk_plan, dim3(1), dim3(1024), 0, s, nU, p.nb, toff, run.flag, run.want);
  return hipGetLastError();
}

int act_grid(const BlockedPlan& p) {
  const int max_tiles = p.nb * (p.ucap / UPAD);
  return 8 * std::min((max_tiles + 7) / 8, MI355X_CUS * K1_WG_PER_CU / 8);
}

// dy = dy_hi + dy_lo, two bf16 terms (round to nearest even, then the rest)
__global__ __launch_bounds__(256) void split_bf16(const float* __restrict__ a, size_t n,
                                                  uint16_t* __restrict__ hi,
                                                  uint16_t* __restrict__ lo,
                                                  const int32_t* run_flag, int run_want) {
  if (gated_out(run_flag, run_want)) return;
  for (size_t i = (size_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (size_t)gridDim.x * 256) {
    const float v = a[i];
    const uint16_t h = bf16_rne(v);
    hi[i] = h;
    lo[i] = bf16_rne(v - __uint_as_float((uint32_t)h << 16));
  }
}

}  // namespace

hipError_t launch_expert_blocked(const void* x, const void* W, const void* V, const int32_t* idx,
                                 const float* gate, const int32_t* order, int L, int d, int K,
                                 float* y, const BlockedPlan& p, void* ws, hipStream_t s,
                                 RunGate run) {
  char* w = (char*)ws;
  const int32_t* U = (const int32_t*)(w + p.off_U);
  const int32_t* toff = (const int32_t*)(w + p.off_toff);
  const float* G = (const float*)(w + p.off_G);
  uint16_t* Ahi = (uint16_t*)(w + p.off_Ahi);
  uint16_t* Alo = (uint16_t*)(w + p.off_Alo);
  hipError_t e = launch_union_plan(idx, gate, order, L, K, p, ws, nullptr, s, run);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(blk_act<BLK_FWD>, dim3(act_grid(p)), dim3(256), K1_S * K1_STAGE, s,
                     (const uint16_t*)x, (const uint16_t*)W, nullptr, nullptr, nullptr, order, U,
                     toff, G, nullptr, L, d, K, p.nb, p.ucap, Ahi, Alo, nullptr, nullptr, nullptr,
                     run.flag, run.want);
  hipLaunchKernelGGL((blk_out<false, 1, false>), dim3(p.nb * (d / K2_COLS)), dim3(256),
                     K2_S * K2_STAGE, s, (const uint16_t*)V, nullptr, order, nullptr, U, toff, Ahi,
                     Alo, L, d, p.ucap, (void*)y, run.flag, run.want);
  return hipGetLastError();
}

BlockedBwdPlan plan_expert_backward_blocked(int64_t L, int64_t d, int64_t N, int64_t K) {
  BlockedBwdPlan p{};
  p.blk = plan_blocked(L, K, N);
  p.bwd = plan_expert_backward(L, d, N, K);
  const int64_t M = L * K;
  p.ucap_e = (int)std::min<int64_t>(N, M);
  p.smax = (p.ucap_e + BT - 1) / BT;
  p.ksort = plan_schedule(p.ucap_e, 1, L + 1, 1);
  // the sets' unions hold at most min(L, tasks) tokens each, in whole tiles
  const size_t tcap = (size_t)M + (size_t)UPAD * p.smax;
  p.set_elems = (size_t)BT * tcap;
  auto a256 = [](size_t n) { return (n + 255) & ~(size_t)255; };
  size_t o = 0;
  p.off_blk = o;    o += a256(p.blk.ws_bytes);
  p.off_kmap = o;   o += a256((size_t)p.blk.nb * BT * p.blk.ucap * 4);
  p.off_dyh = o;    o += a256((size_t)L * d * 2);
  p.off_dyl = o;    o += a256((size_t)L * d * 2);
  p.off_bwd = o;    o += a256(p.bwd.ws_bytes);
  p.off_pos = o;    o += a256((size_t)L * 4);
  p.off_key = o;    o += a256((size_t)p.ucap_e * 4);
  p.off_eord = o;   o += a256((size_t)p.ucap_e * 4);
  p.off_ksort = o;  o += a256(p.ksort.ws_bytes);
  p.off_ns = o;     o += a256((size_t)p.smax * 4);
  p.off_stoff = o;  o += a256((size_t)(p.smax + 1) * 4);
  p.off_T = o;      o += a256(tcap * 4);
  p.off_dht = o;    o += 2 * a256(p.set_elems * 2);
  p.off_gat = o;    o += 2 * a256(p.set_elems * 2);
  p.ws_bytes = o;
  return p;
}

hipError_t launch_expert_backward_blocked(const void* x, const void* W, const void* V,
                                          const int32_t* idx, const float* gate, const float* dy,
                                          const int32_t* order, int L, int d, int N, int K,
                                          float* dx, float* dgate, int32_t* uniq, int32_t* n_uniq,
                                          omni_dtype grad_dt, void* dW_rows, void* dV_rows,
                                          const BlockedBwdPlan& p, void* ws, hipStream_t s,
                                          RunGate run, bool segments_done) {
  char* w = (char*)ws;
  char* wb = w + p.off_blk;
  const BlockedPlan& bp = p.blk;
  const int32_t* U = (const int32_t*)(wb + bp.off_U);
  const int32_t* toff = (const int32_t*)(wb + bp.off_toff);
  const float* G = (const float*)(wb + bp.off_G);
  uint16_t* dHhi = (uint16_t*)(wb + bp.off_Ahi);
  uint16_t* dHlo = (uint16_t*)(wb + bp.off_Alo);
  int32_t* kmap = (int32_t*)(w + p.off_kmap);
  uint16_t* dyh = (uint16_t*)(w + p.off_dyh);
  uint16_t* dyl = (uint16_t*)(w + p.off_dyl);
  char* wr = w + p.off_bwd;
  float* dh = (float*)(wr + p.bwd.off_dh);
  float* ga = (float*)(wr + p.bwd.off_ga);
  const int32_t* perm = (const int32_t*)(wr + p.bwd.off_perm);
  const int32_t* seg = (const int32_t*)(wr + p.bwd.off_seg);
  int32_t* pos = (int32_t*)(w + p.off_pos);
  int32_t* key = (int32_t*)(w + p.off_key);
  int32_t* eord = (int32_t*)(w + p.off_eord);
  int32_t* nS = (int32_t*)(w + p.off_ns);
  int32_t* stoff = (int32_t*)(w + p.off_stoff);
  int32_t* T = (int32_t*)(w + p.off_T);
  const size_t term = ((p.set_elems * 2) + 255) & ~(size_t)255;
  uint16_t* dht_hi = (uint16_t*)(w + p.off_dht);
  uint16_t* dht_lo = (uint16_t*)(w + p.off_dht + term);
  uint16_t* gat_hi = (uint16_t*)(w + p.off_gat);
  uint16_t* gat_lo = (uint16_t*)(w + p.off_gat + term);
  // 1. per token block: dgate, the per-task terms dh and g SiLU(h), and dx
  hipError_t e = launch_union_plan(idx, gate, order, L, K, bp, wb, kmap, s, run);
  if (e != hipSuccess) return e;
  const size_t n = (size_t)L * d;
  hipLaunchKernelGGL(split_bf16, dim3((unsigned)std::min<size_t>((n + 255) / 256, 8192)), dim3(256),
                     0, s, dy, n, dyh, dyl, run.flag, run.want);
  hipLaunchKernelGGL(blk_act<BLK_BWD>, dim3(act_grid(bp)), dim3(256), K1_S * K1_STAGE, s,
                     (const uint16_t*)x, (const uint16_t*)W, dyh, dyl, (const uint16_t*)V, order, U,
                     toff, G, kmap, L, d, K, bp.nb, bp.ucap, dHhi, dHlo, dgate, dh, ga, run.flag,
                     run.want);
  // dx = dH W[U], the forward's second product with W in place of V
  hipLaunchKernelGGL((blk_out<false, 1, false>), dim3(bp.nb * (d / K2_COLS)), dim3(256),
                     K2_S * K2_STAGE, s, (const uint16_t*)W, nullptr, order, nullptr, U, toff, dHhi,
                     dHlo, L, d, bp.ucap, (void*)dx, run.flag, run.want);
  // 2. the used experts (unless the caller has them already), then the expert
  // sets and their dW, dV rows
  if (!segments_done &&
      (e = launch_expert_segments(idx, N, uniq, n_uniq, p.bwd, wr, s)) != hipSuccess)
    return e;
  hipLaunchKernelGGL(inv_order, dim3((L + 255) / 256), dim3(256), 0, s, order, L, pos, run.flag,
                     run.want);
  hipLaunchKernelGGL(set_keys, dim3((unsigned)std::min(2048, (p.ucap_e + 3) / 4)), dim3(256), 0, s,
                     perm, seg, n_uniq, pos, K, L, p.ucap_e, key, run.flag, run.want);
  if ((e = launch_sort_keys(key, p.ucap_e, (int64_t)L + 1, eord, w + p.off_ksort, s, run)) !=
      hipSuccess)
    return e;
  const size_t lds_s = (size_t)2 * ((L + 31) / 32) * 4;
  const dim3 sgrid((unsigned)std::min(p.smax, MI355X_CUS));
  hipLaunchKernelGGL(set_union<true>, sgrid, dim3(1024), lds_s, s, eord, n_uniq, perm, seg, K, L,
                     nullptr, nullptr, nullptr, nS, nullptr, nullptr, nullptr, nullptr, nullptr,
                     run.flag, run.want);
  hipLaunchKernelGGL(set_plan, dim3(1), dim3(1024), 0, s, nS, n_uniq, p.smax, stoff, run.flag,
                     run.want);
  hipLaunchKernelGGL(set_union<false>, sgrid, dim3(1024), lds_s, s, eord, n_uniq, perm, seg, K, L,
                     stoff, dh, ga, nullptr, T, dht_hi, dht_lo, gat_hi, gat_lo, run.flag,
                     run.want);
  const bool obf = grad_dt == OMNI_BF16;
  const dim3 ogrid((unsigned)std::min(p.smax * (d / K2_COLS), 2 * MI355X_CUS));
  const dim3 ogrid2((unsigned)std::min(p.smax * (d / K2_COLS), MI355X_CUS));
  constexpr size_t lds1 = K2_S * (K2_VT + 2 * K2_AT), lds2 = K2_S * (2 * K2_VT + 2 * K2_AT);
  if (obf) {
    hipLaunchKernelGGL((blk_out<true, 1, true>), ogrid, dim3(256), lds1, s, (const uint16_t*)x,
                       nullptr, eord, n_uniq, T, stoff, dht_hi, dht_lo, L, d, 0, dW_rows, run.flag,
                       run.want);
    hipLaunchKernelGGL((blk_out<true, 2, true>), ogrid2, dim3(256), lds2, s, dyh, dyl, eord, n_uniq,
                       T, stoff, gat_hi, gat_lo, L, d, 0, dV_rows, run.flag, run.want);
  } else {
    hipLaunchKernelGGL((blk_out<true, 1, false>), ogrid, dim3(256), lds1, s, (const uint16_t*)x,
                       nullptr, eord, n_uniq, T, stoff, dht_hi, dht_lo, L, d, 0, dW_rows, run.flag,
                       run.want);
    hipLaunchKernelGGL((blk_out<true, 2, false>), ogrid2, dim3(256), lds2, s, dyh, dyl, eord,
                       n_uniq, T, stoff, gat_hi, gat_lo, L, d, 0, dV_rows, run.flag, run.want);
  }
  return hipGetLastError();
}

AutoBwdPlan plan_expert_backward_auto(int64_t L, int64_t d, int64_t N, int64_t K, omni_dtype dt) {
  auto a256 = [](size_t n) { return (n + 255) & ~(size_t)255; };
  AutoBwdPlan p{};
  p.blocked_ok = dt == OMNI_BF16 && d % BLK_D_TILE == 0 && L <= BLK_BWD_MAX_L;
  size_t o = 0;
  if (p.blocked_ok) {
    p.blk = plan_expert_backward_blocked(L, d, N, K);
    p.order_sort = plan_schedule(L, 1, N, 1);
    p.off_flag = o;   o += 256;  // [1] distinct experts in the sample, [2] the sample size
    p.off_bits = o;   o += a256((size_t)((N + 31) / 32) * 4);
    p.off_order = o;  o += a256((size_t)L * 4);
    p.off_osort = o;  o += a256(p.order_sort.ws_bytes);
    p.off_main = o;   o += a256(p.blk.ws_bytes);
  } else {
    p.bwd = plan_expert_backward(L, d, N, K);
    p.off_flag = p.off_bits = p.off_order = p.off_osort = 0;
    p.off_main = o;   o += a256(p.bwd.ws_bytes);
  }
  p.ws_bytes = o;
  return p;
}

hipError_t launch_expert_backward_auto(const void* x, const void* W, const void* V,
                                       const int32_t* idx, const float* gate, const float* dy,
                                       int L, int d, int N, int K, omni_dtype dt, float* dx,
                                       float* dgate, int32_t* uniq, int32_t* n_uniq,
                                       omni_dtype grad_dt, void* dW_rows, void* dV_rows,
                                       int32_t* chosen, const AutoBwdPlan& p, void* ws,
                                       hipStream_t s) {
  char* w = (char*)ws;
  hipError_t e;
  if (!p.blocked_ok) {  // the blocked form cannot take these inputs
    if (chosen && (e = launch_set_i32(chosen, 0, s)) != hipSuccess) return e;
    return launch_expert_backward(x, W, V, idx, gate, dy, L, d, N, K, dt, dx, dgate, uniq, n_uniq,
                                  grad_dt, dW_rows, dV_rows, p.bwd, w + p.off_main, s);
  }
  int32_t* choice = (int32_t*)(w + p.off_flag);
  if ((e = launch_auto_sample(idx, L * K, N, (uint32_t*)(w + p.off_bits), choice, s)) !=
      hipSuccess)
    return e;
  const RunGate per_task{choice, 0}, blocked{choice, 1};
  char* wm = w + p.off_main;
  char* wt = wm + p.blk.off_bwd;  // the per-task plan's region, used by both forms
  int32_t* order = (int32_t*)(w + p.off_order);
  // the blocked form's token order (tokens sorted by their first expert);
  // its first launch records the choice
  if ((e = launch_token_order(idx, L, K, N, 1, order, w + p.off_osort, s, blocked, chosen)) !=
      hipSuccess)
    return e;
  // both forms: the tasks sorted by expert, the used experts and segments
  if ((e = launch_expert_segments(idx, N, uniq, n_uniq, p.blk.bwd, wt, s)) != hipSuccess) return e;
  // per-task form
  if ((e = launch_expert_bwd_token(x, W, V, idx, gate, dy, L, d, K, dt, dx, dgate, n_uniq,
                                   p.blk.bwd, wt, s, per_task)) != hipSuccess)
    return e;
  if ((e = launch_expert_grad_rows(x, dy, d, K, dt, n_uniq, grad_dt, dW_rows, dV_rows, p.blk.bwd,
                                   wt, s, per_task)) != hipSuccess)
    return e;
  // blocked form
  return launch_expert_backward_blocked(x, W, V, idx, gate, dy, order, L, d, N, K, dx, dgate, uniq,
                                        n_uniq, grad_dt, dW_rows, dV_rows, p.blk, wm, s, blocked,
                                        /*segments_done=*/true);
}

}  // namespace omni
