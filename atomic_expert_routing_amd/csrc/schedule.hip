// Expert-centric scheduling on gfx950.
//
// OmniMoE digest (paper.rainbus.top), method paragraph, step 3: the L*K
// routing tasks are sorted by expert id into contiguous groups of size B,
// group id first, token id second; gist.science resume section 2.2: groups
// are contiguous ranges of expert ids.
//
// Task m = t*K + k lists the tasks token-major, so the task order already
// sorts by (token, m).  A STABLE sort of the tasks by group id alone
// therefore yields the order (group, token, m): the key needs only
// ceil(log2 G) bits.  It is an LSD radix sort with up to 8-bit digits:
//   sched_hist     per-tile digit histograms (digit-major table)
//   sched_scan_digits  per digit: exclusive scan over tiles, digit total
//   sched_scatter  stable scatter: in-tile ranks from wave ballots
// followed by sched_offsets, which turns the sorted group ids into
// group_off[q] = first sorted position whose group is >= q.
//
// The same sort, over the L tokens keyed by the group of each token's first
// expert, gives the token order the output pass may follow: tokens whose
// leading experts coincide run next to each other (and on one XCD).

#include "omni_internal.h"

namespace omni {
namespace {

constexpr int SCHED_THREADS = 256;
// A tile is `rounds` x 256 elements, rounds a power of two from 2 to 16:
// the smallest that keeps the tile count at or below SCHED_MAX_TILES.  The
// passes are latency bound; measured (one pass pair + offsets) at 2^19
// elements 36 us with 1024 tiles against 42 us with 256, at 2^22 elements
// 95 us with 1024 tiles against 100 us with 2048 and 122 us with 8192.
constexpr int SCHED_MAX_TILES = 1024;

// Element p's key: its group, idx[p * stride] / B, in the first pass; the
// previous pass's sorted key afterwards.
__device__ __forceinline__ int load_key(const int32_t* __restrict__ idx,
                                        const int32_t* __restrict__ keys_in, int p, int stride,
                                        int B) {
  return keys_in ? keys_in[p] : idx[(size_t)p * stride] / B;
}

__global__ __launch_bounds__(SCHED_THREADS) void sched_hist(const int32_t* __restrict__ idx,
                                                            const int32_t* __restrict__ keys_in,
                                                            int M, int stride, int B, int shift,
                                                            int radix, int rounds,
                                                            int ntiles, int* __restrict__ hist) {
  __shared__ int h[256];
  const int tid = threadIdx.x, tile = blockIdx.x;
  if (tid < radix) h[tid] = 0;
  __syncthreads();
  const int base = tile * rounds * SCHED_THREADS;
  for (int r = 0; r < rounds; ++r) {
    const int p = base + r * SCHED_THREADS + tid;
    if (p < M) atomicAdd(&h[(load_key(idx, keys_in, p, stride, B) >> shift) & (radix - 1)], 1);
  }
  __syncthreads();
  if (tid < radix) hist[tid * ntiles + tile] = h[tid];
}

// Row d of the digit-major table holds digit d's count in every tile.  One
// workgroup per digit turns its row into an exclusive scan over tiles and
// stores the digit's total.
__global__ __launch_bounds__(SCHED_THREADS) void sched_scan_digits(int* __restrict__ hist,
                                                                   int ntiles,
                                                                   int* __restrict__ totals) {
  __shared__ int wsum[SCHED_THREADS / 64];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  int* row = hist + (size_t)blockIdx.x * ntiles;
  int carry = 0;
  for (int base = 0; base < ntiles; base += SCHED_THREADS * 4) {
    const int i0 = base + tid * 4;
    int v[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) v[q] = i0 + q < ntiles ? row[i0 + q] : 0;
    const int s = v[0] + v[1] + v[2] + v[3];
    const int inc = wave_incl_scan(s);
    if (lane == 63) wsum[wave] = inc;
    __syncthreads();
    int woff = 0, tot = 0;
#pragma unroll
    for (int w = 0; w < SCHED_THREADS / 64; ++w) {
      woff += w < wave ? wsum[w] : 0;
      tot += wsum[w];
    }
    int run = carry + woff + inc - s;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      if (i0 + q < ntiles) row[i0 + q] = run;
      run += v[q];
    }
    carry += tot;
    __syncthreads();
  }
  if (tid == 0) totals[blockIdx.x] = carry;
}

__global__ __launch_bounds__(SCHED_THREADS) void sched_scatter(
    const int32_t* __restrict__ idx, const int32_t* __restrict__ keys_in,
    const int32_t* __restrict__ vals_in, int M, int stride, int B, int shift, int radix,
    int rounds, int ntiles,
    const int* __restrict__ hist, const int* __restrict__ totals, int32_t* __restrict__ keys_out,
    int32_t* __restrict__ vals_out) {
  __shared__ int run[256];
  __shared__ int wcnt[SCHED_THREADS / 64][256];
  const int tid = threadIdx.x, tile = blockIdx.x;
  const int wave = tid >> 6, lane = tid & 63;
  const int dbits = 31 - __clz(radix);
  if (wave == 0) {
    // exclusive scan of the digit totals (radix <= 256: 4 per lane)
    int v[4], s = 0;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      v[q] = 4 * lane + q < radix ? totals[4 * lane + q] : 0;
      s += v[q];
    }
    const int inc = wave_incl_scan(s);
    int b = inc - s;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      if (4 * lane + q < radix) run[4 * lane + q] = b;
      b += v[q];
    }
  }
  if (tid < radix) {
#pragma unroll
    for (int w = 0; w < SCHED_THREADS / 64; ++w) wcnt[w][tid] = 0;
  }
  __syncthreads();
  if (tid < radix) run[tid] += hist[(size_t)tid * ntiles + tile];
  __syncthreads();
  const unsigned long long lt = (1ull << lane) - 1ull;
  const int base = tile * rounds * SCHED_THREADS;
  for (int r = 0; r < rounds; ++r) {
    const int p = base + r * SCHED_THREADS + tid;
    const bool act = p < M;
    int key = 0, val = 0, dig = 0;
    if (act) {
      key = load_key(idx, keys_in, p, stride, B);
      val = vals_in ? vals_in[p] : p;
      dig = (key >> shift) & (radix - 1);
    }
    // lanes of this wave holding the same digit (ballot per digit bit)
    unsigned long long peers = __ballot(act);
    for (int b = 0; b < dbits; ++b) {
      const unsigned long long m = __ballot((dig >> b) & 1);
      peers &= ((dig >> b) & 1) ? m : ~m;
    }
    const int rank = __popcll(peers & lt);
    if (act && (peers >> lane) == 1ull) wcnt[wave][dig] = __popcll(peers);  // highest peer
    __syncthreads();
    if (act) {
      int pos = run[dig] + rank;
      for (int w = 0; w < wave; ++w) pos += wcnt[w][dig];
      keys_out[pos] = key;
      vals_out[pos] = val;
    }
    __syncthreads();
    if (tid < radix) {
      int s = 0;
#pragma unroll
      for (int w = 0; w < SCHED_THREADS / 64; ++w) {
        s += wcnt[w][tid];
        wcnt[w][tid] = 0;
      }
      run[tid] += s;
    }
    __syncthreads();
  }
}

// group_off[q] = first sorted position p with key[p] >= q, for q in [0, G]:
// position p owns the entries prev+1 .. cur between its key and the one
// before.  Short runs are written by their owner; a wave writes its lanes'
// long runs together, 64 entries per store (with one expert per group and
// clustered routing the runs of unused ids reach thousands: one lane
// writing them took 108 us).
__global__ __launch_bounds__(256) void sched_offsets(const int32_t* __restrict__ keys, int M,
                                                     int G, int32_t* __restrict__ off) {
  const int p = blockIdx.x * blockDim.x + threadIdx.x, lane = threadIdx.x & 63;
  // ids outside [0, N) break the precondition; clamping keeps the writes in
  // bounds (the offsets are then meaningless, but nothing is corrupted)
  int prev = 0, cur = 0;  // past M: an empty run
  if (p <= M) {
    prev = p == 0 ? -1 : max(-1, min(G, keys[p - 1]));
    cur = p == M ? G : max(-1, min(G, keys[p]));
  }
  const int n = cur - prev;
  if (n > 0 && n <= 16)
    for (int q = prev + 1; q <= cur; ++q) off[q] = p;
  unsigned long long longs = __ballot(n > 16);  // every lane of the wave is here
  while (longs) {
    const int l = __builtin_ctzll(longs);
    longs &= longs - 1;
    const int owner = __builtin_amdgcn_readlane(p, l);
    const int hi = __builtin_amdgcn_readlane(cur, l);
    for (int q = __builtin_amdgcn_readlane(prev, l) + 1 + lane; q <= hi; q += 64) off[q] = owner;
  }
}

size_t align256(size_t n) { return (n + 255) & ~(size_t)255; }

}  // namespace

SchedPlan plan_schedule(int64_t L, int64_t K, int64_t N, int64_t B) {
  SchedPlan p{};
  p.M = (int)(L * K);
  p.G = (int)((N + B - 1) / B);
  int bits = 1;
  while (bits < 31 && (1ll << bits) < p.G) ++bits;  // groups 0 .. G-1 fit in `bits`
  p.passes = (bits + 7) / 8;
  p.digit_bits = (bits + p.passes - 1) / p.passes;
  p.rounds = 2;
  while (p.rounds < 16 && ((int64_t)p.M + SCHED_THREADS * p.rounds - 1) / (SCHED_THREADS * p.rounds) >
                              SCHED_MAX_TILES)
    p.rounds *= 2;
  p.ntiles = (p.M + SCHED_THREADS * p.rounds - 1) / (SCHED_THREADS * p.rounds);
  const size_t arr = align256((size_t)p.M * 4);
  p.off_keys_a = 0;
  p.off_vals_a = arr;
  p.off_keys_b = 2 * arr;
  p.off_vals_b = 3 * arr;
  p.off_hist = 4 * arr;
  p.off_totals = p.off_hist + align256((size_t)(1 << p.digit_bits) * p.ntiles * 4);
  p.ws_bytes = p.off_totals + align256(256 * 4);
  return p;
}

const int32_t* schedule_sorted_keys(const SchedPlan& plan, const void* ws) {
  const char* w = (const char*)ws;
  return (const int32_t*)(w + (((plan.passes - 1) & 1) ? plan.off_keys_b : plan.off_keys_a));
}

namespace {

// Stable LSD sort of the elements p < M by group idx[p * stride] / B; the
// last pass writes the element indices in sorted order to `vals_last` and
// leaves the sorted keys in the workspace.
void sort_by_group(const int32_t* idx, int stride, int M, int B, const SchedPlan& plan,
                   int32_t* vals_last, void* ws, hipStream_t s) {
  char* w = (char*)ws;
  int32_t* ka = (int32_t*)(w + plan.off_keys_a);
  int32_t* va = (int32_t*)(w + plan.off_vals_a);
  int32_t* kb = (int32_t*)(w + plan.off_keys_b);
  int32_t* vb = (int32_t*)(w + plan.off_vals_b);
  int* hist = (int*)(w + plan.off_hist);
  int* totals = (int*)(w + plan.off_totals);
  const int radix = 1 << plan.digit_bits;
  const int32_t* kin = nullptr;  // pass 0 derives keys from idx
  const int32_t* vin = nullptr;  // pass 0 values are the element ids
  for (int pass = 0; pass < plan.passes; ++pass) {
    const bool last = pass + 1 == plan.passes;
    int32_t* kout = (pass & 1) ? kb : ka;
    int32_t* vout = last ? vals_last : ((pass & 1) ? vb : va);
    const int shift = pass * plan.digit_bits;
    hipLaunchKernelGGL(sched_hist, dim3(plan.ntiles), dim3(SCHED_THREADS), 0, s, idx, kin, M,
                       stride, B, shift, radix, plan.rounds, plan.ntiles, hist);
    hipLaunchKernelGGL(sched_scan_digits, dim3(radix), dim3(SCHED_THREADS), 0, s, hist,
                       plan.ntiles, totals);
    hipLaunchKernelGGL(sched_scatter, dim3(plan.ntiles), dim3(SCHED_THREADS), 0, s, idx, kin, vin,
                       M, stride, B, shift, radix, plan.rounds, plan.ntiles, hist, totals, kout,
                       vout);
    kin = kout;
    vin = vout;
  }
}

}  // namespace

hipError_t launch_schedule(const int32_t* idx, int M, int B, int G, const SchedPlan& plan,
                           int32_t* perm, int32_t* group_off, void* ws, hipStream_t s) {
  sort_by_group(idx, 1, M, B, plan, perm, ws, s);
  hipLaunchKernelGGL(sched_offsets, dim3((M + 1 + 255) / 256), dim3(256), 0, s,
                     schedule_sorted_keys(plan, ws), M, G, group_off);
  return hipGetLastError();
}

hipError_t launch_sort_keys(const int32_t* keys, int M, int64_t key_bound, int32_t* order,
                            void* ws, hipStream_t s) {
  const SchedPlan plan = plan_schedule(M, 1, key_bound, 1);
  sort_by_group(keys, 1, M, 1, plan, order, ws, s);
  return hipGetLastError();
}

hipError_t launch_token_order(const int32_t* idx, int L, int K, int64_t N, int B,
                              int32_t* order, void* ws, hipStream_t s) {
  // the plan for L elements needs no more workspace than the one for L*K
  const SchedPlan plan = plan_schedule(L, 1, N, B);
  sort_by_group(idx, K, L, B, plan, order, ws, s);
  return hipGetLastError();
}

}  // namespace omni
