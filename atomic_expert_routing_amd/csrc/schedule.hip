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
// ceil(log2 G) bits.  It is an LSD radix sort with up to 8-bit digits, three
// launches per pass:
//   sched_hist     per-tile digit counts of the current order
//   sched_scan     per digit: exclusive scan over tiles, digit total
//   sched_scatter  stable scatter: in-tile ranks from wave ballots; the first
//                  pass also counts the tasks of every group, and the last
//                  workgroup of the last pass turns those counts into
//                  group_off[q] = number of tasks whose group is < q.
// With more groups than fit a workgroup's LDS, sched_offsets takes the group
// offsets from the sorted group ids instead (one more launch).
//
// The same sort, over the L tokens keyed by the group of each token's first
// expert, gives the token order the output pass may follow: tokens whose
// leading experts coincide run next to each other (and on one XCD).

#include "omni_internal.h"

namespace omni {
namespace {


// The histogram and scatter kernels run 16 waves per workgroup over tiles of
// `rounds` x 1024 elements, rounds the smallest power of two that keeps the
// tile count at or below SORT_MAX_TILES (so that one workgroup of the scan
// kernel covers a digit's whole row of tiles with one thread per tile).
constexpr int SORT_THREADS = 1024;
constexpr int SORT_WAVES = SORT_THREADS / 64;
constexpr int SORT_MAX_TILES = 256;


// Element p's key: its group, idx[p * stride] / B, in the first pass; the
// previous pass's sorted key afterwards.
__device__ __forceinline__ int load_key(const int32_t* __restrict__ idx,
                                        const int32_t* __restrict__ keys_in, int p, int stride,
                                        int B) {
  return keys_in ? keys_in[p] : idx[(size_t)p * stride] / B;
}

// Digit counts of one pass for each tile of the current order:
// hist[digit * ntiles + tile].  The first pass's launch also clears the group
// counts and the ticket that the scatter passes accumulate into.
__global__ __launch_bounds__(SORT_THREADS) void sched_hist(
    const int32_t* __restrict__ idx, const int32_t* __restrict__ keys_in, int M, int stride,
    int B, int shift, int dbits, int rounds, int ntiles, int* __restrict__ hist,
    int* __restrict__ gcount, int gclear, int* __restrict__ ticket, const int32_t* run_flag,
    int run_want) {
  if (gated_out(run_flag, run_want)) return;
  __shared__ int h[256];
  const int tid = threadIdx.x, tile = blockIdx.x;
  const int radix = 1 << dbits;
  if (tid < 256) h[tid] = 0;
  __syncthreads();
  const int base = tile * rounds * SORT_THREADS;
  for (int r = 0; r < rounds; ++r) {
    const int p = base + r * SORT_THREADS + tid;
    if (p < M) atomicAdd(&h[(load_key(idx, keys_in, p, stride, B) >> shift) & (radix - 1)], 1);
  }
  __syncthreads();
  if (tid < radix) hist[(size_t)tid * ntiles + tile] = h[tid];
  for (int g = tile * SORT_THREADS + tid; g < gclear; g += ntiles * SORT_THREADS) gcount[g] = 0;
  if (gclear && tile == 0 && tid == 0) ticket[0] = 0;
}

// One workgroup per digit: exclusive scan of the digit's row over the tiles
// (one thread per tile) in place, and the digit's total.
__global__ __launch_bounds__(SORT_MAX_TILES) void sched_scan(int* __restrict__ hist, int ntiles,
                                                             int* __restrict__ totals,
                                                             const int32_t* run_flag,
                                                             int run_want) {
  if (gated_out(run_flag, run_want)) return;
  __shared__ int wsum[SORT_MAX_TILES / 64];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  int* row = hist + (size_t)blockIdx.x * ntiles;
  const int v = tid < ntiles ? row[tid] : 0;
  const int inc = wave_incl_scan(v);
  if (lane == 63) wsum[wave] = inc;
  __syncthreads();
  int off = 0, tot = 0;
#pragma unroll
  for (int w = 0; w < SORT_MAX_TILES / 64; ++w) {
    off += w < wave ? wsum[w] : 0;
    tot += wsum[w];
  }
  if (tid < ntiles) row[tid] = off + inc - v;
  if (tid == 0) totals[blockIdx.x] = tot;
}

// Stable scatter of one pass.  In-tile ranks come from 64-bit wave ballots
// over the digit bits; the waves of a round then take their places in wave
// order from a per-digit prefix over the waves.
// With the group counts gcount (G <= GROUP_HIST_MAX, cleared by the first
// pass's sched_hist):
//   count (first pass): the tile's group counts are gathered in LDS, two
//     16-bit counters to a word (a tile holds at most 32768 elements), and
//     added into gcount;
//   off != null (last pass): the workgroup that finishes last (a ticket after
//     a device-scope fence) turns gcount into the group offsets
//     off[q] = sum of gcount[0 .. q), off[G] = M.
// Positions outside [0, M) are never written (they cannot occur when the
// counts match the keys; the guard keeps any mismatch from writing out of
// bounds).
__global__ __launch_bounds__(SORT_THREADS) void sched_scatter(
    const int32_t* __restrict__ idx, const int32_t* __restrict__ keys_in,
    const int32_t* __restrict__ vals_in, int M, int stride, int B, int shift, int dbits,
    int rounds, int ntiles, const int* __restrict__ hist, const int* __restrict__ totals,
    int32_t* __restrict__ keys_out, int32_t* __restrict__ vals_out, int G,
    int* __restrict__ gcount, int count, int32_t* __restrict__ off, int* __restrict__ ticket,
    const int32_t* run_flag, int run_want) {
  if (gated_out(run_flag, run_want)) return;
  if (!gcount) {  // no group counts: neither counting nor offsets
    count = 0;
    off = nullptr;
  }
  extern __shared__ unsigned ghist[];  // [(G + 1) / 2] when counting: group g in half g & 1
  __shared__ int run[256];
  __shared__ unsigned short wcnt[SORT_WAVES][256];  // counts <= 64, prefixes <= 1024
  __shared__ int wsum[SORT_WAVES];
  __shared__ int is_last;
  const int tid = threadIdx.x, tile = blockIdx.x;
  const int wave = tid >> 6, lane = tid & 63;
  const int radix = 1 << dbits;
  const int gwords = (G + 1) / 2;
  if (count)
    for (int g = tid; g < gwords; g += SORT_THREADS) ghist[g] = 0u;
  if (wave == 0) {
    // exclusive scan of the digit totals (radix <= 256: 4 per lane), plus the
    // tile's exclusive prefix per digit
    int v[4], sum = 0;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      v[q] = 4 * lane + q < radix ? totals[4 * lane + q] : 0;
      sum += v[q];
    }
    const int inc = wave_incl_scan(sum);
    int b = inc - sum;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      if (4 * lane + q < radix) run[4 * lane + q] = b + hist[(size_t)(4 * lane + q) * ntiles + tile];
      b += v[q];
    }
  }
  __syncthreads();
  const unsigned long long lt = (1ull << lane) - 1ull;
  const int base = tile * rounds * SORT_THREADS;
  for (int r = 0; r < rounds; ++r) {
    const int p = base + r * SORT_THREADS + tid;
    const bool act = p < M;
    int key = 0, val = 0, dig = 0;
    if (act) {
      key = load_key(idx, keys_in, p, stride, B);
      val = vals_in ? vals_in[p] : p;
      dig = (key >> shift) & (radix - 1);
      if (count) {
        const int g = min(max(key, 0), G - 1);
        atomicAdd(&ghist[g >> 1], 1u << ((g & 1) * 16));
      }
    }
    // lanes of this wave holding the same digit (ballot per digit bit)
    unsigned long long peers = __ballot(act);
    for (int b = 0; b < dbits; ++b) {
      const unsigned long long m = __ballot((dig >> b) & 1);
      peers &= ((dig >> b) & 1) ? m : ~m;
    }
    const int rank = __popcll(peers & lt);
    for (int d = tid; d < SORT_WAVES * 256; d += SORT_THREADS) (&wcnt[0][0])[d] = 0;
    __syncthreads();
    if (act && (peers >> lane) == 1ull)  // highest peer
      wcnt[wave][dig] = (unsigned short)__popcll(peers);
    __syncthreads();
    // per digit: exclusive prefix over the waves, in place; the total moves run
    int tot = 0;
    if (tid < radix) {
#pragma unroll
      for (int w = 0; w < SORT_WAVES; ++w) {
        const int c = wcnt[w][tid];
        wcnt[w][tid] = (unsigned short)tot;
        tot += c;
      }
    }
    __syncthreads();
    if (act) {
      const int pos = run[dig] + wcnt[wave][dig] + rank;
      if ((unsigned)pos < (unsigned)M) {
        keys_out[pos] = key;
        vals_out[pos] = val;
      }
    }
    __syncthreads();
    if (tid < radix) run[tid] += tot;
  }
  if (count) {
    __syncthreads();
    for (int g2 = tid; g2 < gwords; g2 += SORT_THREADS) {
      const unsigned v = ghist[g2];
      if (v & 0xffffu) atomicAdd(&gcount[2 * g2], (int)(v & 0xffffu));
      if (v >> 16) atomicAdd(&gcount[2 * g2 + 1], (int)(v >> 16));  // then 2 * g2 + 1 < G
    }
  }
  if (!off) return;
  // the last workgroup to finish turns the group counts into offsets
  // counts added in this launch (a single pass) are made visible before the
  // ticket; with more passes they were completed by an earlier launch, and the
  // device-scope fence in every wave (an L2 write-back on this chip) would
  // cost more than the whole scatter
  if (count) __threadfence();
  __syncthreads();
  if (tid == 0) is_last = atomicAdd(ticket, 1) == ntiles - 1;
  __syncthreads();
  if (!is_last) return;
  __threadfence();
  const int per = (G + SORT_THREADS - 1) / SORT_THREADS;  // <= GROUP_HIST_MAX / 1024
  int cnt[GROUP_HIST_MAX / SORT_THREADS], sum = 0;
#pragma unroll
  for (int i = 0; i < GROUP_HIST_MAX / SORT_THREADS; ++i) {
    const int g = tid * per + i;
    cnt[i] = (i < per && g < G) ? __hip_atomic_load(&gcount[g], __ATOMIC_RELAXED,
                                                    __HIP_MEMORY_SCOPE_AGENT)
                                : 0;
    sum += cnt[i];
  }
  const int inc = wave_incl_scan(sum);
  if (lane == 63) wsum[wave] = inc;
  __syncthreads();
  int before = inc - sum;
  for (int w = 0; w < wave; ++w) before += wsum[w];
#pragma unroll
  for (int i = 0; i < GROUP_HIST_MAX / SORT_THREADS; ++i) {
    const int g = tid * per + i;
    if (i < per && g < G) off[g] = before;
    before += cnt[i];
  }
  if (tid == SORT_THREADS - 1) off[G] = before;  // = M
}

// group_off[q] = first sorted position p with key[p] >= q, for q in [0, G]:
// position p owns the entries prev+1 .. cur between its key and the one
// before.  Short runs are written by their owner; a wave writes its lanes'
// long runs together, 64 entries per store (with one expert per group and
// clustered routing the runs of unused ids reach thousands: one lane
// writing them took 108 us).
__global__ __launch_bounds__(256) void sched_offsets(const int32_t* __restrict__ keys, int M,
                                                     int G, int32_t* __restrict__ off,
                                                     const int32_t* run_flag, int run_want) {
  if (gated_out(run_flag, run_want)) return;
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
  p.rounds = 1;
  while (((int64_t)p.M + (int64_t)SORT_THREADS * p.rounds - 1) /
             ((int64_t)SORT_THREADS * p.rounds) > SORT_MAX_TILES)
    p.rounds *= 2;
  p.ntiles = (int)(((int64_t)p.M + (int64_t)SORT_THREADS * p.rounds - 1) /
                   ((int64_t)SORT_THREADS * p.rounds));
  // the scatter's 16-bit LDS group counters hold a tile of at most 32768 elements
  p.group_hist = p.G <= GROUP_HIST_MAX && p.rounds * SORT_THREADS <= 32768;
  const int radix = 1 << p.digit_bits;
  const size_t arr = align256((size_t)p.M * 4);
  p.off_keys_a = 0;
  p.off_vals_a = arr;
  p.off_keys_b = 2 * arr;
  p.off_vals_b = 3 * arr;
  p.off_hist = 4 * arr;
  p.off_totals = p.off_hist + align256((size_t)radix * p.ntiles * 4);
  p.off_gcount = p.off_totals + align256((size_t)radix * 4);
  p.off_ticket = p.off_gcount + (p.group_hist ? align256((size_t)p.G * 4) : 0);
  p.ws_bytes = p.off_ticket + 256;
  return p;
}

const int32_t* schedule_sorted_keys(const SchedPlan& plan, const void* ws) {
  const char* w = (const char*)ws;
  return (const int32_t*)(w + (((plan.passes - 1) & 1) ? plan.off_keys_b : plan.off_keys_a));
}

namespace {

// Stable LSD sort of the elements p < M by group idx[p * stride] / B; the
// last pass writes the element indices in sorted order to `vals_last` and
// leaves the sorted keys in the workspace.  With group_off given (and at most
// GROUP_HIST_MAX groups) the last pass also writes the group offsets.
// Launches: the digit counts of all passes, their scan, one scatter per pass.
void sort_by_group(const int32_t* idx, int stride, int M, int B, const SchedPlan& plan,
                   int32_t* vals_last, int32_t* group_off, void* ws, hipStream_t s,
                   RunGate run = {}) {
  char* w = (char*)ws;
  int32_t* ka = (int32_t*)(w + plan.off_keys_a);
  int32_t* va = (int32_t*)(w + plan.off_vals_a);
  int32_t* kb = (int32_t*)(w + plan.off_keys_b);
  int32_t* vb = (int32_t*)(w + plan.off_vals_b);
  int* hist = (int*)(w + plan.off_hist);
  int* totals = (int*)(w + plan.off_totals);
  int* gcount = (int*)(w + plan.off_gcount);
  int* ticket = (int*)(w + plan.off_ticket);
  const int radix = 1 << plan.digit_bits;
  const bool offsets = group_off && plan.group_hist;
  const int32_t* kin = nullptr;  // pass 0 derives keys from idx
  const int32_t* vin = nullptr;  // pass 0 values are the element ids
  for (int pass = 0; pass < plan.passes; ++pass) {
    const bool first = pass == 0, last = pass + 1 == plan.passes;
    int32_t* kout = (pass & 1) ? kb : ka;
    int32_t* vout = last ? vals_last : ((pass & 1) ? vb : va);
    const int shift = pass * plan.digit_bits;
    hipLaunchKernelGGL(sched_hist, dim3(plan.ntiles), dim3(SORT_THREADS), 0, s, idx, kin, M,
                       stride, B, shift, plan.digit_bits, plan.rounds, plan.ntiles, hist, gcount,
                       offsets && first ? plan.G : 0, ticket, run.flag, run.want);
    hipLaunchKernelGGL(sched_scan, dim3(radix), dim3(SORT_MAX_TILES), 0, s, hist, plan.ntiles,
                       totals, run.flag, run.want);
    // the group counts: gathered by the first pass, turned into offsets by
    // the last (the same pass when there is one)
    const size_t lds = offsets && first ? (size_t)(plan.G + 1) / 2 * 4 : 0;
    hipLaunchKernelGGL(sched_scatter, dim3(plan.ntiles), dim3(SORT_THREADS), lds, s, idx, kin,
                       vin, M, stride, B, shift, plan.digit_bits, plan.rounds, plan.ntiles, hist,
                       totals, kout, vout, plan.G, offsets ? gcount : nullptr,
                       offsets && first ? 1 : 0, offsets && last ? group_off : nullptr, ticket,
                       run.flag, run.want);
    kin = kout;
    vin = vout;
  }
}

}  // namespace

hipError_t launch_schedule(const int32_t* idx, int M, int B, int G, const SchedPlan& plan,
                           int32_t* perm, int32_t* group_off, void* ws, hipStream_t s,
                           RunGate run) {
  sort_by_group(idx, 1, M, B, plan, perm, group_off, ws, s, run);
  if (!plan.group_hist)  // too many groups for the scatter's LDS: offsets from the sorted keys
    hipLaunchKernelGGL(sched_offsets, dim3((M + 1 + 255) / 256), dim3(256), 0, s,
                       schedule_sorted_keys(plan, ws), M, G, group_off, run.flag, run.want);
  return hipGetLastError();
}

hipError_t launch_sort_keys(const int32_t* keys, int M, int64_t key_bound, int32_t* order,
                            void* ws, hipStream_t s) {
  const SchedPlan plan = plan_schedule(M, 1, key_bound, 1);
  sort_by_group(keys, 1, M, 1, plan, order, nullptr, ws, s);
  return hipGetLastError();
}

hipError_t launch_token_order(const int32_t* idx, int L, int K, int64_t N, int B,
                              int32_t* order, void* ws, hipStream_t s, RunGate run) {
  // the plan for L elements needs no more workspace than the one for L*K
  const SchedPlan plan = plan_schedule(L, 1, N, B);
  sort_by_group(idx, K, L, B, plan, order, nullptr, ws, s, run);
  return hipGetLastError();
}

}  // namespace omni
