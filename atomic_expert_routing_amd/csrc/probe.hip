// Measurement aid: the rate at which this GPU gathers whole rows of a large
// matrix at random, the access pattern of the expert assembly (each W or V
// row is one atomic expert's vector).  The benchmark times it on the rows a
// step actually uses, so that the assembly's achieved HBM rate can be set
// against what the memory system delivers for that pattern, besides the
// nominal peak.

#include "omni_internal.h"

namespace omni {
namespace {

constexpr int PROBE_ROWS = 8;  // rows in flight per wave

// Wave w of the grid reads rows w, w + waves, ... of the list, each row as
// 16-byte chunks spread over the 64 lanes, PROBE_ROWS rows at a time, and
// stores one checksum per lane so that no load is dead.  The loads are
// non-temporal, the fastest form measured for rows read once: the 447,367
// used rows (4 KB each) of the 4096-token, 1.7M-expert step gather at
// 6.1 TB/s this way against 4.8 TB/s with plain loads (buffer loads and 4 to
// 16 rows in flight within 2%); the used 1.5 KB rows at 280,900 experts at
// 4.7 against 2.4 TB/s.
__global__ __launch_bounds__(256) void gather_rows(const unsigned char* __restrict__ A,
                                                   int64_t nA, const int32_t* __restrict__ rows,
                                                   int64_t n, int row_bytes,
                                                   float* __restrict__ sink) {
  const int lane = threadIdx.x & 63;
  const int64_t wave = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  const int64_t waves = (int64_t)gridDim.x * 4;
  const int chunks = row_bytes / 16;
  float acc = 0.f;
  for (int64_t r0 = wave * PROBE_ROWS; r0 < n; r0 += waves * PROBE_ROWS) {
    for (int c0 = 0; c0 < chunks; c0 += 64) {
      const int c = c0 + lane;
      u32x4 v[PROBE_ROWS];
#pragma unroll
      for (int j = 0; j < PROBE_ROWS; ++j) {
        const int64_t r = r0 + j;
        const int64_t row = r < n ? rows[r] : -1;  // ids outside [0, nA) are skipped
        v[j] = (row >= 0 && row < nA && c < chunks)
                   ? __builtin_nontemporal_load(
                         (const u32x4*)(A + (size_t)row * (size_t)row_bytes + (size_t)c * 16))
                   : u32x4{0u, 0u, 0u, 0u};
      }
#pragma unroll
      for (int j = 0; j < PROBE_ROWS; ++j)
        acc += __uint_as_float(v[j].x & 0x3fffffffu) + __uint_as_float(v[j].w & 0x3fffffffu);
    }
  }
  sink[(size_t)blockIdx.x * 256 + threadIdx.x] = acc;
}

}  // namespace

int gather_probe_blocks(int64_t n) {
  const int64_t want = (n + 4 * PROBE_ROWS - 1) / (4 * PROBE_ROWS);
  return (int)(want < 8192 ? (want < 1 ? 1 : want) : 8192);
}

hipError_t launch_gather_probe(const void* A, int64_t nA, const int32_t* rows, int64_t n,
                               int row_bytes, float* sink, hipStream_t s) {
  hipLaunchKernelGGL(gather_rows, dim3(gather_probe_blocks(n)), dim3(256), 0, s,
                     (const unsigned char*)A, nA, rows, n, row_bytes, sink);
  return hipGetLastError();
}

}  // namespace omni
