// Pipelined MFMA product C = A . B^T on gfx950 (bf16 in, fp32 accumulate).
//
// It computes the router's logits x [W_r; W_c]^T (OmniMoE digest,
// paper.rainbus.top, method paragraph, step 2), the router backward's
// products, and the shared dense MLP's gate/up and down projections
// (digest, step 1: the + MLP(x) branch).

#include "mfma_pipe.h"

namespace omni {
namespace {

constexpr int GEMM_PLAIN = 0, GEMM_SWIGLU = 1;

// ------------------------------------------------------------------ bf16 GEMM, pipelined
// Output tiles per workgroup (below), with the k-tiles (BK deep)
// streamed through S LDS stages by direct global->LDS loads
// (global_load_lds_dwordx4: each instruction writes 64 lanes x 16 bytes of
// LDS without register staging), so S-1 k-tiles are in flight while one is
// multiplied.  A stage holds the A and B tiles as rows of 2*BK bytes; the
// 16-byte chunk c of row r sits in slot c ^ swz(r), which spreads the 16
// rows read by one ds_read_b128 over 16 distinct bank groups.  Rows past L
// or N_r+N_c are loaded from a clamped row (their results are never
// stored).  Needs d % BK == 0 (no partial k-tile).

// MODE GEMM_PLAIN writes fp32 C.  MODE GEMM_SWIGLU is the first half of a
// SwiGLU block: the B rows are taken as alternating 16-row blocks of B0
// (gate projection) and B1 (up projection), N = 2 d_ff, and the epilogue
// writes bf16 SiLU(gate) * up to Cb [M, ldc = d_ff].
//
// Tiles are (16 MI WVM) x (16 NJ WVN): WVM x WVN waves, each 16 MI x 16 NJ
// outputs held as MI x NJ MFMA 16x16 accumulators (three shapes, chosen
// per product; see below).  The grid is one-dimensional and the tile
// order is XCD-aware: workgroup b runs on XCD b % 8 and takes tile
// (b % 8) * per_xcd + b / 8 of the row-major tile order, so that each XCD
// sweeps a contiguous band of output rows and the x and W panels its
// concurrent workgroups share are fetched into its own L2 once.
//
// General form: C[M, N] = A[M, Kd] . B[N, Kd]^T (or C += when `accumulate`),
// A and B bf16 row-major with Kd contiguous (Kd % BK == 0).  B rows n < n_split
// come from B0, the others from B1 (the router stacks W_r over W_c); C rows
// m < m_split go to C0, the others to C1 (row stride ldc), so that one product
// can fill two separately owned matrices.
template <int BK, int S, int NJ, int MI, int WVM, int WVN, int MODE>
__global__ __launch_bounds__(64 * WVM * WVN) void gemm_bt_bf16_pipe(const uint16_t* __restrict__ A,
                                                         const uint16_t* __restrict__ B0,
                                                         const uint16_t* __restrict__ B1,
                                                         int M, int N, int Kd, int n_split,
                                                         int tiles_n, int per_xcd,
                                                         float* __restrict__ C0,
                                                         float* __restrict__ C1, int m_split,
                                                         int ldc, int accumulate,
                                                         uint16_t* __restrict__ Cb) {
  extern __shared__ __attribute__((aligned(16))) unsigned char gsm[];
  constexpr int NW = WVM * WVN;           // waves per workgroup
  constexpr int TM = WVM * MI * 16;       // tile rows
  constexpr int TN = WVN * NJ * 16;       // tile columns
  constexpr int ROWB = 2 * BK;            // bytes per tile row
  constexpr int TILEA = TM * ROWB;        // bytes of the A tile
  constexpr int TILEB = TN * ROWB;        // bytes of the B tile
  constexpr int STAGE = TILEA + TILEB;
  constexpr int CPR = ROWB / 16;          // 16-byte chunks per row
  constexpr int RPI = 64 / CPR;           // rows per 1 KB load instruction
  constexpr int NLA = TILEA / 1024;       // 1 KB loads per k-tile, A
  constexpr int NL = NLA + TILEB / 1024;  // and with B
  constexpr int LPW = (NL + NW - 1) / NW; // loads per wave per k-tile
  static_assert(TILEA % 1024 == 0 && TILEB % 1024 == 0, "tiles must split into 1 KB loads");
  static_assert(MODE != GEMM_SWIGLU || NJ % 2 == 0, "SwiGLU pairs MFMA column tiles");
  static_assert(S >= 2 && S <= 5, "pipeline depth");
  const int t = (blockIdx.x % 8) * per_xcd + blockIdx.x / 8;
  const int tiles_m = (M + TM - 1) / TM;
  if (t >= tiles_m * tiles_n) return;  // whole workgroup, before any barrier
  const int tile_m = (t / tiles_n) * TM, tile_n = (t % tiles_n) * TN;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = (wave / WVN) * (16 * MI), wn = (wave % WVN) * (16 * NJ);

  // The k-tile's A and B bytes form one list of NL 1 KB loads; wave w issues
  // loads w*LPW .. w*LPW+LPW-1.  When NL is not a multiple of the wave count
  // the surplus slots repeat the last load (the same bytes to the same LDS
  // address), so that every wave issues exactly LPW loads and its waits
  // count exactly.
  const uint16_t* src[LPW];
  int dst[LPW];
#pragma unroll
  for (int j = 0; j < LPW; ++j) {
    const int l = min(wave * LPW + j, NL - 1);
    const bool is_a = l < NLA;
    const int lb = is_a ? l : l - NLA;
    const int r = lb * RPI + lane / CPR;
    const int chunk = (lane % CPR) ^ chunk_swz<BK>(r);
    dst[j] = (is_a ? 0 : TILEA) + lb * 1024;
    if (is_a) {
      src[j] = A + (size_t)min(tile_m + r, M - 1) * Kd + chunk * 8;
    } else {
      const int gn = min(tile_n + r, N - 1);
      if constexpr (MODE == GEMM_SWIGLU) {
        // fused row gn: 16-row blocks alternate gate (B0) and up (B1) rows
        const int row = (gn >> 5) * 16 + (gn & 15);
        src[j] = (((gn >> 4) & 1) ? B1 : B0) + (size_t)row * Kd + chunk * 8;
      } else {
        src[j] = (gn < n_split ? B0 + (size_t)gn * Kd : B1 + (size_t)(gn - n_split) * Kd) +
                 chunk * 8;
      }
    }
  }
  auto issue = [&](int kt) {
    unsigned char* st = gsm + (kt % S) * STAGE;
    const int k0 = kt * BK;
#pragma unroll
    for (int j = 0; j < LPW; ++j)
      __builtin_amdgcn_global_load_lds((const void*)(src[j] + k0), (lds_void*)(st + dst[j]), 16,
                                       0, 0);
  };

  f32x4 acc[MI][NJ];
#pragma unroll
  for (int i = 0; i < MI; ++i)
#pragma unroll
    for (int j = 0; j < NJ; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  // fragments of k-step ks of a stage: A rows wm.., B rows wn.. of the tile
  auto load_frags = [&](const unsigned char* st, int ks, bf16x8* af, bf16x8* bfr) {
    const int kc = ks * 4 + (lane >> 4);  // 16-byte chunk of the k-slice
#pragma unroll
    for (int i = 0; i < MI; ++i) {
      const int r = wm + i * 16 + (lane & 15);
      af[i] = *(const bf16x8*)(st + r * ROWB + ((kc ^ chunk_swz<BK>(r)) << 4));
    }
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
      const int r = wn + j * 16 + (lane & 15);
      bfr[j] = *(const bf16x8*)(st + TILEA + r * ROWB + ((kc ^ chunk_swz<BK>(r)) << 4));
    }
  };

  const int nk = Kd / BK;
  for (int kt = 0; kt < S - 1 && kt < nk; ++kt) issue(kt);
  for (int kt = 0; kt < nk; ++kt) {
    // tile kt landed for this wave; after the barrier it has for every wave,
    // and every wave has finished reading tile kt-1, whose stage is refilled
    wait_vm_tiles<LPW, S - 2>(min(S - 2, nk - 1 - kt));
    block_sync_lds();
    if (kt + S - 1 < nk) issue(kt + S - 1);
    const unsigned char* st = gsm + (kt % S) * STAGE;
    bf16x8 af[2][MI], bfr[2][NJ];
    load_frags(st, 0, af[0], bfr[0]);
#pragma unroll
    for (int ks = 0; ks < BK / 32; ++ks) {
      if (ks + 1 < BK / 32) load_frags(st, ks + 1, af[(ks + 1) & 1], bfr[(ks + 1) & 1]);
#pragma unroll
      for (int i = 0; i < MI; ++i)
#pragma unroll
        for (int j = 0; j < NJ; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[ks & 1][i], bfr[ks & 1][j],
                                                              acc[i][j], 0, 0, 0);
    }
  }
  if constexpr (MODE == GEMM_SWIGLU) {
    // MFMA tiles 2q and 2q+1 of a wave hold the gate and up projections of
    // the same 16 hidden units: out = SiLU(g) * u, rounded to bf16
#pragma unroll
    for (int i = 0; i < MI; ++i)
#pragma unroll
      for (int q = 0; q < NJ / 2; ++q) {
        const int col = (((tile_n + wn) >> 5) + q) * 16 + (lane & 15);
        if (col >= (N >> 1)) continue;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int row = tile_m + wm + i * 16 + (lane >> 4) * 4 + r;
          if (row >= M) continue;
          const float g = acc[i][2 * q][r], u = acc[i][2 * q + 1][r];
          const float a = g / (1.f + expf(-g)) * u;
          const unsigned ub = __float_as_uint(a);
          Cb[(size_t)row * ldc + col] = (uint16_t)((ub + 0x7fffu + ((ub >> 16) & 1u)) >> 16);
        }
      }
    return;
  }
#pragma unroll
  for (int i = 0; i < MI; ++i)
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
      const int col = tile_n + wn + j * 16 + (lane & 15);
      if (col >= N) continue;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int row = tile_m + wm + i * 16 + (lane >> 4) * 4 + r;
        if (row >= M) continue;
        float* c = row < m_split ? C0 + (size_t)row * ldc + col
                                 : C1 + (size_t)(row - m_split) * ldc + col;
        *c = accumulate ? *c + acc[i][j][r] : acc[i][j][r];
      }
    }
}

// Three tile shapes, chosen per product by its tile count.  More waves per
// CU hide the operand loads better than deeper LDS rings: every shape below
// beat its 4- or 8-wave form, and 3 to 5 stages of 32-deep k-tiles lost to
// 2 stages of 64-deep ones (by 5-20%).  Measured, us (TFLOP/s on the
// 2.5 PFLOP/s bf16 peak), previous shape in brackets:
//   huge:  256 x 256, 16 waves (8 x 2) of 32 x 128, 128 KB of LDS.  From two
//          full rounds (512 tiles): 4096 x 11008 x 2048 170 (1088) [200, 8
//          waves], 4096 x 65536 x 2048 1096 (1003) [1132], 16384 x 2608 x
//          2048 174 (1007) [179].
//   big:   256 x 192, 12 waves (4 x 3) of 64 x 64, 112 KB.  From ~200 tiles:
//          the router product 4096 x 2608 x 2048 49 (893) [59, 8 waves of
//          64 x 96]; 16 waves of 32 x 96 or 64 x 48 took 50-53.
//   small: 128 x 128, 8 waves (4 x 2) of 32 x 64, 64 KB (two workgroups per
//          CU).  Below that: 4096 x 2048 x 1024 25.5 [27.4, 4 waves],
//          4096 x 1060 x 768 19.4 [22.2], 4096 x 2048 x 5504 88 [90],
//          2608 x 2048 x 4096 59 [62].
// Also measured and dropped: 128 x 336 (12 or 14 waves; 49.6-50.9 on the
// router product, slower elsewhere), 128 x 192 and 128 x 256 with 8 waves,
// 256 x 176, 256 x 128.  hipBLASLt (torch.matmul, bf16 out) takes 56 / 186 /
// 163 / 780 / 84 us on 4096 x 2608 x 2048, 16384 x 2608 x 2048, 4096 x
// 11008 x 2048, 4096 x 65536 x 2048 and 4096 x 2048 x 5504.
struct GemmCfgHuge {
  static constexpr int BK = GEMM_KTILE, S = 2, NJ = 8, MI = 2, WVM = 8, WVN = 2;
};
struct GemmCfgBig {
  static constexpr int BK = GEMM_KTILE, S = 2, NJ = 4, MI = 4, WVM = 4, WVN = 3;
};
struct GemmCfgSmall {
  static constexpr int BK = GEMM_KTILE, S = 2, NJ = 4, MI = 2, WVM = 4, WVN = 2;
};
using GemmCfg = GemmCfgBig;
constexpr int GEMM_BIG_MIN_TILES = 200;
constexpr int GEMM_HUGE_MIN_TILES = 512;  // two full rounds of 256 x 256 tiles

// ------------------------------------------------------------------ fp32 product
// C[m, n] (+)= sum_k A[m*sam + k*sak] * B[n*sbn + k*sbk], 64 x 64 tiles.
constexpr int GF = 64, GFK = 16;

__global__ __launch_bounds__(256) void gemm_f32_strided(const float* __restrict__ A, long sam,
                                                        long sak, const float* __restrict__ B,
                                                        long sbn, long sbk, int M, int N, int Kd,
                                                        float* __restrict__ C, int ldc,
                                                        int accumulate) {
  __shared__ float As[GFK][GF + 1];
  __shared__ float Bs[GFK][GF + 1];
  const int tile_m = blockIdx.y * GF, tile_n = blockIdx.x * GF;
  const int tid = threadIdx.x, ty = tid >> 4, tx = tid & 15;
  float acc[4][4] = {};
  for (int k0 = 0; k0 < Kd; k0 += GFK) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int c = tid + 256 * i, r = c % GF, k = c / GF;  // r fastest: m/n-contiguous reads
      const int gm = tile_m + r, gn = tile_n + r, gk = k0 + k;
      As[k][r] = (gm < M && gk < Kd) ? A[gm * sam + gk * sak] : 0.f;
      Bs[k][r] = (gn < N && gk < Kd) ? B[gn * sbn + gk * sbk] : 0.f;
    }
    __syncthreads();
#pragma unroll
    for (int k = 0; k < GFK; ++k) {
      float a[4], b[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) a[i] = As[k][ty * 4 + i];
#pragma unroll
      for (int j = 0; j < 4; ++j) b[j] = Bs[k][tx * 4 + j];
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
    if (row >= M) continue;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int col = tile_n + tx * 4 + j;
      if (col >= N) continue;
      float* c = C + (size_t)row * ldc + col;
      *c = accumulate ? *c + acc[i][j] : acc[i][j];
    }
  }
}

template <int MODE, class C = GemmCfg>
hipError_t launch_t(const void* A, const void* B0, const void* B1, int n_split, int M, int N,
                    int Kd, float* C0, float* C1, int m_split, int ldc, bool accumulate,
                    uint16_t* Cb, hipStream_t s) {
  constexpr int TM = C::WVM * C::MI * 16, TN = C::WVN * C::NJ * 16;
  if (Kd % C::BK != 0 || M <= 0 || N <= 0) return hipErrorInvalidValue;
  const int tiles_n = (N + TN - 1) / TN;
  const int tiles = ((M + TM - 1) / TM) * tiles_n;
  const int per_xcd = (tiles + 7) / 8;
  const size_t lds = (size_t)C::S * (TM + TN) * 2 * C::BK;
  hipLaunchKernelGGL((gemm_bt_bf16_pipe<C::BK, C::S, C::NJ, C::MI, C::WVM, C::WVN, MODE>),
                     dim3(8 * per_xcd), dim3(64 * C::WVM * C::WVN), lds, s, (const uint16_t*)A,
                     (const uint16_t*)B0, (const uint16_t*)B1, M, N, Kd, n_split, tiles_n,
                     per_xcd, C0, C1, m_split, ldc, accumulate ? 1 : 0, Cb);
  return hipGetLastError();
}

template <int MODE>
hipError_t launch_sel(const void* A, const void* B0, const void* B1, int n_split, int M, int N,
                      int Kd, float* C0, float* C1, int m_split, int ldc, bool accumulate,
                      uint16_t* Cb, hipStream_t s) {
  const int huge_tiles = ((M + 255) / 256) * ((N + 255) / 256);
  const int big_tiles = ((M + 255) / 256) * ((N + 191) / 192);
  if (huge_tiles >= GEMM_HUGE_MIN_TILES)
    return launch_t<MODE, GemmCfgHuge>(A, B0, B1, n_split, M, N, Kd, C0, C1, m_split, ldc,
                                       accumulate, Cb, s);
  if (big_tiles >= GEMM_BIG_MIN_TILES)
    return launch_t<MODE, GemmCfgBig>(A, B0, B1, n_split, M, N, Kd, C0, C1, m_split, ldc,
                                      accumulate, Cb, s);
  return launch_t<MODE, GemmCfgSmall>(A, B0, B1, n_split, M, N, Kd, C0, C1, m_split, ldc,
                                      accumulate, Cb, s);
}

}  // namespace

hipError_t launch_gemm_bt_bf16(const void* A, const void* B0, const void* B1, int n_split, int M,
                               int N, int Kd, float* C0, float* C1, int m_split, int ldc,
                               bool accumulate, hipStream_t s) {
  return launch_sel<GEMM_PLAIN>(A, B0, B1, n_split, M, N, Kd, C0, C1, m_split, ldc, accumulate,
                                nullptr, s);
}

hipError_t launch_gemm_swiglu_bf16(const void* A, const void* Wg, const void* Wu, int M, int F,
                                   int Kd, uint16_t* out, hipStream_t s) {
  if (F % 16 != 0) return hipErrorInvalidValue;
  return launch_sel<GEMM_SWIGLU>(A, Wg, Wu, 0, M, 2 * F, Kd, nullptr, nullptr, 0, F, false, out,
                                 s);
}

hipError_t gemm_f32(const float* A, long sam, long sak, const float* B, long sbn, long sbk, int M,
                    int N, int Kd, float* C, int ldc, bool accumulate, hipStream_t s) {
  const dim3 grid((N + GF - 1) / GF, (M + GF - 1) / GF);
  hipLaunchKernelGGL(gemm_f32_strided, grid, dim3(256), 0, s, A, sam, sak, B, sbn, sbk, M, N, Kd,
                     C, ldc, accumulate ? 1 : 0);
  return hipGetLastError();
}

}  // namespace omni
