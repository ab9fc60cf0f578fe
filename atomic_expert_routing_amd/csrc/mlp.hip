// Shared dense MLP branch on gfx950.
//
// OmniMoE digest (paper.rainbus.top), method paragraph, step 1: the layer
// output is the routed assembly plus MLP(x), a dense branch active for every
// token (gist.science resume section 2.1: a standard dense MLP).  The pages
// give no shape; it is read as a SwiGLU block
//   MLP(x) = (SiLU(x W_g^T) * (x W_u^T)) W_d^T,  W_g, W_u [F, d], W_d [d, F].
//
// bf16: the gate and up projections run as one MFMA product whose epilogue
// forms SiLU(g) * u and stores it as bf16 (the precision of the weights it
// then multiplies, as bf16 MLPs do); the down projection is the plain MFMA
// product, accumulating into y when asked.  fp32: VALU products, the
// intermediate kept in fp32.

#include "omni_internal.h"

namespace omni {
namespace {

__global__ __launch_bounds__(256) void swiglu_f32(float* __restrict__ g, const float* __restrict__ u,
                                                  size_t n) {
  const size_t i = blockIdx.x * (size_t)256 + threadIdx.x;
  if (i < n) {
    const float a = g[i];
    g[i] = a / (1.f + expf(-a)) * u[i];
  }
}

}  // namespace

size_t shared_mlp_ws_bytes(int64_t L, int64_t F, omni_dtype dt) {
  const size_t n = (size_t)L * (size_t)F;
  return dt == OMNI_BF16 ? ((n * 2 + 255) & ~(size_t)255) : 2 * ((n * 4 + 255) & ~(size_t)255);
}

hipError_t launch_shared_mlp(const void* x, const void* Wg, const void* Wu, const void* Wd, int L,
                             int d, int F, omni_dtype dt, float* y, bool accumulate, void* ws,
                             hipStream_t s) {
  hipError_t e;
  if (dt == OMNI_BF16) {
    uint16_t* a = (uint16_t*)ws;  // [L, F] bf16
    if ((e = launch_gemm_swiglu_bf16(x, Wg, Wu, L, F, d, a, s)) != hipSuccess) return e;
    return launch_gemm_bt_bf16(a, Wd, Wd, d, L, d, F, y, y, L, d, accumulate, s);
  }
  const size_t n = (size_t)L * (size_t)F;
  float* hg = (float*)ws;
  float* hu = (float*)((char*)ws + ((n * 4 + 255) & ~(size_t)255));
  const float* xf = (const float*)x;
  // hg[t, j] = x_t . Wg[j], hu likewise
  if ((e = gemm_f32(xf, d, 1, (const float*)Wg, d, 1, L, F, d, hg, F, false, s))) return e;
  if ((e = gemm_f32(xf, d, 1, (const float*)Wu, d, 1, L, F, d, hu, F, false, s))) return e;
  hipLaunchKernelGGL(swiglu_f32, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, hg, hu, n);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  // y[t, i] (+)= sum_j a[t, j] Wd[i, j]
  return gemm_f32(hg, F, 1, (const float*)Wd, F, 1, L, d, F, y, d, accumulate, s);
}

}  // namespace omni
