// sinkhorn.hip -- batched Sinkhorn-Knopp forward/backward, one matrix per lane.
#include "internal.h"
#include "sinkhorn.h"

namespace mhc {

__global__ __launch_bounds__(256) void sinkhorn_fwd_kernel(const float *__restrict__ L,
                                                           float *__restrict__ H, int64_t count,
                                                           int iters, float eps) {
  const int64_t m = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (m >= count) return;
  float v[16], M[16];
  load16(L + m * 16, v);
  sk_exp(v, M);
  sk_forward(M, iters, eps);
  store16(H + m * 16, M);
}

__global__ __launch_bounds__(256) void sinkhorn_bwd_kernel(const float *__restrict__ dH,
                                                           const float *__restrict__ L,
                                                           float *__restrict__ dL, int64_t count,
                                                           int iters, float eps) {
  const int64_t m = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (m >= count) return;
  float l[16], G[16];
  load16(L + m * 16, l);
  load16(dH + m * 16, G);
  sk_backward(l, G, iters, eps);
  store16(dL + m * 16, G);
}

void launch_sinkhorn_fwd(hipStream_t s, int64_t count, const float *L, float *H, int iters,
                         float eps) {
  const unsigned blocks = (unsigned)((count + 255) / 256);
  hipLaunchKernelGGL(sinkhorn_fwd_kernel, dim3(blocks), dim3(256), 0, s, L, H, count, iters, eps);
}

void launch_sinkhorn_bwd(hipStream_t s, int64_t count, const float *dH, const float *L, float *dL,
                         int iters, float eps) {
  const unsigned blocks = (unsigned)((count + 255) / 256);
  hipLaunchKernelGGL(sinkhorn_bwd_kernel, dim3(blocks), dim3(256), 0, s, dH, L, dL, count, iters,
                     eps);
}

}  // namespace mhc
