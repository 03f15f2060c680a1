// norm.hip -- RMSNorm of the aggregated stream: forward, backward, and the
// forward fused into the h_aggregate pass.
//
// Per token row x [C] (activation type), optional gain gamma [C] (fp32):
//   q = sqrt(sum_c x_c^2 / C),  r = 1 / (q + eps),  y_c = gamma_c r x_c
//   dx_k = r gamma_k dy_k - S r^2 x_k / (C q),  S = sum_c gamma_c dy_c x_c
//          (the second term is 0 for an all-zero row, q == 0)
//   dgamma_c = sum over tokens of dy_c r x_c
// [rwkv-ops mhu_ffi.cu, RMSNorm forward/backward FFI: [N, C] in and out, one
// eps attribute, no weight; RL-Kernel PR #383: rmsnorm_residual carries a
// norm gain (its dgamma is summed across ranks) and removes the zero-row
// singularity with r = 1/(q + eps).]
//
// Geometry as the other streaming kernels: a workgroup owns whole tokens, a
// thread owns 8-channel groups g = tid + j*TPB, every element is read once
// with a 128-bit access, and per-token sums go lane -> wave (DPP) ->
// workgroup (LDS, fixed wave order), so results are bitwise reproducible.
// dgamma: per-workgroup partial rows (TG tokens each, fixed token order) in
// the workspace, summed over rows in a fixed order (launch_rows_sum).
#include "device.h"
#include "internal.h"

namespace mhc {

namespace {

constexpr int kNormTG = 16;  // tokens per workgroup when dgamma is produced

__device__ __forceinline__ int group_of(int j, int G) {
  return min((int)threadIdx.x + j * (int)blockDim.x, G - 1);
}

// Sum of NV per-thread values over the workgroup (at most 8 waves); every
// thread receives the totals.  `red` is reused across calls: the trailing
// barrier keeps the next call's writes behind this call's reads.
template <int NV>
__device__ __forceinline__ void block_sum(float v[NV], float (*red)[NV]) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63, nw = blockDim.x >> 6;
#pragma unroll
  for (int k = 0; k < NV; ++k) v[k] = wave_sum(v[k]);
  if (lane == 0) {
#pragma unroll
    for (int k = 0; k < NV; ++k) red[wave][k] = v[k];
  }
  __syncthreads();
#pragma unroll
  for (int k = 0; k < NV; ++k) {
    float s = 0.f;
    for (int w = 0; w < nw; ++w) s += red[w][k];
    v[k] = s;
  }
  __syncthreads();
}

// The norm's input gradient of one element, r (gamma dy) + coef x, as one
// explicit fma (the rounding does not depend on the compiler's contraction).
__device__ __forceinline__ float norm_dx(float r, float gdy, float coef, float x) {
  return fmaf(coef, x, r * gdy);
}

__device__ __forceinline__ void load_gamma(const float *gamma, int g, float gv[8]) {
  const float4 a = *reinterpret_cast<const float4 *>(gamma + 8 * g);
  const float4 b = *reinterpret_cast<const float4 *>(gamma + 8 * g + 4);
  gv[0] = a.x; gv[1] = a.y; gv[2] = a.z; gv[3] = a.w;
  gv[4] = b.x; gv[5] = b.y; gv[6] = b.z; gv[7] = b.w;
}

// The value a float takes once stored in the activation type.
template <typename T> __device__ __forceinline__ float stored(float v);
template <> __device__ __forceinline__ float stored<float>(float v) { return v; }
template <> __device__ __forceinline__ float stored<bf16_t>(float v) { return bf16_lo(pack_bf16x2(v, 0.f)); }

__device__ __forceinline__ float rms_r(float ss, int64_t C, float eps) {
  const float q = sqrtf(ss / (float)C);
  return 1.0f / (q + eps);
}

// ============================================================ forward
template <typename T, int GPT, bool GAMMA>
__global__ __launch_bounds__(512) void rmsnorm_fwd_kernel(const T *__restrict__ x,
                                                          const float *__restrict__ gamma,
                                                          T *__restrict__ y, int64_t C, float eps) {
  using R = typename Io8<T>::raw_t;
  __shared__ float red[8][1];
  const int64_t t = blockIdx.x;
  const int G = (int)(C / 8);
  R rx[GPT];
#pragma unroll
  for (int j = 0; j < GPT; ++j) rx[j] = Io8<T>::ld_nt(x + t * C + 8 * group_of(j, G));
  float v[GPT][8];
  float ss[1] = {0.f};
#pragma unroll
  for (int j = 0; j < GPT; ++j) {
    Io8<T>::cvt(rx[j], v[j]);
    if ((int)threadIdx.x + j * (int)blockDim.x < G) {
#pragma unroll
      for (int e = 0; e < 8; ++e) ss[0] += v[j][e] * v[j][e];
    }
  }
  block_sum<1>(ss, red);
  const float r = rms_r(ss[0], C, eps);
#pragma unroll
  for (int j = 0; j < GPT; ++j) {
    const int g = threadIdx.x + j * blockDim.x;
    if (g < G) {
      float o[8], gv[8];
      if (GAMMA) load_gamma(gamma, g, gv);
#pragma unroll
      for (int e = 0; e < 8; ++e) o[e] = GAMMA ? gv[e] * (r * v[j][e]) : r * v[j][e];
      Io8<T>::store(y + t * C + 8 * g, o);
    }
  }
}

// ============================================================ h_aggregate + RMSNorm forward
// agg[c] = sum_i H_pre[i] X[i][c] is stored (the fork that stays the
// aggregated stream), and y = RMSNorm(agg) is computed from the stored
// (rounded) agg values, so the fused pass equals h_aggregate followed by
// the standalone forward on its output.  Last token first, as h_aggregate:
// the projection pass before it has just walked the tokens upwards.
template <typename T, int GPT, bool GAMMA>
__global__ __launch_bounds__(512) void h_aggregate_rmsnorm_fwd_kernel(
    const T *__restrict__ X, const float *__restrict__ Hpre, const float *__restrict__ gamma,
    T *__restrict__ agg, T *__restrict__ y, int64_t C, float eps) {
  using R = typename Io8<T>::raw_t;
  __shared__ float red[8][1];
  const int64_t t = (int64_t)gridDim.x - 1 - blockIdx.x;
  const int G = (int)(C / 8);
  const T *xt = X + t * 4 * C;
  R rx[GPT][4];
#pragma unroll
  for (int j = 0; j < GPT; ++j) {
    const int gc = group_of(j, G);
#pragma unroll
    for (int i = 0; i < 4; ++i) rx[j][i] = Io8<T>::ld_nt(xt + i * C + 8 * gc);
  }
  const float h0 = Hpre[t * 4 + 0], h1 = Hpre[t * 4 + 1], h2 = Hpre[t * 4 + 2], h3 = Hpre[t * 4 + 3];
  float a[GPT][8];
  float ss[1] = {0.f};
#pragma unroll
  for (int j = 0; j < GPT; ++j) {
    float v[4][8];
#pragma unroll
    for (int i = 0; i < 4; ++i) Io8<T>::cvt(rx[j][i], v[i]);
#pragma unroll
    for (int e = 0; e < 8; ++e) a[j][e] = h0 * v[0][e] + h1 * v[1][e] + h2 * v[2][e] + h3 * v[3][e];
    const int g = threadIdx.x + j * blockDim.x;
    if (g < G) {
      Io8<T>::store(agg + t * C + 8 * g, a[j]);
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        a[j][e] = stored<T>(a[j][e]);
        ss[0] += a[j][e] * a[j][e];
      }
    }
  }
  block_sum<1>(ss, red);
  const float r = rms_r(ss[0], C, eps);
#pragma unroll
  for (int j = 0; j < GPT; ++j) {
    const int g = threadIdx.x + j * blockDim.x;
    if (g < G) {
      float o[8], gv[8];
      if (GAMMA) load_gamma(gamma, g, gv);
#pragma unroll
      for (int e = 0; e < 8; ++e) o[e] = GAMMA ? gv[e] * (r * a[j][e]) : r * a[j][e];
      Io8<T>::store(y + t * C + 8 * g, o);
    }
  }
}

// ============================================================ backward
// TG tokens per workgroup (TG > 1 only with dgamma: the partial row of this
// workgroup's tokens, in token order, goes to part[blockIdx.x][C]).
template <typename T, int GPT, bool GAMMA, bool ACCUM, bool DGAMMA>
__global__ __launch_bounds__(512) void rmsnorm_bwd_kernel(
    const T *__restrict__ dy, const T *__restrict__ x, const float *__restrict__ gamma,
    T *__restrict__ dx, float *__restrict__ part, int64_t N, int64_t C, float eps, int TG) {
  using R = typename Io8<T>::raw_t;
  __shared__ float red[8][2];
  const int G = (int)(C / 8);
  float gv[GPT][8], dg[GPT][8];
#pragma unroll
  for (int j = 0; j < GPT; ++j) {
    const int gc = group_of(j, G);
#pragma unroll
    for (int e = 0; e < 8; ++e) { gv[j][e] = 1.f; dg[j][e] = 0.f; }
    if (GAMMA) load_gamma(gamma, gc, gv[j]);
  }
  const int64_t t0 = (int64_t)blockIdx.x * TG;
  const int64_t t1 = min(t0 + (int64_t)TG, N);
  // The next token's rows are loaded while this token is reduced and
  // written, so a workgroup always has one token's loads in flight.
  R nx[GPT], ng[GPT], nd[GPT];
  auto issue = [&](int64_t tt) {
#pragma unroll
    for (int j = 0; j < GPT; ++j) {
      const int gc = group_of(j, G);
      nx[j] = Io8<T>::ld_nt(x + tt * C + 8 * gc);
      ng[j] = Io8<T>::ld_nt(dy + tt * C + 8 * gc);
      if (ACCUM) nd[j] = Io8<T>::ld_nt(dx + tt * C + 8 * gc);
    }
  };
  // One token: reduce, then write dx and add to the dgamma partials.  The
  // loop issues token t+1 unconditionally and the last token is peeled, so
  // the waits for token t never have to cover the prefetch.
  auto token = [&](int64_t t) {
    R rx[GPT], rg[GPT], rd[GPT];
#pragma unroll
    for (int j = 0; j < GPT; ++j) {
      rx[j] = nx[j];
      rg[j] = ng[j];
      if (ACCUM) rd[j] = nd[j];
    }
    if (t + 1 < t1) issue(t + 1);
    float xv[GPT][8], gy[GPT][8];
    float sums[2] = {0.f, 0.f};  // sum x^2, sum gamma dy x
#pragma unroll
    for (int j = 0; j < GPT; ++j) {
      Io8<T>::cvt(rx[j], xv[j]);
      Io8<T>::cvt(rg[j], gy[j]);
      if ((int)threadIdx.x + j * (int)blockDim.x < G) {
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          sums[0] = fmaf(xv[j][e], xv[j][e], sums[0]);
          sums[1] = fmaf(gv[j][e] * gy[j][e], xv[j][e], sums[1]);
        }
      }
    }
    block_sum<2>(sums, red);
    const float q = sqrtf(sums[0] / (float)C);
    const float r = 1.0f / (q + eps);
    const float coef = q > 0.f ? -sums[1] * r * r / ((float)C * q) : 0.f;
#pragma unroll
    for (int j = 0; j < GPT; ++j) {
      const int g = threadIdx.x + j * blockDim.x;
      if (g < G) {
        float o[8], din[8];
        if (ACCUM) Io8<T>::cvt(rd[j], din);
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          o[e] = norm_dx(r, gv[j][e] * gy[j][e], coef, xv[j][e]);
          if (ACCUM) o[e] += din[e];
          if (DGAMMA) dg[j][e] = fmaf(gy[j][e], r * xv[j][e], dg[j][e]);
        }
        Io8<T>::store(dx + t * C + 8 * g, o);
      }
    }
  };
  if (t0 < t1) {
    issue(t0);
    for (int64_t t = t0; t + 1 < t1; ++t) token(t);
    token(t1 - 1);
  }
  if (DGAMMA) {
#pragma unroll
    for (int j = 0; j < GPT; ++j) {
      const int g = threadIdx.x + j * blockDim.x;
      if (g < G) {
        float *p = part + (int64_t)blockIdx.x * C + 8 * g;
        *reinterpret_cast<float4 *>(p) = make_float4(dg[j][0], dg[j][1], dg[j][2], dg[j][3]);
        *reinterpret_cast<float4 *>(p + 4) = make_float4(dg[j][4], dg[j][5], dg[j][6], dg[j][7]);
      }
    }
  }
}

#define MHC_NORM_GPT_DISPATCH(GPT_VAL, ...)                  \
  switch (GPT_VAL) {                                         \
    case 1: { constexpr int GPT = 1; __VA_ARGS__; } break;   \
    case 2: { constexpr int GPT = 2; __VA_ARGS__; } break;   \
    default: { constexpr int GPT = 4; __VA_ARGS__; } break;  \
  }

template <typename T, bool GAMMA>
void norm_fwd(hipStream_t s, int64_t N, int64_t C, const void *x, const float *gamma, float eps, void *y) {
  const StreamGeom g = stream_geom(C);
  MHC_NORM_GPT_DISPATCH(g.gpt, hipLaunchKernelGGL((rmsnorm_fwd_kernel<T, GPT, GAMMA>), dim3((unsigned)N),
                                                  dim3(g.tpb), 0, s, (const T *)x, gamma, (T *)y, C, eps));
}

template <typename T, bool GAMMA>
void agg_norm_fwd(hipStream_t s, int64_t N, int64_t C, const void *X, const float *H, const float *gamma,
                  float eps, void *agg, void *y) {
  const StreamGeom g = stream_geom(C);
  MHC_NORM_GPT_DISPATCH(g.gpt, hipLaunchKernelGGL((h_aggregate_rmsnorm_fwd_kernel<T, GPT, GAMMA>),
                                                  dim3((unsigned)N), dim3(g.tpb), 0, s, (const T *)X, H,
                                                  gamma, (T *)agg, (T *)y, C, eps));
}

template <typename T, bool GAMMA, bool ACCUM, bool DGAMMA>
void norm_bwd4(hipStream_t s, int64_t N, int64_t C, const void *dy, const void *x, const float *gamma,
               float eps, void *dx, float *part) {
  const StreamGeom g = stream_geom(C);
  const int TG = DGAMMA ? kNormTG : 1;
  const unsigned blocks = (unsigned)((N + TG - 1) / TG);
  MHC_NORM_GPT_DISPATCH(g.gpt, hipLaunchKernelGGL((rmsnorm_bwd_kernel<T, GPT, GAMMA, ACCUM, DGAMMA>),
                                                  dim3(blocks), dim3(g.tpb), 0, s, (const T *)dy,
                                                  (const T *)x, gamma, (T *)dx, part, N, C, eps, TG));
}

template <typename T, bool GAMMA>
void norm_bwd(hipStream_t s, int64_t N, int64_t C, const void *dy, const void *x, const float *gamma,
              float eps, void *dx, bool acc, float *dgamma, void *ws) {
  float *part = (float *)ws;
  if (dgamma) {
    if (acc)
      norm_bwd4<T, GAMMA, true, true>(s, N, C, dy, x, gamma, eps, dx, part);
    else
      norm_bwd4<T, GAMMA, false, true>(s, N, C, dy, x, gamma, eps, dx, part);
    const int64_t R = (N + kNormTG - 1) / kNormTG;
    launch_rows_sum(s, part, R, C, part + R * C, dgamma, false);
  } else if (acc) {
    norm_bwd4<T, GAMMA, true, false>(s, N, C, dy, x, gamma, eps, dx, nullptr);
  } else {
    norm_bwd4<T, GAMMA, false, false>(s, N, C, dy, x, gamma, eps, dx, nullptr);
  }
}

}  // namespace

void launch_rmsnorm_fwd(hipStream_t s, bool f32, int64_t N, int64_t C, const void *x, const float *gamma,
                        float eps, void *y) {
  if (f32)
    gamma ? norm_fwd<float, true>(s, N, C, x, gamma, eps, y) : norm_fwd<float, false>(s, N, C, x, gamma, eps, y);
  else
    gamma ? norm_fwd<bf16_t, true>(s, N, C, x, gamma, eps, y) : norm_fwd<bf16_t, false>(s, N, C, x, gamma, eps, y);
}

void launch_h_aggregate_rmsnorm_fwd(hipStream_t s, bool f32, int64_t N, int64_t C, const void *X,
                                    const float *H_pre, const float *gamma, float eps, void *agg, void *y) {
  if (f32)
    gamma ? agg_norm_fwd<float, true>(s, N, C, X, H_pre, gamma, eps, agg, y)
          : agg_norm_fwd<float, false>(s, N, C, X, H_pre, gamma, eps, agg, y);
  else
    gamma ? agg_norm_fwd<bf16_t, true>(s, N, C, X, H_pre, gamma, eps, agg, y)
          : agg_norm_fwd<bf16_t, false>(s, N, C, X, H_pre, gamma, eps, agg, y);
}

size_t rmsnorm_bwd_ws(int64_t N, int64_t C, bool with_dgamma) {
  return with_dgamma ? ((size_t)((N + kNormTG - 1) / kNormTG) + kRowSumSlices) * (size_t)C * 4 : 0;
}

void launch_rmsnorm_bwd(hipStream_t s, bool f32, int64_t N, int64_t C, const void *dy, const void *x,
                        const float *gamma, float eps, void *dx, bool accumulate, float *dgamma, void *ws) {
  if (f32)
    gamma ? norm_bwd<float, true>(s, N, C, dy, x, gamma, eps, dx, accumulate, dgamma, ws)
          : norm_bwd<float, false>(s, N, C, dy, x, gamma, eps, dx, accumulate, dgamma, ws);
  else
    gamma ? norm_bwd<bf16_t, true>(s, N, C, dy, x, gamma, eps, dx, accumulate, dgamma, ws)
          : norm_bwd<bf16_t, false>(s, N, C, dy, x, gamma, eps, dx, accumulate, dgamma, ws);
}

}  // namespace mhc
