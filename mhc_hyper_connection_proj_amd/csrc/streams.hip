// streams.hip -- HBM-streaming kernels: h_aggregate and h_post_bda, fwd + bwd.
//
// Layout: X/G/dX [tokens][4][C], x/agg/dx [tokens][C], bias [C] (activation
// type), H_pre/H_post [tokens][4], H_res [tokens][4][4] (fp32).
//
// Each workgroup owns whole tokens.  A thread owns 8-channel groups
// g = tid + j*TPB (j < GPT) and touches every stream of those channels, so
// each tensor element is read exactly once with a 128-bit (bf16) access and
// the 4x4 mix stays in registers.  The per-token H values are wave-uniform
// (scalar loads).  Per-token reductions over C go lane -> wave (DPP) ->
// workgroup (LDS, fixed wave order); cross-token sums (dbias) go through
// per-workgroup partials summed in a fixed order by launch_rows_sum (reduce.hip).
//
// Token order: the kernels that follow a full pass over X walk the tokens in
// the opposite direction of that pass (h_aggregate forward and h_post_bda
// backward run from the last token down), so their first reads hit the
// data the previous kernel left in the 256 MB Infinity Cache.
//
// Outputs that the next kernel of the step reads (agg, dx) and the new
// residual are written with non-temporal stores: with the default policy
// their dirty lines were written back in the middle of the following
// kernels' reads (mHC step at 16384 x 7168: 2055-2060 -> 2030-2033 us, the
// layer stand-in between them unchanged).
#include "device.h"
#include "internal.h"

namespace mhc {

// Threads per workgroup (a multiple of 64, at most 512) and 8-channel groups
// per thread (1, 2 or 4; C <= 16384 gives at most 2048 groups), chosen so
// that tpb * gpt covers C/8 with the fewest idle groups (exactly, when C is
// a multiple of 512 * gpt or of the size below it: C = 7168 gives 448 x 2).
StreamGeom stream_geom(int64_t C) {
  const int64_t G = C / 8;
  const int gpt = G <= 512 ? 1 : G <= 1024 ? 2 : 4;
  const int64_t per = (G + gpt - 1) / gpt;
  return {(int)((per + 63) / 64 * 64), gpt};
}

// Each kernel first issues every load of a token (all groups of the thread,
// raw and unconditional: a group past C/8 re-reads the last real group and
// is never stored or summed), then converts and computes.  Loads issued
// inside per-group branches are waited for group by group, which leaves a
// fraction of the bytes in flight.
__device__ __forceinline__ int clamp_group(int j, int G) {
  return min((int)threadIdx.x + j * (int)blockDim.x, G - 1);
}

// ============================================================ h_aggregate fwd
// hs: H_pre's token stride, 4 (one row per token) or 0 (one row for all).
template <typename T, int GPT>
__global__ __launch_bounds__(512) void h_aggregate_fwd_kernel(const T *__restrict__ X,
                                                               const float *__restrict__ Hpre,
                                                               T *__restrict__ out, int64_t C, int64_t hs) {
  using R = typename Io8<T>::raw_t;
  const int64_t t = (int64_t)gridDim.x - 1 - blockIdx.x;  // last token first
  const int G = (int)(C / 8);
  const T *xt = X + t * 4 * C;
  R rx[GPT][4];
#pragma unroll
  for (int j = 0; j < GPT; ++j) {
    const int gc = clamp_group(j, G);
#pragma unroll
    for (int i = 0; i < 4; ++i) rx[j][i] = Io8<T>::ld_nt(xt + i * C + 8 * gc);
  }
  const float h0 = Hpre[t * hs + 0], h1 = Hpre[t * hs + 1], h2 = Hpre[t * hs + 2], h3 = Hpre[t * hs + 3];
#pragma unroll
  for (int j = 0; j < GPT; ++j) {
    const int g = threadIdx.x + j * blockDim.x;
    if (g < G) {
      float v[4][8], o[8];
#pragma unroll
      for (int i = 0; i < 4; ++i) Io8<T>::cvt(rx[j][i], v[i]);
#pragma unroll
      for (int e = 0; e < 8; ++e) o[e] = h0 * v[0][e] + h1 * v[1][e] + h2 * v[2][e] + h3 * v[3][e];
      Io8<T>::store_nt(out + t * C + 8 * g, o);
    }
  }
}

// ============================================================ h_aggregate bwd
// dH_pre[t][i] = sum_c g[t][c] X[t][i][c];  optionally dX (+)= H_pre[i] g
// (H_pre's token stride hs as in the forward).
template <typename T, int GPT, bool WRITE_DX, bool ACCUM>
__global__ __launch_bounds__(512) void h_aggregate_bwd_kernel(
    const T *__restrict__ gr, const T *__restrict__ X, const float *__restrict__ Hpre,
    T *__restrict__ dX, float *__restrict__ dHpre, int64_t C, int64_t hs) {
  using R = typename Io8<T>::raw_t;
  __shared__ float red[8][4];
  const int64_t t = blockIdx.x;
  const int G = (int)(C / 8);
  const T *xt = X + t * 4 * C;
  R rg[GPT], rx[GPT][4], rd[GPT][4];
#pragma unroll
  for (int j = 0; j < GPT; ++j) {
    const int gc = clamp_group(j, G);
    rg[j] = Io8<T>::ld_nt(gr + t * C + 8 * gc);
#pragma unroll
    for (int i = 0; i < 4; ++i) rx[j][i] = Io8<T>::ld_nt(xt + i * C + 8 * gc);
    if (WRITE_DX && ACCUM) {
#pragma unroll
      for (int i = 0; i < 4; ++i) rd[j][i] = Io8<T>::ld_nt(dX + (t * 4 + i) * C + 8 * gc);
    }
  }
  float acc[4] = {0.f, 0.f, 0.f, 0.f};
  float h[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) h[i] = Hpre[t * hs + i];
#pragma unroll
  for (int j = 0; j < GPT; ++j) {
    const int g = threadIdx.x + j * blockDim.x;
    if (g < G) {
      float gv[8], xv[4][8];
      Io8<T>::cvt(rg[j], gv);
#pragma unroll
      for (int i = 0; i < 4; ++i) Io8<T>::cvt(rx[j][i], xv[i]);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        float s = 0.f;
#pragma unroll
        for (int e = 0; e < 8; ++e) s = fmaf(gv[e], xv[i][e], s);
        acc[i] += s;
      }
      if (WRITE_DX) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          float d[8];
          if (ACCUM) {
            Io8<T>::cvt(rd[j][i], d);
#pragma unroll
            for (int e = 0; e < 8; ++e) d[e] += h[i] * gv[e];
          } else {
#pragma unroll
            for (int e = 0; e < 8; ++e) d[e] = h[i] * gv[e];
          }
          Io8<T>::store(dX + (t * 4 + i) * C + 8 * g, d);
        }
      }
    }
  }
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const float s = wave_sum(acc[i]);
    if (lane == 0) red[wave][i] = s;
  }
  __syncthreads();
  if (threadIdx.x < 4) {
    const int nw = blockDim.x >> 6;
    float s = 0.f;
    for (int w = 0; w < nw; ++w) s += red[w][threadIdx.x];
    dHpre[t * 4 + threadIdx.x] = s;
  }
}

// dH_pre[i] = sum over tokens of the per-token rows part[t][i], for one
// shared H_pre row: thread k adds tokens k, k + 256, ... in order (eight
// loads in flight), then a fixed pairwise tree over the 256 thread sums.
__global__ __launch_bounds__(256) void hpre_rows_sum_kernel(const float *__restrict__ part,
                                                            float *__restrict__ dH, int64_t N) {
  __shared__ float4 red[256];
  float4 s = make_float4(0.f, 0.f, 0.f, 0.f);
  const float4 *p = reinterpret_cast<const float4 *>(part);
#pragma unroll 8
  for (int64_t t = threadIdx.x; t < N; t += 256) {
    const float4 v = p[t];
    s.x += v.x; s.y += v.y; s.z += v.z; s.w += v.w;
  }
  red[threadIdx.x] = s;
  __syncthreads();
  for (int w = 128; w > 0; w >>= 1) {
    if ((int)threadIdx.x < w) {
      const float4 a = red[threadIdx.x], b = red[threadIdx.x + w];
      red[threadIdx.x] = make_float4(a.x + b.x, a.y + b.y, a.z + b.z, a.w + b.w);
    }
    __syncthreads();
  }
  if (threadIdx.x == 0) {
    dH[0] = red[0].x; dH[1] = red[0].y; dH[2] = red[0].z; dH[3] = red[0].w;
  }
}

// ============================================================ h_post_bda fwd
// MODE: kPostFull  out[i] = sum_j H_res[j][i] X[j] + H_post[i] (x + bias)
//       kPostMix   out[i] = sum_j H_res[j][i] X[j]          (x, H_post unused)
//       kPostDist  out[i] = H_post[i] x                      (X, H_res unused)
// The new residual is written with non-temporal stores: its 8C bytes per
// token otherwise sit dirty in the caches when the kernel ends, and their
// write-back then lands in the next kernel's read stream (on MI355X the
// following h_post_bda backward measured ~50 us slower at C = 7168, 16384
// tokens; this kernel itself ran no slower).
enum : int { kPostFull = 0, kPostMix = 1, kPostDist = 2 };

template <typename T, int GPT, bool HAS_BIAS, int MODE>
__global__ __launch_bounds__(512) void h_post_bda_fwd_kernel(
    const T *__restrict__ X, const float *__restrict__ Hres, const float *__restrict__ Hpost,
    const T *__restrict__ x, const T *__restrict__ bias, T *__restrict__ out, int64_t C) {
  using R = typename Io8<T>::raw_t;
  constexpr bool MIX = MODE != kPostDist, DIST = MODE != kPostMix;
  const int64_t t = blockIdx.x;
  const int G = (int)(C / 8);
  const T *xt = X + t * 4 * C;
  R rx[GPT][4], rl[GPT];
#pragma unroll
  for (int j = 0; j < GPT; ++j) {
    const int gc = clamp_group(j, G);
    if (MIX) {
#pragma unroll
      for (int i = 0; i < 4; ++i) rx[j][i] = Io8<T>::ld_nt(xt + i * C + 8 * gc);
    }
    if (DIST) rl[j] = Io8<T>::ld_nt(x + t * C + 8 * gc);
  }
  float hr[16], hp[4];
  if (MIX) {
#pragma unroll
    for (int e = 0; e < 16; ++e) hr[e] = Hres[t * 16 + e];
  }
  if (DIST) {
#pragma unroll
    for (int i = 0; i < 4; ++i) hp[i] = Hpost[t * 4 + i];
  }
  T *ot = out + t * 4 * C;
#pragma unroll
  for (int j = 0; j < GPT; ++j) {
    const int g = threadIdx.x + j * blockDim.x;
    if (g < G) {
      float xv[4][8], lv[8];
      if (MIX) {
#pragma unroll
        for (int i = 0; i < 4; ++i) Io8<T>::cvt(rx[j][i], xv[i]);
      }
      if (DIST) {
        Io8<T>::cvt(rl[j], lv);
        if (HAS_BIAS) {
          float bv[8];
          Io8<T>::load(bias + 8 * g, bv);
#pragma unroll
          for (int e = 0; e < 8; ++e) lv[e] += bv[e];
        }
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        float o[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          if (MODE == kPostFull)
            o[e] = (hr[0 * 4 + i] * xv[0][e] + hr[1 * 4 + i] * xv[1][e]) +
                   (hr[2 * 4 + i] * xv[2][e] + hr[3 * 4 + i] * xv[3][e]) + hp[i] * lv[e];
          else if (MODE == kPostMix)
            o[e] = (hr[0 * 4 + i] * xv[0][e] + hr[1 * 4 + i] * xv[1][e]) +
                   (hr[2 * 4 + i] * xv[2][e] + hr[3 * 4 + i] * xv[3][e]);
          else
            o[e] = hp[i] * lv[e];
        }
        Io8<T>::store_nt(ot + i * C + 8 * g, o);
      }
    }
  }
}

// ============================================================ h_post_bda bwd
// Workgroup b owns tokens [b*TG, b*TG + TG).  Per token: dX (unless null) and
// dx streamed out; 16 dH_res + 4 dH_post dot products reduced to LDS; after
// the token loop one barrier and the per-token sums are written.  With
// DBIAS, each thread keeps the fp32 dx sums of its channels over the
// workgroup's tokens and writes them as one partial row.
// This kernel keeps 256-thread workgroups with the loads of a group issued
// and consumed together (about 120 registers, four workgroups per CU): the
// two-phase form of the other streaming kernels needs ~190 registers here,
// which leaves one workgroup per CU and measured slower.
constexpr int kPostTG = 16;

// MODE as in the forward: kPostMix computes dX and dH_res only (x, H_post,
// dx, dH_post unused), kPostDist dx and dH_post only (X, H_res, dX, dH_res
// unused).
template <typename T, int GPT, bool HAS_BIAS, bool DBIAS, int MODE>
__global__ __launch_bounds__(256) void h_post_bda_bwd_kernel(
    const T *__restrict__ Gr, const T *__restrict__ X, const float *__restrict__ Hres,
    const float *__restrict__ Hpost, const T *__restrict__ x, const T *__restrict__ bias,
    T *__restrict__ dX, float *__restrict__ dHres, float *__restrict__ dHpost, T *__restrict__ dx,
    float *__restrict__ dbias_part, int64_t N, int64_t C, int TG) {
  extern __shared__ float red[];  // [nwaves][TG][20]
  constexpr bool MIX = MODE != kPostDist, DIST = MODE != kPostMix;
  constexpr int E0 = MIX ? 0 : 16, E1 = DIST ? 20 : 16;  // sums used: dH_res 0..15, dH_post 16..19
  const int G = (int)(C / 8);
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  float dbp[GPT][8];
  if (DBIAS) {
#pragma unroll
    for (int j = 0; j < GPT; ++j)
#pragma unroll
      for (int e = 0; e < 8; ++e) dbp[j][e] = 0.f;
  }
  const int64_t t0 = ((int64_t)gridDim.x - 1 - blockIdx.x) * TG;  // last tokens first
  const int ntok = (int)min((int64_t)TG, N - t0);
  for (int tt = 0; tt < ntok; ++tt) {
    const int64_t t = t0 + tt;
    float hr[16], hp[4];
    if (MIX) {
#pragma unroll
      for (int e = 0; e < 16; ++e) hr[e] = Hres[t * 16 + e];
    }
    if (DIST) {
#pragma unroll
      for (int i = 0; i < 4; ++i) hp[i] = Hpost[t * 4 + i];
    }
    float acc[20];
#pragma unroll
    for (int e = 0; e < 20; ++e) acc[e] = 0.f;
    const T *gt = Gr + t * 4 * C;
    const T *xt = X + t * 4 * C;
#pragma unroll
    for (int j = 0; j < GPT; ++j) {
      const int g = threadIdx.x + j * blockDim.x;
      if (g < G) {
        float gv[4][8], xv[4][8], lv[8];
#pragma unroll
        for (int i = 0; i < 4; ++i) Io8<T>::load_nt(gt + i * C + 8 * g, gv[i]);
        if (MIX) {
#pragma unroll
          for (int i = 0; i < 4; ++i) Io8<T>::load_nt(xt + i * C + 8 * g, xv[i]);
        }
        if (DIST) Io8<T>::load_nt(x + t * C + 8 * g, lv);
        if (DIST && HAS_BIAS) {
          float bv[8];
          Io8<T>::load(bias + 8 * g, bv);
#pragma unroll
          for (int e = 0; e < 8; ++e) lv[e] += bv[e];
        }
        // dX[j] = sum_i H_res[j][i] G[i]  (skipped when the caller folds it
        // into the pre pass backward; dX is then null for every thread)
#pragma unroll
        for (int js = 0; js < 4 && MIX && dX != nullptr; ++js) {
          float o[8];
#pragma unroll
          for (int e = 0; e < 8; ++e)
            o[e] = (hr[js * 4 + 0] * gv[0][e] + hr[js * 4 + 1] * gv[1][e]) +
                   (hr[js * 4 + 2] * gv[2][e] + hr[js * 4 + 3] * gv[3][e]);
          Io8<T>::store(dX + (t * 4 + js) * C + 8 * g, o);
        }
        // dx = sum_i H_post[i] G[i]
        if (DIST) {
          float o[8];
#pragma unroll
          for (int e = 0; e < 8; ++e)
            o[e] = (hp[0] * gv[0][e] + hp[1] * gv[1][e]) + (hp[2] * gv[2][e] + hp[3] * gv[3][e]);
          Io8<T>::store_nt(dx + t * C + 8 * g, o);
          if (DBIAS) {
#pragma unroll
            for (int e = 0; e < 8; ++e) dbp[j][e] += o[e];
          }
        }
        // dH_res[js][i] += X[js] . G[i];  dH_post[i] += G[i] . (x + bias)
        if (MIX) {
#pragma unroll
          for (int js = 0; js < 4; ++js)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              float s = 0.f;
#pragma unroll
              for (int e = 0; e < 8; ++e) s += xv[js][e] * gv[i][e];
              acc[js * 4 + i] += s;
            }
        }
        if (DIST) {
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            float s = 0.f;
#pragma unroll
            for (int e = 0; e < 8; ++e) s += gv[i][e] * lv[e];
            acc[16 + i] += s;
          }
        }
      }
    }
#pragma unroll
    for (int e = E0; e < E1; ++e) {
      const float s = wave_sum(acc[e]);
      if (lane == 0) red[(wave * TG + tt) * 20 + e] = s;
    }
  }
  __syncthreads();
  const int nw = blockDim.x >> 6;
  for (int k = threadIdx.x; k < ntok * (E1 - E0); k += blockDim.x) {
    const int tt = k / (E1 - E0), e = E0 + k % (E1 - E0);
    float s = 0.f;
    for (int w = 0; w < nw; ++w) s += red[(w * TG + tt) * 20 + e];
    const int64_t t = t0 + tt;
    if (e < 16)
      dHres[t * 16 + e] = s;
    else
      dHpost[t * 4 + (e - 16)] = s;
  }
  if (DBIAS) {
#pragma unroll
    for (int j = 0; j < GPT; ++j) {
      const int g = threadIdx.x + j * blockDim.x;
      if (g < G) {
        float *p = dbias_part + (t0 / TG) * C + 8 * g;
        *reinterpret_cast<float4 *>(p) = make_float4(dbp[j][0], dbp[j][1], dbp[j][2], dbp[j][3]);
        *reinterpret_cast<float4 *>(p + 4) = make_float4(dbp[j][4], dbp[j][5], dbp[j][6], dbp[j][7]);
      }
    }
  }
}

// ---------------------------------------------- h_post_bda bwd with dbias, bf16
// The kernel above walks a workgroup's 16 tokens one after another and issues
// a token's loads only once the previous token is done; with the bias
// gradient its N/16 workgroups fill the GPU about once, so no other
// workgroup hides that latency.  For bf16 rows of up to 1024 8-channel groups
// this kernel gives each thread one group (a workgroup spans the row) and
// loads token t + 1 while token t is computed: two register sets used in
// turn, every load unconditional (a lane past C/8 re-reads the last group and
// neither stores nor sums it), so the wait for one set counts only the loads
// issued after it.  Results per token and the dbias partial rows follow the
// same arithmetic as above with one group per thread.
// The rows loaded a token ahead are G and x (20 registers a set); X, used
// last (dH_res), is loaded when its token's turn comes, before the next
// token's G and x, so its latency is covered by the dX, dx and dH_post work
// (and its wait leaves the next token's loads in flight), and the two sets
// plus the working values stay within the 128 registers of a 1024-thread
// workgroup (holding X a token ahead too had spilled).
struct PostRowsBf16 {
  nt_u32x4 g[4], x;
};

__device__ __forceinline__ void post_rows_issue(PostRowsBf16 &r, const bf16_t *__restrict__ Gr,
                                                const bf16_t *__restrict__ x, int64_t t, int64_t C, int c8) {
#pragma unroll
  for (int i = 0; i < 4; ++i) r.g[i] = Io8<bf16_t>::ld_nt(Gr + (t * 4 + i) * C + c8);
  r.x = Io8<bf16_t>::ld_nt(x + t * C + c8);
}

__device__ __forceinline__ void post_x_issue(nt_u32x4 xr[4], const bf16_t *__restrict__ X, int64_t t, int64_t C,
                                             int c8) {
#pragma unroll
  for (int i = 0; i < 4; ++i) xr[i] = Io8<bf16_t>::ld_nt(X + (t * 4 + i) * C + c8);
}

template <bool DXO>
__device__ __forceinline__ void post_rows_compute(const PostRowsBf16 &r, const nt_u32x4 xr[4],
                                                  const float *__restrict__ Hres,
                                                  const float *__restrict__ Hpost, nt_u32x4 braw,
                                                  bf16_t *__restrict__ dX, bf16_t *__restrict__ dx, float dbp[8],
                                                  float *__restrict__ red, int64_t t, int tt, int64_t C, int c8,
                                                  bool live) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  float gv[4][8], lv[8], bv[8];
#pragma unroll
  for (int i = 0; i < 4; ++i) Io8<bf16_t>::cvt(r.g[i], gv[i]);
  Io8<bf16_t>::cvt(r.x, lv);
  Io8<bf16_t>::cvt(braw, bv);
#pragma unroll
  for (int e = 0; e < 8; ++e) lv[e] += bv[e];
  if (DXO) {
#pragma unroll
    for (int js = 0; js < 4; ++js) {
      float o[8];
#pragma unroll
      for (int e = 0; e < 8; ++e)
        o[e] = (Hres[t * 16 + js * 4 + 0] * gv[0][e] + Hres[t * 16 + js * 4 + 1] * gv[1][e]) +
               (Hres[t * 16 + js * 4 + 2] * gv[2][e] + Hres[t * 16 + js * 4 + 3] * gv[3][e]);
      if (live) Io8<bf16_t>::store(dX + (t * 4 + js) * C + c8, o);
    }
  }
  {
    float o[8];
#pragma unroll
    for (int e = 0; e < 8; ++e)
      o[e] = (Hpost[t * 4 + 0] * gv[0][e] + Hpost[t * 4 + 1] * gv[1][e]) +
             (Hpost[t * 4 + 2] * gv[2][e] + Hpost[t * 4 + 3] * gv[3][e]);
    if (live) {
      Io8<bf16_t>::store_nt(dx + t * C + c8, o);
#pragma unroll
      for (int e = 0; e < 8; ++e) dbp[e] += o[e];
    }
  }
  // dH_res[js][i] = X[js] . G[i], dH_post[i] = G[i] . (x + bias), each summed
  // over the wave as soon as it is formed
#pragma unroll
  for (int js = 0; js < 4; ++js) {
    float xv[8];
    Io8<bf16_t>::cvt(xr[js], xv);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      float a = 0.f;
#pragma unroll
      for (int e = 0; e < 8; ++e) a += xv[e] * gv[i][e];
      const float sum = wave_sum(live ? a : 0.f);
      if (lane == 0) red[(wave * kPostTG + tt) * 20 + js * 4 + i] = sum;
    }
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    float a = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) a += gv[i][e] * lv[e];
    const float sum = wave_sum(live ? a : 0.f);
    if (lane == 0) red[(wave * kPostTG + tt) * 20 + 16 + i] = sum;
  }
}

template <bool DXO>
__global__ __launch_bounds__(1024) void h_post_bda_bwd_dbias_bf16_kernel(
    const bf16_t *__restrict__ Gr, const bf16_t *__restrict__ X, const float *__restrict__ Hres,
    const float *__restrict__ Hpost, const bf16_t *__restrict__ x, const bf16_t *__restrict__ bias,
    bf16_t *__restrict__ dX, float *__restrict__ dHres, float *__restrict__ dHpost, bf16_t *__restrict__ dx,
    float *__restrict__ dbias_part, int64_t N, int64_t C) {
  extern __shared__ float red[];  // [nwaves][kPostTG][20]
  const int G = (int)(C / 8);
  const bool live = (int)threadIdx.x < G;
  const int c8 = 8 * min((int)threadIdx.x, G - 1);
  const int64_t t0 = ((int64_t)gridDim.x - 1 - blockIdx.x) * kPostTG;  // last tokens first
  const int ntok = (int)min((int64_t)kPostTG, N - t0);
  float dbp[8];
  const nt_u32x4 braw = *reinterpret_cast<const nt_u32x4 *>(bias + c8);
#pragma unroll
  for (int e = 0; e < 8; ++e) dbp[e] = 0.f;
  PostRowsBf16 ra, rb;
  nt_u32x4 xr[4];
  post_rows_issue(ra, Gr, x, t0, C, c8);
  int tt = 0;
  // two tokens per trip, both prefetches unconditional inside the loop
  for (; tt + 2 < ntok; tt += 2) {
    post_x_issue(xr, X, t0 + tt, C, c8);
    post_rows_issue(rb, Gr, x, t0 + tt + 1, C, c8);
    post_rows_compute<DXO>(ra, xr, Hres, Hpost, braw, dX, dx, dbp, red, t0 + tt, tt, C, c8, live);
    post_x_issue(xr, X, t0 + tt + 1, C, c8);
    post_rows_issue(ra, Gr, x, t0 + tt + 2, C, c8);
    post_rows_compute<DXO>(rb, xr, Hres, Hpost, braw, dX, dx, dbp, red, t0 + tt + 1, tt + 1, C, c8, live);
  }
  if (tt + 1 < ntok) {
    post_x_issue(xr, X, t0 + tt, C, c8);
    post_rows_issue(rb, Gr, x, t0 + tt + 1, C, c8);
    post_rows_compute<DXO>(ra, xr, Hres, Hpost, braw, dX, dx, dbp, red, t0 + tt, tt, C, c8, live);
    post_x_issue(xr, X, t0 + tt + 1, C, c8);
    post_rows_compute<DXO>(rb, xr, Hres, Hpost, braw, dX, dx, dbp, red, t0 + tt + 1, tt + 1, C, c8, live);
  } else {
    post_x_issue(xr, X, t0 + tt, C, c8);
    post_rows_compute<DXO>(ra, xr, Hres, Hpost, braw, dX, dx, dbp, red, t0 + tt, tt, C, c8, live);
  }
  __syncthreads();
  const int nw = blockDim.x >> 6;
  for (int k = threadIdx.x; k < ntok * 20; k += blockDim.x) {
    const int t1 = k / 20, e = k % 20;
    float s = 0.f;
    for (int w = 0; w < nw; ++w) s += red[(w * kPostTG + t1) * 20 + e];
    const int64_t t = t0 + t1;
    if (e < 16)
      dHres[t * 16 + e] = s;
    else
      dHpost[t * 4 + (e - 16)] = s;
  }
  if (live) {
    float *p = dbias_part + (t0 / kPostTG) * C + c8;
    *reinterpret_cast<float4 *>(p) = make_float4(dbp[0], dbp[1], dbp[2], dbp[3]);
    *reinterpret_cast<float4 *>(p + 4) = make_float4(dbp[4], dbp[5], dbp[6], dbp[7]);
  }
}

// ============================================================ launchers
#define MHC_GPT_DISPATCH(GPT_VAL, ...)                       \
  switch (GPT_VAL) {                                         \
    case 1: { constexpr int GPT = 1; __VA_ARGS__; } break;   \
    case 2: { constexpr int GPT = 2; __VA_ARGS__; } break;   \
    default: { constexpr int GPT = 4; __VA_ARGS__; } break;  \
  }
#define MHC_GPT_DISPATCH8(GPT_VAL, ...)                      \
  switch (GPT_VAL) {                                         \
    case 1: { constexpr int GPT = 1; __VA_ARGS__; } break;   \
    case 2: { constexpr int GPT = 2; __VA_ARGS__; } break;   \
    case 4: { constexpr int GPT = 4; __VA_ARGS__; } break;   \
    default: { constexpr int GPT = 8; __VA_ARGS__; } break;  \
  }

template <typename T>
static void agg_fwd(hipStream_t s, int64_t N, int64_t C, const void *X, const float *H, void *out, int64_t hs) {
  const StreamGeom g = stream_geom(C);
  MHC_GPT_DISPATCH(g.gpt, hipLaunchKernelGGL((h_aggregate_fwd_kernel<T, GPT>), dim3((unsigned)N),
                                              dim3(g.tpb), 0, s, (const T *)X, H, (T *)out, C, hs));
}

void launch_h_aggregate_fwd(hipStream_t s, bool f32, int64_t N, int64_t C, const void *X,
                            const float *H_pre, void *out, int64_t h_stride) {
  if (f32)
    agg_fwd<float>(s, N, C, X, H_pre, out, h_stride);
  else
    agg_fwd<bf16_t>(s, N, C, X, H_pre, out, h_stride);
}

template <typename T, bool WRITE_DX, bool ACCUM>
static void agg_bwd3(hipStream_t s, int64_t N, int64_t C, const void *g, const void *X,
                     const float *H, void *dX, float *dH, int64_t hs) {
  const StreamGeom geo = stream_geom(C);
  MHC_GPT_DISPATCH(geo.gpt,
                   hipLaunchKernelGGL((h_aggregate_bwd_kernel<T, GPT, WRITE_DX, ACCUM>),
                                      dim3((unsigned)N), dim3(geo.tpb), 0, s, (const T *)g,
                                      (const T *)X, H, (T *)dX, dH, C, hs));
}

template <typename T>
static void agg_bwd(hipStream_t s, int64_t N, int64_t C, const void *g, const void *X,
                    const float *H, void *dX, bool acc, float *dH, int64_t hs) {
  if (!dX)
    agg_bwd3<T, false, false>(s, N, C, g, X, H, dX, dH, hs);
  else if (acc)
    agg_bwd3<T, true, true>(s, N, C, g, X, H, dX, dH, hs);
  else
    agg_bwd3<T, true, false>(s, N, C, g, X, H, dX, dH, hs);
}

void launch_h_aggregate_bwd(hipStream_t s, bool f32, int64_t N, int64_t C, const void *g,
                            const void *X, const float *H_pre, void *dX, bool accumulate,
                            float *dH_pre) {
  if (f32)
    agg_bwd<float>(s, N, C, g, X, H_pre, dX, accumulate, dH_pre, 4);
  else
    agg_bwd<bf16_t>(s, N, C, g, X, H_pre, dX, accumulate, dH_pre, 4);
}

size_t h_aggregate_static_bwd_ws(int64_t N) { return (size_t)N * 16; }

void launch_h_aggregate_static_bwd(hipStream_t s, bool f32, int64_t N, int64_t C, const void *g,
                                   const void *X, const float *H_pre, void *dX, bool accumulate,
                                   float *dH_pre, void *ws) {
  float *rows = (float *)ws;  // per-token dH_pre rows [N][4]
  if (f32)
    agg_bwd<float>(s, N, C, g, X, H_pre, dX, accumulate, rows, 0);
  else
    agg_bwd<bf16_t>(s, N, C, g, X, H_pre, dX, accumulate, rows, 0);
  hipLaunchKernelGGL(hpre_rows_sum_kernel, dim3(1), dim3(256), 0, s, rows, dH_pre, N);
}

template <typename T, int MODE>
static void post_fwd(hipStream_t s, int64_t N, int64_t C, const void *X, const float *Hr,
                     const float *Hp, const void *x, const void *b, void *out) {
  const StreamGeom geo = stream_geom(C);
  if (b) {
    MHC_GPT_DISPATCH(geo.gpt, hipLaunchKernelGGL((h_post_bda_fwd_kernel<T, GPT, true, MODE>),
                                                  dim3((unsigned)N), dim3(geo.tpb), 0, s,
                                                  (const T *)X, Hr, Hp, (const T *)x,
                                                  (const T *)b, (T *)out, C));
  } else {
    MHC_GPT_DISPATCH(geo.gpt, hipLaunchKernelGGL((h_post_bda_fwd_kernel<T, GPT, false, MODE>),
                                                  dim3((unsigned)N), dim3(geo.tpb), 0, s,
                                                  (const T *)X, Hr, Hp, (const T *)x,
                                                  (const T *)nullptr, (T *)out, C));
  }
}

void launch_h_post_bda_fwd(hipStream_t s, bool f32, int64_t N, int64_t C, const void *X,
                           const float *H_res, const float *H_post, const void *x,
                           const void *bias, void *out) {
  if (f32)
    post_fwd<float, kPostFull>(s, N, C, X, H_res, H_post, x, bias, out);
  else
    post_fwd<bf16_t, kPostFull>(s, N, C, X, H_res, H_post, x, bias, out);
}

void launch_stream_mix_fwd(hipStream_t s, bool f32, int64_t N, int64_t C, const void *X, const float *M,
                           void *out) {
  if (f32)
    post_fwd<float, kPostMix>(s, N, C, X, M, nullptr, nullptr, nullptr, out);
  else
    post_fwd<bf16_t, kPostMix>(s, N, C, X, M, nullptr, nullptr, nullptr, out);
}

void launch_stream_distribute_fwd(hipStream_t s, bool f32, int64_t N, int64_t C, const void *x,
                                  const float *H_post, void *out) {
  if (f32)
    post_fwd<float, kPostDist>(s, N, C, nullptr, nullptr, H_post, x, nullptr, out);
  else
    post_fwd<bf16_t, kPostDist>(s, N, C, nullptr, nullptr, H_post, x, nullptr, out);
}

size_t h_post_bda_bwd_ws(int64_t N, int64_t C, bool with_dbias) {
  if (!with_dbias) return 0;
  const int64_t rows = (N + kPostTG - 1) / kPostTG;
  return (size_t)((rows + kRowSumSlices) * C) * sizeof(float);
}

template <typename T, bool HAS_BIAS, bool DBIAS, int MODE = kPostFull>
static void post_bwd3(hipStream_t s, int64_t N, int64_t C, const void *G, const void *X,
                      const float *Hr, const float *Hp, const void *x, const void *b, void *dX,
                      float *dHr, float *dHp, void *dx, float *part) {
  const int64_t ng = C / 8;  // 8-channel groups; 256 threads take 1, 2, 4 or 8 each
  const StreamGeom geo = ng <= 64 ? StreamGeom{64, 1} : ng <= 128 ? StreamGeom{128, 1}
                         : ng <= 256 ? StreamGeom{256, 1} : ng <= 512 ? StreamGeom{256, 2}
                         : ng <= 1024 ? StreamGeom{256, 4} : StreamGeom{256, 8};
  const int TG = DBIAS ? kPostTG : 1;
  const unsigned blocks = (unsigned)((N + TG - 1) / TG);
  const size_t lds = (size_t)(geo.tpb / 64) * TG * 20 * sizeof(float);
  MHC_GPT_DISPATCH8(geo.gpt,
                   hipLaunchKernelGGL((h_post_bda_bwd_kernel<T, GPT, HAS_BIAS, DBIAS, MODE>),
                                      dim3(blocks), dim3(geo.tpb), lds, s, (const T *)G,
                                      (const T *)X, Hr, Hp, (const T *)x, (const T *)b, (T *)dX,
                                      dHr, dHp, (T *)dx, part, N, C, TG));
}

template <typename T>
static void post_bwd(hipStream_t s, int64_t N, int64_t C, const void *G, const void *X,
                     const float *Hr, const float *Hp, const void *x, const void *b, void *dX,
                     float *dHr, float *dHp, void *dx, void *db, void *ws) {
  if (b && db) {
    float *part = (float *)ws;
    const int64_t rows = (N + kPostTG - 1) / kPostTG;
    if (sizeof(T) == 2 && C / 8 <= 1024) {
      const unsigned tpb = (unsigned)((C / 8 + 63) / 64 * 64);
      const size_t lds = (size_t)(tpb / 64) * kPostTG * 20 * sizeof(float);
      if (dX)
        hipLaunchKernelGGL(h_post_bda_bwd_dbias_bf16_kernel<true>, dim3((unsigned)rows), dim3(tpb), lds, s,
                           (const bf16_t *)G, (const bf16_t *)X, Hr, Hp, (const bf16_t *)x, (const bf16_t *)b,
                           (bf16_t *)dX, dHr, dHp, (bf16_t *)dx, part, N, C);
      else
        hipLaunchKernelGGL(h_post_bda_bwd_dbias_bf16_kernel<false>, dim3((unsigned)rows), dim3(tpb), lds, s,
                           (const bf16_t *)G, (const bf16_t *)X, Hr, Hp, (const bf16_t *)x, (const bf16_t *)b,
                           nullptr, dHr, dHp, (bf16_t *)dx, part, N, C);
    } else {
      post_bwd3<T, true, true>(s, N, C, G, X, Hr, Hp, x, b, dX, dHr, dHp, dx, part);
    }
    launch_rows_sum(s, part, rows, C, part + rows * C, db, sizeof(T) == 2);
  } else if (b) {
    post_bwd3<T, true, false>(s, N, C, G, X, Hr, Hp, x, b, dX, dHr, dHp, dx, nullptr);
  } else {
    post_bwd3<T, false, false>(s, N, C, G, X, Hr, Hp, x, b, dX, dHr, dHp, dx, nullptr);
  }
}

void launch_stream_mix_bwd(hipStream_t s, bool f32, int64_t N, int64_t C, const void *G, const void *X,
                           const float *M, void *dX, float *dM) {
  if (f32)
    post_bwd3<float, false, false, kPostMix>(s, N, C, G, X, M, nullptr, nullptr, nullptr, dX, dM, nullptr,
                                             nullptr, nullptr);
  else
    post_bwd3<bf16_t, false, false, kPostMix>(s, N, C, G, X, M, nullptr, nullptr, nullptr, dX, dM, nullptr,
                                              nullptr, nullptr);
}

void launch_stream_distribute_bwd(hipStream_t s, bool f32, int64_t N, int64_t C, const void *G,
                                  const void *x, const float *H_post, void *dx, float *dH_post) {
  if (f32)
    post_bwd3<float, false, false, kPostDist>(s, N, C, G, nullptr, nullptr, H_post, x, nullptr, nullptr,
                                              nullptr, dH_post, dx, nullptr);
  else
    post_bwd3<bf16_t, false, false, kPostDist>(s, N, C, G, nullptr, nullptr, H_post, x, nullptr, nullptr,
                                               nullptr, dH_post, dx, nullptr);
}

void launch_h_post_bda_bwd(hipStream_t s, bool f32, int64_t N, int64_t C, const void *G,
                           const void *X, const float *H_res, const float *H_post, const void *x,
                           const void *bias, void *dX, float *dH_res, float *dH_post, void *dx,
                           void *dbias, void *ws) {
  if (f32)
    post_bwd<float>(s, N, C, G, X, H_res, H_post, x, bias, dX, dH_res, dH_post, dx, dbias, ws);
  else
    post_bwd<bf16_t>(s, N, C, G, X, H_res, H_post, x, bias, dX, dH_res, dH_post, dx, dbias, ws);
}

}  // namespace mhc
