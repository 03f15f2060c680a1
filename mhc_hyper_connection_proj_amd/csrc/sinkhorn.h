// sinkhorn.h -- register-resident Sinkhorn-Knopp on one 4x4 matrix per lane.
//
// Forward (Megatron Core fused_mhc_kernels, operation sinkhorn; rwkv-ops
// "Sinkhorn Knopp FFI"): M = exp(L), then `iters` times a row pass
// M[a][:] *= 1/(rowsum_a + eps) followed by a column pass.  One lane owns the
// 16 entries, so row and column sums need no cross-lane traffic and each
// reciprocal is computed once (4 v_rcp_f32 per half-step).
//
// Floating-point contraction is off in the passes and in the quad sum: a
// row pass's scaling (M *= 1/d) would otherwise be fused into the next
// column sum as an fma, which rounds one term fewer, and differently in the
// one-lane and the quad layouts.  Every entry is rounded after its scaling,
// so both layouts run the same operation sequence.
//
// Backward: exact reverse mode of the unrolled map.  A half-step M' = M / d
// (d = line sum + eps) has the adjoint dM = (G - <G, M'>_line) / d.  The
// replay stores each half-step's 4 denominators in registers and walks back
// by reconstructing the half-step input as M' * d, so no matrix history is
// kept.  Replay runs in segments of SK_SEG iterations from the last segment
// backwards (each segment re-runs the forward from the logits), which bounds
// both the register footprint and the reconstruction drift to one segment.
#pragma once

#include "device.h"

namespace mhc {

constexpr int SK_SEG = 20;

__device__ __forceinline__ void sk_row_pass(float M[16], float eps, float d[4]) {
#pragma clang fp contract(off)
#pragma unroll
  for (int a = 0; a < 4; ++a) {
    d[a] = ((M[4 * a] + M[4 * a + 1]) + (M[4 * a + 2] + M[4 * a + 3])) + eps;
    const float inv = fast_rcp(d[a]);
#pragma unroll
    for (int b = 0; b < 4; ++b) M[4 * a + b] *= inv;
  }
}

__device__ __forceinline__ void sk_col_pass(float M[16], float eps, float d[4]) {
#pragma clang fp contract(off)
#pragma unroll
  for (int b = 0; b < 4; ++b) {
    d[b] = ((M[b] + M[4 + b]) + (M[8 + b] + M[12 + b])) + eps;
    const float inv = fast_rcp(d[b]);
#pragma unroll
    for (int a = 0; a < 4; ++a) M[4 * a + b] *= inv;
  }
}

__device__ __forceinline__ void sk_exp(const float L[16], float M[16]) {
#pragma unroll
  for (int e = 0; e < 16; ++e) M[e] = expf(L[e]);
}

// In place: L (logits) -> H_res.
__device__ __forceinline__ void sk_forward(float M[16], int iters, float eps) {
  float d[4];
  for (int it = 0; it < iters; ++it) {
    sk_row_pass(M, eps, d);
    sk_col_pass(M, eps, d);
  }
}

// Adjoint of a row half-step with output M (in place: M becomes the input).
__device__ __forceinline__ void sk_row_back(float G[16], float M[16], const float d[4]) {
#pragma unroll
  for (int a = 0; a < 4; ++a) {
    const float dot = (G[4 * a] * M[4 * a] + G[4 * a + 1] * M[4 * a + 1]) +
                      (G[4 * a + 2] * M[4 * a + 2] + G[4 * a + 3] * M[4 * a + 3]);
    const float inv = fast_rcp(d[a]);
#pragma unroll
    for (int b = 0; b < 4; ++b) {
      G[4 * a + b] = (G[4 * a + b] - dot) * inv;
      M[4 * a + b] *= d[a];
    }
  }
}

__device__ __forceinline__ void sk_col_back(float G[16], float M[16], const float d[4]) {
#pragma unroll
  for (int b = 0; b < 4; ++b) {
    const float dot = (G[b] * M[b] + G[4 + b] * M[4 + b]) + (G[8 + b] * M[8 + b] + G[12 + b] * M[12 + b]);
    const float inv = fast_rcp(d[b]);
#pragma unroll
    for (int a = 0; a < 4; ++a) {
      G[4 * a + b] = (G[4 * a + b] - dot) * inv;
      M[4 * a + b] *= d[b];
    }
  }
}

// G: in = dH_res, out = dL.  L: logits.
__device__ __forceinline__ void sk_backward(const float L[16], float G[16], int iters, float eps) {
  const int nseg = (iters + SK_SEG - 1) / SK_SEG;
  for (int s = nseg - 1; s >= 0; --s) {
    float M[16];
    float drow[SK_SEG][4], dcol[SK_SEG][4];
    sk_exp(L, M);
    for (int it = 0; it < s * SK_SEG; ++it) {
      sk_row_pass(M, eps, drow[0]);
      sk_col_pass(M, eps, dcol[0]);
    }
    const int cnt = min(iters - s * SK_SEG, SK_SEG);
#pragma unroll
    for (int j = 0; j < SK_SEG; ++j) {
      if (j < cnt) {
        sk_row_pass(M, eps, drow[j]);
        sk_col_pass(M, eps, dcol[j]);
      }
    }
#pragma unroll
    for (int j = SK_SEG - 1; j >= 0; --j) {
      if (j < cnt) {
        sk_col_back(G, M, dcol[j]);
        sk_row_back(G, M, drow[j]);
      }
    }
  }
  float E[16];
  sk_exp(L, E);
#pragma unroll
  for (int e = 0; e < 16; ++e) G[e] *= E[e];
}

// ---------------------------------------------------------------- quad layout
// Four lanes per matrix (lanes 4k..4k+3 of a wave): lane r = threadIdx.x & 3
// holds row r in m[4].  Row sums stay in the lane; a column sum adds the
// four lanes' entries with two quad permutes, (r0 + r1) + (r2 + r3) on every
// lane, the same association as the one-lane code above, so the forward is
// bit-identical to it.  Used where one layer's tokens give too few waves for
// one matrix per lane to fill the chip.
__device__ __forceinline__ float quad_sum(float v) {
#pragma clang fp contract(off)
  v += dpp<DPP_QUAD_1032>(v);
  v += dpp<DPP_QUAD_2301>(v);
  return v;
}

// value of lane b of the quad, on every lane of it
template <int B>
__device__ __forceinline__ float quad_bcast(float v) {
  return dpp<B * 0x55>(v);
}

__device__ __forceinline__ void sk_exp4(const float l[4], float m[4]) {
#pragma unroll
  for (int b = 0; b < 4; ++b) m[b] = expf(l[b]);
}

__device__ __forceinline__ void sk_row_pass_q(float m[4], float eps, float &d) {
#pragma clang fp contract(off)
  d = ((m[0] + m[1]) + (m[2] + m[3])) + eps;
  const float inv = fast_rcp(d);
#pragma unroll
  for (int b = 0; b < 4; ++b) m[b] *= inv;
}

// dcol: this lane's own column's denominator (column r)
__device__ __forceinline__ void sk_col_pass_q(float m[4], float eps, int r, float &dcol) {
#pragma clang fp contract(off)
#pragma unroll
  for (int b = 0; b < 4; ++b) {
    const float d = quad_sum(m[b]) + eps;
    dcol = r == b ? d : dcol;
    m[b] *= fast_rcp(d);
  }
}

// In place: logits row -> H_res row.
__device__ __forceinline__ void sk_forward_q(float m[4], int iters, float eps, int r) {
  float d, dc = 0.f;
  for (int it = 0; it < iters; ++it) {
    sk_row_pass_q(m, eps, d);
    sk_col_pass_q(m, eps, r, dc);
  }
}

// g: in = dH_res row r, out = dL row r.  l: logits row r.  Same replay as
// sk_backward; each lane keeps its row's and its own column's denominators
// and takes the other columns' from their lanes.
__device__ __forceinline__ void sk_backward_q(const float l[4], float g[4], int iters, float eps, int r) {
  const int nseg = (iters + SK_SEG - 1) / SK_SEG;
  for (int s = nseg - 1; s >= 0; --s) {
    float m[4];
    float drow[SK_SEG], dcol[SK_SEG];
#pragma unroll
    for (int j = 0; j < SK_SEG; ++j) dcol[j] = 0.f;
    sk_exp4(l, m);
    for (int it = 0; it < s * SK_SEG; ++it) {
      sk_row_pass_q(m, eps, drow[0]);
      sk_col_pass_q(m, eps, r, dcol[0]);
    }
    const int cnt = min(iters - s * SK_SEG, SK_SEG);
#pragma unroll
    for (int j = 0; j < SK_SEG; ++j) {
      if (j < cnt) {
        sk_row_pass_q(m, eps, drow[j]);
        sk_col_pass_q(m, eps, r, dcol[j]);
      }
    }
#pragma unroll
    for (int j = SK_SEG - 1; j >= 0; --j) {
      if (j < cnt) {
        const float dc[4] = {quad_bcast<0>(dcol[j]), quad_bcast<1>(dcol[j]), quad_bcast<2>(dcol[j]),
                             quad_bcast<3>(dcol[j])};
#pragma unroll
        for (int b = 0; b < 4; ++b) {
          const float dot = quad_sum(g[b] * m[b]);
          g[b] = (g[b] - dot) * fast_rcp(dc[b]);
          m[b] *= dc[b];
        }
        const float dot = (g[0] * m[0] + g[1] * m[1]) + (g[2] * m[2] + g[3] * m[3]);
        const float inv = fast_rcp(drow[j]);
#pragma unroll
        for (int b = 0; b < 4; ++b) {
          g[b] = (g[b] - dot) * inv;
          m[b] *= drow[j];
        }
      }
    }
  }
  float e[4];
  sk_exp4(l, e);
#pragma unroll
  for (int b = 0; b < 4; ++b) g[b] *= e[b];
}

__device__ __forceinline__ void load16(const float *p, float v[16]) {
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const float4 w = reinterpret_cast<const float4 *>(p)[q];
    v[4 * q] = w.x; v[4 * q + 1] = w.y; v[4 * q + 2] = w.z; v[4 * q + 3] = w.w;
  }
}

__device__ __forceinline__ void store16(float *p, const float v[16]) {
#pragma unroll
  for (int q = 0; q < 4; ++q)
    reinterpret_cast<float4 *>(p)[q] = make_float4(v[4 * q], v[4 * q + 1], v[4 * q + 2], v[4 * q + 3]);
}

}  // namespace mhc
