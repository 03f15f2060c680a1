// internal.h -- launchers shared between the C-ABI layer and the kernel files.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace mhc {

constexpr int kN = 4;            // residual streams supported on the GPU
constexpr int kJ = kN * kN + 2 * kN;  // 24 controller outputs
constexpr int kSavedStride = 32;

// ---- launch geometry for per-token streaming kernels
struct StreamGeom {
  int tpb;  // threads per block (a multiple of 64, at most 512)
  int gpt;  // 8-channel groups per thread (1, 2 or 4): C <= 16384
};
constexpr int64_t kMaxC = 16384;
// Largest token (or matrix) count an entry point accepts: a launch runs at
// most 512 threads per token, so every grid stays below 2^31 threads.
constexpr int64_t kMaxTokens = int64_t(1) << 22;
StreamGeom stream_geom(int64_t C);

// Measurement hook (mhc_set_kernel_events): records the registered start /
// stop event on s around a launch of kernel `id` (ids of mhc_kernel_id).
constexpr int kKernelProjBwdDxDw = 1;  // MHC_KERNEL_PROJ_BWD_DXDW
void kernel_event(int id, hipStream_t s, bool start);

// ---- bandwidth probe (measurement only): read `bytes` of src (checksums to a
// kProbeSinkWords-word sink at dst) or copy them to dst; bytes % 16 == 0.
constexpr int kProbeSinkWords = 1024;
void launch_bandwidth_probe(hipStream_t s, bool copy, bool nt, const void *src, void *dst, int64_t bytes);

// ---- Sinkhorn
void launch_sinkhorn_fwd(hipStream_t s, int64_t count, const float *L, float *H, int iters, float eps);
void launch_sinkhorn_bwd(hipStream_t s, int64_t count, const float *dH, const float *L, float *dL,
                         int iters, float eps);

// ---- streaming ops; `f32` selects fp32 activations, else bf16
// h_stride: H_pre's token stride, 4 (a row per token) or 0 (one shared row).
void launch_h_aggregate_fwd(hipStream_t s, bool f32, int64_t N, int64_t C, const void *X,
                            const float *H_pre, void *out, int64_t h_stride = 4);
// dX may be NULL (only dH_pre is produced).
void launch_h_aggregate_bwd(hipStream_t s, bool f32, int64_t N, int64_t C, const void *g,
                            const void *X, const float *H_pre, void *dX, bool accumulate,
                            float *dH_pre);
void launch_h_post_bda_fwd(hipStream_t s, bool f32, int64_t N, int64_t C, const void *X,
                           const float *H_res, const float *H_post, const void *x,
                           const void *bias, void *out);
// One H_pre row [4] for all tokens: dX as above, dH_pre [4] = sum over tokens
// (per-token rows in ws, then a fixed-order sum).
size_t h_aggregate_static_bwd_ws(int64_t N);
void launch_h_aggregate_static_bwd(hipStream_t s, bool f32, int64_t N, int64_t C, const void *g,
                                   const void *X, const float *H_pre, void *dX, bool accumulate,
                                   float *dH_pre, void *ws);
// The two halves of h_post_bda on their own: stream mix out[i] = sum_j M[j][i] X[j]
// and stream distribute out[i] = H_post[i] x, with their backwards.
void launch_stream_mix_fwd(hipStream_t s, bool f32, int64_t N, int64_t C, const void *X, const float *M,
                           void *out);
void launch_stream_mix_bwd(hipStream_t s, bool f32, int64_t N, int64_t C, const void *G, const void *X,
                           const float *M, void *dX, float *dM);
void launch_stream_distribute_fwd(hipStream_t s, bool f32, int64_t N, int64_t C, const void *x,
                                  const float *H_post, void *out);
void launch_stream_distribute_bwd(hipStream_t s, bool f32, int64_t N, int64_t C, const void *G,
                                  const void *x, const float *H_post, void *dx, float *dH_post);
size_t h_post_bda_bwd_ws(int64_t N, int64_t C, bool with_dbias);
void launch_h_post_bda_bwd(hipStream_t s, bool f32, int64_t N, int64_t C, const void *G,
                           const void *X, const float *H_res, const float *H_post, const void *x,
                           const void *bias, void *dX, float *dH_res, float *dH_post, void *dx,
                           void *dbias, void *ws);

// ---- fixed-order column sums of per-workgroup partial rows part[R][C] (fp32)
// into out[C] (fp32 or bf16); mid: kRowSumSlices * C floats of scratch.
constexpr int kRowSumSlices = 16;
void launch_rows_sum(hipStream_t s, const float *part, int64_t R, int64_t C, float *mid, void *out,
                     bool out_bf16);

// ---- RMSNorm of the aggregated stream [N][C]; gamma [C] fp32 or NULL (unit gain)
void launch_rmsnorm_fwd(hipStream_t s, bool f32, int64_t N, int64_t C, const void *x, const float *gamma,
                        float eps, void *y);
// h_aggregate writing agg, then y = RMSNorm(agg as stored), in one pass (H_pre [N][4]).
void launch_h_aggregate_rmsnorm_fwd(hipStream_t s, bool f32, int64_t N, int64_t C, const void *X,
                                    const float *H_pre, const float *gamma, float eps, void *agg, void *y);
// dx (+)= the RMSNorm input gradient; dgamma (may be NULL) = sum over tokens,
// through per-workgroup partial rows in ws (rmsnorm_bwd_ws bytes).
size_t rmsnorm_bwd_ws(int64_t N, int64_t C, bool with_dgamma);
void launch_rmsnorm_bwd(hipStream_t s, bool f32, int64_t N, int64_t C, const void *dy, const void *x,
                        const float *gamma, float eps, void *dx, bool accumulate, float *dgamma, void *ws);

// ---- projection (forward)
size_t proj_fwd_ws(int64_t N, int64_t C, bool f32);
// Writes H_pre, H_post, logits, saved (may be NULL); if H_res != NULL also
// runs Sinkhorn on the logits.
void launch_proj_fwd(hipStream_t s, bool f32, int64_t N, int64_t C, const void *X, const float *W,
                     const float *alpha, const float *hbias, float rms_eps, float *H_pre,
                     float *H_post, float *logits, float *saved, float *H_res, int iters,
                     float eps, void *ws);

// The same forward (bf16 activations) with x @ W on the VALU: the comparison
// point for the MFMA projection (same workspace layout, Sinkhorn not run).
void launch_proj_fwd_fma(hipStream_t s, int64_t N, int64_t C, const void *X, const float *W, const float *alpha,
                         const float *hbias, float rms_eps, float *H_pre, float *H_post, float *logits,
                         float *saved, void *ws);

// ---- projection (backward).  Two front ends share the dX / dW kernels:
//  - proj_rms_h_bwd: dL given directly (dH_res_logits)
//  - pre_bwd: dH_pre from g.X, dL from the Sinkhorn backward of dH_res, and
//    the aggregate term H_pre * g added into dX.
size_t proj_bwd_ws(int64_t N, int64_t C, bool f32);
struct ProjBwdArgs {
  bool f32;
  int64_t N, C;
  const void *X;
  const float *W, *alpha, *saved, *H_pre, *H_post;
  const float *dH_pre;   // NULL in the fused pre backward (computed from g)
  const float *dH_post;
  const float *dL;       // logits gradient, or NULL when dH_res + logits are given
  const float *dH_res, *logits;
  int iters;
  float eps;
  const void *g;         // gradient of the aggregated stream (fused pre backward) or NULL
  void *dX;
  bool accumulate;
  float *dW, *dalpha, *dhbias;
  float *dH_pre_out, *dL_out;
  void *ws;
  const void *post_G;       // h_post_bda upstream gradient, or NULL (see mhc_pre_bwd)
  const float *post_H_res;  // H_res of the h_post_bda pass, with post_G
};
void launch_proj_bwd(hipStream_t s, const ProjBwdArgs &a);

// ---- any stream count 1 <= n <= 8 other than 4 (generic.hip); same
// arguments as the n = 4 launchers above, with n explicit.
constexpr int kMaxN = 8;
// Row stride of the saved forward state {r, q, z[J], 0...}: 32 while
// 2 + J fits, else 2 + J rounded up to a multiple of 8.
int saved_stride(int n);
void glaunch_sinkhorn_fwd(hipStream_t s, int n, int64_t count, const float *L, float *H, int iters, float eps);
void glaunch_sinkhorn_bwd(hipStream_t s, int n, int64_t count, const float *dH, const float *L, float *dL,
                          int iters, float eps);
void glaunch_h_aggregate_fwd(hipStream_t s, bool f32, int n, int64_t N, int64_t C, const void *X,
                             const float *H_pre, void *out, int64_t hs);
void glaunch_h_aggregate_bwd(hipStream_t s, bool f32, int n, int64_t N, int64_t C, const void *g, const void *X,
                             const float *H_pre, void *dX, bool accumulate, float *dH_pre);
size_t gh_aggregate_static_bwd_ws(int n, int64_t N);
void glaunch_h_aggregate_static_bwd(hipStream_t s, bool f32, int n, int64_t N, int64_t C, const void *g,
                                    const void *X, const float *H_pre, void *dX, bool accumulate, float *dH_pre,
                                    void *ws);
void glaunch_h_post_bda_fwd(hipStream_t s, bool f32, int n, int64_t N, int64_t C, const void *X,
                            const float *H_res, const float *H_post, const void *x, const void *bias, void *out);
void glaunch_stream_mix_fwd(hipStream_t s, bool f32, int n, int64_t N, int64_t C, const void *X, const float *M,
                            void *out);
void glaunch_stream_distribute_fwd(hipStream_t s, bool f32, int n, int64_t N, int64_t C, const void *x,
                                   const float *H_post, void *out);
size_t gh_post_bda_bwd_ws(int64_t N, int64_t C, bool with_dbias);
void glaunch_h_post_bda_bwd(hipStream_t s, bool f32, int n, int64_t N, int64_t C, const void *G, const void *X,
                            const float *H_res, const float *H_post, const void *x, const void *bias, void *dX,
                            float *dH_res, float *dH_post, void *dx, void *dbias, void *ws);
void glaunch_stream_mix_bwd(hipStream_t s, bool f32, int n, int64_t N, int64_t C, const void *G, const void *X,
                            const float *M, void *dX, float *dM);
void glaunch_stream_distribute_bwd(hipStream_t s, bool f32, int n, int64_t N, int64_t C, const void *G,
                                   const void *x, const float *H_post, void *dx, float *dH_post);
size_t gproj_fwd_ws(int n, int64_t N, int64_t C, bool f32);
void glaunch_proj_fwd(hipStream_t s, bool f32, int n, int64_t N, int64_t C, const void *X, const float *W,
                      const float *alpha, const float *hbias, float rms_eps, float *H_pre, float *H_post,
                      float *logits, float *saved, float *H_res, int iters, float eps, void *ws);
// terms: the fused pre backward (aggregate and h_post_bda residual terms formed first)
size_t gproj_bwd_ws(int n, int64_t N, int64_t C, bool terms, bool f32);
void glaunch_proj_bwd(hipStream_t s, int n, const ProjBwdArgs &a);

}  // namespace mhc
