/*
 * mhc.h -- C ABI of libmhc: the per-token mHC (Manifold-Constrained
 * Hyper-Connections) residual-mixing path on AMD Instinct MI355X (gfx950).
 *
 * Notation (per token): n residual streams of C channels; K = n*C; the
 * flattened stream index is k = i*C + c; J = n*n + 2n controller outputs,
 * ordered PRE [0,n) | POST [n,2n) | RES [2n, 2n+n*n) with RES row-major.
 * Every entry point takes 1 <= n <= 8 (the pages' kernels read n from the
 * tensor shapes).  n == 4 (J = 24, every benchmark workload) runs on kernels
 * laid out for it; other n run on simpler kernels templated on n, with the
 * same definitions, layouts, validation and determinism.
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 *  - `stream` is a hipStream_t passed as void* (NULL = the default stream).
 *    Calls only enqueue work on it and return; results are ready when the
 *    stream has reached the call.
 *  - Every tensor pointer is caller-owned DEVICE memory, dense, row-major,
 *    16-byte aligned.  The library allocates nothing and keeps no state
 *    between calls; scratch for cross-token reductions comes from the
 *    caller's `workspace` (sized by the matching *_workspace_size query,
 *    256-byte aligned).  Calls on different streams with disjoint buffers
 *    may run concurrently.
 *  - Activation tensors (residual X and its gradients, the layer input/output
 *    x, bias, the aggregated stream) are stored as `act` (bf16 or fp32) and
 *    computed in fp32; H tensors, logits, W, alpha, hbias and all of their
 *    gradients are fp32.  bf16 outputs are rounded once, to nearest even.
 *  - Every output is fully overwritten; `accumulate_dX = 1` is the only
 *    read-modify-write (dX += this op's gradient, for summing the residual
 *    gradient contributions).  No float atomics: results are bitwise
 *    deterministic from run to run.
 *  - Fail-closed validation BEFORE anything is enqueued: a bad argument
 *    returns an error and leaves every output untouched.  MHC_ERR_NULL for a
 *    missing required pointer, MHC_ERR_SHAPE for negative/zero sizes,
 *    MHC_ERR_UNSUPPORTED for n > 8, C % 8 != 0, C > 16384, iters > 4096 or
 *    tokens (count) > 4194304 (2^22; each launch then stays below 2^31 threads),
 *    MHC_ERR_ALIGN for pointers not 16-byte aligned, MHC_ERR_ALIAS when an
 *    output overlaps an input or another output, MHC_ERR_WORKSPACE when the
 *    workspace is missing or too small, MHC_ERR_ARG for eps < 0, a
 *    non-finite eps or an unknown dtype, MHC_ERR_HIP when a launch fails.
 *    tokens == 0 (or count == 0) is a successful no-op.  mhc_last_error()
 *    describes the most recent failure on the calling thread.
 */
#ifndef MHC_H_
#define MHC_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum mhc_status {
  MHC_OK = 0,
  MHC_ERR_NULL = 1,
  MHC_ERR_SHAPE = 2,
  MHC_ERR_UNSUPPORTED = 3,
  MHC_ERR_ALIGN = 4,
  MHC_ERR_ALIAS = 5,
  MHC_ERR_WORKSPACE = 6,
  MHC_ERR_ARG = 7,
  MHC_ERR_HIP = 8
} mhc_status;

typedef enum mhc_dtype { MHC_BF16 = 0, MHC_F32 = 1 } mhc_dtype;

/* Per-token record written by the projection forward and read by its
 * backward: fp32 [tokens][mhc_saved_stride(n)] = { r, q, z[0..J), 0 ... }
 * with q = sqrt(sum x^2 / K), r = 1/(q + rms_eps) and z = r * (x @ W)
 * (pre-gain).  The stride is MHC_SAVED_STRIDE (32) while 2 + J <= 32
 * (n <= 4), else 2 + J rounded up to a multiple of 8; mhc_saved_stride
 * returns 0 for n outside [1, 8]. */
#define MHC_SAVED_STRIDE 32
int32_t mhc_saved_stride(int32_t n);

const char *mhc_status_string(mhc_status s);
const char *mhc_last_error(void);
const char *mhc_version(void);

/* -------------------------------------------------------------------------
 * Measurement hook (benchmarks and profilers; nothing is computed through it).
 * A call such as mhc_pre_bwd launches several kernels; to time one of them
 * alone, register two caller-owned HIP events (hipEvent_t, passed as void *)
 * for it.  While registered, on the calling host thread only, every launch of
 * that kernel by a libmhc call made from this thread is bracketed by
 * hipEventRecord(start_event) and hipEventRecord(stop_event) on the call's
 * stream.  kernel = MHC_KERNEL_NONE, or both events NULL, clears the hook.
 * Returns MHC_ERR_ARG for an unknown kernel id or exactly one NULL event.
 * A failed event record is ignored: it cannot change any result.
 *   MHC_KERNEL_PROJ_BWD_DXDW: the projection backward's dX / dW kernel
 *   (launched by mhc_proj_rms_h_bwd and mhc_pre_bwd).
 * ---------------------------------------------------------------------- */
typedef enum mhc_kernel_id { MHC_KERNEL_NONE = 0, MHC_KERNEL_PROJ_BWD_DXDW = 1 } mhc_kernel_id;
mhc_status mhc_set_kernel_events(int32_t kernel, void *start_event, void *stop_event);

/* Measurement hook: the practical memory rates of the device, reported beside
 * its HBM peak; nothing of the mHC path is computed.  Streams `bytes` (a
 * multiple of 16) of src with 16-byte vector loads, four per thread in
 * flight, 8192 workgroups of 256 threads each taking one contiguous share.
 * kind = MHC_PROBE_READ: read only; dst (at least 4096 bytes) receives an
 * unspecified checksum.  kind = MHC_PROBE_COPY: src is copied to dst (bytes
 * each, not overlapping).  Add MHC_PROBE_NONTEMPORAL for loads (and copy
 * stores) with the non-temporal cache policy.  Validation as for every
 * entry point. */
typedef enum mhc_probe_kind {
  MHC_PROBE_READ = 0, MHC_PROBE_COPY = 1, MHC_PROBE_NONTEMPORAL = 2
} mhc_probe_kind;
mhc_status mhc_bandwidth_probe(void *stream, int32_t kind, const void *src, void *dst, size_t bytes);

/* -------------------------------------------------------------------------
 * Projection + RMS + compute_h, forward.
 * Megatron Core "core.fusions.fused_mhc_kernels", operation
 * proj_rms_compute_h (`_torch_proj_rms_compute_h(x, weight, alpha_pre,
 * alpha_post, alpha_res, bias, n, eps)`); RL-Kernel PR #383 review of the RMS
 * leg (r = 1/(q + eps)) and the commit making alpha three segment gains.
 *
 *   q = sqrt(sum_k x_k^2 / K), r = 1/(q + rms_eps), z = r * (x @ W)
 *   zh_j = alpha[seg(j)] * z_j + hbias[j]
 *   H_pre = sigmoid(zh_PRE), H_post = 2 sigmoid(zh_POST), logits = zh_RES
 *
 * X [tokens][n][C] (act); W [K][J] fp32; alpha [3] fp32 (pre, post, res) or
 * NULL for ones; hbias [J] fp32 or NULL for zeros.  Outputs (fp32): H_pre
 * [tokens][n], H_post [tokens][n], H_res_logits [tokens][n][n], saved
 * [tokens][mhc_saved_stride(n)].  `saved` may be NULL when no backward follows.
 * ---------------------------------------------------------------------- */
size_t mhc_proj_rms_h_workspace_size(int64_t tokens, int32_t n, int64_t C, mhc_dtype act);
mhc_status mhc_proj_rms_h(void *stream, int64_t tokens, int32_t n, int64_t C, mhc_dtype act,
                          const void *X, const float *W, const float *alpha, const float *hbias,
                          float rms_eps, float *H_pre, float *H_post, float *H_res_logits,
                          float *saved, void *workspace, size_t workspace_bytes);

/* The same forward with the contraction x @ W as fp32 FMAs on the vector ALUs
 * instead of the matrix cores: the comparison point that the MFMA choice is
 * measured against (n == 4 and bf16 activations only, else
 * MHC_ERR_UNSUPPORTED; the workspace of mhc_proj_rms_h_workspace_size).
 * Results agree with mhc_proj_rms_h to fp32 rounding (a different summation
 * order), not bit for bit. */
mhc_status mhc_proj_rms_h_fma(void *stream, int64_t tokens, int32_t n, int64_t C, mhc_dtype act,
                              const void *X, const float *W, const float *alpha, const float *hbias,
                              float rms_eps, float *H_pre, float *H_post, float *H_res_logits,
                              float *saved, void *workspace, size_t workspace_bytes);

/* -------------------------------------------------------------------------
 * Projection + RMS + compute_h, backward (RL-Kernel PR #383: the RMS
 * backward is the GEMM leg plus the RMS leg, with the RMS leg zero for an
 * all-zero row; d_alpha is three scalars).
 *
 *   dzh_PRE = dH_pre * H_pre (1 - H_pre), dzh_POST = dH_post * H_post (1 -
 *   H_post/2), dzh_RES = dH_res_logits; dz = alpha * dzh; dr = sum_j dz_j z_j / r;
 *   dX (+)= r dz @ W^T - dr r^2 x / (K q)     (RMS term 0 when q == 0)
 *   dW = sum_t r x^T dz, dalpha[s] = sum_t sum_{j in s} dzh_j z_j,
 *   dhbias = sum_t dzh
 *
 * Inputs: X, W, alpha (NULL = ones), saved/H_pre/H_post from the forward,
 * upstream gradients dH_pre [tokens][n], dH_post [tokens][n], dH_res_logits
 * [tokens][n][n] (fp32).  Outputs: dX [tokens][n][C] (act; overwritten, or
 * accumulated into when accumulate_dX != 0); dW [K][J], dalpha [3], dhbias
 * [J] (fp32; each may be NULL to skip it).
 * ---------------------------------------------------------------------- */
size_t mhc_proj_rms_h_bwd_workspace_size(int64_t tokens, int32_t n, int64_t C, mhc_dtype act);
mhc_status mhc_proj_rms_h_bwd(void *stream, int64_t tokens, int32_t n, int64_t C, mhc_dtype act,
                              const void *X, const float *W, const float *alpha, const float *saved,
                              const float *H_pre, const float *H_post, const float *dH_pre,
                              const float *dH_post, const float *dH_res_logits, void *dX,
                              int32_t accumulate_dX, float *dW, float *dalpha, float *dhbias,
                              void *workspace, size_t workspace_bytes);

/* -------------------------------------------------------------------------
 * Sinkhorn-Knopp projection of each n x n logit matrix (Megatron Core
 * fused_mhc_kernels, operation sinkhorn / `fused_sinkhorn`: project logits to
 * a doubly stochastic matrix; rwkv-ops mhu_ffi.cu, "Sinkhorn Knopp FFI",
 * attributes num_iters and eps).
 *
 *   M = exp(logits); iters times: each row /= (row sum + eps), then each
 *   column /= (column sum + eps).   H_res = M.
 *
 * logits, H_res: fp32 [count][n][n].  iters in [0, 4096], eps >= 0.
 * ---------------------------------------------------------------------- */
mhc_status mhc_sinkhorn_fwd(void *stream, int64_t count, int32_t n, const float *logits,
                            float *H_res, int32_t iters, float eps);

/* Exact reverse mode of the unrolled forward map (every half-step, eps
 * included), replayed from the logits (rwkv-ops "Sinkhorn Knopp FFI"
 * backward takes the forward input, iters and eps).  dH_res, logits,
 * dlogits: fp32 [count][n][n]. */
mhc_status mhc_sinkhorn_bwd(void *stream, int64_t count, int32_t n, const float *dH_res,
                            const float *logits, float *dlogits, int32_t iters, float eps);

/* -------------------------------------------------------------------------
 * h_aggregate: weighted n-stream -> 1-stream aggregation (Megatron Core
 * fused_mhc_kernels `fused_h_aggregate` / `FusedHAggregate`; rwkv-ops
 * "Stream Aggregate FFI", per-token weights).
 *
 *   out[t][c] = sum_i H_pre[t][i] X[t][i][c]
 *
 * X [tokens][n][C] (act), H_pre [tokens][n] fp32, out [tokens][C] (act).
 * ---------------------------------------------------------------------- */
mhc_status mhc_h_aggregate_fwd(void *stream, int64_t tokens, int32_t n, int64_t C, mhc_dtype act,
                               const void *X, const float *H_pre, void *out);

/* Backward (`_torch_h_aggregate_bwd(grad_output, x, h_pre)`):
 *   dX[t][i][c] (+)= H_pre[t][i] g[t][c],   dH_pre[t][i] = sum_c g[t][c] X[t][i][c]
 * g [tokens][C] (act); dX (act, overwritten or accumulated); dH_pre fp32. */
mhc_status mhc_h_aggregate_bwd(void *stream, int64_t tokens, int32_t n, int64_t C, mhc_dtype act,
                               const void *g, const void *X, const float *H_pre, void *dX,
                               int32_t accumulate_dX, float *dH_pre);

/* -------------------------------------------------------------------------
 * h_post_bda: H_res^T @ residual + H_post * (x + bias) (Megatron Core
 * fused_mhc_kernels `fused_h_post_bda` / `FusedHPostBDA`; rwkv-ops "MHC
 * Post-Op FFI", which has no bias).
 *
 *   out[t][i][c] = sum_j H_res[t][j][i] X[t][j][c] + H_post[t][i] (x[t][c] + bias[c])
 *
 * X [tokens][n][C] (act), H_res [tokens][n][n] fp32, H_post [tokens][n] fp32,
 * x [tokens][C] (act), bias [C] (act) or NULL, out [tokens][n][C] (act).
 * ---------------------------------------------------------------------- */
mhc_status mhc_h_post_bda_fwd(void *stream, int64_t tokens, int32_t n, int64_t C, mhc_dtype act,
                              const void *X, const float *H_res, const float *H_post, const void *x,
                              const void *bias, void *out);

/* Backward (`_torch_h_post_bda_bwd(grad_output, h_res, original_residual,
 * h_post, x, bias)` -> five gradients, the last optional):
 *   dX[j][c] = sum_i H_res[j][i] G[i][c]          (act, overwritten; dX may be
 *                                                  NULL to skip it when the
 *                                                  caller has mhc_pre_bwd add
 *                                                  this term from G instead)
 *   dH_res[j][i] = sum_c X[j][c] G[i][c]          (fp32)
 *   dH_post[i] = sum_c G[i][c] (x[c] + bias[c])   (fp32)
 *   dx[c] = sum_i H_post[i] G[i][c]               (act)
 *   dbias[c] = sum_t dx_t[c]                      (act; only if dbias != NULL,
 *                                                  which requires bias != NULL)
 * G [tokens][n][C] (act). */
size_t mhc_h_post_bda_bwd_workspace_size(int64_t tokens, int32_t n, int64_t C, mhc_dtype act,
                                         int32_t with_dbias);
mhc_status mhc_h_post_bda_bwd(void *stream, int64_t tokens, int32_t n, int64_t C, mhc_dtype act,
                              const void *G, const void *X, const float *H_res,
                              const float *H_post, const void *x, const void *bias, void *dX,
                              float *dH_res, float *dH_post, void *dx, void *dbias,
                              void *workspace, size_t workspace_bytes);

/* -------------------------------------------------------------------------
 * The two halves of h_post_bda as operations of their own (rwkv-ops
 * mhu_ffi.cu, sections "Stream Mix FFI" and "Stream Distribute FFI"); the
 * mix uses the same orientation as h_post_bda's H_res term.
 *   stream mix:        out[i][c] = sum_j M[j][i] X[j][c]
 *                      dX[j][c] = sum_i M[j][i] G[i][c], dM[j][i] = sum_c X[j][c] G[i][c]
 *   stream distribute: out[i][c] = H_post[i] x[c]
 *                      dx[c] = sum_i H_post[i] G[i][c], dH_post[i] = sum_c G[i][c] x[c]
 * X, G, out, dX [tokens][n][C] (act); x, dx [tokens][C] (act); M, dM
 * [tokens][n][n] fp32; H_post, dH_post [tokens][n] fp32.  Every output is
 * written in full; none may overlap an input or another output.
 * ---------------------------------------------------------------------- */
mhc_status mhc_stream_mix_fwd(void *stream, int64_t tokens, int32_t n, int64_t C, mhc_dtype act,
                              const void *X, const float *M, void *out);
mhc_status mhc_stream_mix_bwd(void *stream, int64_t tokens, int32_t n, int64_t C, mhc_dtype act,
                              const void *G, const void *X, const float *M, void *dX, float *dM);
mhc_status mhc_stream_distribute_fwd(void *stream, int64_t tokens, int32_t n, int64_t C, mhc_dtype act,
                                     const void *x, const float *H_post, void *out);
mhc_status mhc_stream_distribute_bwd(void *stream, int64_t tokens, int32_t n, int64_t C, mhc_dtype act,
                                     const void *G, const void *x, const float *H_post, void *dx,
                                     float *dH_post);

/* -------------------------------------------------------------------------
 * h_aggregate with one H_pre row for all tokens (rwkv-ops "Stream Aggregate
 * FFI" with per_token = false): H_pre and dH_pre are fp32 [n].
 *   agg[t][c] = sum_i H_pre[i] X[t][i][c]
 *   dX[t][i][c] (+)= H_pre[i] g[t][c],  dH_pre[i] = sum_t sum_c g[t][c] X[t][i][c]
 * dH_pre is a fixed-order sum over tokens (per-token rows in the workspace,
 * then one reduction); with tokens == 0 it is set to zero.
 * ---------------------------------------------------------------------- */
mhc_status mhc_h_aggregate_static_fwd(void *stream, int64_t tokens, int32_t n, int64_t C, mhc_dtype act,
                                      const void *X, const float *H_pre, void *out);
size_t mhc_h_aggregate_static_bwd_workspace_size(int64_t tokens, int32_t n, int64_t C, mhc_dtype act);
mhc_status mhc_h_aggregate_static_bwd(void *stream, int64_t tokens, int32_t n, int64_t C, mhc_dtype act,
                                      const void *g, const void *X, const float *H_pre, void *dX,
                                      int32_t accumulate_dX, float *dH_pre, void *workspace,
                                      size_t workspace_bytes);

/* -------------------------------------------------------------------------
 * Fused pre pass (rwkv-ops "MHC Pre-Op FFI" fuses aggregate + sigmoid +
 * Sinkhorn; here the projection is fused in as well):
 *   forward  = proj_rms_h -> sinkhorn(H_res_logits) -> h_aggregate(X, H_pre)
 * Outputs: H_pre, H_post, H_res (Sinkhorn output), H_res_logits, saved (as
 * mhc_proj_rms_h) and agg [tokens][C] (act).
 * ---------------------------------------------------------------------- */
size_t mhc_pre_fwd_workspace_size(int64_t tokens, int32_t n, int64_t C, mhc_dtype act);
mhc_status mhc_pre_fwd(void *stream, int64_t tokens, int32_t n, int64_t C, mhc_dtype act,
                       const void *X, const float *W, const float *alpha, const float *hbias,
                       float rms_eps, int32_t iters, float eps, float *H_pre, float *H_post,
                       float *H_res, float *H_res_logits, float *saved, void *agg,
                       void *workspace, size_t workspace_bytes);

/* For callers that cannot allocate (code under HIP graph capture, tight
 * serving loops, harnesses that forbid hipMalloc): mhc_pre_fwd with the same
 * arguments and results, bit for bit, but no workspace.  Its scratch is a
 * static device array of MHC_NOALLOC_SCRATCH_BYTES (64 MiB) that every GPU
 * loading the library holds until the process ends; the call itself
 * allocates nothing.  A call whose scratch need, mhc_pre_fwd_workspace_size
 * for the same arguments, exceeds it returns MHC_ERR_UNSUPPORTED before
 * anything is enqueued (16384 tokens at C = 7168, n = 4, need about 22 MiB).
 * All calls on one GPU share that GPU's array: calls that can overlap on one
 * GPU (other streams, other host threads) race and must be ordered by the
 * caller.  Every scratch byte a call reads is written earlier in the same
 * call, so nothing is carried over from the previous call.  The first call
 * on a device looks up that device's array (hipGetSymbolAddress) and may
 * return MHC_ERR_HIP if the lookup fails. */
#define MHC_NOALLOC_SCRATCH_BYTES (64u << 20)
mhc_status mhc_pre_fwd_noalloc(void *stream, int64_t tokens, int32_t n, int64_t C, mhc_dtype act,
                               const void *X, const float *W, const float *alpha, const float *hbias,
                               float rms_eps, int32_t iters, float eps, float *H_pre, float *H_post,
                               float *H_res, float *H_res_logits, float *saved, void *agg);

/* Fused pre pass backward: h_aggregate backward (dH_pre and the H_pre * g
 * residual term) + Sinkhorn backward (dH_res -> logits) + projection
 * backward, with the residual gradient terms summed into dX (Megatron Core
 * `fused_add_3` sums the three residual-gradient contributions).
 *
 * g [tokens][C] (act) is the gradient of the aggregated stream; dH_post
 * [tokens][n] and dH_res [tokens][n][n] (fp32) come from the h_post_bda
 * backward.  The third residual term, the h_post_bda dX, is supplied one of
 * two ways:
 *   * post_G = NULL, post_H_res = NULL: pass the h_post_bda dX as dX with
 *     accumulate_dX != 0 (dX is read and overwritten with the sum);
 *   * post_G [tokens][n][C] (act, the h_post_bda upstream gradient G) and
 *     post_H_res [tokens][n][n] (fp32): the term sum_i H_res[j][i] G[i][c]
 *     is computed here, and mhc_h_post_bda_bwd can skip its dX (dX = NULL),
 *     which saves writing and re-reading one residual-sized tensor.
 *     Both must be given or both NULL.
 * dX (act): overwritten, or accumulated into when accumulate_dX != 0.
 * dW/dalpha/dhbias as mhc_proj_rms_h_bwd.  dH_pre_out [tokens][n] and
 * dlogits_out [tokens][n][n] (fp32) optionally receive the intermediate
 * gradients; pass NULL to skip them.
 * ---------------------------------------------------------------------- */
size_t mhc_pre_bwd_workspace_size(int64_t tokens, int32_t n, int64_t C, mhc_dtype act);
mhc_status mhc_pre_bwd(void *stream, int64_t tokens, int32_t n, int64_t C, mhc_dtype act,
                       const void *g, const float *dH_post, const float *dH_res, const void *X,
                       const float *W, const float *alpha, const float *saved, const float *H_pre,
                       const float *H_post, const float *H_res_logits, int32_t iters, float eps,
                       const void *post_G, const float *post_H_res, void *dX,
                       int32_t accumulate_dX, float *dW, float *dalpha, float *dhbias,
                       float *dH_pre_out, float *dlogits_out, void *workspace,
                       size_t workspace_bytes);

/* -------------------------------------------------------------------------
 * RMSNorm of the aggregated stream, the step right after h_aggregate
 * (rwkv-ops mhu_ffi.cu, RMSNorm forward/backward FFI: a [N][C] row norm with
 * one eps; RL-Kernel PR #383, P1-5 rmsnorm_residual, which adds a norm gain
 * whose gradient dgamma is summed over tokens (and ranks), and removes the
 * zero-row singularity with r = 1/(q + eps)).  Per token row x [C]:
 *   q = sqrt(sum_c x_c^2 / C),  r = 1/(q + eps),  y_c = gamma_c r x_c
 *   dx_k (+)= r gamma_k dy_k - S r^2 x_k / (C q),  S = sum_c gamma_c dy_c x_c
 *             (the second term is 0 for an all-zero row)
 *   dgamma_c = sum_t dy_{t,c} r_t x_{t,c}
 * x, y, dy, dx [tokens][C] (act); gamma, dgamma [C] fp32.  gamma == NULL
 * means a unit gain (the weightless norm); dgamma == NULL skips it (it may
 * be requested with gamma == NULL).  The residual fork: the aggregated
 * stream x is kept as a tensor of its own beside y; its own gradient is
 * added by passing it in dx with accumulate_dx != 0.  dgamma is a
 * fixed-order sum over tokens through the workspace
 * (mhc_rmsnorm_bwd_workspace_size; 0 bytes without dgamma); with
 * tokens == 0 it is set to zero.  n plays no part: C % 8 == 0 and
 * C <= 16384 as elsewhere.
 * ---------------------------------------------------------------------- */
mhc_status mhc_rmsnorm_fwd(void *stream, int64_t tokens, int64_t C, mhc_dtype act, const void *x,
                           const float *gamma, float eps, void *y);
size_t mhc_rmsnorm_bwd_workspace_size(int64_t tokens, int64_t C, mhc_dtype act, int32_t with_dgamma);
mhc_status mhc_rmsnorm_bwd(void *stream, int64_t tokens, int64_t C, mhc_dtype act, const void *dy,
                           const void *x, const float *gamma, float eps, void *dx,
                           int32_t accumulate_dx, float *dgamma, void *workspace,
                           size_t workspace_bytes);

/* Fused pre pass with the norm as its epilogue: mhc_pre_fwd, and in the
 * same pass over the residual that writes agg, normed = RMSNorm(agg) as
 * stored (the values after rounding to act), so the result equals
 * mhc_pre_fwd followed by mhc_rmsnorm_fwd on its agg.  gamma [C] fp32 or
 * NULL, norm_eps >= 0, normed [tokens][C] (act).  The backward is
 * mhc_pre_rmsnorm_bwd (or mhc_rmsnorm_bwd followed by mhc_pre_bwd).
 * ---------------------------------------------------------------------- */
mhc_status mhc_pre_rmsnorm_fwd(void *stream, int64_t tokens, int32_t n, int64_t C, mhc_dtype act,
                               const void *X, const float *W, const float *alpha, const float *hbias,
                               float rms_eps, int32_t iters, float eps, const float *gamma,
                               float norm_eps, float *H_pre, float *H_post, float *H_res,
                               float *H_res_logits, float *saved, void *agg, void *normed,
                               void *workspace, size_t workspace_bytes);

/* Fused pre pass backward with the norm's backward in front, the backward of
 * mhc_pre_rmsnorm_fwd (RL-Kernel PR #383, P1-5 rmsnorm_residual: the norm and
 * its residual fork in front of the pre pass).  Results equal, bit for bit,
 *   mhc_rmsnorm_bwd(dy, agg, gamma, norm_eps, dx = g_fork copy, accumulate_dx =
 *                   g_fork != NULL, dgamma)          -> d_agg (act, rounded)
 *   mhc_pre_bwd(g = d_agg, dH_post, dH_res, X, ...)  -> dX, dW, dalpha, dhbias
 * in one call (the two kernels run in sequence on the caller's stream; one
 * pass forming d_agg and dH_pre together measured slower on MI355X).
 * dy [tokens][C] (act): gradient of the normed output; agg [tokens][C] (act):
 * the norm's input as the forward stored it; gamma [C] fp32 or NULL (unit
 * gain); g_fork [tokens][C] (act) or NULL: agg's own upstream gradient (the
 * residual fork), added to the norm's input gradient.  dgamma [C] fp32 or
 * NULL; d_agg_out [tokens][C] (act) or NULL: receives d_agg.  The other
 * arguments as mhc_pre_bwd (without the intermediate outputs).  tokens == 0
 * zero-fills dW, dalpha, dhbias and dgamma. */
size_t mhc_pre_rmsnorm_bwd_workspace_size(int64_t tokens, int32_t n, int64_t C, mhc_dtype act,
                                          int32_t with_dgamma);
mhc_status mhc_pre_rmsnorm_bwd(void *stream, int64_t tokens, int32_t n, int64_t C, mhc_dtype act,
                               const void *dy, const void *agg, const float *gamma, float norm_eps,
                               const void *g_fork, const float *dH_post, const float *dH_res, const void *X,
                               const float *W, const float *alpha, const float *saved, const float *H_pre,
                               const float *H_post, const float *H_res_logits, int32_t iters, float eps,
                               const void *post_G, const float *post_H_res, void *dX, int32_t accumulate_dX,
                               float *dW, float *dalpha, float *dhbias, float *dgamma, void *d_agg_out,
                               void *workspace, size_t workspace_bytes);

#ifdef __cplusplus
}
#endif

#endif /* MHC_H_ */
