/*
 * mhc_oracle.c -- plain, slow fp64 CPU reference of the per-token mHC
 * (Manifold-Constrained Hyper-Connections) residual-mixing path.
 *
 * TEST INFRASTRUCTURE ONLY.  This file is the parity oracle for the HIP
 * library: only the test suite, the package's smoke check and the benchmark's
 * CPU-baseline leg may load it.  It shares no code, header, table or constant
 * with the GPU path and it never calls into it.
 *
 * Every function loops over tokens and does the arithmetic exactly as the
 * operation is defined, in double precision, in the obvious order.  No
 * blocking, fusion or reordering.  Inputs arrive as double arrays (the caller
 * converts bf16/fp32 storage exactly); outputs are double and the caller
 * rounds them once to their storage type.
 *
 * Notation (per token): n residual streams of C channels, K = n*C, the
 * flattened stream index k = i*C + c, J = n*n + 2n controller outputs laid out
 * PRE [0,n) | POST [n,2n) | RES [2n, 2n+n*n) (RES row-major a*n+b).
 *
 * Sources (pages on the method):
 *  [MCORE] Megatron Core developer guide, "core.fusions.fused_mhc_kernels":
 *          module summary listing the four fused operations (sinkhorn,
 *          h_aggregate, h_post_bda, proj_rms_compute_h) and the API entries
 *          `_torch_proj_rms_compute_h`, `_torch_h_aggregate_bwd`,
 *          `_torch_h_post_bda_bwd`.
 *  [RWKV]  rwkv-ops 0.6.1 wheel, rwkv_ops/mhc_kernel/jax_kernel/mhu_ffi.cu:
 *          sections "Sinkhorn Knopp FFI", "Stream Aggregate FFI",
 *          "MHC Post-Op FFI", "MHC Pre-Op FFI".
 *  [RLK]   RL-Kernel pull request #383, "[DSv4][P1-S0] Start kit for the P1
 *          work package (mHC + RMSNorm)": review comment on the RMS backward
 *          (zero-row guard, r = 1/(q+eps)), and the commit message on the
 *          three segment gains alpha_pre/alpha_post/alpha_res.
 */
#include <math.h>
#include <stddef.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

static int seg_of(int j, int n) { return j < n ? 0 : (j < 2 * n ? 1 : 2); }

static double sigmoid(double v) { return 1.0 / (1.0 + exp(-v)); }

/* ------------------------------------------------------------------------
 * F1  proj_rms_compute_h forward  [MCORE proj_rms_compute_h; RLK RMS note]
 *
 *   s = sum_k x_k^2,  q = sqrt(s / K),  r = 1 / (q + eps_rms)
 *   p_j = sum_k x_k W[k][j],  z_j = r * p_j
 *   zh_j = alpha[seg(j)] * z_j + hbias[j]
 *   H_pre[i] = sigmoid(zh_i), H_post[i] = 2 sigmoid(zh_{n+i}),
 *   L[a][b] = zh_{2n + a n + b}   (logits handed to Sinkhorn)
 *
 * r_out/q_out/z_out receive r, q and z (pre-gain) per token.
 * ---------------------------------------------------------------------- */
void mhc_oracle_proj_rms_h(int64_t N, int n, int64_t C, const double *X,
                           const double *W, const double *alpha,
                           const double *hbias, double eps_rms, double *H_pre,
                           double *H_post, double *L, double *r_out,
                           double *q_out, double *z_out) {
  const int64_t K = (int64_t)n * C;
  const int J = n * n + 2 * n;
  for (int64_t t = 0; t < N; ++t) {
    const double *x = X + t * K;
    double s = 0.0;
    for (int64_t k = 0; k < K; ++k) s += x[k] * x[k];
    const double q = sqrt(s / (double)K);
    const double r = 1.0 / (q + eps_rms);
    for (int j = 0; j < J; ++j) {
      double p = 0.0;
      for (int64_t k = 0; k < K; ++k) p += x[k] * W[k * J + j];
      const double z = r * p;
      const int sg = seg_of(j, n);
      const double zh = alpha[sg] * z + hbias[j];
      if (sg == 0)
        H_pre[t * n + j] = sigmoid(zh);
      else if (sg == 1)
        H_post[t * n + (j - n)] = 2.0 * sigmoid(zh);
      else
        L[t * n * n + (j - 2 * n)] = zh;
      if (z_out) z_out[t * J + j] = z;
    }
    if (r_out) r_out[t] = r;
    if (q_out) q_out[t] = q;
  }
}

/* ------------------------------------------------------------------------
 * F2  Sinkhorn-Knopp forward  [MCORE sinkhorn; RWKV Sinkhorn Knopp FFI]
 *
 *   M = exp(L); repeat iters times:
 *     every row    a: M[a][:] /= (sum_b M[a][b] + eps)
 *     every column b: M[:][b] /= (sum_a M[a][b] + eps)
 * ---------------------------------------------------------------------- */
void mhc_oracle_sinkhorn_fwd(int64_t count, int n, const double *L, int iters,
                             double eps, double *H) {
  const int nn = n * n;
  double *M = (double *)malloc(sizeof(double) * nn);
  for (int64_t m = 0; m < count; ++m) {
    for (int e = 0; e < nn; ++e) M[e] = exp(L[m * nn + e]);
    for (int it = 0; it < iters; ++it) {
      for (int a = 0; a < n; ++a) {
        double s = 0.0;
        for (int b = 0; b < n; ++b) s += M[a * n + b];
        const double d = s + eps;
        for (int b = 0; b < n; ++b) M[a * n + b] /= d;
      }
      for (int b = 0; b < n; ++b) {
        double s = 0.0;
        for (int a = 0; a < n; ++a) s += M[a * n + b];
        const double d = s + eps;
        for (int a = 0; a < n; ++a) M[a * n + b] /= d;
      }
    }
    memcpy(H + m * nn, M, sizeof(double) * nn);
  }
  free(M);
}

/* ------------------------------------------------------------------------
 * B2  Sinkhorn-Knopp backward: exact reverse mode of the unrolled F2 map
 * (2*iters half-steps, eps included).  [RWKV Sinkhorn Knopp FFI: the
 * backward takes the forward input, the iteration count and eps.]
 *
 * A half-step maps M -> M' = M / d with d = sum(M along the line) + eps, so
 * for an upstream gradient G on M':  dM = (G - <G, M'>_line) / d  on each
 * row (row half-step) or column (column half-step).  Finally
 * dL = dM0 * exp(L).  Every intermediate M and d is stored.
 * ---------------------------------------------------------------------- */
void mhc_oracle_sinkhorn_bwd(int64_t count, int n, const double *dH,
                             const double *L, int iters, double eps,
                             double *dL) {
  const int nn = n * n;
  const int steps = 2 * iters;
  double *Ms = (double *)malloc(sizeof(double) * nn * (steps + 1));
  double *ds = (double *)malloc(sizeof(double) * n * (steps + 1));
  double *G = (double *)malloc(sizeof(double) * nn);
  for (int64_t m = 0; m < count; ++m) {
    /* forward replay, keeping every state */
    for (int e = 0; e < nn; ++e) Ms[e] = exp(L[m * nn + e]);
    for (int h = 1; h <= steps; ++h) {
      const double *P = Ms + (h - 1) * nn;
      double *Q = Ms + h * nn;
      double *d = ds + h * n;
      const int row_step = (h % 2) == 1;
      for (int u = 0; u < n; ++u) {
        double s = 0.0;
        for (int v = 0; v < n; ++v)
          s += row_step ? P[u * n + v] : P[v * n + u];
        d[u] = s + eps;
      }
      for (int a = 0; a < n; ++a)
        for (int b = 0; b < n; ++b)
          Q[a * n + b] = P[a * n + b] / (row_step ? d[a] : d[b]);
    }
    /* reverse sweep */
    for (int e = 0; e < nn; ++e) G[e] = dH[m * nn + e];
    for (int h = steps; h >= 1; --h) {
      const double *Q = Ms + h * nn;
      const double *d = ds + h * n;
      const int row_step = (h % 2) == 1;
      for (int u = 0; u < n; ++u) {
        double dot = 0.0;
        for (int v = 0; v < n; ++v) {
          const int e = row_step ? u * n + v : v * n + u;
          dot += G[e] * Q[e];
        }
        for (int v = 0; v < n; ++v) {
          const int e = row_step ? u * n + v : v * n + u;
          G[e] = (G[e] - dot) / d[u];
        }
      }
    }
    for (int e = 0; e < nn; ++e) dL[m * nn + e] = G[e] * Ms[e];
  }
  free(Ms);
  free(ds);
  free(G);
}

/* ------------------------------------------------------------------------
 * F3  h_aggregate forward  [MCORE h_aggregate: weighted n-stream -> 1-stream]
 *   agg[c] = sum_i H_pre[i] * X[i][c]
 * ---------------------------------------------------------------------- */
void mhc_oracle_h_aggregate_fwd(int64_t N, int n, int64_t C, const double *X,
                                const double *H_pre, double *agg) {
  for (int64_t t = 0; t < N; ++t)
    for (int64_t c = 0; c < C; ++c) {
      double acc = 0.0;
      for (int i = 0; i < n; ++i)
        acc += H_pre[t * n + i] * X[(t * n + i) * C + c];
      agg[t * C + c] = acc;
    }
}

/* ------------------------------------------------------------------------
 * B3  h_aggregate backward  [MCORE _torch_h_aggregate_bwd(grad_output, x,
 * h_pre) -> (d_x, d_h_pre); RWKV Stream Aggregate FFI backward]
 *   dX[i][c] = H_pre[i] * g[c],   dH_pre[i] = sum_c g[c] * X[i][c]
 * ---------------------------------------------------------------------- */
void mhc_oracle_h_aggregate_bwd(int64_t N, int n, int64_t C, const double *g,
                                const double *X, const double *H_pre,
                                double *dX, double *dH_pre) {
  for (int64_t t = 0; t < N; ++t)
    for (int i = 0; i < n; ++i) {
      double acc = 0.0;
      for (int64_t c = 0; c < C; ++c) {
        dX[(t * n + i) * C + c] = H_pre[t * n + i] * g[t * C + c];
        acc += g[t * C + c] * X[(t * n + i) * C + c];
      }
      dH_pre[t * n + i] = acc;
    }
}

/* ------------------------------------------------------------------------
 * F4  h_post_bda forward  [MCORE h_post_bda: H_res.T @ residual +
 * H_post * (x + bias); RWKV MHC Post-Op FFI]
 *   out[i][c] = sum_j H_res[j][i] X[j][c] + H_post[i] (x[c] + bias[c])
 * bias may be NULL (treated as zero).
 * ---------------------------------------------------------------------- */
void mhc_oracle_h_post_bda_fwd(int64_t N, int n, int64_t C, const double *X,
                               const double *H_res, const double *H_post,
                               const double *x, const double *bias,
                               double *out) {
  for (int64_t t = 0; t < N; ++t)
    for (int i = 0; i < n; ++i)
      for (int64_t c = 0; c < C; ++c) {
        double acc = 0.0;
        for (int j = 0; j < n; ++j)
          acc += H_res[t * n * n + j * n + i] * X[(t * n + j) * C + c];
        const double xb = x[t * C + c] + (bias ? bias[c] : 0.0);
        out[(t * n + i) * C + c] = acc + H_post[t * n + i] * xb;
      }
}

/* ------------------------------------------------------------------------
 * B4  h_post_bda backward  [MCORE _torch_h_post_bda_bwd(grad_output, h_res,
 * original_residual, h_post, x, bias) -> five tensors, the last optional]
 *   dX[j][c]     = sum_i H_res[j][i] G[i][c]
 *   dH_res[j][i] = sum_c X[j][c] G[i][c]
 *   dH_post[i]   = sum_c G[i][c] (x[c] + bias[c])
 *   dx[c]        = sum_i H_post[i] G[i][c]
 *   dbias[c]     = sum_t dx_t[c]           (only when dbias != NULL)
 * ---------------------------------------------------------------------- */
void mhc_oracle_h_post_bda_bwd(int64_t N, int n, int64_t C, const double *G,
                               const double *X, const double *H_res,
                               const double *H_post, const double *x,
                               const double *bias, double *dX, double *dH_res,
                               double *dH_post, double *dx, double *dbias) {
  if (dbias)
    for (int64_t c = 0; c < C; ++c) dbias[c] = 0.0;
  for (int64_t t = 0; t < N; ++t) {
    for (int j = 0; j < n; ++j)
      for (int64_t c = 0; c < C; ++c) {
        double acc = 0.0;
        for (int i = 0; i < n; ++i)
          acc += H_res[t * n * n + j * n + i] * G[(t * n + i) * C + c];
        dX[(t * n + j) * C + c] = acc;
      }
    for (int j = 0; j < n; ++j)
      for (int i = 0; i < n; ++i) {
        double acc = 0.0;
        for (int64_t c = 0; c < C; ++c)
          acc += X[(t * n + j) * C + c] * G[(t * n + i) * C + c];
        dH_res[t * n * n + j * n + i] = acc;
      }
    for (int i = 0; i < n; ++i) {
      double acc = 0.0;
      for (int64_t c = 0; c < C; ++c)
        acc += G[(t * n + i) * C + c] *
               (x[t * C + c] + (bias ? bias[c] : 0.0));
      dH_post[t * n + i] = acc;
    }
    for (int64_t c = 0; c < C; ++c) {
      double acc = 0.0;
      for (int i = 0; i < n; ++i)
        acc += H_post[t * n + i] * G[(t * n + i) * C + c];
      dx[t * C + c] = acc;
      if (dbias) dbias[c] += acc;
    }
  }
}

/* ------------------------------------------------------------------------
 * F5  stream mix  [RWKV Stream Mix FFI: inp [B,T,n,C], M [B,T,n,n] -> out
 * [B,T,n,C]; the mixing orientation read as the post-op's H_res mix]
 *   out[i][c] = sum_j M[j][i] X[j][c]
 * B5  its backward (d_inp, d_M)
 *   dX[j][c] = sum_i M[j][i] G[i][c],   dM[j][i] = sum_c X[j][c] G[i][c]
 * ---------------------------------------------------------------------- */
void mhc_oracle_stream_mix_fwd(int64_t N, int n, int64_t C, const double *X,
                               const double *M, double *out) {
  for (int64_t t = 0; t < N; ++t)
    for (int i = 0; i < n; ++i)
      for (int64_t c = 0; c < C; ++c) {
        double acc = 0.0;
        for (int j = 0; j < n; ++j)
          acc += M[t * n * n + j * n + i] * X[(t * n + j) * C + c];
        out[(t * n + i) * C + c] = acc;
      }
}

void mhc_oracle_stream_mix_bwd(int64_t N, int n, int64_t C, const double *G,
                               const double *X, const double *M, double *dX,
                               double *dM) {
  for (int64_t t = 0; t < N; ++t) {
    for (int j = 0; j < n; ++j)
      for (int64_t c = 0; c < C; ++c) {
        double acc = 0.0;
        for (int i = 0; i < n; ++i)
          acc += M[t * n * n + j * n + i] * G[(t * n + i) * C + c];
        dX[(t * n + j) * C + c] = acc;
      }
    for (int j = 0; j < n; ++j)
      for (int i = 0; i < n; ++i) {
        double acc = 0.0;
        for (int64_t c = 0; c < C; ++c)
          acc += X[(t * n + j) * C + c] * G[(t * n + i) * C + c];
        dM[t * n * n + j * n + i] = acc;
      }
  }
}

/* ------------------------------------------------------------------------
 * F6  stream distribute  [RWKV Stream Distribute FFI: inp [B,T,C], H_post
 * [B,T,n] -> out [B,T,n,C]]
 *   out[i][c] = H_post[i] x[c]
 * B6  its backward (d_inp, d_H_post: the dx and dh kernels of that section)
 *   dx[c] = sum_i H_post[i] G[i][c],   dH_post[i] = sum_c G[i][c] x[c]
 * ---------------------------------------------------------------------- */
void mhc_oracle_stream_distribute_fwd(int64_t N, int n, int64_t C, const double *x,
                                      const double *H_post, double *out) {
  for (int64_t t = 0; t < N; ++t)
    for (int i = 0; i < n; ++i)
      for (int64_t c = 0; c < C; ++c)
        out[(t * n + i) * C + c] = H_post[t * n + i] * x[t * C + c];
}

void mhc_oracle_stream_distribute_bwd(int64_t N, int n, int64_t C, const double *G,
                                      const double *x, const double *H_post,
                                      double *dx, double *dH_post) {
  for (int64_t t = 0; t < N; ++t) {
    for (int64_t c = 0; c < C; ++c) {
      double acc = 0.0;
      for (int i = 0; i < n; ++i)
        acc += H_post[t * n + i] * G[(t * n + i) * C + c];
      dx[t * C + c] = acc;
    }
    for (int i = 0; i < n; ++i) {
      double acc = 0.0;
      for (int64_t c = 0; c < C; ++c)
        acc += G[(t * n + i) * C + c] * x[t * C + c];
      dH_post[t * n + i] = acc;
    }
  }
}

/* ------------------------------------------------------------------------
 * F3s / B3s  h_aggregate with one H_pre row for all tokens  [RWKV Stream
 * Aggregate FFI with per_token = false: H_pre [n], d_H_pre [n]]
 *   agg[t][c] = sum_i H_pre[i] X[t][i][c]
 *   dX[t][i][c] = H_pre[i] g[t][c],   dH_pre[i] = sum_t sum_c g[t][c] X[t][i][c]
 * ---------------------------------------------------------------------- */
void mhc_oracle_h_aggregate_static_fwd(int64_t N, int n, int64_t C, const double *X,
                                       const double *H_pre, double *agg) {
  for (int64_t t = 0; t < N; ++t)
    for (int64_t c = 0; c < C; ++c) {
      double acc = 0.0;
      for (int i = 0; i < n; ++i) acc += H_pre[i] * X[(t * n + i) * C + c];
      agg[t * C + c] = acc;
    }
}

void mhc_oracle_h_aggregate_static_bwd(int64_t N, int n, int64_t C, const double *g,
                                       const double *X, const double *H_pre,
                                       double *dX, double *dH_pre) {
  for (int i = 0; i < n; ++i) dH_pre[i] = 0.0;
  for (int64_t t = 0; t < N; ++t)
    for (int i = 0; i < n; ++i)
      for (int64_t c = 0; c < C; ++c) {
        dX[(t * n + i) * C + c] = H_pre[i] * g[t * C + c];
        dH_pre[i] += g[t * C + c] * X[(t * n + i) * C + c];
      }
}

/* ------------------------------------------------------------------------
 * B1  proj_rms_compute_h backward  [RLK review comment on the RMS backward:
 * dx = dx_gemm + dx_rms, with the q == 0 guard; RLK commit message: three
 * segment gains, so d_alpha is three scalars]
 *
 * Recomputes F1 in fp64 from X, then per token
 *   dzh_pre  = dH_pre  * s (1 - s),          s = sigmoid(zh_pre)
 *   dzh_post = dH_post * 2 s (1 - s),        s = sigmoid(zh_post)
 *   dzh_res  = dL
 *   dhbias_j += dzh_j,   dalpha_seg += dzh_j z_j,   dz_j = alpha_seg dzh_j
 *   dr = sum_j dz_j p_j,  dp_j = r dz_j
 *   dX_gemm[k] = sum_j dp_j W[k][j],   dW[k][j] += x_k dp_j
 *   dX_rms[k]  = -dr r^2 x_k / (K q)   (0 when q == 0)
 *   dX = dX_gemm + dX_rms   (this operation's own contribution)
 * dW, dalpha, dhbias are sums over all N tokens and are overwritten.
 * ---------------------------------------------------------------------- */
void mhc_oracle_proj_rms_h_bwd(int64_t N, int n, int64_t C, const double *X,
                               const double *W, const double *alpha,
                               const double *hbias, double eps_rms,
                               const double *dH_pre, const double *dH_post,
                               const double *dL, double *dX, double *dW,
                               double *dalpha, double *dhbias) {
  const int64_t K = (int64_t)n * C;
  const int J = n * n + 2 * n;
  double *p = (double *)malloc(sizeof(double) * J);
  double *dp = (double *)malloc(sizeof(double) * J);
  for (int64_t e = 0; e < K * J; ++e) dW[e] = 0.0;
  for (int s = 0; s < 3; ++s) dalpha[s] = 0.0;
  for (int j = 0; j < J; ++j) dhbias[j] = 0.0;
  for (int64_t t = 0; t < N; ++t) {
    const double *x = X + t * K;
    double s = 0.0;
    for (int64_t k = 0; k < K; ++k) s += x[k] * x[k];
    const double q = sqrt(s / (double)K);
    const double r = 1.0 / (q + eps_rms);
    double dr = 0.0;
    for (int j = 0; j < J; ++j) {
      double acc = 0.0;
      for (int64_t k = 0; k < K; ++k) acc += x[k] * W[k * J + j];
      p[j] = acc;
      const double z = r * acc;
      const int sg = seg_of(j, n);
      const double zh = alpha[sg] * z + hbias[j];
      double dzh;
      if (sg == 0) {
        const double sv = sigmoid(zh);
        dzh = dH_pre[t * n + j] * sv * (1.0 - sv);
      } else if (sg == 1) {
        const double sv = sigmoid(zh);
        dzh = dH_post[t * n + (j - n)] * 2.0 * sv * (1.0 - sv);
      } else {
        dzh = dL[t * n * n + (j - 2 * n)];
      }
      dhbias[j] += dzh;
      dalpha[sg] += dzh * z;
      const double dz = alpha[sg] * dzh;
      dr += dz * p[j];
      dp[j] = r * dz;
    }
    const double rms_coef = (q > 0.0) ? (-dr * r * r / ((double)K * q)) : 0.0;
    for (int64_t k = 0; k < K; ++k) {
      double acc = 0.0;
      for (int j = 0; j < J; ++j) {
        acc += dp[j] * W[k * J + j];
        dW[k * J + j] += x[k] * dp[j];
      }
      dX[t * K + k] = acc + rms_coef * x[k];
    }
  }
  free(p);
  free(dp);
}

/* ------------------------------------------------------------------------
 * F7  RMSNorm of one activation row  [RWKV: the RMSNorm forward/backward FFI
 * handlers (inp [N,C] -> out [N,C], attribute eps; no weight); RLK: P1-5
 * rmsnorm_residual with a norm gain whose gradient dgamma is summed across
 * ranks; RLK review comment: r = 1/(q+eps) removes the zero-row singularity]
 *
 *   q = sqrt(sum_c x_c^2 / C),  r = 1/(q + eps),  y_c = gamma_c r x_c
 *   gamma == NULL means gamma_c = 1 (the weightless form).
 * B7  its backward
 *   S = sum_c gamma_c dy_c x_c
 *   dx_k = r gamma_k dy_k - S r^2 x_k / (C q)        (second term 0 when q == 0)
 *   dgamma_c = sum_t dy_{t,c} r_t x_{t,c}            (when dgamma != NULL)
 * r_out (may be NULL) receives r per row.
 * ---------------------------------------------------------------------- */
void mhc_oracle_rmsnorm_fwd(int64_t N, int64_t C, const double *x,
                            const double *gamma, double eps, double *y,
                            double *r_out) {
  for (int64_t t = 0; t < N; ++t) {
    const double *xt = x + t * C;
    double s = 0.0;
    for (int64_t c = 0; c < C; ++c) s += xt[c] * xt[c];
    const double q = sqrt(s / (double)C);
    const double r = 1.0 / (q + eps);
    for (int64_t c = 0; c < C; ++c)
      y[t * C + c] = (gamma ? gamma[c] : 1.0) * r * xt[c];
    if (r_out) r_out[t] = r;
  }
}

void mhc_oracle_rmsnorm_bwd(int64_t N, int64_t C, const double *dy,
                            const double *x, const double *gamma, double eps,
                            double *dx, double *dgamma) {
  if (dgamma)
    for (int64_t c = 0; c < C; ++c) dgamma[c] = 0.0;
  for (int64_t t = 0; t < N; ++t) {
    const double *xt = x + t * C;
    const double *gt = dy + t * C;
    double s = 0.0;
    for (int64_t c = 0; c < C; ++c) s += xt[c] * xt[c];
    const double q = sqrt(s / (double)C);
    const double r = 1.0 / (q + eps);
    double S = 0.0;
    for (int64_t c = 0; c < C; ++c) S += (gamma ? gamma[c] : 1.0) * gt[c] * xt[c];
    const double coef = (q > 0.0) ? (-S * r * r / ((double)C * q)) : 0.0;
    for (int64_t c = 0; c < C; ++c) {
      dx[t * C + c] = r * (gamma ? gamma[c] : 1.0) * gt[c] + coef * xt[c];
      if (dgamma) dgamma[c] += gt[c] * r * xt[c];
    }
  }
}
