/* Runs every oracle function once on small seeded inputs, each buffer
 * allocated at exactly its documented size, so that an AddressSanitizer /
 * UndefinedBehaviorSanitizer build of the oracle reports any read or write
 * outside the buffers.  Built and run by tests/test_oracle_sanitize.py (host
 * code only, gcc). */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

void mhc_oracle_proj_rms_h(int64_t, int, int64_t, const double *, const double *, const double *,
                           const double *, double, double *, double *, double *, double *, double *, double *);
void mhc_oracle_sinkhorn_fwd(int64_t, int, const double *, int, double, double *);
void mhc_oracle_sinkhorn_bwd(int64_t, int, const double *, const double *, int, double, double *);
void mhc_oracle_h_aggregate_fwd(int64_t, int, int64_t, const double *, const double *, double *);
void mhc_oracle_h_aggregate_bwd(int64_t, int, int64_t, const double *, const double *, const double *, double *,
                                double *);
void mhc_oracle_h_post_bda_fwd(int64_t, int, int64_t, const double *, const double *, const double *,
                               const double *, const double *, double *);
void mhc_oracle_h_post_bda_bwd(int64_t, int, int64_t, const double *, const double *, const double *,
                               const double *, const double *, const double *, double *, double *, double *,
                               double *, double *);
void mhc_oracle_stream_mix_fwd(int64_t, int, int64_t, const double *, const double *, double *);
void mhc_oracle_stream_mix_bwd(int64_t, int, int64_t, const double *, const double *, const double *, double *,
                               double *);
void mhc_oracle_stream_distribute_fwd(int64_t, int, int64_t, const double *, const double *, double *);
void mhc_oracle_stream_distribute_bwd(int64_t, int, int64_t, const double *, const double *, const double *,
                                      double *, double *);
void mhc_oracle_h_aggregate_static_fwd(int64_t, int, int64_t, const double *, const double *, double *);
void mhc_oracle_h_aggregate_static_bwd(int64_t, int, int64_t, const double *, const double *, const double *,
                                       double *, double *);
void mhc_oracle_proj_rms_h_bwd(int64_t, int, int64_t, const double *, const double *, const double *,
                               const double *, double, const double *, const double *, const double *, double *,
                               double *, double *, double *);
void mhc_oracle_rmsnorm_fwd(int64_t, int64_t, const double *, const double *, double, double *, double *);
void mhc_oracle_rmsnorm_bwd(int64_t, int64_t, const double *, const double *, const double *, double, double *,
                            double *);

static uint64_t state = 0x9E3779B97F4A7C15ull;
static double rnd(void) { /* xorshift64*, uniform in [-1, 1) */
  state ^= state >> 12; state ^= state << 25; state ^= state >> 27;
  return (double)((state * 2685821657736338717ull) >> 11) / 9007199254740992.0 * 2.0 - 1.0;
}
static double *buf(size_t n) {
  double *p = (double *)malloc(n * sizeof(double));
  for (size_t i = 0; i < n; ++i) p[i] = rnd();
  return p;
}

int main(void) {
  const int ns[] = {1, 3, 4, 8};
  for (int a = 0; a < 4; ++a) {
    const int n = ns[a];
    const int64_t N = 3, C = 12, K = n * C, J = n * n + 2 * n;
    double *X = buf(N * K), *W = buf(K * J), *al = buf(3), *hb = buf(J), *G = buf(N * K), *x = buf(N * C);
    double *g = buf(N * C), *bias = buf(C), *Hp = buf(N * n), *Hq = buf(N * n), *Hr = buf(N * n * n);
    double *dHp = buf(N * n), *dHq = buf(N * n), *dL = buf(N * n * n), *h = buf(n);
    double *o1 = buf(N * n), *o2 = buf(N * n), *o3 = buf(N * n * n), *r = buf(N), *q = buf(N), *z = buf(N * J);
    double *oK = buf(N * K), *oK2 = buf(N * K), *oC = buf(N * C), *oNN = buf(N * n * n), *oN = buf(N * n);
    double *oC1 = buf(C), *dW = buf(K * J), *da = buf(3), *db = buf(J), *on = buf(n);
    mhc_oracle_proj_rms_h(N, n, C, X, W, al, hb, 1e-6, o1, o2, o3, r, q, z);
    mhc_oracle_sinkhorn_fwd(N, n, o3, 20, 1e-6, oNN);
    mhc_oracle_sinkhorn_bwd(N, n, dL, o3, 20, 1e-6, oNN);
    mhc_oracle_h_aggregate_fwd(N, n, C, X, Hp, oC);
    mhc_oracle_h_aggregate_bwd(N, n, C, g, X, Hp, oK, oN);
    mhc_oracle_h_post_bda_fwd(N, n, C, X, Hr, Hq, x, bias, oK);
    mhc_oracle_h_post_bda_bwd(N, n, C, G, X, Hr, Hq, x, bias, oK, oNN, oN, oC, oC1);
    mhc_oracle_h_post_bda_bwd(N, n, C, G, X, Hr, Hq, x, NULL, oK, oNN, oN, oC, NULL);
    mhc_oracle_stream_mix_fwd(N, n, C, X, Hr, oK);
    mhc_oracle_stream_mix_bwd(N, n, C, G, X, Hr, oK, oNN);
    mhc_oracle_stream_distribute_fwd(N, n, C, x, Hq, oK);
    mhc_oracle_stream_distribute_bwd(N, n, C, G, x, Hq, oC, oN);
    mhc_oracle_h_aggregate_static_fwd(N, n, C, X, h, oC);
    mhc_oracle_h_aggregate_static_bwd(N, n, C, g, X, h, oK, on);
    mhc_oracle_proj_rms_h_bwd(N, n, C, X, W, al, hb, 1e-6, dHp, dHq, dL, oK2, dW, da, db);
    mhc_oracle_rmsnorm_fwd(N, C, x, bias, 1e-6, oC, r);
    mhc_oracle_rmsnorm_fwd(N, C, x, NULL, 1e-6, oC, NULL);
    mhc_oracle_rmsnorm_bwd(N, C, g, x, bias, 1e-6, oC, oC1);
    mhc_oracle_rmsnorm_bwd(N, C, g, x, NULL, 1e-6, oC, NULL);
    double *all[] = {X, W, al, hb, G, x, g, bias, Hp, Hq, Hr, dHp, dHq, dL, h, o1, o2, o3, r, q, z,
                     oK, oK2, oC, oNN, oN, oC1, dW, da, db, on};
    for (size_t i = 0; i < sizeof(all) / sizeof(all[0]); ++i) free(all[i]);
  }
  puts("oracle sanitizer run: ok");
  return 0;
}
