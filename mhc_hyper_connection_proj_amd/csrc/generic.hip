// generic.hip -- the whole mHC path for a stream count n other than 4
// (1 <= n <= 8), on straightforward kernels templated on n.
//
// The kernels for n = 4 (proj.hip, streams.hip, sinkhorn.hip) are laid out
// for that n: the 4x4 mix and the 24 projection columns live in registers
// and the MFMA tiles hold exactly one column tile.  The pages' kernels take
// n at run time (rwkv-ops reads it from the tensor shape), so the same
// operations are provided here for any n up to 8, with the same
// definitions, layouts, determinism (fixed-order reductions, no atomics)
// and boundary checks, but simpler, less tuned kernels:
//  * projection forward: split-K over 8 slices.  bf16: W split once per call
//    into three exact bf16 terms and packed in 64-k chunks; 8 waves x 32
//    tokens per workgroup copy each chunk and their X tiles into an LDS ring
//    (global_load_lds) and multiply on the bf16 MFMA (32x32x16).  fp32: the
//    fp32 MFMA (32x32x2) with each 64-k W chunk staged once per workgroup.
//    A per-token finalize sums the slices in order and applies RMS, gains,
//    sigmoid and Sinkhorn;
//  * projection backward: a per-token kernel (sigmoid / Sinkhorn backward,
//    dp = r alpha dzh and the RMS coefficient), then dX and dW, with the
//    aggregate and h_post_bda terms formed in the dX epilogue.  bf16, n <= 3:
//    one MFMA kernel on tiles of 64-128 channels of all n streams (so the
//    h_post_bda gradient G, which every output stream mixes, is loaded
//    once), dp W^T on fp32 MFMA with W's rows in registers and x^T dp on
//    bf16 MFMA with dp split exactly into three bf16 terms.  bf16, n >= 5:
//    the same two contractions as two kernels (dX on 64-channel tiles of all
//    n streams, dW on 256-k tiles), dp split and transposed once for dW.
//    fp32: a per-token pass forming the epilogue terms in an fp32 workspace,
//    then a VALU kernel with one thread per k that owns W's row k and its dW
//    row, walking a token block;
//  * Sinkhorn: n >= 3 on groups of 4 or 8 lanes, one rotated line per lane
//    (row and column passes in-lane, layouts swapped by lane moves); the
//    backward records every half-step's line sums and a checkpoint every 8
//    half-steps.  n <= 2 (and records too large for LDS): one matrix per
//    thread, with stored sums where they fit, else a replay of the forward
//    from checkpoints spaced ~sqrt(2 iters) half-steps apart;
//  * streaming ops: one workgroup (or wave) per token, 8-channel groups per
//    thread, once-read rows loaded non-temporally, per-token sums lane ->
//    wave -> workgroup in fixed order.
#include <algorithm>

#include "device.h"
#include "internal.h"
#include "ring.h"

namespace mhc {

namespace {

typedef __attribute__((ext_vector_type(16))) float gf32x16;

// h_post_bda parts, as in the n = 4 kernels: the whole op, its H_res mix
// alone (stream mix), its H_post distribution alone (stream distribute).
enum : int { kPostFull = 0, kPostMix = 1, kPostDist = 2 };

template <int NS> struct Dim {
  static constexpr int J = NS * NS + 2 * NS;   // controller outputs
  static constexpr int JT = (J + 31) / 32;     // 32-column MFMA tiles
  static constexpr int PS = J + 1;             // partial row: x @ W, then sum x^2
  // Backward record of a token: dp[0..J), zeros up to RC, c_rms at RC, row
  // stride RS (a multiple of 4 floats).  The fp32 MFMA of the dX kernels
  // takes dp in equal parts, one per lane group, read as whole 16-byte
  // words: two halves of JC values (32x32x2, n <= 3: lane half h holds
  // j = h JC + c) or four quarters of JQ values (16x16x4, n >= 5: lane group
  // g holds j = g JQ + c).
  static constexpr int JC = ((J + 1) / 2 + 3) / 4 * 4;
  static constexpr int JQ = ((J + 3) / 4 + 3) / 4 * 4;
  static constexpr int RC = NS >= 5 ? 4 * JQ : 2 * JC;
  static constexpr int RS = (RC + 1 + 3) / 4 * 4;
};

constexpr int kGSplitK = 8;   // k slices of the forward projection
constexpr int kGTok = 32;     // tokens per wave in the forward projection (one MFMA tile)
constexpr int kGBwdK = 256;   // k per backward workgroup (one per thread)
constexpr int kGMaxTB = 32;   // at most this many token blocks in the backward
constexpr int64_t kGDwBudget = 512ll << 20;  // bytes of dW partials the token blocks may take

// ------------------------------------------------------------------ helpers
template <typename T> struct Ld;
template <> struct Ld<float> {
  static __device__ __forceinline__ float one(const float *p) { return *p; }
};
template <> struct Ld<bf16_t> {
  static __device__ __forceinline__ float one(const bf16_t *p) { return __uint_as_float((uint32_t)*p << 16); }
};

template <typename T> __device__ __forceinline__ void st_one(T *p, float v);
template <> __device__ __forceinline__ void st_one<float>(float *p, float v) { *p = v; }
template <> __device__ __forceinline__ void st_one<bf16_t>(bf16_t *p, float v) {
  const __bf16 h = (__bf16)v;
  *p = __builtin_bit_cast(uint16_t, h);
}

__device__ __forceinline__ float sigm(float v) { return 1.0f / (1.0f + __expf(-v)); }

typedef __attribute__((ext_vector_type(4))) unsigned int gu32x4;

// Sum of NV per-thread values over a workgroup of at most 512 threads; the
// totals go to every thread.  Fixed order: wave DPP tree, then waves in order.
template <int NV>
__device__ __forceinline__ void gblock_sum(float v[NV], float (*red)[NV]) {
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

// ------------------------------------------------------------------ Sinkhorn, one matrix per thread
template <int NS>
__device__ __forceinline__ void sk_half(float m[NS * NS], int h, float eps) {
  if ((h & 1) == 0) {
#pragma unroll
    for (int a = 0; a < NS; ++a) {
      float s = 0.f;
#pragma unroll
      for (int b = 0; b < NS; ++b) s += m[a * NS + b];
      const float d = 1.0f / (s + eps);
#pragma unroll
      for (int b = 0; b < NS; ++b) m[a * NS + b] *= d;
    }
  } else {
#pragma unroll
    for (int b = 0; b < NS; ++b) {
      float s = 0.f;
#pragma unroll
      for (int a = 0; a < NS; ++a) s += m[a * NS + b];
      const float d = 1.0f / (s + eps);
#pragma unroll
      for (int a = 0; a < NS; ++a) m[a * NS + b] *= d;
    }
  }
}

// Reverse of half-step h given its input state m (left unchanged): dm := d(input).
// For a row pass with line sum s_a, d_a = 1/(s_a + eps), M' = M d_a:
//   dM[a][b] = d_a (dM'[a][b] - sum_b' dM'[a][b'] M'[a][b'])
//            = d_a (sum_b' (dM'[a][b] - dM'[a][b']) M'[a][b'] + dM'[a][b] eps d_a)
// using 1 - sum_b' M'[a][b'] = eps d_a.  The second form has no cancellation
// when the line is nearly normalised (with one stream the first form loses
// everything but eps d_a of dM'); a column pass is the same over columns.
template <int NS>
__device__ __forceinline__ void sk_half_bwd(const float m[NS * NS], float dm[NS * NS], int h, float eps) {
  const bool rows = (h & 1) == 0;
#pragma unroll
  for (int a = 0; a < NS; ++a) {
    // line a: elements e(b) = a*NS + b (row pass) or b*NS + a (column pass)
    float s = 0.f;
#pragma unroll
    for (int b = 0; b < NS; ++b) s += m[rows ? a * NS + b : b * NS + a];
    const float d = 1.0f / (s + eps);
    float mp[NS], g[NS], o[NS];
#pragma unroll
    for (int b = 0; b < NS; ++b) {
      const int e = rows ? a * NS + b : b * NS + a;
      mp[b] = m[e] * d;
      g[b] = dm[e];
    }
#pragma unroll
    for (int b = 0; b < NS; ++b) {
      float acc = g[b] * (eps * d);
#pragma unroll
      for (int bp = 0; bp < NS; ++bp) acc += (g[b] - g[bp]) * mp[bp];
      o[b] = d * acc;
    }
#pragma unroll
    for (int b = 0; b < NS; ++b) dm[rows ? a * NS + b : b * NS + a] = o[b];
  }
}

template <int NS>
__device__ __forceinline__ void sk_exp(const float *L, float m[NS * NS]) {
#pragma unroll
  for (int e = 0; e < NS * NS; ++e) m[e] = __expf(L[e]);
}

template <int NS>
__device__ void sk_forward(const float *L, float m[NS * NS], int iters, float eps) {
  sk_exp<NS>(L, m);
  for (int h = 0; h < 2 * iters; ++h) sk_half<NS>(m, h, eps);
}

// dL for logits L (global, NS*NS) given dH in dm; dm is overwritten with dL.
// Checkpoints every `seg` half-steps: the state at a segment's start is
// replayed from exp(L), each half-step's input inside the segment from the
// segment start, so the cost is ~H^2/(2 seg) + H seg/2 half-steps.
template <int NS>
__device__ void sk_backward(const float *L, float dm[NS * NS], int iters, float eps) {
  const int H = 2 * iters;
  int seg = 1;
  while (seg * seg < H) ++seg;
  float ms[NS * NS], m[NS * NS];
  const int nseg = (H + seg - 1) / seg;
  for (int sgi = nseg - 1; sgi >= 0; --sgi) {
    const int h0 = sgi * seg, h1 = min(H, h0 + seg);
    sk_exp<NS>(L, ms);
    for (int h = 0; h < h0; ++h) sk_half<NS>(ms, h, eps);
    for (int h = h1 - 1; h >= h0; --h) {
#pragma unroll
      for (int e = 0; e < NS * NS; ++e) m[e] = ms[e];
      for (int hh = h0; hh < h; ++hh) sk_half<NS>(m, hh, eps);
      sk_half_bwd<NS>(m, dm, h, eps);
    }
  }
  sk_exp<NS>(L, m);
#pragma unroll
  for (int e = 0; e < NS * NS; ++e) dm[e] *= m[e];
}

// The same gradient with each half-step's line sums kept instead of
// replayed: one forward pass records e_a = s_a + eps per line, and the state
// at every kSkCkpt-th half-step, in the caller's thread-private LDS slots
// (word w of the thread at es[w * stride]); the reverse walk takes each
// half-step's output M', applies the half-step backward with d = 1/e (the
// forward's reciprocal, recomputed bit-identically) and rebuilds the
// half-step's input as M' e, restarting from the exact recorded state at
// every checkpoint so that rebuilt states carry at most kSkCkpt - 1
// roundings (rebuilding across all 40 half-steps of 20 iterations had put
// n = 5 gradients ~5e-6 off).  2 iters half-steps forward and back instead
// of ~2 iters sqrt(2 iters).
constexpr int kSkCkpt = 8;

inline size_t sk_stored_words(int n, int iters) {
  const int H = 2 * iters;
  return (size_t)H * n + (size_t)((H + kSkCkpt - 1) / kSkCkpt) * n * n;
}

template <int NS>
__device__ void sk_backward_stored(const float *L, float dm[NS * NS], int iters, float eps, float *es,
                                   int stride) {
  const int H = 2 * iters;
  float *ck = es + (size_t)H * NS * stride;  // checkpoints: state before half-steps 0, kSkCkpt, ...
  float m[NS * NS];
  sk_exp<NS>(L, m);
  for (int h = 0; h < H; ++h) {
    if (h % kSkCkpt == 0) {
#pragma unroll
      for (int e = 0; e < NS * NS; ++e) ck[((h / kSkCkpt) * NS * NS + e) * stride] = m[e];
    }
    const bool rows = (h & 1) == 0;
#pragma unroll
    for (int a = 0; a < NS; ++a) {
      float sum = 0.f;
#pragma unroll
      for (int b = 0; b < NS; ++b) sum += m[rows ? a * NS + b : b * NS + a];
      const float e = sum + eps;
      es[(h * NS + a) * stride] = e;
      const float d = 1.0f / e;
#pragma unroll
      for (int b = 0; b < NS; ++b) m[rows ? a * NS + b : b * NS + a] *= d;
    }
  }
  for (int h = H - 1; h >= 0; --h) {
    if ((h + 1) % kSkCkpt == 0 && h + 1 < H) {  // exact state after half-step h
#pragma unroll
      for (int e = 0; e < NS * NS; ++e) m[e] = ck[(((h + 1) / kSkCkpt) * NS * NS + e) * stride];
    }
    const bool rows = (h & 1) == 0;
#pragma unroll
    for (int a = 0; a < NS; ++a) {
      const float e = es[(h * NS + a) * stride];
      const float d = 1.0f / e;
      float mp[NS], g[NS], o[NS];
#pragma unroll
      for (int b = 0; b < NS; ++b) {
        const int el = rows ? a * NS + b : b * NS + a;
        mp[b] = m[el];
        g[b] = dm[el];
      }
#pragma unroll
      for (int b = 0; b < NS; ++b) {
        float acc = g[b] * (eps * d);
#pragma unroll
        for (int bp = 0; bp < NS; ++bp) acc += (g[b] - g[bp]) * mp[bp];
        o[b] = d * acc;
      }
#pragma unroll
      for (int b = 0; b < NS; ++b) {
        const int el = rows ? a * NS + b : b * NS + a;
        dm[el] = o[b];
        m[el] = mp[b] * e;
      }
    }
  }
  sk_exp<NS>(L, m);
#pragma unroll
  for (int e = 0; e < NS * NS; ++e) dm[e] *= m[e];
}

// Threads per block and whether the recorded sums and checkpoints fit in
// LDS (64 KB of dynamic LDS per block) for a Sinkhorn backward of `iters`
// iterations.
struct SkBwdGeom {
  int threads;
  bool stored;
  size_t lds;
};
inline SkBwdGeom sk_bwd_geom(int n, int iters) {
  const size_t per = sk_stored_words(n, iters) * sizeof(float);
  for (int t : {64, 32, 16})
    if (per * t <= 65536) return {t, true, per * t};
  return {64, false, 0};
}

// Row per lane (n >= 3): token i's matrix on a group of GW = n rounded up
// to a power of two lanes, each lane holding one line rotated by its lane
// index a: in the row layout v[c] = M[a][(a + c) % GW], in the column layout
// v[k] = M[(a + k) % GW][a] (entries past n are zero, lanes a >= n hold
// zeros).  A row pass sums and scales in-lane in the row layout, a column
// pass in-lane in the column layout, and sk_rotate turns either layout into
// the other with GW shuffles whose source register is the same on every lane
// (lane a reads lane (a + k) % GW's v[(GW - k) % GW]).  Every line sum runs
// in the rotated order (line a from entry a on), so every path that uses
// these functions (the fused finalize, the batched forward) gives the same
// bits for the same logits.
constexpr int sk_group(int n) { return n <= 1 ? 1 : n <= 2 ? 2 : n <= 4 ? 4 : 8; }

template <int GW>
__device__ __forceinline__ void sk_rotate(float v[GW], int a, int base) {
  float o[GW];
#pragma unroll
  for (int k = 0; k < GW; ++k) o[k] = __shfl(v[(GW - k) & (GW - 1)], base + ((a + k) & (GW - 1)), 64);
#pragma unroll
  for (int k = 0; k < GW; ++k) v[k] = o[k];
}

// 2 iters half-steps on the row layout (act: lane a < n of a real token);
// the state ends in the row layout.
template <int NS>
__device__ __forceinline__ void sk_forward_lanes(float v[sk_group(NS)], int a, int base, bool act, int iters,
                                                 float eps) {
  constexpr int GW = sk_group(NS);
  for (int h = 0; h < 2 * iters; ++h) {
    float s = 0.f;
#pragma unroll
    for (int c = 0; c < GW; ++c) s += v[c];
    const float d = act ? 1.0f / (s + eps) : 0.f;
#pragma unroll
    for (int c = 0; c < GW; ++c) v[c] *= d;
    sk_rotate<GW>(v, a, base);
  }
}

// Lanes records of the backward: e of the lane's line for every half-step,
// and the lane's row every kSkCkpt-th half-step.
inline size_t sk_lane_words(int n, int iters) {
  const int H = 2 * iters;
  return (size_t)H + (size_t)((H + kSkCkpt - 1) / kSkCkpt) * sk_group(n);
}

// The gradient on the lanes layout: the forward records each half-step's
// line sum (+ eps) and the state every kSkCkpt half-steps in the lane's own
// LDS slots (word w at lds[w * blockDim]); the reverse walk turns m (the
// half-step's output) and dm into the half-step's layout, applies the
// half-step backward in-lane with d = 1/e (the forward's reciprocal,
// recomputed bit-identically) and rebuilds the input as m e, restarting from
// the exact recorded state at every checkpoint.
template <int NS>
__global__ __launch_bounds__(256) void gsinkhorn_bwd_lanes_kernel(int64_t count, const float *__restrict__ dH,
                                                                 const float *__restrict__ L,
                                                                 float *__restrict__ dL, int iters, float eps) {
  constexpr int GW = sk_group(NS);
  extern __shared__ float sk_lds[];
  const int T = blockDim.x;
  float *my = sk_lds + threadIdx.x;
  const int64_t i = ((int64_t)blockIdx.x * T + threadIdx.x) / GW;
  const int a = threadIdx.x % GW;
  const int base = (threadIdx.x & 63) - a;  // the group's first lane within the wave
  const bool act = a < NS && i < count;
  const int H = 2 * iters;
  float *ck = my + (size_t)H * T;
  // real[c]: entry c of the lane's line is a matrix entry (the same test in both layouts)
  bool real[GW];
  float m[GW], dm[GW];
#pragma unroll
  for (int c = 0; c < GW; ++c) {
    const int col = (a + c) & (GW - 1);
    real[c] = act && col < NS;
    m[c] = real[c] ? __expf(L[(i * NS + a) * NS + col]) : 0.f;
    dm[c] = real[c] ? dH[(i * NS + a) * NS + col] : 0.f;
  }
  for (int h = 0; h < H; ++h) {
    if (h % kSkCkpt == 0) {
#pragma unroll
      for (int c = 0; c < GW; ++c) ck[((h / kSkCkpt) * GW + c) * T] = m[c];
    }
    float s = 0.f;
#pragma unroll
    for (int c = 0; c < GW; ++c) s += m[c];
    const float e = s + eps;
    my[h * T] = e;
    const float d = act ? 1.0f / e : 0.f;
#pragma unroll
    for (int c = 0; c < GW; ++c) m[c] *= d;
    sk_rotate<GW>(m, a, base);
  }
  // m: the output of half-step H - 1 and dm its gradient, both in the row
  // layout; each step below turns them into half-step h's layout first
  for (int h = H - 1; h >= 0; --h) {
    if ((h + 1) % kSkCkpt == 0 && h + 1 < H) {  // exact state after half-step h (row layout)
#pragma unroll
      for (int c = 0; c < GW; ++c) m[c] = ck[(((h + 1) / kSkCkpt) * GW + c) * T];
    }
    sk_rotate<GW>(m, a, base);
    sk_rotate<GW>(dm, a, base);
    const float e = my[h * T];
    const float d = act ? 1.0f / e : 0.f;
    float o[GW];
#pragma unroll
    for (int c = 0; c < GW; ++c) {
      float acc = dm[c] * (eps * d);
#pragma unroll
      for (int cp = 0; cp < GW; ++cp) acc += (dm[c] - dm[cp]) * m[cp];
      o[c] = real[c] ? d * acc : 0.f;
    }
#pragma unroll
    for (int c = 0; c < GW; ++c) {
      dm[c] = o[c];
      m[c] *= act ? e : 0.f;
    }
  }
#pragma unroll
  for (int c = 0; c < GW; ++c) {
    const int col = (a + c) & (GW - 1);
    if (real[c]) dL[(i * NS + a) * NS + col] = dm[c] * __expf(L[(i * NS + a) * NS + col]);
  }
}

// The forward on the lanes layout (n >= 3).
template <int NS>
__global__ __launch_bounds__(256) void gsinkhorn_fwd_lanes_kernel(int64_t count, const float *__restrict__ L,
                                                                 float *__restrict__ H, int iters, float eps) {
  constexpr int GW = sk_group(NS);
  const int64_t i = ((int64_t)blockIdx.x * 256 + threadIdx.x) / GW;
  const int a = threadIdx.x % GW;
  const int base = (threadIdx.x & 63) - a;
  const bool act = a < NS && i < count;
  float v[GW];
#pragma unroll
  for (int c = 0; c < GW; ++c) {
    const int col = (a + c) & (GW - 1);
    v[c] = act && col < NS ? __expf(L[(i * NS + a) * NS + col]) : 0.f;
  }
  sk_forward_lanes<NS>(v, a, base, act, iters, eps);
#pragma unroll
  for (int c = 0; c < GW; ++c) {
    const int col = (a + c) & (GW - 1);
    if (act && col < NS) H[(i * NS + a) * NS + col] = v[c];
  }
}

// Threads per block of the row-per-lane kernel whose records fit in 64 KB of
// LDS (0: they do not, or n <= 2, where a token per lane measured faster:
// the per-token kernels serve those cases).
inline int sk_lane_threads(int n, int iters) {
  if (n <= 2) return 0;
  const size_t per = sk_lane_words(n, iters) * sizeof(float);
  for (int t : {256, 128, 64})
    if (per * t <= 65536) return t;
  return 0;
}

template <int NS>
__global__ __launch_bounds__(64) void gsinkhorn_fwd_kernel(int64_t count, const float *__restrict__ L,
                                                          float *__restrict__ H, int iters, float eps) {
  const int64_t i = (int64_t)blockIdx.x * 64 + threadIdx.x;
  if (i >= count) return;
  float m[NS * NS];
  sk_forward<NS>(L + i * NS * NS, m, iters, eps);
#pragma unroll
  for (int e = 0; e < NS * NS; ++e) H[i * NS * NS + e] = m[e];
}

template <int NS, bool STORED>
__global__ __launch_bounds__(64) void gsinkhorn_bwd_kernel(int64_t count, const float *__restrict__ dH,
                                                          const float *__restrict__ L, float *__restrict__ dL,
                                                          int iters, float eps) {
  extern __shared__ float sk_lds[];  // STORED: line sums, thread-private slots
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= count) return;
  float dm[NS * NS];
#pragma unroll
  for (int e = 0; e < NS * NS; ++e) dm[e] = dH[i * NS * NS + e];
  if (STORED)
    sk_backward_stored<NS>(L + i * NS * NS, dm, iters, eps, sk_lds + threadIdx.x, blockDim.x);
  else
    sk_backward<NS>(L + i * NS * NS, dm, iters, eps);
#pragma unroll
  for (int e = 0; e < NS * NS; ++e) dL[i * NS * NS + e] = dm[e];
}

// ------------------------------------------------------------------ streaming ops
// One workgroup per token (per TG tokens for the dbias partials); thread
// owns 8-channel groups g = tid, tid + TPB, ...
template <typename T, int NS>
__global__ __launch_bounds__(256) void gagg_fwd_kernel(const T *__restrict__ X, const float *__restrict__ Hpre,
                                                      int64_t hs, T *__restrict__ out, int64_t C) {
  const int64_t t = blockIdx.x;
  const int64_t G = C / 8;
  float h[NS];
#pragma unroll
  for (int i = 0; i < NS; ++i) h[i] = Hpre[t * hs + i];
  for (int64_t g = threadIdx.x; g < G; g += blockDim.x) {
    float o[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int i = 0; i < NS; ++i) {
      float v[8];
      Io8<T>::load_nt(X + (t * NS + i) * C + 8 * g, v);
#pragma unroll
      for (int e = 0; e < 8; ++e) o[e] += h[i] * v[e];
    }
    Io8<T>::store(out + t * C + 8 * g, o);
  }
}

// dH_pre rows [N][NS] (dHrow), optionally dX (+)= H_pre g.
template <typename T, int NS>
__global__ __launch_bounds__(256) void gagg_bwd_kernel(const T *__restrict__ gr, const T *__restrict__ X,
                                                      const float *__restrict__ Hpre, int64_t hs,
                                                      T *__restrict__ dX, float *__restrict__ dHrow, int64_t C,
                                                      bool WRITE_DX, bool ACCUM) {
  __shared__ float red[4][NS];
  const int64_t t = blockIdx.x;
  const int64_t G = C / 8;
  float h[NS], acc[NS];
#pragma unroll
  for (int i = 0; i < NS; ++i) { h[i] = Hpre[t * hs + i]; acc[i] = 0.f; }
  for (int64_t g = threadIdx.x; g < G; g += blockDim.x) {
    float gv[8];
    Io8<T>::load_nt(gr + t * C + 8 * g, gv);
#pragma unroll
    for (int i = 0; i < NS; ++i) {
      float v[8];
      Io8<T>::load_nt(X + (t * NS + i) * C + 8 * g, v);
      float s = 0.f;
#pragma unroll
      for (int e = 0; e < 8; ++e) s += gv[e] * v[e];
      acc[i] += s;
      if (WRITE_DX) {
        float d[8];
        if (ACCUM) Io8<T>::load(dX + (t * NS + i) * C + 8 * g, d);
#pragma unroll
        for (int e = 0; e < 8; ++e) d[e] = (ACCUM ? d[e] : 0.f) + h[i] * gv[e];
        Io8<T>::store(dX + (t * NS + i) * C + 8 * g, d);
      }
    }
  }
  gblock_sum<NS>(acc, red);
  if (threadIdx.x == 0) {
#pragma unroll
    for (int i = 0; i < NS; ++i) dHrow[t * NS + i] = acc[i];
  }
}

// Column sums of rows[R][NC] in a fixed order: block b sums column b, thread
// i takes rows i, i + 256, ..., then the workgroup tree.
__global__ __launch_bounds__(256) void gcol_sum_kernel(const float *__restrict__ rows, float *__restrict__ out,
                                                      int64_t R, int NC) {
  __shared__ float red[4][1];
  const int col = blockIdx.x;
  float s[1] = {0.f};
  for (int64_t r = threadIdx.x; r < R; r += 256) s[0] += rows[r * NC + col];
  gblock_sum<1>(s, red);
  if (threadIdx.x == 0) out[col] = s[0];
}

// Sums over tokens of the per-token parameter terms rows[R][NC] (dhbias and
// dalpha of the projection backward), in two fixed-order stages.  Stage 1:
// thread i adds column i % NC over rows i / NC + kGParts m, m = 0, 1, ... in
// order, so consecutive threads read consecutive floats.
constexpr int kGParts = 1024;

__global__ __launch_bounds__(256) void gparam_part_kernel(const float *__restrict__ rows, float *__restrict__ part,
                                                         int64_t R, int NC) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= (int64_t)kGParts * NC) return;
  float s = 0.f;
#pragma unroll 8
  for (int64_t f = i; f < R * NC; f += (int64_t)kGParts * NC) s += rows[f];
  part[i] = s;
}

// Stage 2: per column, 32 lanes each add every 32nd of the kGParts partials
// in order, then a pairwise tree over the 32; columns [0, J) go to dhbias,
// [J, J + 3) to dalpha (either may be NULL).
__global__ __launch_bounds__(1024) void gparam_final_kernel(const float *__restrict__ part, int NC, int J,
                                                           float *__restrict__ dhbias, float *__restrict__ dalpha) {
  __shared__ float red[32][33];
  const int e = threadIdx.x & 31, q = threadIdx.x >> 5;
  const int col = blockIdx.x * 32 + e;
  float s = 0.f;
  if (col < NC) {
#pragma unroll 4
    for (int p = q; p < kGParts; p += 32) s += part[(int64_t)p * NC + col];
  }
  red[q][e] = s;
  __syncthreads();
  for (int w = 16; w > 0; w >>= 1) {
    if (q < w) red[q][e] += red[q + w][e];
    __syncthreads();
  }
  if (q != 0 || col >= NC) return;
  if (col < J) {
    if (dhbias) dhbias[col] = red[0][e];
  } else if (dalpha) {
    dalpha[col - J] = red[0][e];
  }
}

// h_post_bda forward and its halves (modes as the n = 4 kernels).
template <typename T, int NS, int MODE>
__global__ __launch_bounds__(256) void gpost_fwd_kernel(const T *__restrict__ X, const float *__restrict__ Hr,
                                                       const float *__restrict__ Hp, const T *__restrict__ x,
                                                       const T *__restrict__ bias, T *__restrict__ out, int64_t C) {
  const bool HAS_BIAS = bias != nullptr;
  const int64_t t = blockIdx.x;
  const int64_t G = C / 8;
  for (int64_t g = threadIdx.x; g < G; g += blockDim.x) {
    float xb[8], xv[NS][8];
    if (MODE != kPostMix) {
      Io8<T>::load_nt(x + t * C + 8 * g, xb);
      if (HAS_BIAS) {
        float b[8];
        Io8<T>::load(bias + 8 * g, b);
#pragma unroll
        for (int e = 0; e < 8; ++e) xb[e] += b[e];
      }
    }
    if (MODE != kPostDist) {
#pragma unroll
      for (int j = 0; j < NS; ++j) Io8<T>::load_nt(X + (t * NS + j) * C + 8 * g, xv[j]);
    }
#pragma unroll
    for (int i = 0; i < NS; ++i) {
      float o[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
      if (MODE != kPostDist) {
#pragma unroll
        for (int j = 0; j < NS; ++j) {
          const float w = Hr[t * NS * NS + j * NS + i];
#pragma unroll
          for (int e = 0; e < 8; ++e) o[e] += w * xv[j][e];
        }
      }
      if (MODE != kPostMix) {
        const float hp = Hp[t * NS + i];
#pragma unroll
        for (int e = 0; e < 8; ++e) o[e] += hp * xb[e];
      }
      // the new residual: written non-temporally (its dirty lines otherwise
      // land in the next kernel's reads when the caches evict them)
      Io8<T>::store_nt(out + (t * NS + i) * C + 8 * g, o);
    }
  }
}

// h_post_bda backward and its halves.  Per token: dX[j] = sum_i H_res[j][i]
// G[i] (WRITE_DX), dH_res[j][i] = <X_j, G_i> (MODE != dist), dH_post[i] =
// <G_i, x + bias> and dx = sum_i H_post[i] G_i (MODE != mix).  One wave per
// token, four waves per workgroup working independently: a lane owns the
// 8-channel groups g = lane, lane + 64, ..., and the per-token sums are wave
// reductions (no barrier).  The rows j of X are taken JB at a time, each
// pass with its own JB * n sums (GPostShape).  DBIAS: each wave walks TG
// tokens and adds its lanes' dx into its own partial row part[wave][C]
// (owned by that lane alone: no atomics).
template <typename T, int NS, int MODE> struct GPostShape {
  // all of X's rows in one pass (G read once) up to n = 7; at n = 8 the
  // n^2 + n sums take the registers to 256 either way, so two passes of
  // four rows, on two waves of the same token at once without dbias (the
  // second G read then comes from L2)
  static constexpr int JB = NS <= 7 ? NS : 4;
  static constexpr int NPASS = MODE != kPostDist ? (NS + JB - 1) / JB : 1;
};

template <typename T, int NS, int MODE, bool WDX>
__global__ __launch_bounds__(256) void gpost_bwd_kernel(const T *__restrict__ Gr, const T *__restrict__ X,
                                                       const float *__restrict__ Hr, const float *__restrict__ Hp,
                                                       const T *__restrict__ x, const T *__restrict__ bias,
                                                       T *__restrict__ dX, float *__restrict__ dHr,
                                                       float *__restrict__ dHp, T *__restrict__ dx,
                                                       float *__restrict__ part, int64_t N, int64_t C, int TG) {
  // WDX = false compiles the dX rows out (fewer registers).  With WDX the
  // test is a compile-time one up to n = 6 and a run-time one at n = 7, 8,
  // where that register allocation measured faster
  const bool HAS_BIAS = bias != nullptr, DBIAS = part != nullptr, WRITE_DX = WDX && (NS <= 6 || dX != nullptr);
  constexpr bool MIX = MODE != kPostDist, DIST = MODE != kPostMix;
  constexpr int JB = GPostShape<T, NS, MODE>::JB, NPASS = GPostShape<T, NS, MODE>::NPASS;
  constexpr int NR = (MIX ? JB * NS : 0) + (DIST ? NS : 0);
  const int lane = threadIdx.x & 63;
  const int64_t wv = (int64_t)blockIdx.x * (blockDim.x >> 6) + (threadIdx.x >> 6);  // global wave index
  // without dbias (one token per wave) the passes of a token run on NPASS
  // consecutive waves of one workgroup
  const bool split = NPASS > 1 && !DBIAS;
  const int pass_lo = split ? (int)(wv % NPASS) : 0, pass_hi = split ? pass_lo + 1 : NPASS;
  const int64_t G = C / 8;
  const int64_t t0 = (split ? wv / NPASS : wv) * TG;
  const int64_t t1 = min(t0 + (int64_t)TG, N);
  for (int64_t t = t0; t < t1; ++t) {
#pragma unroll 1
    for (int pass = pass_lo; pass < pass_hi; ++pass) {
      const int j0 = pass * JB;
      const bool dist_here = DIST && pass == 0;
      float acc[NR];
#pragma unroll
      for (int r = 0; r < NR; ++r) acc[r] = 0.f;
      for (int64_t g = lane; g < G; g += 64) {
        if constexpr (sizeof(T) == 2) {
          // bf16: G rows stay packed; dot products as bf16 pairs, other terms converted where used
          gu32x4 gw[NS];
#pragma unroll
          for (int i = 0; i < NS; ++i) {
            const gu32x4 *gp = reinterpret_cast<const gu32x4 *>(Gr + (t * NS + i) * C + 8 * g);
            gw[i] = NPASS > 1 ? *gp : __builtin_nontemporal_load(gp);  // two passes: G kept for the second
          }
          auto gval = [&](int i, int e) {
            const uint32_t w = (e >> 1) == 0 ? gw[i].x : (e >> 1) == 1 ? gw[i].y : (e >> 1) == 2 ? gw[i].z : gw[i].w;
            return (e & 1) ? bf16_hi(w) : bf16_lo(w);
          };
          // the dwords go through plain variables: bit-casting ext-vector
          // elements directly has been lowered with dword 0 in every position
          typedef __attribute__((ext_vector_type(2))) __bf16 pbf16x2;
          auto dot8 = [&](const gu32x4 &u, const gu32x4 &v, float a) {
            const uint32_t uw[4] = {u.x, u.y, u.z, u.w}, vw[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
            for (int q = 0; q < 4; ++q)
              a = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(pbf16x2, uw[q]),
                                                  __builtin_bit_cast(pbf16x2, vw[q]), a, false);
            return a;
          };
          if (MIX) {
#pragma unroll
            for (int jj = 0; jj < JB; ++jj) {
              const int j = j0 + jj;
              if (j < NS) {
                const gu32x4 xw =
                    __builtin_nontemporal_load(reinterpret_cast<const gu32x4 *>(X + (t * NS + j) * C + 8 * g));
#pragma unroll
                for (int i = 0; i < NS; ++i) acc[jj * NS + i] = dot8(xw, gw[i], acc[jj * NS + i]);
                if (WRITE_DX) {
                  float d[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
#pragma unroll
                  for (int i = 0; i < NS; ++i) {
                    const float w = Hr[t * NS * NS + j * NS + i];
#pragma unroll
                    for (int e = 0; e < 8; ++e) d[e] += w * gval(i, e);
                  }
                  Io8<T>::store(dX + (t * NS + j) * C + 8 * g, d);
                }
              }
            }
          }
          if (DIST && dist_here) {
            constexpr int off = MIX ? JB * NS : 0;
            float xb[8], o[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
            Io8<T>::load_nt(x + t * C + 8 * g, xb);
            if (HAS_BIAS) {
              float bv[8];
              Io8<T>::load(bias + 8 * g, bv);
#pragma unroll
              for (int e = 0; e < 8; ++e) xb[e] += bv[e];
            }
#pragma unroll
            for (int i = 0; i < NS; ++i) {
              const float hp = Hp[t * NS + i];
              float sdot = 0.f;
#pragma unroll
              for (int e = 0; e < 8; ++e) {
                const float gvi = gval(i, e);
                sdot += gvi * xb[e];
                o[e] += hp * gvi;
              }
              acc[off + i] += sdot;
            }
            Io8<T>::store(dx + t * C + 8 * g, o);
            if (DBIAS) {
              float *p = part + wv * C + 8 * g;
#pragma unroll
              for (int e = 0; e < 8; ++e) p[e] = (t == t0 ? 0.f : p[e]) + o[e];
            }
          }
          continue;
        }
        float gv[NS][8];
#pragma unroll
        for (int i = 0; i < NS; ++i) {
          if (NPASS > 1)
            Io8<T>::load(Gr + (t * NS + i) * C + 8 * g, gv[i]);  // two passes: G kept for the second
          else
            Io8<T>::load_nt(Gr + (t * NS + i) * C + 8 * g, gv[i]);
        }
        if (MIX) {
#pragma unroll
          for (int jj = 0; jj < JB; ++jj) {
            const int j = j0 + jj;
            if (j < NS) {
              float xv[8];
              Io8<T>::load_nt(X + (t * NS + j) * C + 8 * g, xv);
#pragma unroll
              for (int i = 0; i < NS; ++i) {
                float sdot = 0.f;
#pragma unroll
                for (int e = 0; e < 8; ++e) sdot += xv[e] * gv[i][e];
                acc[jj * NS + i] += sdot;
              }
              if (WRITE_DX) {
                float d[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int i = 0; i < NS; ++i) {
                  const float w = Hr[t * NS * NS + j * NS + i];
#pragma unroll
                  for (int e = 0; e < 8; ++e) d[e] += w * gv[i][e];
                }
                Io8<T>::store(dX + (t * NS + j) * C + 8 * g, d);
              }
            }
          }
        }
        if (DIST && dist_here) {
          constexpr int off = MIX ? JB * NS : 0;
          float xb[8], o[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
          Io8<T>::load_nt(x + t * C + 8 * g, xb);
          if (HAS_BIAS) {
            float bv[8];
            Io8<T>::load(bias + 8 * g, bv);
#pragma unroll
            for (int e = 0; e < 8; ++e) xb[e] += bv[e];
          }
#pragma unroll
          for (int i = 0; i < NS; ++i) {
            const float hp = Hp[t * NS + i];
            float sdot = 0.f;
#pragma unroll
            for (int e = 0; e < 8; ++e) {
              sdot += gv[i][e] * xb[e];
              o[e] += hp * gv[i][e];
            }
            acc[off + i] += sdot;
          }
          Io8<T>::store(dx + t * C + 8 * g, o);
          if (DBIAS) {
            float *p = part + wv * C + 8 * g;
#pragma unroll
            for (int e = 0; e < 8; ++e) p[e] = (t == t0 ? 0.f : p[e]) + o[e];
          }
        }
      }
#pragma unroll
      for (int r = 0; r < NR; ++r) acc[r] = wave_sum(acc[r]);
      if (lane == 0) {
        if (MIX) {
#pragma unroll
          for (int jj = 0; jj < JB; ++jj)
            if (j0 + jj < NS) {
#pragma unroll
              for (int i = 0; i < NS; ++i) dHr[t * NS * NS + (j0 + jj) * NS + i] = acc[jj * NS + i];
            }
        }
        if (dist_here) {
          constexpr int off = MIX ? JB * NS : 0;
#pragma unroll
          for (int i = 0; i < NS; ++i) dHp[t * NS + i] = acc[off + i];
        }
      }
    }
  }
}

// ------------------------------------------------------------------ projection forward
// Grid: ceil(N / 128) * kGSplitK workgroups of 4 waves; workgroup b takes
// token block b / kGSplitK (128 tokens, 32 per wave) and k slice
// b % kGSplitK.  The slice's 64-k chunks are walked by all four waves
// together: each chunk of W (64 k x J) is loaded once per workgroup into LDS,
// transposed to [column][k] so a lane reads its 32 k values with 128-bit
// reads, and every wave multiplies it with its own tokens' x on the fp32
// MFMA (32x32x2).  Each chunk is summed from zero and then added to the
// running sum (two-level blocking).  part[slice][t][0..J) = partial x @ W,
// part[slice][t][J] = partial sum x^2.
constexpr int kGTokWG = 4 * kGTok;  // tokens per forward workgroup

template <typename T, int NS>
__global__ __launch_bounds__(256) void gproj_partial_kernel(const T *__restrict__ X, const float *__restrict__ W,
                                                           float *__restrict__ part, int64_t N, int64_t K) {
  constexpr int J = Dim<NS>::J, JT = Dim<NS>::JT, PS = Dim<NS>::PS;
  constexpr int SWS = 64 + 4;  // LDS row stride of the transposed W chunk (floats)
  __shared__ __align__(16) float sW[32 * JT][SWS];
  const int slice = blockIdx.x % kGSplitK;
  const int64_t tb = blockIdx.x / kGSplitK;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int row = lane & 31, h = lane >> 5;
  const int64_t nch = (K + 63) / 64;
  const int64_t cps = (nch + kGSplitK - 1) / kGSplitK;
  const int64_t c_begin = slice * cps;
  const int64_t c_end = min(nch, c_begin + cps);
  const int64_t trow = tb * kGTokWG + wave * kGTok + row;
  const bool tvalid = trow < N;

  gf32x16 outer[JT];
#pragma unroll
  for (int u = 0; u < JT; ++u)
#pragma unroll
    for (int r = 0; r < 16; ++r) outer[u][r] = 0.f;
  float ss = 0.f;

  // The next chunk's W values and x groups are loaded into registers while
  // the current chunk is multiplied (K % 8 == 0 and k0 % 32 == 0: an 8-value
  // x group is either wholly inside K or wholly past it).
  constexpr int WPT = (64 * 32 * JT + 255) / 256;  // W values per thread per chunk
  using R = typename Io8<T>::raw_t;
  float wreg[WPT];
  R xr[4];
  bool xok[4];
  auto fetch = [&](int64_t c) {
    const int64_t kc = c * 64;
#pragma unroll
    for (int q = 0; q < WPT; ++q) {
      const int idx = threadIdx.x + q * 256;
      const int kk = idx / (32 * JT), j = idx % (32 * JT);
      wreg[q] = (idx < 64 * 32 * JT && j < J && kc + kk < K) ? W[(kc + kk) * J + j] : 0.f;
    }
    const int64_t k0 = kc + 32 * h;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      xok[q] = tvalid && k0 + 8 * q < K;
      if (xok[q]) xr[q] = Io8<T>::ld_nt(X + trow * K + k0 + 8 * q);
    }
  };
  if (c_begin < c_end) fetch(c_begin);
  for (int64_t c = c_begin; c < c_end; ++c) {
    __syncthreads();  // the previous chunk's reads of sW are done
#pragma unroll
    for (int q = 0; q < WPT; ++q) {
      const int idx = threadIdx.x + q * 256;
      if (idx < 64 * 32 * JT) sW[idx % (32 * JT)][idx / (32 * JT)] = wreg[q];
    }
    float a[32];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      if (xok[q]) {
        Io8<T>::cvt(xr[q], a + 8 * q);
      } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) a[8 * q + e] = 0.f;
      }
    }
    __syncthreads();
    if (c + 1 < c_end) fetch(c + 1);
    float sq = 0.f;
#pragma unroll
    for (int e = 0; e < 32; ++e) sq = fmaf(a[e], a[e], sq);
    ss += sq;
#pragma unroll
    for (int u = 0; u < JT; ++u) {
      float b[32];
      const float4 *src = reinterpret_cast<const float4 *>(&sW[32 * u + row][32 * h]);
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        const float4 v = src[q];
        b[4 * q] = v.x; b[4 * q + 1] = v.y; b[4 * q + 2] = v.z; b[4 * q + 3] = v.w;
      }
      gf32x16 acc;
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[r] = 0.f;
#pragma unroll
      for (int e = 0; e < 32; ++e) acc = __builtin_amdgcn_mfma_f32_32x32x2f32(a[e], b[e], acc, 0, 0, 0);
#pragma unroll
      for (int r = 0; r < 16; ++r) outer[u][r] += acc[r];
    }
  }
  // accumulator layout of a 32x32 MFMA: lane (col, h), register r holds row
  // 8*(r/4) + 4*h + (r%4), column col.  Sum of squares: the two k halves of a
  // token's row sit on lanes row and row + 32.
#pragma unroll
  for (int u = 0; u < JT; ++u) {
    const int col = 32 * u + row;
    if (col < J) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int64_t t = tb * kGTokWG + wave * kGTok + 8 * (r >> 2) + 4 * h + (r & 3);
        if (t < N) part[((int64_t)slice * N + t) * PS + col] = outer[u][r];
      }
    }
  }
  const float ss_other = __shfl_xor(ss, 32);
  if (h == 0 && tvalid) part[((int64_t)slice * N + trow) * PS + J] = ss + ss_other;
}

// bf16 activations: the same split-K on the bf16 MFMA (32x32x16).  Each W
// value is split exactly into three bf16 terms (hi = W rounded to bf16,
// mid = the rest rounded, lo = what remains: 8 + 8 + 8 significant bits
// cover fp32's 24), and bf16 x times a bf16 term is exact in the fp32
// accumulator, so the three products give x @ W to fp32 accumulation.
// gpack_w_kernel splits W once per call into Wp[chunk][piece of 8 k][term]
// [column][8 k] (64 k per chunk, 32 JT columns, zero past K and J), so a
// chunk is one contiguous block of 12 JT KB that a workgroup copies verbatim
// into LDS, and the 32 columns of one piece and term (a B fragment for each
// lane of a half-wave) are 512 contiguous bytes, read without bank conflicts.  A workgroup is 8
// waves x 32 tokens on one k slice; each 64-k chunk of W (shared) and of
// every wave's X tile (4 KB, 8 lanes per 128-byte row segment, piece p of
// row r in slot p ^ (r & 7)) goes through an LDS ring filled by
// global_load_lds_dwordx4 (3 stages where they fit in LDS, else 2).  A
// lane's A operand is the 8 x values of its token at k = 32h + 8q and its B
// operand the same 8 k of its column (the k order inside an MFMA is free as
// long as A and B agree).  Each chunk is summed from zero and then added to
// the running sum, as in the fp32 kernel.  With NSUB > 1 the slice's chunks
// form NSUB sub-slices, each with its own running sum, and workgroup tb starts
// its walk at sub-slice tb % NSUB (wrapping around); the sub-slice sums are
// added in sub-slice order at the end, so a token's result still depends on K
// alone.  Rows whose stride is a multiple of 16 KB otherwise put the same k
// offsets of all tokens in flight at once, which reads slower.
typedef __attribute__((ext_vector_type(8))) __bf16 gbf16x8;

template <int NS> struct GPj {
  static constexpr int JT = Dim<NS>::JT;
  static constexpr int WB = 3 * 32 * JT * 128;          // bytes of one packed 64-k W chunk
  static constexpr int XT = 32 * 128;                   // bytes of one wave's X tile
  // waves (32 tokens each) per workgroup, and ring stages: three where they
  // fit in LDS (one column tile), else two.  Four waves with three stages
  // for the wider W chunks measured 40% slower (W read per token doubles).
  static constexpr int WAVES = 8;
  static constexpr int SB = WB + WAVES * XT;            // bytes of one stage
  static constexpr int STAGES = 3 * SB <= 160 * 1024 ? 3 : 2;
  static constexpr int TOK = 32 * WAVES;                // tokens per workgroup
};

template <int NS>
__global__ __launch_bounds__(256) void gpack_w_kernel(const float *__restrict__ W, bf16_t *__restrict__ Wp,
                                                     int64_t K) {
  constexpr int J = Dim<NS>::J, JT = Dim<NS>::JT;
  const int64_t nch = (K + 63) / 64;
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;  // (chunk, piece, column)
  if (i >= nch * 32 * JT * 8) return;
  const int j = (int)(i % (32 * JT)), p = (int)((i / (32 * JT)) & 7);
  const int64_t c = i / (32 * JT * 8);
  float hi[8], mid[8], lo[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const int64_t k = c * 64 + 8 * p + e;
    const float w = (k < K && j < J) ? W[k * J + j] : 0.f;
    hi[e] = (float)(__bf16)w;
    const float r1 = w - hi[e];
    mid[e] = (float)(__bf16)r1;
    lo[e] = r1 - mid[e];
  }
  const float *terms[3] = {hi, mid, lo};
#pragma unroll
  for (int m = 0; m < 3; ++m) {
    const float *v = terms[m];
    uint4 w4;
    w4.x = pack_bf16x2(v[0], v[1]);
    w4.y = pack_bf16x2(v[2], v[3]);
    w4.z = pack_bf16x2(v[4], v[5]);
    w4.w = pack_bf16x2(v[6], v[7]);
    *reinterpret_cast<uint4 *>(Wp + (((c * 8 + p) * 3 + m) * 32 * JT + j) * 8) = w4;
  }
}

template <int NS, int NSUB>
__global__ __launch_bounds__(512) void gproj_partial_dma_kernel(const bf16_t *__restrict__ X,
                                                               const bf16_t *__restrict__ Wp,
                                                               float *__restrict__ part, int64_t N, int64_t K) {
  using G = GPj<NS>;
  constexpr int J = Dim<NS>::J, JT = G::JT, PS = Dim<NS>::PS, STG = G::STAGES;
  extern __shared__ __attribute__((aligned(16))) char gpl[];
  const int slice = blockIdx.x % kGSplitK;
  const int64_t tb = blockIdx.x / kGSplitK;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int row = lane & 31, h = lane >> 5;
  const int64_t nch = (K + 63) / 64;
  const int64_t cps = (nch + kGSplitK - 1) / kGSplitK;
  const int64_t c_begin = min(nch, slice * cps);
  const int nc = (int)(min(nch, c_begin + cps) - c_begin);
  const int64_t tw = tb * G::TOK + kGTok * wave;  // this wave's first token
  constexpr int QW = G::WB / 1024;                       // 1 KB copies of a W chunk, over the waves
  const int nq = (QW - wave + G::WAVES - 1) / G::WAVES + 4;  // this wave's copies per chunk
  // the slice's chunks fall into NSUB sub-slices of sps chunks; the walk
  // starts at sub-slice tb % NSUB and wraps around
  const int sps = (nc + NSUB - 1) / NSUB;
  const int cstart = sps * (int)(tb % NSUB) < nc ? sps * (int)(tb % NSUB) : 0;
  auto chunk = [&](int v) { return cstart + v < nc ? cstart + v : cstart + v - nc; };

  auto issue = [&](int v) {  // the copies of walk position v
    char *st = gpl + (v % STG) * G::SB;
    const int64_t c = c_begin + chunk(v);
    const char *wsrc = reinterpret_cast<const char *>(Wp) + c * G::WB;
    for (int q = wave; q < QW; q += G::WAVES) dma16(wsrc + q * 1024 + lane * 16, st + q * 1024);
    char *xs = st + G::WB + wave * G::XT;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int rr = 8 * q + (lane >> 3);   // row within the wave's 32
      const int p = (lane & 7) ^ (rr & 7);  // global 8-k piece for this slot
      const int64_t t = min(tw + rr, N - 1);  // rows past N re-read row N-1 (never stored)
      const int64_t k = c * 64 + 8 * p < K ? c * 64 + 8 * p : c * 64;  // past K: a real k (W is 0 there)
      dma16_nt(X + t * K + k, xs + q * 1024);  // X is streamed once
    }
  };

  gf32x16 outer[NSUB][JT];  // one running sum per sub-slice
  float ss[NSUB];
#pragma unroll
  for (int q = 0; q < NSUB; ++q) {
#pragma unroll
    for (int u = 0; u < JT; ++u)
#pragma unroll
      for (int r = 0; r < 16; ++r) outer[q][u][r] = 0.f;
    ss[q] = 0.f;
  }
  if (nc > 0) issue(0);
  if (STG == 3 && nc > 1) issue(1);
  for (int v = 0; v < nc; ++v) {
    // this wave's copies of position v are complete once at most those of v + 1 remain
    if (STG == 3 && v + 1 < nc) wait_vmcnt_le(nq); else wait_vmcnt<0>();
    lds_barrier();
    if (v + STG - 1 < nc) issue(v + STG - 1);  // that slot was last read in iteration v - 1
    const char *st = gpl + (v % STG) * G::SB;
    const char *xs = st + G::WB + wave * G::XT;
    const int ci = chunk(v);
    const int sub = NSUB == 1 ? 0 : ci / sps;  // workgroup-uniform
    const int64_t k0 = (c_begin + ci) * 64;
    gu32x4 a[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int p = 4 * h + q;
      a[q] = *reinterpret_cast<const gu32x4 *>(xs + (row * 8 + (p ^ (row & 7))) * 16);
    }
    float sq = 0.f;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      if (k0 + 32 * h + 8 * q < K) {
        const uint32_t w4[4] = {a[q].x, a[q].y, a[q].z, a[q].w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float v0 = bf16_lo(w4[e]), v1 = bf16_hi(w4[e]);
          sq = fmaf(v0, v0, sq);
          sq = fmaf(v1, v1, sq);
        }
      }
    }
#pragma unroll
    for (int q = 0; q < NSUB; ++q)
      if (sub == q) ss[q] += sq;
#pragma unroll
    for (int u = 0; u < JT; ++u) {
      gf32x16 acc;
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[r] = 0.f;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int p = 4 * h + q;
#pragma unroll
        for (int m = 0; m < 3; ++m) {
          const gu32x4 bw = *reinterpret_cast<const gu32x4 *>(st + ((p * 3 + m) * 32 * JT + 32 * u + row) * 16);
          acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(gbf16x8, a[q]),
                                                        __builtin_bit_cast(gbf16x8, bw), acc, 0, 0, 0);
        }
      }
#pragma unroll
      for (int q = 0; q < NSUB; ++q)
        if (sub == q) {
#pragma unroll
          for (int r = 0; r < 16; ++r) outer[q][u][r] += acc[r];
        }
    }
  }
  // the sub-slice sums in sub-slice order: a token's summation order depends
  // on K alone, not on where the walk started
#pragma unroll
  for (int q = 1; q < NSUB; ++q) {
#pragma unroll
    for (int u = 0; u < JT; ++u)
#pragma unroll
      for (int r = 0; r < 16; ++r) outer[0][u][r] += outer[q][u][r];
    ss[0] += ss[q];
  }
  // accumulator layout of a 32x32 MFMA: lane (col, h), register r holds row
  // 8*(r/4) + 4*h + (r%4), column col.  Sum of squares: the two k halves of a
  // token's row sit on lanes row and row + 32.
#pragma unroll
  for (int u = 0; u < JT; ++u) {
    const int col = 32 * u + row;
    if (col < J) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int64_t t = tw + 8 * (r >> 2) + 4 * h + (r & 3);
        if (t < N) part[((int64_t)slice * N + t) * PS + col] = outer[0][u][r];
      }
    }
  }
  const float ss_other = __shfl_xor(ss[0], 32);
  if (h == 0 && tw + row < N) part[((int64_t)slice * N + tw + row) * PS + J] = ss[0] + ss_other;
}

// One thread per token: slices summed in order, then RMS, gains, sigmoid;
// saved[t] = {r, q, z[0..J), 0...} (stride SS); Sinkhorn when Hres != NULL.
template <int NS>
__global__ __launch_bounds__(64) void gproj_finalize_kernel(const float *__restrict__ part, int64_t N, int64_t K,
                                                           const float *__restrict__ alpha,
                                                           const float *__restrict__ hbias, float rms_eps,
                                                           float *__restrict__ Hpre, float *__restrict__ Hpost,
                                                           float *__restrict__ logits, float *__restrict__ saved,
                                                           int SS, float *__restrict__ Hres, int iters, float eps) {
  constexpr int J = Dim<NS>::J, PS = Dim<NS>::PS;
  const int64_t t = (int64_t)blockIdx.x * 64 + threadIdx.x;
  if (t >= N) return;
  float p[PS];
#pragma unroll
  for (int j = 0; j < PS; ++j) p[j] = 0.f;
  for (int sl = 0; sl < kGSplitK; ++sl) {
#pragma unroll
    for (int j = 0; j < PS; ++j) p[j] += part[((int64_t)sl * N + t) * PS + j];
  }
  const float q = sqrtf(p[J] / (float)K);
  const float r = 1.0f / (q + rms_eps);
  const float a0 = alpha ? alpha[0] : 1.f, a1 = alpha ? alpha[1] : 1.f, a2 = alpha ? alpha[2] : 1.f;
  float L[NS * NS];
#pragma unroll
  for (int j = 0; j < J; ++j) {
    const float z = r * p[j];
    const float a = j < NS ? a0 : j < 2 * NS ? a1 : a2;
    const float zh = a * z + (hbias ? hbias[j] : 0.f);
    if (j < NS)
      Hpre[t * NS + j] = sigm(zh);
    else if (j < 2 * NS)
      Hpost[t * NS + j - NS] = 2.0f * sigm(zh);
    else
      L[j - 2 * NS] = zh;
    if (saved) saved[t * SS + 2 + j] = z;
  }
#pragma unroll
  for (int e = 0; e < NS * NS; ++e) logits[t * NS * NS + e] = L[e];
  if (saved) {
    saved[t * SS + 0] = r;
    saved[t * SS + 1] = q;
    for (int j = 2 + J; j < SS; ++j) saved[t * SS + j] = 0.f;
  }
  if (Hres) {
    float m[NS * NS];
    sk_forward<NS>(L, m, iters, eps);
#pragma unroll
    for (int e = 0; e < NS * NS; ++e) Hres[t * NS * NS + e] = m[e];
  }
}

// The same for n >= 3 on GW = sk_group(n) lanes per token: lane a < n sums
// the slices of its entries (H_pre a, H_post a, logits row a) in slice order,
// every lane the sum of squares (so all lanes hold the same r), and the
// Sinkhorn runs on the lanes layout, as the batched forward does.
template <int NS>
__global__ __launch_bounds__(256) void gproj_finalize_lanes_kernel(
    const float *__restrict__ part, int64_t N, int64_t K, const float *__restrict__ alpha,
    const float *__restrict__ hbias, float rms_eps, float *__restrict__ Hpre, float *__restrict__ Hpost,
    float *__restrict__ logits, float *__restrict__ saved, int SS, float *__restrict__ Hres, int iters, float eps) {
  constexpr int J = Dim<NS>::J, PS = Dim<NS>::PS, GW = sk_group(NS);
  const int64_t t = ((int64_t)blockIdx.x * 256 + threadIdx.x) / GW;
  const int a = threadIdx.x % GW;
  const int base = (threadIdx.x & 63) - a;
  const bool tv = t < N;
  const bool act = tv && a < NS;
  const int64_t tt = tv ? t : N - 1;  // lanes past N compute on a real row and store nothing
  const int ar = a < NS ? a : 0;      // lanes a >= n likewise
  // p[0] = H_pre column a, p[1] = H_post column a, p[2 + b] = logit (a, b)
  float ss = 0.f, p[NS + 2];
#pragma unroll
  for (int e = 0; e < NS + 2; ++e) p[e] = 0.f;
  for (int sl = 0; sl < kGSplitK; ++sl) {
    const float *pr = part + ((int64_t)sl * N + tt) * PS;
    ss += pr[J];
    p[0] += pr[ar];
    p[1] += pr[NS + ar];
#pragma unroll
    for (int b = 0; b < NS; ++b) p[2 + b] += pr[2 * NS + ar * NS + b];
  }
  const float q = sqrtf(ss / (float)K);
  const float r = 1.0f / (q + rms_eps);
  const float a0 = alpha ? alpha[0] : 1.f, a1 = alpha ? alpha[1] : 1.f, a2 = alpha ? alpha[2] : 1.f;
  float L[NS];
  {
    const float z0 = r * p[0], z1 = r * p[1];
    const float zh0 = a0 * z0 + (hbias ? hbias[ar] : 0.f);
    const float zh1 = a1 * z1 + (hbias ? hbias[NS + ar] : 0.f);
    if (act) {
      Hpre[t * NS + a] = sigm(zh0);
      Hpost[t * NS + a] = 2.0f * sigm(zh1);
      if (saved) {
        saved[t * SS + 2 + a] = z0;
        saved[t * SS + 2 + NS + a] = z1;
      }
    }
#pragma unroll
    for (int b = 0; b < NS; ++b) {
      const int j = 2 * NS + ar * NS + b;
      const float z = r * p[2 + b];
      L[b] = a2 * z + (hbias ? hbias[j] : 0.f);
      if (act) {
        logits[t * NS * NS + a * NS + b] = L[b];
        if (saved) saved[t * SS + 2 + j] = z;
      }
    }
  }
  if (saved && tv && a == 0) {
    saved[t * SS + 0] = r;
    saved[t * SS + 1] = q;
    for (int j = 2 + J; j < SS; ++j) saved[t * SS + j] = 0.f;
  }
  if (Hres) {
    float v[GW];
#pragma unroll
    for (int c = 0; c < GW; ++c) {
      const int col = (a + c) & (GW - 1);
      float x = 0.f;
#pragma unroll
      for (int b = 0; b < NS; ++b) x = b == col ? L[b] : x;
      v[c] = act && col < NS ? __expf(x) : 0.f;
    }
    sk_forward_lanes<NS>(v, a, base, act, iters, eps);
#pragma unroll
    for (int c = 0; c < GW; ++c) {
      const int col = (a + c) & (GW - 1);
      if (act && col < NS) Hres[(t * NS + a) * NS + col] = v[c];
    }
  }
}

// ------------------------------------------------------------------ projection backward
// Per token (one thread): dzh from the saved forward state; rec[t] (stride
// RS) = {dp[0..J) = r alpha dzh, zeros up to RC, c_rms = -r sum_j dz_j z_j /
// (K q) (0 if q == 0) at RC};
// prm[t] = {dzh[0..J) (dhbias terms), sum_seg dzh z (dalpha terms, 3)}.
// dH_res and the logits (Sinkhorn backward) replace dL when dL == NULL.
template <int NS, bool STORED>
__global__ __launch_bounds__(64) void gproj_bwd_token_kernel(
    int64_t N, int64_t K, const float *__restrict__ alpha, const float *__restrict__ saved, int SS,
    const float *__restrict__ Hpre, const float *__restrict__ Hpost, const float *__restrict__ dHpre,
    const float *__restrict__ dHpost, const float *__restrict__ dL, const float *__restrict__ dHres,
    const float *__restrict__ logits, int iters, float eps, float *__restrict__ rec, float *__restrict__ prm,
    float *__restrict__ dL_out) {
  extern __shared__ float sk_lds[];  // STORED: Sinkhorn line sums, thread-private slots
  constexpr int J = Dim<NS>::J;
  const int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (t >= N) return;
  const float r = saved[t * SS], q = saved[t * SS + 1];
  const float al[3] = {alpha ? alpha[0] : 1.f, alpha ? alpha[1] : 1.f, alpha ? alpha[2] : 1.f};
  float dl[NS * NS];
  if (dL) {
#pragma unroll
    for (int e = 0; e < NS * NS; ++e) dl[e] = dL[t * NS * NS + e];
  } else {
#pragma unroll
    for (int e = 0; e < NS * NS; ++e) dl[e] = dHres[t * NS * NS + e];
    if (STORED)
      sk_backward_stored<NS>(logits + t * NS * NS, dl, iters, eps, sk_lds + threadIdx.x, blockDim.x);
    else
      sk_backward<NS>(logits + t * NS * NS, dl, iters, eps);
  }
  if (dL_out) {
#pragma unroll
    for (int e = 0; e < NS * NS; ++e) dL_out[t * NS * NS + e] = dl[e];
  }
  float S = 0.f, da[3] = {0.f, 0.f, 0.f};
#pragma unroll
  for (int j = 0; j < J; ++j) {
    float dzh;
    int sg;
    if (j < NS) {
      const float sv = Hpre[t * NS + j];
      dzh = dHpre[t * NS + j] * sv * (1.f - sv);
      sg = 0;
    } else if (j < 2 * NS) {
      const float sv = 0.5f * Hpost[t * NS + j - NS];
      dzh = dHpost[t * NS + j - NS] * 2.f * sv * (1.f - sv);
      sg = 1;
    } else {
      dzh = dl[j - 2 * NS];
      sg = 2;
    }
    const float z = saved[t * SS + 2 + j];
    const float dz = al[sg] * dzh;
    S += dz * z;
    da[sg] += dzh * z;
    rec[t * Dim<NS>::RS + j] = r * dz;
    prm[t * (J + 3) + j] = dzh;
  }
#pragma unroll
  for (int j = J; j < Dim<NS>::RC; ++j) rec[t * Dim<NS>::RS + j] = 0.f;
  rec[t * Dim<NS>::RS + Dim<NS>::RC] = q > 0.f ? -S * r / ((float)K * q) : 0.f;
  prm[t * (J + 3) + J] = da[0];
  prm[t * (J + 3) + J + 1] = da[1];
  prm[t * (J + 3) + J + 2] = da[2];
}

// The residual-gradient terms of the fused pre backward that need no
// projection state, formed per token with 128-bit loads into an fp32
// workspace row term[t][k], k = j*C + c:
//   term = H_pre[t][j] g[t][c]  (g given)  +  sum_i H_res[t][j][i] G[t][i][c]  (G given)
// so the dX/dW kernel reads one value per element instead of n + 1 narrow
// ones.  One workgroup per token, H values staged in LDS.
template <typename T, int NS>
__global__ __launch_bounds__(256) void gpre_terms_kernel(const T *__restrict__ gr, const float *__restrict__ Hpre,
                                                        const T *__restrict__ Gp, const float *__restrict__ Hr,
                                                        float *__restrict__ term, int64_t C) {
  __shared__ float sH[NS + NS * NS];
  const int64_t t = blockIdx.x;
  const bool HAS_G = gr != nullptr, POST = Gp != nullptr;
  for (int e = threadIdx.x; e < NS + NS * NS; e += blockDim.x)
    sH[e] = e < NS ? (HAS_G ? Hpre[t * NS + e] : 0.f) : (POST ? Hr[t * NS * NS + e - NS] : 0.f);
  __syncthreads();
  const int64_t G = C / 8;
  for (int64_t g = threadIdx.x; g < G; g += blockDim.x) {
    float gv[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f}, Gv[NS][8];
    if (HAS_G) Io8<T>::load(gr + t * C + 8 * g, gv);
#pragma unroll
    for (int i = 0; i < NS; ++i) {
      if (POST) {
        Io8<T>::load(Gp + (t * NS + i) * C + 8 * g, Gv[i]);
      } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) Gv[i][e] = 0.f;
      }
    }
#pragma unroll
    for (int j = 0; j < NS; ++j) {
      float o[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) o[e] = sH[j] * gv[e];
#pragma unroll
      for (int i = 0; i < NS; ++i) {
        const float w = sH[NS + j * NS + i];
#pragma unroll
        for (int e = 0; e < 8; ++e) o[e] += w * Gv[i][e];
      }
      float *dst = term + (t * NS + j) * C + 8 * g;
      *reinterpret_cast<float4 *>(dst) = make_float4(o[0], o[1], o[2], o[3]);
      *reinterpret_cast<float4 *>(dst + 4) = make_float4(o[4], o[5], o[6], o[7]);
    }
  }
}

// dX and dW.  Grid: (K / 256 k tiles) x (token blocks); thread = one k =
// i*C + c, holding W[k][0..J) and its dW partial.  For each token of the
// block (records staged in LDS, four tokens' loads issued together):
//   dX[t][k] = (dX_in) + term[t][k] + sum_j dp[t][j] W[k][j] + c_rms[t] x[t][k]
// all in fp32 with one rounding at the store; dW[k][j] += x[t][k] dp[t][j].
template <typename T, int NS, bool DW>
__global__ __launch_bounds__(256) void gproj_bwd_dx_kernel(
    const T *__restrict__ X, const float *__restrict__ W, const float *__restrict__ rec,
    const float *__restrict__ term, T *__restrict__ dX, float *__restrict__ dwpart, int64_t N, int64_t C,
    int64_t TB, bool ACCUM) {
  constexpr int J = Dim<NS>::J;
  constexpr int RT = 16;  // tokens per LDS record stage
  constexpr int UB = 4;   // tokens whose global loads are issued together
  constexpr int JP = (J + 1 + 3) / 4 * 4;  // record row padded to 16 bytes (128-bit LDS reads)
  __shared__ __align__(16) float srec[RT][JP];
  const int64_t K = NS * C;
  const int64_t k = (int64_t)blockIdx.x * kGBwdK + threadIdx.x;
  const bool kv = k < K;
  float w[J], dw[J];
#pragma unroll
  for (int j = 0; j < J; ++j) {
    w[j] = kv ? W[k * J + j] : 0.f;
    dw[j] = 0.f;
  }
  const int64_t t0 = (int64_t)blockIdx.y * TB;
  const int64_t t1 = min(t0 + TB, N);
  for (int64_t ts = t0; ts < t1; ts += RT) {
    const int nt = (int)min((int64_t)RT, t1 - ts);
    __syncthreads();
    for (int idx = threadIdx.x; idx < nt * (J + 1); idx += blockDim.x) {
      const int u = idx / (J + 1), j = idx % (J + 1);
      srec[u][j] = rec[(ts + u) * Dim<NS>::RS + (j < J ? j : Dim<NS>::RC)];
    }
    __syncthreads();
    if (kv) {
      for (int u0 = 0; u0 < nt; u0 += UB) {
        // loads of UB tokens first (a token past the block re-reads the last one; it is not stored)
        float xv[UB], tv[UB];
#pragma unroll
        for (int q = 0; q < UB; ++q) {
          const int64_t t = ts + min(u0 + q, nt - 1);
          xv[q] = Ld<T>::one(X + t * K + k);
          tv[q] = (term ? term[t * K + k] : 0.f) + (ACCUM ? Ld<T>::one(dX + t * K + k) : 0.f);
        }
#pragma unroll
        for (int q = 0; q < UB; ++q) {
          const int u = u0 + q;
          if (u < nt) {
            float s0 = 0.f, s1 = 0.f;  // two chains for the J-long dot product
#pragma unroll
            for (int j = 0; j < J; ++j) {
              if (j & 1) s1 += srec[u][j] * w[j];
              else s0 += srec[u][j] * w[j];
              if (DW) dw[j] += xv[q] * srec[u][j];
            }
            st_one<T>(dX + (ts + u) * K + k, tv[q] + (s0 + s1) + srec[u][J] * xv[q]);
          }
        }
      }
    }
  }
  if (DW && kv) {
#pragma unroll
    for (int j = 0; j < J; ++j) dwpart[((int64_t)blockIdx.y * K + k) * J + j] = dw[j];
  }
}

// ------------------------------------------------------------------ MFMA dX / dW kernel (bf16 activations, n <= 3)
// The same dX and dW as the VALU kernel above, with the aggregate and
// h_post_bda residual terms formed in place (no fp32 term workspace):
//   dX[t][j][c] = (dX_in) + dp[t] . W[k] + c_rms[t] x[t][j][c] + H_pre[t][j] g[t][c]
//                 + sum_i H_res[t][j][i] G[t][i][c],      k = j C + c
//   dW[k][.]   += x[t][k] dp[t][.]
// Workgroup = 8 waves on one token block and one tile of CW channels of all
// NS streams (so the G tile, needed by every output stream, is loaded once),
// walked in 32-token sub-tiles through a 3-stage LDS ring:
//  * waves 4..7 (loaders) fill each stage with global_load_lds_dwordx4 two
//    sub-tiles ahead: the X tile, the G tile, the g tile and the sub-tile's
//    32 backward records; then dW = x^T dp on bf16 MFMA (32x32x16), A = 16
//    tokens of a k column of X (exact in bf16), B = dp split exactly into
//    three bf16 terms (8 + 8 + 8 significant bits);
//  * waves 0..3 own 32-k column blocks: dp W^T on fp32 MFMA (32x32x2), W's
//    rows held in registers (a lane half holds j = h JC + c), the 32 x 32
//    accumulator transposed through a private LDS area, then the epilogue
//    with 16-byte row pieces and 16-byte stores; H_pre, H_res and dX_in rows
//    are prefetched one sub-tile ahead.
// fp32 MFMA keeps W's rows in registers (J / 2 values per lane per block,
// where the six three-term bf16 products would need 3 J).  n >= 5 uses the
// two kernels further below.
// Synchronisation as in the n = 4 kernel: loaders issue no other global
// memory operation in the loop (exact vmcnt), dX waves never issue DMA, one
// barrier per sub-tile.

// 32-channel blocks per stream in a channel tile of the MFMA dX/dW kernel
// (n <= 3): as wide as the 3-stage ring fits in LDS.
constexpr int gmf_cb(int n) { return n <= 2 ? 4 : n == 3 ? 2 : 1; }
constexpr int64_t gmf_cw(int n) { return 32 * gmf_cb(n); }

template <int NS> struct GMf {
  static constexpr int J = Dim<NS>::J, JT = Dim<NS>::JT, JC = Dim<NS>::JC, RC = Dim<NS>::RC, RS = Dim<NS>::RS;
  static constexpr int CB = gmf_cb(NS);                     // 32-channel blocks per stream in a tile
  static constexpr int CW = 32 * CB;                        // channels of a tile
  static constexpr int PW = CW / 8;                         // 16-byte pieces of a tile row
  static constexpr int NB = NS * CB;                        // 32-k column blocks of a tile
  static constexpr int MB = (NB + 3) / 4;                   // blocks per wave (round robin over 4 waves)
  static constexpr int XB = NS * 32 * CW * 2;               // bytes of the X tile (and of the G tile)
  static constexpr int GB = 32 * CW * 2;                    // bytes of the g tile
  static constexpr int RB = (RS * 32 * 4 + 1023) / 1024 * 1024;  // record tile, whole 1 KB copies
  static constexpr int AS = 40;                             // row stride (floats) of a wave's accumulator tile
  static constexpr int ACC = 4 * 32 * AS * 4;               // the four dX waves' accumulator tiles
  static_assert(NB >= 4, "every dX wave owns a block (its first block waits for the prefetched rows)");
  static_assert(3 * (2 * XB + GB + RB) + ACC <= 160 * 1024, "LDS of one workgroup");
  // Byte offset of 16-byte piece `slot` of row (stream j, token t) in an X
  // or G tile ([stream][token][CW], j = 0 for the g tile).  Tokens t and
  // t + 8, which one column read takes together, land on different banks:
  // rows of 64 bytes are permuted (t ^ bit 3 of t), wider rows have their
  // pieces rotated by half a row.  The map is its own inverse in t.
  static __device__ __forceinline__ int off(int j, int t, int slot) {
    const int b3 = (t >> 3) & 1;
    if (PW == 4) return ((j * 32 + (t ^ b3)) * PW + slot) * 16;
    return ((j * 32 + t) * PW + (slot ^ (b3 * (PW / 2)))) * 16;
  }
};

// flags: bit 0 g given, bit 1 h_post_bda term (G, H_res), bit 2 accumulate into dX
template <int NS, bool DW>
__global__ __launch_bounds__(512) void gproj_bwd_mfma_kernel(
    const bf16_t *__restrict__ X, const float *__restrict__ W, const float *__restrict__ rec,
    const float *__restrict__ Hpre, const bf16_t *__restrict__ gr, const bf16_t *__restrict__ Gp,
    const float *__restrict__ Hres, bf16_t *__restrict__ dX, float *__restrict__ dwpart, int64_t N, int64_t C,
    int64_t tbsz, int64_t ntb, int flags) {
  using M = GMf<NS>;
  constexpr int J = M::J, JT = M::JT, JC = M::JC, RC = M::RC, RS = M::RS, CB = M::CB, CW = M::CW, PW = M::PW;
  constexpr int NB = M::NB, MB = M::MB;
  extern __shared__ __attribute__((aligned(16))) char glds[];
  const bool has_g = flags & 1, post = (flags >> 1) & 1, accum = (flags >> 2) & 1;
  const int64_t K = (int64_t)NS * C;
  const int64_t nct = (C + CW - 1) / CW;
  // XCD-contiguous tile order (as the n = 4 kernel): XCD b % 8 walks tiles
  // [x per, (x + 1) per) in order, neighbouring channel tiles of one block
  const int64_t T = nct * ntb, per = (T + 7) / 8;
  const int64_t tile = (int64_t)(blockIdx.x % 8) * per + blockIdx.x / 8;
  if (tile >= T) return;  // grid padding to a multiple of 8 (whole workgroup)
  // token blocks from the last down: the dH_pre pass before read X and g in
  // token order, so the first blocks here may still sit in the Infinity Cache
  const int64_t tb = ntb - 1 - tile / nct;
  const int64_t c0 = (tile % nct) * CW;
  const int64_t t_begin = min(N, tb * tbsz);
  const int64_t t_end = min(N, t_begin + tbsz);
  const int nsub = (int)((t_end - t_begin + 31) / 32);

  // stage layout: X tile, G tile (post), g tile (has_g), records
  const int oG = M::XB, og = oG + (post ? M::XB : 0), oR = og + (has_g ? M::GB : 0), SB = oR + M::RB;
  const int QX = M::XB / 1024, QG = post ? QX : 0, Qg = has_g ? M::GB / 1024 : 0, QR = M::RB / 1024;
  const int Q = QX + QG + Qg + QR;

  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int col = lane & 31, h = lane >> 5;
  const bool loader = wave >= 4;
  const int w4 = wave & 3;

  // ---- loaders: copy q of a stage (lane -> 16 bytes)
  auto issue = [&](int i) {
    char *st = glds + (i % 3) * SB;
    const int64_t t0 = t_begin + 32 * (int64_t)i;
    for (int q = w4; q < Q; q += 4) {
      if (q < QX + QG + Qg) {
        const bool is_g = q >= QX + QG;
        const int qq = is_g ? q - QX - QG : q < QX ? q : q - QX;
        const int p16 = qq * 64 + lane;  // 16-byte piece index inside the tile
        const int row = p16 / PW, ps = p16 % PW;
        const int j = row / 32, tp = row % 32;
        const int b3 = (tp >> 3) & 1;
        const int t = PW == 4 ? tp ^ b3 : tp;
        const int slot = PW == 4 ? ps : ps ^ (b3 * (PW / 2));
        const int64_t tt = min(t0 + t, N - 1);  // rows past N re-read row N-1 (never stored, dW-masked)
        const int64_t ch = c0 + 8 * slot < C ? c0 + 8 * slot : c0;  // pieces past C: a real channel
        const bf16_t *src = is_g ? gr + tt * C + ch : (q < QX ? X : Gp) + (tt * NS + j) * C + ch;
        char *dst = st + (is_g ? og : q < QX ? 0 : oG) + qq * 1024;
        dma16(src, dst);
      } else {
        // records are contiguous; the workspace holds them up to the 32-token padding plus 1 KB
        const int qq = q - QX - QG - Qg;
        dma16(reinterpret_cast<const char *>(rec + t0 * RS) + qq * 1024 + lane * 16, st + oR + qq * 1024);
      }
    }
  };

  // ---- dX waves: blocks b = w4 + 4 bi; stream j = b / CB, channels c0 + 32 (b % CB) + [0, 32)
  float wf[MB][JC];
  if (!loader) {
#pragma unroll
    for (int bi = 0; bi < MB; ++bi) {
      const int b = w4 + 4 * bi;
      const int64_t c = c0 + 32 * (b % CB) + col;
      const bool ok = b < NB && c < C;
      const float *wr = W + ((int64_t)(b / CB) * C + c) * J;
#pragma unroll
      for (int e = 0; e < JC; ++e) {
        const int jj = h * JC + e;
        wf[bi][e] = ok && jj < J ? wr[jj] : 0.f;
      }
    }
  }
  // prefetched per sub-tile: rows er and er + 16 of each block
  const int er = lane >> 2, pk = lane & 3;
  float hp[MB][2], hr[MB][2][NS];
  gu32x4 din[MB][2];
  auto prefetch = [&](int i) {
    const int64_t t0 = t_begin + 32 * (int64_t)i;
#pragma unroll
    for (int bi = 0; bi < MB; ++bi) {
      const int b = w4 + 4 * bi, j = b / CB;
      const int64_t ch = c0 + 32 * (b % CB) + 8 * pk;
#pragma unroll
      for (int rr = 0; rr < 2; ++rr) {
        const int64_t t = t0 + er + 16 * rr;
        const bool v = b < NB && t < N;
        hp[bi][rr] = v && has_g ? Hpre[t * NS + j] : 0.f;
#pragma unroll
        for (int e = 0; e < NS; ++e) hr[bi][rr][e] = v && post ? Hres[(t * NS + j) * NS + e] : 0.f;
        din[bi][rr] = v && accum && ch < C ? *reinterpret_cast<const gu32x4 *>(dX + (t * NS + j) * C + ch)
                                           : gu32x4{0u, 0u, 0u, 0u};
      }
    }
  };

  gf32x16 accW[MB][JT];
#pragma unroll
  for (int bi = 0; bi < MB; ++bi)
#pragma unroll
    for (int u = 0; u < JT; ++u)
#pragma unroll
      for (int r = 0; r < 16; ++r) accW[bi][u][r] = 0.f;

  if (loader) {
    const int nq = (Q - w4 + 3) / 4;  // this wave's copies per stage
    if (nsub > 0) issue(0);
    if (nsub > 1) issue(1);
    for (int i = 0; i < nsub; ++i) {
      if (i + 1 < nsub) wait_vmcnt_le(nq); else wait_vmcnt<0>();
      lds_barrier();
      if (i + 2 < nsub) issue(i + 2);
      if (DW) {
        const char *st = glds + (i % 3) * SB;
        const float *rt = reinterpret_cast<const float *>(st + oR);
        const int64_t t0 = t_begin + 32 * (int64_t)i;
        // per 16-token half s: B = the three bf16 terms of dp[token][j],
        // j = 32 u + col, for the 8 tokens 16 s + 8 h + p of the lane (tokens
        // past N give 0); A = x[token][kk] of the same tokens for each block
#pragma unroll
        for (int s = 0; s < 2; ++s) {
          gu32x4 bfr[JT][3];
#pragma unroll
          for (int u = 0; u < JT; ++u) {
            uint32_t tw[3][4];
#pragma unroll
            for (int p = 0; p < 4; ++p) {
              float v2[2];
#pragma unroll
              for (int e = 0; e < 2; ++e) {
                const int tok = 16 * s + 8 * h + 2 * p + e;
                const int jj = 32 * u + col;
                v2[e] = (jj < J && t0 + tok < N) ? rt[tok * RS + jj] : 0.f;
              }
              float th[2], tm[2], tl[2];
#pragma unroll
              for (int e = 0; e < 2; ++e) {
                th[e] = (float)(__bf16)v2[e];
                const float r1 = v2[e] - th[e];
                tm[e] = (float)(__bf16)r1;
                tl[e] = r1 - tm[e];
              }
              tw[0][p] = pack_bf16x2(th[0], th[1]);
              tw[1][p] = pack_bf16x2(tm[0], tm[1]);
              tw[2][p] = pack_bf16x2(tl[0], tl[1]);
            }
#pragma unroll
            for (int m = 0; m < 3; ++m) bfr[u][m] = gu32x4{tw[m][0], tw[m][1], tw[m][2], tw[m][3]};
          }
#pragma unroll
          for (int bi = 0; bi < MB; ++bi) {
            const int b = w4 + 4 * bi;
            if (b >= NB) continue;
            const int j = b / CB, kk = 32 * (b % CB) + col;  // column of the tile
            uint32_t w4v[4];
#pragma unroll
            for (int p = 0; p < 4; ++p) {
              const int tr0 = 16 * s + 8 * h + 2 * p;
              const uint32_t lo = *reinterpret_cast<const uint16_t *>(st + M::off(j, tr0, kk >> 3) + 2 * (kk & 7));
              const uint32_t hi =
                  *reinterpret_cast<const uint16_t *>(st + M::off(j, tr0 + 1, kk >> 3) + 2 * (kk & 7));
              w4v[p] = lo | (hi << 16);
            }
            const gu32x4 xa = gu32x4{w4v[0], w4v[1], w4v[2], w4v[3]};
#pragma unroll
            for (int m = 0; m < 3; ++m)
#pragma unroll
              for (int u = 0; u < JT; ++u)
                accW[bi][u] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(gbf16x8, xa),
                                                                      __builtin_bit_cast(gbf16x8, bfr[u][m]),
                                                                      accW[bi][u], 0, 0, 0);
          }
        }
      }
    }
  } else {
    float *acc_t = reinterpret_cast<float *>(glds + 3 * SB) + w4 * 32 * M::AS;
    wait_vmcnt<0>();  // W in registers: only the prefetches are pending inside the loop
    prefetch(0);
    for (int i = 0; i < nsub; ++i) {
      lds_barrier();
      const char *st = glds + (i % 3) * SB;
      const float *rt = reinterpret_cast<const float *>(st + oR);
      const int64_t t0 = t_begin + 32 * (int64_t)i;
#pragma unroll
      for (int bi = 0; bi < MB; ++bi) {
        const int b = w4 + 4 * bi;
        if (b >= NB) continue;
        const int j = b / CB, cb = b % CB;
        // dp W^T: A = dp[token col][h JC + e], B = W[k col][h JC + e]
        gf32x16 acc;
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[r] = 0.f;
        const float *ar = rt + col * RS + h * JC;
#pragma unroll
        for (int e4 = 0; e4 < JC / 4; ++e4) {
          const float4 a4 = *reinterpret_cast<const float4 *>(ar + 4 * e4);
          acc = __builtin_amdgcn_mfma_f32_32x32x2f32(a4.x, wf[bi][4 * e4], acc, 0, 0, 0);
          acc = __builtin_amdgcn_mfma_f32_32x32x2f32(a4.y, wf[bi][4 * e4 + 1], acc, 0, 0, 0);
          acc = __builtin_amdgcn_mfma_f32_32x32x2f32(a4.z, wf[bi][4 * e4 + 2], acc, 0, 0, 0);
          acc = __builtin_amdgcn_mfma_f32_32x32x2f32(a4.w, wf[bi][4 * e4 + 3], acc, 0, 0, 0);
        }
        if (bi == 0) {
          // the prefetched rows, waited for once, after the first MFMAs
          __builtin_amdgcn_sched_barrier(0);
          wait_vmcnt<0>();
        }
#pragma unroll
        for (int r = 0; r < 16; ++r) acc_t[(8 * (r >> 2) + 4 * h + (r & 3)) * M::AS + col] = acc[r];
        wave_lds_sync();
#pragma unroll
        for (int rr = 0; rr < 2; ++rr) {
          const int row = er + 16 * rr;
          const int64_t t = t0 + row;
          const int64_t ch = c0 + 32 * cb + 8 * pk;
          if (!(t < N && ch < C)) continue;
          const int slot = 4 * cb + pk;
          const float4 a0 = *reinterpret_cast<const float4 *>(&acc_t[row * M::AS + 8 * pk]);
          const float4 a1 = *reinterpret_cast<const float4 *>(&acc_t[row * M::AS + 8 * pk + 4]);
          float o[8] = {a0.x, a0.y, a0.z, a0.w, a1.x, a1.y, a1.z, a1.w};
          const float crms = rt[row * RS + RC];
          const gu32x4 xv = *reinterpret_cast<const gu32x4 *>(st + M::off(j, row, slot));
          const uint32_t xw[4] = {xv.x, xv.y, xv.z, xv.w};
#pragma unroll
          for (int p = 0; p < 4; ++p) {
            o[2 * p] += crms * bf16_lo(xw[p]);
            o[2 * p + 1] += crms * bf16_hi(xw[p]);
          }
          if (has_g) {
            const gu32x4 gv = *reinterpret_cast<const gu32x4 *>(st + og + M::off(0, row, slot));
            const uint32_t gw[4] = {gv.x, gv.y, gv.z, gv.w};
            const float hv = hp[bi][rr];
#pragma unroll
            for (int p = 0; p < 4; ++p) {
              o[2 * p] += hv * bf16_lo(gw[p]);
              o[2 * p + 1] += hv * bf16_hi(gw[p]);
            }
          }
          if (post) {  // sum_i H_res[t][j][i] G[t][i], i in order
            float s8[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int e = 0; e < NS; ++e) {
              const gu32x4 v = *reinterpret_cast<const gu32x4 *>(st + oG + M::off(e, row, slot));
              const uint32_t vw[4] = {v.x, v.y, v.z, v.w};
              const float hv = hr[bi][rr][e];
#pragma unroll
              for (int p = 0; p < 4; ++p) {
                s8[2 * p] += hv * bf16_lo(vw[p]);
                s8[2 * p + 1] += hv * bf16_hi(vw[p]);
              }
            }
#pragma unroll
            for (int e = 0; e < 8; ++e) o[e] += s8[e];
          }
          if (accum) {
            const uint32_t dw4[4] = {din[bi][rr].x, din[bi][rr].y, din[bi][rr].z, din[bi][rr].w};
#pragma unroll
            for (int p = 0; p < 4; ++p) {
              o[2 * p] += bf16_lo(dw4[p]);
              o[2 * p + 1] += bf16_hi(dw4[p]);
            }
          }
          uint4 ow;
          ow.x = pack_bf16x2(o[0], o[1]);
          ow.y = pack_bf16x2(o[2], o[3]);
          ow.z = pack_bf16x2(o[4], o[5]);
          ow.w = pack_bf16x2(o[6], o[7]);
          *reinterpret_cast<uint4 *>(dX + (t * NS + j) * C + ch) = ow;
        }
        wave_lds_sync();  // the accumulator tile's reads precede the next block's writes
      }
      if (i + 1 < nsub) prefetch(i + 1);
    }
  }
  if (DW && loader) {
#pragma unroll
    for (int bi = 0; bi < MB; ++bi) {
      const int b = w4 + 4 * bi;
      if (b >= NB) continue;
      const int64_t kb = (int64_t)(b / CB) * C + c0 + 32 * (b % CB);  // k of the block's first column
      const int64_t cb0 = c0 + 32 * (b % CB);
#pragma unroll
      for (int u = 0; u < JT; ++u) {
        const int jj = 32 * u + col;
        if (jj >= J) continue;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int e = 8 * (r >> 2) + 4 * h + (r & 3);
          if (cb0 + e < C) dwpart[(tb * K + kb + e) * J + jj] = accW[bi][u][r];
        }
      }
    }
  }
}

// ------------------------------------------------------------------ dX and dW as two kernels (bf16, n >= 5)
// For n >= 5 W's rows and the dW accumulators of a channel tile do not both
// fit on chip beside a ring at more than 32 channels (64-byte row pieces, one
// DRAM page opened per 64 bytes).  There dW = x^T dp runs alone on tiles of
// 256 consecutive k (512-byte pieces), and dX, freed of the accumulators, on
// tiles of 64 channels of all n streams with eight dX waves.
typedef __attribute__((ext_vector_type(4))) float gf32x4;

// dp split once per call into its three exact bf16 terms, transposed per
// 32-token sub-tile: dpT[sub][term][column (32 JT, zero past J)][32 tokens]
// (zero for tokens past N), so a dW B fragment (8 tokens of one column) is
// one 16-byte read.  In each column's 64-byte row the 8-token group p sits in
// slot p ^ ((column >> 2) & 3): the 32 columns one read takes then spread
// over the banks (rows 64 bytes apart would put 8 of them on each bank).
// Thread = (sub-tile, column, token), tokens fastest.
template <int NS>
__global__ __launch_bounds__(256) void gsplit_dp_kernel(const float *__restrict__ rec, bf16_t *__restrict__ dpT,
                                                       int64_t N) {
  constexpr int J = Dim<NS>::J, JT = Dim<NS>::JT, RS = Dim<NS>::RS;
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t nsub = (N + 31) / 32;
  if (i >= nsub * 32 * JT * 32) return;
  const int tok = (int)(i & 31), jj = (int)((i >> 5) % (32 * JT));
  const int64_t sb = (i >> 5) / (32 * JT);
  const int64_t t = sb * 32 + tok;
  const float v = (t < N && jj < J) ? rec[t * RS + jj] : 0.f;
  const float hi = (float)(__bf16)v, r1 = v - hi, mid = (float)(__bf16)r1, lo = r1 - mid;
  const float terms[3] = {hi, mid, lo};
#pragma unroll
  for (int m = 0; m < 3; ++m) {
    const __bf16 b = (__bf16)terms[m];
    dpT[((sb * 3 + m) * 32 * JT + jj) * 32 + 8 * ((tok >> 3) ^ ((jj >> 2) & 3)) + (tok & 7)] =
        __builtin_bit_cast(uint16_t, b);
  }
}

// dW kernel: eight waves on one token block and 256 consecutive k, walked in
// 32-token sub-tiles through a 2-stage ring that all eight waves fill with
// global_load_lds_dwordx4 (no other global memory operation in the loop):
// the X tile (512-byte row pieces) and the sub-tile's block of dpT.  Two
// stages (68 KB at n = 8) let two workgroups share a CU: 4% faster for the
// n = 8 pre backward than three stages and one workgroup.  Wave w owns the 32 k at 32 w: bf16 MFMA
// (32x32x16), A = 8 tokens of a k column of the X tile (exact in bf16), B =
// one bf16 term of dp for the same 8 tokens (one 16-byte read).  Piece p of
// X row t sits in slot p ^ (4 ((t >> 3) & 1)), so the two 8-token halves of
// a column read fall on different banks.
template <int NS> struct GDw {
  static constexpr int JT = Dim<NS>::JT;
  static constexpr int XB = 32 * 512;           // X tile: 32 tokens x 256 k
  static constexpr int DB = 3 * 32 * JT * 64;   // dpT block of one sub-tile
  static constexpr int SB = XB + DB;
  static constexpr int STG = 2;
  static_assert(DB % 1024 == 0, "whole 1 KB copies");
  static __device__ __forceinline__ int off(int t, int slot) { return (t * 32 + (slot ^ (4 * ((t >> 3) & 1)))) * 16; }
};

template <int NS>
__global__ __launch_bounds__(512) void gproj_dw_mfma_kernel(const bf16_t *__restrict__ X,
                                                           const bf16_t *__restrict__ dpT,
                                                           float *__restrict__ dwpart, int64_t N, int64_t K,
                                                           int64_t tbsz, int64_t ntb) {
  using M = GDw<NS>;
  constexpr int J = Dim<NS>::J, JT = Dim<NS>::JT;
  extern __shared__ __attribute__((aligned(16))) char gdl[];
  const int64_t nkt = (K + 255) / 256;
  const int64_t T = nkt * ntb, per = (T + 7) / 8;
  const int64_t tile = (int64_t)(blockIdx.x % 8) * per + blockIdx.x / 8;  // XCD-contiguous order
  if (tile >= T) return;  // grid padding to a multiple of 8 (whole workgroup)
  const int64_t tb = tile / nkt;
  const int64_t k0 = (tile % nkt) * 256;
  const int64_t t_begin = min(N, tb * tbsz), t_end = min(N, t_begin + tbsz);
  const int nsub = (int)((t_end - t_begin + 31) / 32);
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63, col = lane & 31, h = lane >> 5;
  constexpr int QX = M::XB / 1024, QD = M::DB / 1024, Q = QX + QD;

  auto issue = [&](int i) {
    char *st = gdl + (i % M::STG) * M::SB;
    const int64_t t0 = t_begin + 32 * (int64_t)i;  // a multiple of 32
    for (int q = wave; q < Q; q += 8) {
      if (q < QX) {
        const int t = 2 * q + (lane >> 5), slot = lane & 31;
        const int p = slot ^ (4 * ((t >> 3) & 1));
        const int64_t tt = min(t0 + t, N - 1);  // rows past N re-read row N-1 (their dp terms are 0)
        const int64_t k = k0 + 8 * p < K ? k0 + 8 * p : k0;
        dma16(X + tt * K + k, st + q * 1024);
      } else {
        const int qq = q - QX;
        dma16(reinterpret_cast<const char *>(dpT) + (t0 / 32) * M::DB + qq * 1024 + lane * 16,
               st + M::XB + qq * 1024);
      }
    }
  };

  gf32x16 accW[JT];
#pragma unroll
  for (int u = 0; u < JT; ++u)
#pragma unroll
    for (int r = 0; r < 16; ++r) accW[u][r] = 0.f;
  const int kk = 32 * wave + col;  // this lane's column of the tile
  // two stages: the slot refilled after the barrier of sub-tile i was read
  // in sub-tile i - 1, so only sub-tile i's copies are outstanding at its wait
  if (nsub > 0) issue(0);
  for (int i = 0; i < nsub; ++i) {
    wait_vmcnt<0>();
    lds_barrier();
    if (i + 1 < nsub) issue(i + 1);
    const char *st = gdl + (i % M::STG) * M::SB;
    const char *dt = st + M::XB;
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      uint32_t w4v[4];
#pragma unroll
      for (int p = 0; p < 4; ++p) {
        const int tr0 = 16 * s + 8 * h + 2 * p;
        const uint32_t lo = *reinterpret_cast<const uint16_t *>(st + M::off(tr0, kk >> 3) + 2 * (kk & 7));
        const uint32_t hi = *reinterpret_cast<const uint16_t *>(st + M::off(tr0 + 1, kk >> 3) + 2 * (kk & 7));
        w4v[p] = lo | (hi << 16);
      }
      const gu32x4 xa = gu32x4{w4v[0], w4v[1], w4v[2], w4v[3]};
#pragma unroll
      for (int m = 0; m < 3; ++m)
#pragma unroll
        for (int u = 0; u < JT; ++u) {
          const int slot = (2 * s + h) ^ ((col >> 2) & 3);  // token group 2s + h of column 32u + col
          const gu32x4 bw = *reinterpret_cast<const gu32x4 *>(dt + ((m * 32 * JT + 32 * u + col) * 32 + 8 * slot) * 2);
          accW[u] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(gbf16x8, xa),
                                                            __builtin_bit_cast(gbf16x8, bw), accW[u], 0, 0, 0);
        }
    }
  }
  const int64_t kb = k0 + 32 * wave;
#pragma unroll
  for (int u = 0; u < JT; ++u) {
    const int jj = 32 * u + col;
    if (jj >= J) continue;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int64_t k = kb + 8 * (r >> 2) + 4 * h + (r & 3);
      if (k < K) dwpart[(tb * K + k) * J + jj] = accW[u][r];
    }
  }
}

// dX kernel: 12 waves on one token block and one tile of 64 channels of all
// NS streams, walked in 16-token sub-tiles through a 3-stage LDS ring:
//  * waves 8..11 (loaders) fill each stage with global_load_lds_dwordx4 two
//    sub-tiles ahead: X and G tiles [stream][token][64 channels], the g tile
//    and the 16 records (piece p of row t in slot p ^ (t & 7));
//  * wave w < NS owns stream w: dp W^T on fp32 MFMA (16x16x4) over four
//    16-column blocks, W's rows in registers (lane group g holds
//    j = g JQ + c), the 16 x 64 result transposed through a private LDS
//    area, then the epilogue with 16-byte row pieces (eight lanes store one
//    token's 128-byte row piece); H_pre, H_res and dX_in rows prefetched one
//    sub-tile ahead.  Waves NS..7 only keep the barrier sequence.
template <int NS> struct GDx {
  static constexpr int J = Dim<NS>::J, JQ = Dim<NS>::JQ, RC = Dim<NS>::RC, RS = Dim<NS>::RS;
  static constexpr int XB = NS * 16 * 128;                        // X (and G) tile
  static constexpr int GB = 16 * 128;                             // g tile
  static constexpr int RB = (RS * 16 * 4 + 1023) / 1024 * 1024;   // records, whole 1 KB copies
  static constexpr int AS = 68;                                   // accumulator tile row stride (floats)
  static constexpr int ACC = 8 * 16 * AS * 4;
  static_assert(NS >= 5 && NS <= 8, "the split kernels serve n = 5..8");
  static_assert(3 * (2 * XB + GB + RB) + ACC <= 160 * 1024, "LDS of one workgroup");
  static __device__ __forceinline__ int off(int j, int t, int slot) {
    return ((j * 16 + t) * 8 + (slot ^ (t & 7))) * 16;
  }
};

// flags: bit 0 g given, bit 1 h_post_bda term (G, H_res), bit 2 accumulate into dX
template <int NS>
__global__ __launch_bounds__(768) void gproj_dx16_mfma_kernel(
    const bf16_t *__restrict__ X, const float *__restrict__ W, const float *__restrict__ rec,
    const float *__restrict__ Hpre, const bf16_t *__restrict__ gr, const bf16_t *__restrict__ Gp,
    const float *__restrict__ Hres, bf16_t *__restrict__ dX, int64_t N, int64_t C, int64_t tbsz, int64_t ntb,
    int flags) {
  using M = GDx<NS>;
  constexpr int J = M::J, JQ = M::JQ, RC = M::RC, RS = M::RS;
  extern __shared__ __attribute__((aligned(16))) char gxl[];
  const bool has_g = flags & 1, post = (flags >> 1) & 1, accum = (flags >> 2) & 1;
  const int64_t nct = (C + 63) / 64;
  const int64_t T = nct * ntb, per = (T + 7) / 8;
  const int64_t tile = (int64_t)(blockIdx.x % 8) * per + blockIdx.x / 8;  // XCD-contiguous order
  if (tile >= T) return;  // grid padding to a multiple of 8 (whole workgroup)
  const int64_t tb = tile / nct;
  const int64_t c0 = (tile % nct) * 64;
  const int64_t t_begin = min(N, tb * tbsz), t_end = min(N, t_begin + tbsz);
  const int nsub = (int)((t_end - t_begin + 15) / 16);

  const int oG = M::XB, og = oG + (post ? M::XB : 0), oR = og + (has_g ? M::GB : 0), SB = oR + M::RB;
  const int QX = M::XB / 1024, QG = post ? QX : 0, Qg = has_g ? M::GB / 1024 : 0, QR = M::RB / 1024;
  const int Q = QX + QG + Qg + QR;

  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const bool loader = wave >= 8;
  const int lw = wave - 8;

  auto issue = [&](int i) {
    char *st = gxl + (i % 3) * SB;
    const int64_t t0 = t_begin + 16 * (int64_t)i;
    for (int q = lw; q < Q; q += 4) {
      if (q < QX + QG + Qg) {
        const bool is_g = q >= QX + QG;
        const int qq = is_g ? q - QX - QG : q < QX ? q : q - QX;
        const int row = 8 * qq + (lane >> 3);  // (stream, token) row of the tile
        const int j = row / 16, t = row % 16;
        const int p = (lane & 7) ^ (t & 7);
        const int64_t tt = min(t0 + t, N - 1);  // rows past N re-read row N-1 (never stored)
        const int64_t ch = c0 + 8 * p < C ? c0 + 8 * p : c0;  // pieces past C: a real channel
        const bf16_t *src = is_g ? gr + tt * C + ch : (q < QX ? X : Gp) + (tt * NS + j) * C + ch;
        dma16(src, st + (is_g ? og : q < QX ? 0 : oG) + qq * 1024);
      } else {
        // records: contiguous, padded to whole 32-token sub-tiles plus 1 KB
        const int qq = q - QX - QG - Qg;
        dma16(reinterpret_cast<const char *>(rec + t0 * RS) + qq * 1024 + lane * 16, st + oR + qq * 1024);
      }
    }
  };

  // ---- dX wave w < NS: stream j = w, columns c0 + 16 bi + (lane & 15)
  const int j = wave;
  const bool active = !loader && wave < NS;
  const int gq = lane >> 4, cl = lane & 15;
  float wf[4][JQ];
  if (active) {
#pragma unroll
    for (int bi = 0; bi < 4; ++bi) {
      const int64_t c = c0 + 16 * bi + cl;
      const float *wr = W + ((int64_t)j * C + c) * J;
#pragma unroll
      for (int e = 0; e < JQ; ++e) {
        const int jj = gq * JQ + e;
        wf[bi][e] = c < C && jj < J ? wr[jj] : 0.f;
      }
    }
  }
  const int er = lane >> 3, pk = lane & 7;  // epilogue: rows er and er + 8, channels 8 pk .. + 8
  float hp[2], hr[2][NS];
  gu32x4 din[2];
  auto prefetch = [&](int i) {
    const int64_t t0 = t_begin + 16 * (int64_t)i;
    const int64_t ch = c0 + 8 * pk;
#pragma unroll
    for (int rr = 0; rr < 2; ++rr) {
      const int64_t t = t0 + er + 8 * rr;
      const bool v = t < N;
      hp[rr] = v && has_g ? Hpre[t * NS + j] : 0.f;
#pragma unroll
      for (int e = 0; e < NS; ++e) hr[rr][e] = v && post ? Hres[(t * NS + j) * NS + e] : 0.f;
      din[rr] = v && accum && ch < C ? *reinterpret_cast<const gu32x4 *>(dX + (t * NS + j) * C + ch)
                                     : gu32x4{0u, 0u, 0u, 0u};
    }
  };

  if (loader) {
    const int nq = (Q - lw + 3) / 4;  // this wave's copies per stage
    if (nsub > 0) issue(0);
    if (nsub > 1) issue(1);
    for (int i = 0; i < nsub; ++i) {
      if (i + 1 < nsub) wait_vmcnt_le(nq); else wait_vmcnt<0>();
      lds_barrier();
      if (i + 2 < nsub) issue(i + 2);
    }
  } else if (!active) {
    for (int i = 0; i < nsub; ++i) lds_barrier();
  } else {
    float *acc_t = reinterpret_cast<float *>(gxl + 3 * SB) + wave * 16 * M::AS;
    wait_vmcnt<0>();  // W in registers: only the prefetches are pending inside the loop
    prefetch(0);
    for (int i = 0; i < nsub; ++i) {
      lds_barrier();
      const char *st = gxl + (i % 3) * SB;
      const float *rt = reinterpret_cast<const float *>(st + oR);
      const int64_t t0 = t_begin + 16 * (int64_t)i;
      // the four blocks' accumulations interleaved (independent chains), each
      // A value read once for the four blocks
      const float *ar = rt + cl * RS + gq * JQ;
      gf32x4 acc[4];
#pragma unroll
      for (int bi = 0; bi < 4; ++bi) acc[bi] = gf32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int e4 = 0; e4 < JQ / 4; ++e4) {
        const float4 a4 = *reinterpret_cast<const float4 *>(ar + 4 * e4);
        const float av[4] = {a4.x, a4.y, a4.z, a4.w};
#pragma unroll
        for (int e = 0; e < 4; ++e)
#pragma unroll
          for (int bi = 0; bi < 4; ++bi)
            acc[bi] = __builtin_amdgcn_mfma_f32_16x16x4f32(av[e], wf[bi][4 * e4 + e], acc[bi], 0, 0, 0);
      }
      // 16x16 accumulator layout: lane (column cl, group gq), register r holds row 4 gq + r
#pragma unroll
      for (int bi = 0; bi < 4; ++bi)
#pragma unroll
        for (int r = 0; r < 4; ++r) acc_t[(4 * gq + r) * M::AS + 16 * bi + cl] = acc[bi][r];
      // the prefetched rows, waited for once, after the MFMAs
      __builtin_amdgcn_sched_barrier(0);
      wait_vmcnt<0>();
      wave_lds_sync();
#pragma unroll
      for (int rr = 0; rr < 2; ++rr) {
        const int row = er + 8 * rr;
        const int64_t t = t0 + row;
        const int64_t ch = c0 + 8 * pk;
        if (!(t < N && ch < C)) continue;
        const float4 a0 = *reinterpret_cast<const float4 *>(&acc_t[row * M::AS + 8 * pk]);
        const float4 a1 = *reinterpret_cast<const float4 *>(&acc_t[row * M::AS + 8 * pk + 4]);
        float o[8] = {a0.x, a0.y, a0.z, a0.w, a1.x, a1.y, a1.z, a1.w};
        const float crms = rt[row * RS + RC];
        const gu32x4 xv = *reinterpret_cast<const gu32x4 *>(st + M::off(j, row, pk));
        const uint32_t xw[4] = {xv.x, xv.y, xv.z, xv.w};
#pragma unroll
        for (int p = 0; p < 4; ++p) {
          o[2 * p] += crms * bf16_lo(xw[p]);
          o[2 * p + 1] += crms * bf16_hi(xw[p]);
        }
        if (has_g) {
          const gu32x4 gv = *reinterpret_cast<const gu32x4 *>(st + og + M::off(0, row, pk));
          const uint32_t gw[4] = {gv.x, gv.y, gv.z, gv.w};
#pragma unroll
          for (int p = 0; p < 4; ++p) {
            o[2 * p] += hp[rr] * bf16_lo(gw[p]);
            o[2 * p + 1] += hp[rr] * bf16_hi(gw[p]);
          }
        }
        if (post) {  // sum_i H_res[t][j][i] G[t][i], i in order
          float s8[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int e = 0; e < NS; ++e) {
            const gu32x4 v = *reinterpret_cast<const gu32x4 *>(st + oG + M::off(e, row, pk));
            const uint32_t vw[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
            for (int p = 0; p < 4; ++p) {
              s8[2 * p] += hr[rr][e] * bf16_lo(vw[p]);
              s8[2 * p + 1] += hr[rr][e] * bf16_hi(vw[p]);
            }
          }
#pragma unroll
          for (int e = 0; e < 8; ++e) o[e] += s8[e];
        }
        if (accum) {
          const uint32_t dw4[4] = {din[rr].x, din[rr].y, din[rr].z, din[rr].w};
#pragma unroll
          for (int p = 0; p < 4; ++p) {
            o[2 * p] += bf16_lo(dw4[p]);
            o[2 * p + 1] += bf16_hi(dw4[p]);
          }
        }
        uint4 ow;
        ow.x = pack_bf16x2(o[0], o[1]);
        ow.y = pack_bf16x2(o[2], o[3]);
        ow.z = pack_bf16x2(o[4], o[5]);
        ow.w = pack_bf16x2(o[6], o[7]);
        *reinterpret_cast<uint4 *>(dX + (t * NS + j) * C + ch) = ow;
      }
      wave_lds_sync();  // the accumulator tile's reads precede the next sub-tile's writes
      if (i + 1 < nsub) prefetch(i + 1);
    }
  }
}

// dW[k][j] = sum over token blocks in block order.
__global__ __launch_bounds__(256) void gdw_reduce_kernel(const float *__restrict__ part, float *__restrict__ dW,
                                                        int64_t ntb, int64_t KJ) {
  const int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (e >= KJ) return;
  float s = 0.f;
  for (int64_t b = 0; b < ntb; ++b) s += part[b * KJ + e];
  dW[e] = s;
}

// ------------------------------------------------------------------ launch helpers
#define MHC_NS_DISPATCH(NV, ...)                                   \
  switch (NV) {                                                    \
    case 1: { constexpr int NS = 1; __VA_ARGS__; } break;          \
    case 2: { constexpr int NS = 2; __VA_ARGS__; } break;          \
    case 3: { constexpr int NS = 3; __VA_ARGS__; } break;          \
    case 5: { constexpr int NS = 5; __VA_ARGS__; } break;          \
    case 6: { constexpr int NS = 6; __VA_ARGS__; } break;          \
    case 7: { constexpr int NS = 7; __VA_ARGS__; } break;          \
    default: { constexpr int NS = 8; __VA_ARGS__; } break;         \
  }

int gtpb(int64_t C) {
  const int64_t G = C / 8;
  return G <= 64 ? 64 : G <= 128 ? 128 : 256;
}

inline size_t al256(size_t b) { return (b + 255) / 256 * 256; }

struct GBwdLay {
  int64_t ntb, tb;
  size_t rec, prm, dw, dhrow, term, dl, dpt, psum, total;
};

// Backward record stride (floats) for a run-time n: Dim<n>::RS.
static int grec_stride(int n) {
  const int J = n * n + 2 * n, JC = ((J + 1) / 2 + 3) / 4 * 4, JQ = ((J + 3) / 4 + 3) / 4 * 4;
  return ((n >= 5 ? 4 * JQ : 2 * JC) + 1 + 3) / 4 * 4;
}

// f32: the VALU dX kernel, with room for the fp32 residual-gradient terms
// (terms: the fused pre backward).  bf16: the MFMA dX kernel, whose records
// are copied in whole 32-token sub-tiles (padded, plus the last 1 KB copy's
// overhang) and which reads g and G itself.
GBwdLay gbwd_layout(int64_t N, int64_t C, int n, bool terms, bool f32) {
  const int64_t J = (int64_t)n * n + 2 * n, K = (int64_t)n * C;
  GBwdLay L;
  const int64_t by_budget = std::max<int64_t>(1, kGDwBudget / (K * J * 4));
  if (f32) {
    // token blocks of >= 64 tokens, at most kGMaxTB, and dW partials within kGDwBudget
    L.ntb = std::min<int64_t>(std::min<int64_t>(kGMaxTB, by_budget), std::max<int64_t>(1, (N + 63) / 64));
    L.tb = (N + L.ntb - 1) / L.ntb;
  } else {
    // about 512 workgroups (two rounds of one per CU) over the tiles of the
    // kernel that forms dW (channel tiles of all n streams for n <= 3, 256
    // consecutive k for n >= 5), token blocks in whole 32-token sub-tiles
    const int64_t nct = n >= 5 ? (K + 255) / 256 : (C + gmf_cw(n) - 1) / gmf_cw(n);
    L.ntb = std::min<int64_t>(std::min<int64_t>(std::max<int64_t>(1, 512 / nct), by_budget),
                              std::max<int64_t>(1, (N + 31) / 32));
    L.tb = ((N + L.ntb - 1) / L.ntb + 31) / 32 * 32;
  }
  const int RS = grec_stride(n);
  L.rec = f32 ? al256((size_t)N * RS * 4) : al256((size_t)(N + 31) / 32 * 32 * RS * 4 + 1024);
  L.prm = al256((size_t)N * (J + 3) * 4);
  L.dw = al256((size_t)L.ntb * K * J * 4);
  L.dhrow = al256((size_t)N * n * 4);
  L.term = terms && f32 ? al256((size_t)N * K * 4) : 0;
  L.dl = al256((size_t)N * n * n * 4);  // the logits' gradient when the row-per-lane Sinkhorn backward forms it
  // bf16, n >= 5: dp's bf16 terms transposed per 32-token sub-tile for the dW kernel
  L.dpt = !f32 && n >= 5 ? al256((size_t)(N + 31) / 32 * 3 * 32 * ((J + 31) / 32) * 64) : 0;
  L.psum = al256((size_t)kGParts * (J + 3) * 4);  // stage-1 partials of the parameter sums
  L.total = L.rec + L.prm + L.dw + L.dhrow + L.term + L.dl + L.dpt + L.psum;
  return L;
}

}  // namespace

// ------------------------------------------------------------------ public launchers
int saved_stride(int n) {
  const int need = 2 + n * n + 2 * n;
  return need <= 32 ? 32 : (need + 7) / 8 * 8;
}

void glaunch_sinkhorn_fwd(hipStream_t s, int n, int64_t count, const float *L, float *H, int iters, float eps) {
  if (n >= 3) {  // the lanes layout, as the fused finalize
    const unsigned b = (unsigned)((count * sk_group(n) + 255) / 256);
    MHC_NS_DISPATCH(n, hipLaunchKernelGGL((gsinkhorn_fwd_lanes_kernel<NS>), dim3(b), dim3(256), 0, s, count, L, H,
                                          iters, eps));
    return;
  }
  const unsigned b = (unsigned)((count + 63) / 64);
  MHC_NS_DISPATCH(n, hipLaunchKernelGGL((gsinkhorn_fwd_kernel<NS>), dim3(b), dim3(64), 0, s, count, L, H, iters,
                                        eps));
}

void glaunch_sinkhorn_bwd(hipStream_t s, int n, int64_t count, const float *dH, const float *L, float *dL,
                          int iters, float eps) {
  const int lt = sk_lane_threads(n, iters);
  if (lt > 0) {
    const int64_t per_block = lt / sk_group(n);
    const unsigned b = (unsigned)((count + per_block - 1) / per_block);
    MHC_NS_DISPATCH(n, hipLaunchKernelGGL((gsinkhorn_bwd_lanes_kernel<NS>), dim3(b), dim3(lt),
                                          sk_lane_words(n, iters) * sizeof(float) * lt, s, count, dH, L, dL,
                                          iters, eps))
    return;
  }
  const SkBwdGeom g = sk_bwd_geom(n, iters);
  const unsigned b = (unsigned)((count + g.threads - 1) / g.threads);
  if (g.stored)
    MHC_NS_DISPATCH(n, hipLaunchKernelGGL((gsinkhorn_bwd_kernel<NS, true>), dim3(b), dim3(g.threads), g.lds, s,
                                          count, dH, L, dL, iters, eps))
  else
    MHC_NS_DISPATCH(n, hipLaunchKernelGGL((gsinkhorn_bwd_kernel<NS, false>), dim3(b), dim3(g.threads), 0, s,
                                          count, dH, L, dL, iters, eps))
}

void glaunch_h_aggregate_fwd(hipStream_t s, bool f32, int n, int64_t N, int64_t C, const void *X,
                             const float *H_pre, void *out, int64_t hs) {
  const int tpb = gtpb(C);
  if (f32)
    MHC_NS_DISPATCH(n, hipLaunchKernelGGL((gagg_fwd_kernel<float, NS>), dim3((unsigned)N), dim3(tpb), 0, s,
                                          (const float *)X, H_pre, hs, (float *)out, C))
  else
    MHC_NS_DISPATCH(n, hipLaunchKernelGGL((gagg_fwd_kernel<bf16_t, NS>), dim3((unsigned)N), dim3(tpb), 0, s,
                                          (const bf16_t *)X, H_pre, hs, (bf16_t *)out, C))
}

template <typename T>
static void gagg_bwd(hipStream_t s, int n, int64_t N, int64_t C, const void *g, const void *X, const float *H,
                     int64_t hs, void *dX, bool acc, float *rows) {
  MHC_NS_DISPATCH(n, hipLaunchKernelGGL((gagg_bwd_kernel<T, NS>), dim3((unsigned)N), dim3(gtpb(C)), 0, s,
                                        (const T *)g, (const T *)X, H, hs, (T *)dX, rows, C, dX != nullptr,
                                        dX != nullptr && acc));
}

void glaunch_h_aggregate_bwd(hipStream_t s, bool f32, int n, int64_t N, int64_t C, const void *g, const void *X,
                             const float *H_pre, void *dX, bool accumulate, float *dH_pre) {
  if (f32)
    gagg_bwd<float>(s, n, N, C, g, X, H_pre, n, dX, accumulate, dH_pre);
  else
    gagg_bwd<bf16_t>(s, n, N, C, g, X, H_pre, n, dX, accumulate, dH_pre);
}

size_t gh_aggregate_static_bwd_ws(int n, int64_t N) { return (size_t)N * n * 4; }

void glaunch_h_aggregate_static_bwd(hipStream_t s, bool f32, int n, int64_t N, int64_t C, const void *g,
                                    const void *X, const float *H_pre, void *dX, bool accumulate, float *dH_pre,
                                    void *ws) {
  float *rows = (float *)ws;
  if (f32)
    gagg_bwd<float>(s, n, N, C, g, X, H_pre, 0, dX, accumulate, rows);
  else
    gagg_bwd<bf16_t>(s, n, N, C, g, X, H_pre, 0, dX, accumulate, rows);
  hipLaunchKernelGGL(gcol_sum_kernel, dim3((unsigned)n), dim3(256), 0, s, rows, dH_pre, N, n);
}

template <typename T, int MODE>
static void gpost_fwd(hipStream_t s, int n, int64_t N, int64_t C, const void *X, const float *Hr, const float *Hp,
                      const void *x, const void *b, void *out) {
  MHC_NS_DISPATCH(n, hipLaunchKernelGGL((gpost_fwd_kernel<T, NS, MODE>), dim3((unsigned)N), dim3(gtpb(C)), 0, s,
                                        (const T *)X, Hr, Hp, (const T *)x, (const T *)b, (T *)out, C));
}

void glaunch_h_post_bda_fwd(hipStream_t s, bool f32, int n, int64_t N, int64_t C, const void *X,
                            const float *H_res, const float *H_post, const void *x, const void *bias, void *out) {
  if (f32)
    gpost_fwd<float, kPostFull>(s, n, N, C, X, H_res, H_post, x, bias, out);
  else
    gpost_fwd<bf16_t, kPostFull>(s, n, N, C, X, H_res, H_post, x, bias, out);
}

void glaunch_stream_mix_fwd(hipStream_t s, bool f32, int n, int64_t N, int64_t C, const void *X, const float *M,
                            void *out) {
  if (f32)
    gpost_fwd<float, kPostMix>(s, n, N, C, X, M, nullptr, nullptr, nullptr, out);
  else
    gpost_fwd<bf16_t, kPostMix>(s, n, N, C, X, M, nullptr, nullptr, nullptr, out);
}

void glaunch_stream_distribute_fwd(hipStream_t s, bool f32, int n, int64_t N, int64_t C, const void *x,
                                   const float *H_post, void *out) {
  if (f32)
    gpost_fwd<float, kPostDist>(s, n, N, C, nullptr, nullptr, H_post, x, nullptr, out);
  else
    gpost_fwd<bf16_t, kPostDist>(s, n, N, C, nullptr, nullptr, H_post, x, nullptr, out);
}

constexpr int kGPostTG = 16;

// dbias partial rows: one per wave slot of the grid (ceil(N / TG) waves rounded up to whole workgroups)
static int64_t gpost_rows(int64_t N) { return ((N + kGPostTG - 1) / kGPostTG + 3) / 4 * 4; }

size_t gh_post_bda_bwd_ws(int64_t N, int64_t C, bool with_dbias) {
  if (!with_dbias) return 0;
  return (size_t)((gpost_rows(N) + kRowSumSlices) * C) * sizeof(float);
}

// part != NULL: dbias partial rows (TG tokens per workgroup), else one token per workgroup.
template <typename T, int MODE>
static void gpost_bwd5(hipStream_t s, int n, int64_t N, int64_t C, const void *G, const void *X, const float *Hr,
                       const float *Hp, const void *x, const void *b, void *dX, float *dHr, float *dHp, void *dx,
                       float *part) {
  const int TG = part ? kGPostTG : 1;
  MHC_NS_DISPATCH(n, {
    // one wave per TG tokens (per pass of a token without dbias), four waves per workgroup
    const int64_t waves = part ? (N + TG - 1) / TG : N * GPostShape<T, NS, MODE>::NPASS;
    const unsigned blocks = (unsigned)((waves + 3) / 4);
    if (dX)
      hipLaunchKernelGGL((gpost_bwd_kernel<T, NS, MODE, true>), dim3(blocks), dim3(256), 0, s, (const T *)G,
                         (const T *)X, Hr, Hp, (const T *)x, (const T *)b, (T *)dX, dHr, dHp, (T *)dx, part, N, C, TG);
    else
      hipLaunchKernelGGL((gpost_bwd_kernel<T, NS, MODE, false>), dim3(blocks), dim3(256), 0, s, (const T *)G,
                         (const T *)X, Hr, Hp, (const T *)x, (const T *)b, (T *)dX, dHr, dHp, (T *)dx, part, N, C, TG);
  });
}

template <typename T>
static void gpost_bwd(hipStream_t s, int n, int64_t N, int64_t C, const void *G, const void *X, const float *Hr,
                      const float *Hp, const void *x, const void *b, void *dX, float *dHr, float *dHp, void *dx,
                      void *db, void *ws) {
  if (b && db) {
    float *part = (float *)ws;
    gpost_bwd5<T, kPostFull>(s, n, N, C, G, X, Hr, Hp, x, b, dX, dHr, dHp, dx, part);
    const int64_t waves = (N + kGPostTG - 1) / kGPostTG, rows = gpost_rows(N);
    launch_rows_sum(s, part, waves, C, part + rows * C, db, sizeof(T) == 2);
  } else {
    gpost_bwd5<T, kPostFull>(s, n, N, C, G, X, Hr, Hp, x, b, dX, dHr, dHp, dx, nullptr);
  }
}

void glaunch_h_post_bda_bwd(hipStream_t s, bool f32, int n, int64_t N, int64_t C, const void *G, const void *X,
                            const float *H_res, const float *H_post, const void *x, const void *bias, void *dX,
                            float *dH_res, float *dH_post, void *dx, void *dbias, void *ws) {
  if (f32)
    gpost_bwd<float>(s, n, N, C, G, X, H_res, H_post, x, bias, dX, dH_res, dH_post, dx, dbias, ws);
  else
    gpost_bwd<bf16_t>(s, n, N, C, G, X, H_res, H_post, x, bias, dX, dH_res, dH_post, dx, dbias, ws);
}

void glaunch_stream_mix_bwd(hipStream_t s, bool f32, int n, int64_t N, int64_t C, const void *G, const void *X,
                            const float *M, void *dX, float *dM) {
  if (f32)
    gpost_bwd5<float, kPostMix>(s, n, N, C, G, X, M, nullptr, nullptr, nullptr, dX, dM, nullptr, nullptr, nullptr);
  else
    gpost_bwd5<bf16_t, kPostMix>(s, n, N, C, G, X, M, nullptr, nullptr, nullptr, dX, dM, nullptr, nullptr,
                                 nullptr);
}

void glaunch_stream_distribute_bwd(hipStream_t s, bool f32, int n, int64_t N, int64_t C, const void *G,
                                   const void *x, const float *H_post, void *dx, float *dH_post) {
  if (f32)
    gpost_bwd5<float, kPostDist>(s, n, N, C, G, nullptr, nullptr, H_post, x, nullptr, nullptr, nullptr, dH_post,
                                 dx, nullptr);
  else
    gpost_bwd5<bf16_t, kPostDist>(s, n, N, C, G, nullptr, nullptr, H_post, x, nullptr, nullptr, nullptr, dH_post,
                                  dx, nullptr);
}

// split-K partials [8][N][J + 1], then (bf16) the packed W chunks
size_t gproj_fwd_ws(int n, int64_t N, int64_t C, bool f32) {
  const int64_t J = (int64_t)n * n + 2 * n, JT = (J + 31) / 32, nch = ((int64_t)n * C + 63) / 64;
  return al256((size_t)kGSplitK * N * (J + 1) * 4) + (f32 ? 0 : al256((size_t)nch * 3 * 32 * JT * 128));
}

void glaunch_proj_fwd(hipStream_t s, bool f32, int n, int64_t N, int64_t C, const void *X, const float *W,
                      const float *alpha, const float *hbias, float rms_eps, float *H_pre, float *H_post,
                      float *logits, float *saved, float *H_res, int iters, float eps, void *ws) {
  const int64_t K = (int64_t)n * C, J = (int64_t)n * n + 2 * n;
  float *part = (float *)ws;
  if (f32) {
    const unsigned pb = (unsigned)(((N + kGTokWG - 1) / kGTokWG) * kGSplitK);
    MHC_NS_DISPATCH(n, hipLaunchKernelGGL((gproj_partial_kernel<float, NS>), dim3(pb), dim3(256), 0, s,
                                          (const float *)X, W, part, N, K))
  } else {
    bf16_t *Wp = (bf16_t *)((char *)ws + al256((size_t)kGSplitK * N * (J + 1) * 4));
    const int64_t nch = (K + 63) / 64;
    MHC_NS_DISPATCH(n, {
      using G = GPj<NS>;
      const unsigned pb = (unsigned)(((N + G::TOK - 1) / G::TOK) * kGSplitK);
      hipLaunchKernelGGL((gpack_w_kernel<NS>), dim3((unsigned)((nch * 32 * G::JT * 8 + 255) / 256)), dim3(256), 0,
                         s, W, Wp, K);
      // rows a multiple of 16 KB apart, 32 KB or more: staggered walk starts
      // over 4 sub-slices where one column tile is summed (n <= 3; with more
      // columns the kernel waits on its MFMAs, and the extra sums slowed it)
      constexpr int NSUB = G::JT == 1 ? 4 : 1;
      if (NSUB > 1 && (2 * K) % 16384 == 0 && 2 * K >= 32768)
        hipLaunchKernelGGL((gproj_partial_dma_kernel<NS, NSUB>), dim3(pb), dim3(64 * G::WAVES),
                           (size_t)G::STAGES * G::SB, s, (const bf16_t *)X, (const bf16_t *)Wp, part, N, K);
      else
        hipLaunchKernelGGL((gproj_partial_dma_kernel<NS, 1>), dim3(pb), dim3(64 * G::WAVES),
                           (size_t)G::STAGES * G::SB, s, (const bf16_t *)X, (const bf16_t *)Wp, part, N, K);
    })
  }
  if (n >= 3) {
    const unsigned fb = (unsigned)((N * sk_group(n) + 255) / 256);
    MHC_NS_DISPATCH(n, hipLaunchKernelGGL((gproj_finalize_lanes_kernel<NS>), dim3(fb), dim3(256), 0, s, part, N, K,
                                          alpha, hbias, rms_eps, H_pre, H_post, logits, saved, saved_stride(n),
                                          H_res, iters, eps));
    return;
  }
  const unsigned fb = (unsigned)((N + 63) / 64);
  MHC_NS_DISPATCH(n, hipLaunchKernelGGL((gproj_finalize_kernel<NS>), dim3(fb), dim3(64), 0, s, part, N, K, alpha,
                                        hbias, rms_eps, H_pre, H_post, logits, saved, saved_stride(n), H_res,
                                        iters, eps));
}

size_t gproj_bwd_ws(int n, int64_t N, int64_t C, bool terms, bool f32) {
  return gbwd_layout(N, C, n, terms, f32).total;
}

template <typename T>
static void gdx(hipStream_t s, int n, const ProjBwdArgs &a, const GBwdLay &L, const float *rec, const float *term,
                float *dwp) {
  const int64_t K = (int64_t)n * a.C;
  const dim3 grid((unsigned)((K + kGBwdK - 1) / kGBwdK), (unsigned)L.ntb);
  if (a.dW)
    MHC_NS_DISPATCH(n, hipLaunchKernelGGL((gproj_bwd_dx_kernel<T, NS, true>), grid, dim3(kGBwdK), 0, s,
                                          (const T *)a.X, a.W, rec, term, (T *)a.dX, dwp, a.N, a.C, L.tb,
                                          a.accumulate))
  else
    MHC_NS_DISPATCH(n, hipLaunchKernelGGL((gproj_bwd_dx_kernel<T, NS, false>), grid, dim3(kGBwdK), 0, s,
                                          (const T *)a.X, a.W, rec, term, (T *)a.dX, dwp, a.N, a.C, L.tb,
                                          a.accumulate))
}

// n >= 5: the dX kernel (about 512 workgroups of 64 channels x a token block
// in whole 16-token sub-tiles), then the dW kernel on the layout's token blocks.
template <int NS>
static void gdx_split(hipStream_t s, const ProjBwdArgs &a, const GBwdLay &L, const float *rec, float *dwp,
                      bf16_t *dpT) {
  using M = GDx<NS>;
  const int64_t nct = (a.C + 63) / 64;
  const int64_t ntbx = std::min<int64_t>(std::max<int64_t>(1, 512 / nct), std::max<int64_t>(1, (a.N + 15) / 16));
  const int64_t tbx = ((a.N + ntbx - 1) / ntbx + 15) / 16 * 16;
  const bool has_g = a.g != nullptr, post = a.post_G != nullptr;
  const int flags = (has_g ? 1 : 0) | (post ? 2 : 0) | (a.accumulate ? 4 : 0);
  const size_t stage = (size_t)M::XB * (post ? 2 : 1) + (has_g ? M::GB : 0) + M::RB;
  hipLaunchKernelGGL((gproj_dx16_mfma_kernel<NS>), dim3((unsigned)((nct * ntbx + 7) / 8 * 8)), dim3(768),
                     3 * stage + M::ACC, s, (const bf16_t *)a.X, a.W, rec, a.H_pre, (const bf16_t *)a.g,
                     (const bf16_t *)a.post_G, a.post_H_res, (bf16_t *)a.dX, a.N, a.C, tbx, ntbx, flags);
  if (a.dW) {
    const int64_t K = (int64_t)NS * a.C, nkt = (K + 255) / 256;
    const int64_t nsp = (a.N + 31) / 32 * 32 * GDw<NS>::JT * 32;
    hipLaunchKernelGGL((gsplit_dp_kernel<NS>), dim3((unsigned)((nsp + 255) / 256)), dim3(256), 0, s, rec, dpT, a.N);
    hipLaunchKernelGGL((gproj_dw_mfma_kernel<NS>), dim3((unsigned)((nkt * L.ntb + 7) / 8 * 8)), dim3(512),
                       GDw<NS>::STG * GDw<NS>::SB, s, (const bf16_t *)a.X, (const bf16_t *)dpT, dwp, a.N, K, L.tb,
                       L.ntb);
  }
}

template <int NS>
static void gdx_mfma(hipStream_t s, const ProjBwdArgs &a, const GBwdLay &L, const float *rec, float *dwp,
                     bf16_t *dpT) {
  if constexpr (NS >= 5) {
    gdx_split<NS>(s, a, L, rec, dwp, dpT);
  } else {
    using M = GMf<NS>;
    const int64_t nct = (a.C + M::CW - 1) / M::CW, T = nct * L.ntb;
    const unsigned blocks = (unsigned)((T + 7) / 8 * 8);
    const bool has_g = a.g != nullptr, post = a.post_G != nullptr;
    const int flags = (has_g ? 1 : 0) | (post ? 2 : 0) | (a.accumulate ? 4 : 0);
    const size_t stage = (size_t)M::XB * (post ? 2 : 1) + (has_g ? M::GB : 0) + M::RB;
    const size_t lds = 3 * stage + M::ACC;
    if (a.dW)
      hipLaunchKernelGGL((gproj_bwd_mfma_kernel<NS, true>), dim3(blocks), dim3(512), lds, s, (const bf16_t *)a.X,
                         a.W, rec, a.H_pre, (const bf16_t *)a.g, (const bf16_t *)a.post_G, a.post_H_res,
                         (bf16_t *)a.dX, dwp, a.N, a.C, L.tb, L.ntb, flags);
    else
      hipLaunchKernelGGL((gproj_bwd_mfma_kernel<NS, false>), dim3(blocks), dim3(512), lds, s, (const bf16_t *)a.X,
                         a.W, rec, a.H_pre, (const bf16_t *)a.g, (const bf16_t *)a.post_G, a.post_H_res,
                         (bf16_t *)a.dX, dwp, a.N, a.C, L.tb, L.ntb, flags);
  }
}

template <typename T>
static void gterms(hipStream_t s, int n, const ProjBwdArgs &a, float *term) {
  MHC_NS_DISPATCH(n, hipLaunchKernelGGL((gpre_terms_kernel<T, NS>), dim3((unsigned)a.N), dim3(gtpb(a.C)), 0, s,
                                        (const T *)a.g, a.H_pre, (const T *)a.post_G, a.post_H_res, term, a.C));
}

void glaunch_proj_bwd(hipStream_t s, int n, const ProjBwdArgs &a) {
  const bool terms = a.g != nullptr || a.post_G != nullptr;
  const GBwdLay L = gbwd_layout(a.N, a.C, n, terms, a.f32);
  const int64_t J = (int64_t)n * n + 2 * n, K = (int64_t)n * a.C;
  char *base = (char *)a.ws;
  float *rec = (float *)base;
  float *prm = (float *)(base + L.rec);
  float *dwp = (float *)(base + L.rec + L.prm);
  float *dhrow = (float *)(base + L.rec + L.prm + L.dw);
  float *term = terms ? (float *)(base + L.rec + L.prm + L.dw + L.dhrow) : nullptr;
  const float *dHpre = a.dH_pre;
  if (a.g) {  // fused pre backward: dH_pre = <g, X_i> first (into dH_pre_out when given)
    float *rows = a.dH_pre_out ? a.dH_pre_out : dhrow;
    if (a.f32)
      gagg_bwd<float>(s, n, a.N, a.C, a.g, a.X, a.H_pre, n, nullptr, false, rows);
    else
      gagg_bwd<bf16_t>(s, n, a.N, a.C, a.g, a.X, a.H_pre, n, nullptr, false, rows);
    dHpre = rows;
  }
  // The logits' gradient, when not given: by the row-per-lane Sinkhorn backward first where its records
  // fit (into dL_out when the caller wants it, else the workspace), else inside the per-token kernel.
  const float *dLin = a.dL;
  float *dLout = a.dL_out;
  if (!dLin && sk_lane_threads(n, a.iters) > 0) {
    float *dst = a.dL_out ? a.dL_out : (float *)(base + L.rec + L.prm + L.dw + L.dhrow + L.term);
    glaunch_sinkhorn_bwd(s, n, a.N, a.dH_res, a.logits, dst, a.iters, a.eps);
    dLin = dst;
    dLout = nullptr;
  }
  const SkBwdGeom g = dLin ? SkBwdGeom{64, false, 0} : sk_bwd_geom(n, a.iters);
  const unsigned tb = (unsigned)((a.N + g.threads - 1) / g.threads);
  if (g.stored)
    MHC_NS_DISPATCH(n, hipLaunchKernelGGL((gproj_bwd_token_kernel<NS, true>), dim3(tb), dim3(g.threads), g.lds, s,
                                          a.N, K, a.alpha, a.saved, saved_stride(n), a.H_pre, a.H_post, dHpre,
                                          a.dH_post, dLin, a.dH_res, a.logits, a.iters, a.eps, rec, prm, dLout))
  else
    MHC_NS_DISPATCH(n, hipLaunchKernelGGL((gproj_bwd_token_kernel<NS, false>), dim3(tb), dim3(g.threads), 0, s,
                                          a.N, K, a.alpha, a.saved, saved_stride(n), a.H_pre, a.H_post, dHpre,
                                          a.dH_post, dLin, a.dH_res, a.logits, a.iters, a.eps, rec, prm, dLout))
  if (a.f32) {
    if (terms) gterms<float>(s, n, a, term);
    gdx<float>(s, n, a, L, rec, term, dwp);
  } else {
    bf16_t *dpT = (bf16_t *)(base + L.rec + L.prm + L.dw + L.dhrow + L.term + L.dl);
    MHC_NS_DISPATCH(n, gdx_mfma<NS>(s, a, L, rec, dwp, dpT));
  }
  if (a.dW)
    hipLaunchKernelGGL(gdw_reduce_kernel, dim3((unsigned)((K * J + 255) / 256)), dim3(256), 0, s, dwp, a.dW, L.ntb,
                       K * J);
  // parameter sums: columns 0..J-1 of prm are dhbias terms, J..J+2 dalpha terms
  if (a.dhbias || a.dalpha) {
    const int NC = (int)(J + 3);
    float *part = (float *)(base + L.rec + L.prm + L.dw + L.dhrow + L.term + L.dl + L.dpt);
    hipLaunchKernelGGL(gparam_part_kernel, dim3((unsigned)((kGParts * NC + 255) / 256)), dim3(256), 0, s, prm, part,
                       a.N, NC);
    hipLaunchKernelGGL(gparam_final_kernel, dim3((unsigned)((NC + 31) / 32)), dim3(1024), 0, s, part, NC, (int)J,
                       a.dhbias, a.dalpha);
  }
}

}  // namespace mhc
