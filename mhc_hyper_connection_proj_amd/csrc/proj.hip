// proj.hip -- projection + RMS + compute_h (forward and backward).
//
// Forward (Megatron Core fused_mhc_kernels, proj_rms_compute_h; RL-Kernel
// PR #383 for r = 1/(q + eps) and the three segment gains), per token:
//   q = sqrt(sum x^2 / K), r = 1/(q + rms_eps), p = x @ W, z = r p,
//   zh = alpha[seg] z + hbias, H_pre = sigmoid, H_post = 2 sigmoid, logits = zh_RES.
//
// The contraction x @ W ([K] x [K, 24] per token, K = 4C up to 64K) is the
// only dense work on the path.  It runs on MFMA:
//  * W (fp32) is split exactly into three bf16 terms hi + mid + lo (8 + 8 + 8
//    significant bits cover fp32's 24), and bf16 x times each term is exact in
//    the fp32 accumulator, so 3 bf16 MFMAs reproduce the fp32 product.  For
//    fp32 activations the fp32 MFMA is used on W directly.
//  * A 32x32x16 MFMA takes 32 tokens x 16 k from X and 16 k x 32 columns
//    (24 used) from W.  The k order inside one MFMA is free as long as A and
//    B agree, so lane (row, h) loads 32 consecutive k of its token (64 bytes)
//    per 64-k chunk and feeds them to four MFMAs; W is packed so the matching
//    B fragment is one 16-byte load.
//  * Split-K: the k range is cut into kSplitK slices and workgroup b works on
//    slice b % 8.  Workgroups are dispatched round-robin over the 8 XCDs, so
//    each XCD streams one slice and its L2 only holds that slice of W.
//  * Accuracy: each 64-k chunk accumulates in a fresh MFMA accumulator and is
//    then added into an fp32 running sum (two-level blocking), the 4 waves of a
//    workgroup and the 8 slices are summed in a fixed order; sum x^2 uses
//    v_dot2_f32_bf16 with the same blocking.  Where the rows are a multiple of
//    16 KB apart, each quarter of a slice keeps its own running sum (so the
//    workgroups can start their walks at different quarters) and the quarters
//    are added in order: the summation order still depends on K alone.
#include "device.h"
#include "internal.h"
#include "ring.h"
#include "sinkhorn.h"

namespace mhc {

constexpr int kSplitK = 8;   // one k slice per XCD
constexpr int kTPW = 2;      // 32-token MFMA tiles per wave
constexpr int kTB = 32 * kTPW;  // tokens per workgroup
constexpr int kPartStride = 32;  // partial record: p[24], sumsq, pad

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(16))) float f32x16;
typedef __attribute__((ext_vector_type(4))) unsigned int u32x4;

static inline int64_t kpad64(int64_t K) { return (K + 63) / 64 * 64; }

constexpr int kWcol = 32;  // bf16 packed W: 24 columns padded to the MFMA's 32

static inline size_t wpack_bytes(int64_t C, bool f32) {
  const int64_t Kp = kpad64(4 * C);
  return (size_t)(f32 ? Kp * kJ * 4 : Kp * kWcol * 3 * 2);
}

static inline size_t align256(size_t b) { return (b + 255) / 256 * 256; }

size_t proj_fwd_ws(int64_t N, int64_t C, bool f32) {
  return align256(wpack_bytes(C, f32)) + align256((size_t)kSplitK * N * kPartStride * 4);
}

// ------------------------------------------------------------------ W pack
// bf16: Wp[kg][term][32][8] (kg = k/8), term 0,1,2 = hi, mid, lo; columns
// 24..31 are zero so a 64-k chunk is one contiguous 12 KB block.
// fp32: Wf[kg][j][8].  Rows k >= K (padding to a multiple of 64) are zero.
__device__ __forceinline__ float bf16_round(float v) {
  const __bf16 h = (__bf16)v;
  return (float)h;
}

// One thread per (8-k group, column): 8 strided reads of W (coalesced over
// the column), 16- or 32-byte contiguous writes of the packed group.
template <bool F32>
__global__ __launch_bounds__(256) void pack_w_kernel(const float *__restrict__ W, void *__restrict__ out,
                                                     int64_t K, int64_t Kp) {
  const int ncol = F32 ? kJ : kWcol;
  const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;  // over Kp / 8 * ncol
  if (idx >= Kp / 8 * ncol) return;
  const int64_t kg = idx / ncol;
  const int j = (int)(idx % ncol);
  float w[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const int64_t k = kg * 8 + e;
    w[e] = (k < K && j < kJ) ? W[k * kJ + j] : 0.f;
  }
  if (F32) {
    float4 *o = reinterpret_cast<float4 *>(reinterpret_cast<float *>(out) + (kg * kJ + j) * 8);
    o[0] = make_float4(w[0], w[1], w[2], w[3]);
    o[1] = make_float4(w[4], w[5], w[6], w[7]);
  } else {
    uint32_t t[3][4];
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      float hi[2], mid[2], lo[2];
#pragma unroll
      for (int q = 0; q < 2; ++q) {
        const float v = w[2 * p + q];
        hi[q] = bf16_round(v);
        const float r1 = v - hi[q];
        mid[q] = bf16_round(r1);
        lo[q] = bf16_round(r1 - mid[q]);
      }
      t[0][p] = pack_bf16x2(hi[0], hi[1]);
      t[1][p] = pack_bf16x2(mid[0], mid[1]);
      t[2][p] = pack_bf16x2(lo[0], lo[1]);
    }
    bf16_t *o = reinterpret_cast<bf16_t *>(out);
#pragma unroll
    for (int m = 0; m < 3; ++m)
      *reinterpret_cast<uint4 *>(o + ((kg * 3 + m) * kWcol + j) * 8) = make_uint4(t[m][0], t[m][1], t[m][2], t[m][3]);
  }
}

// ------------------------------------------------------------------ partial projection
// fp32 activations.  Grid: ceil(N / kTB) * kSplitK workgroups of 256 threads; workgroup b handles
// token block b / kSplitK and k slice b % kSplitK.  Wave w takes the slice's
// 64-k chunks w, w+4, ...  Output: part[slice][t][0..24) = partial x @ W,
// part[slice][t][24] = partial sum x^2.
__global__ __launch_bounds__(256) void proj_partial_f32_kernel(const void *__restrict__ Xv,
                                                           const void *__restrict__ Wpk,
                                                           float *__restrict__ part, int64_t N,
                                                           int64_t K) {
  __shared__ float red_p[4][kTB][kJ + 1];
  __shared__ float red_s[4][kTB][2];
  const int slice = blockIdx.x % kSplitK;
  const int64_t tb = blockIdx.x / kSplitK;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int row = lane & 31, h = lane >> 5;
  const int64_t nch = (K + 63) / 64;
  const int64_t cps = (nch + kSplitK - 1) / kSplitK;
  const int64_t c_begin = slice * cps;
  const int64_t c_end = min(nch, c_begin + cps);

  f32x16 outer[kTPW];
  float ss[kTPW];
#pragma unroll
  for (int u = 0; u < kTPW; ++u) {
#pragma unroll
    for (int r = 0; r < 16; ++r) outer[u][r] = 0.f;
    ss[u] = 0.f;
  }
  int64_t trow[kTPW];
  bool tvalid[kTPW];
#pragma unroll
  for (int u = 0; u < kTPW; ++u) {
    trow[u] = tb * kTB + 32 * u + row;
    tvalid[u] = trow[u] < N;
  }
  const bool bcol = row < kJ;  // B lanes with a real W column

  for (int64_t c = c_begin + wave; c < c_end; c += 4) {
    const int64_t k0 = c * 64;
    const bool kvalid = (k0 + 32 * h) < K;
    f32x16 acc[kTPW];
#pragma unroll
    for (int u = 0; u < kTPW; ++u)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[u][r] = 0.f;
    {
      const float *X = reinterpret_cast<const float *>(Xv);
      const float *Wf = reinterpret_cast<const float *>(Wpk);
      float a[kTPW][32];
#pragma unroll
      for (int u = 0; u < kTPW; ++u) {
        const float4 *src = reinterpret_cast<const float4 *>(X + trow[u] * K + k0 + 32 * h);
#pragma unroll
        for (int q = 0; q < 8; ++q) {
          const float4 v = (tvalid[u] && kvalid) ? src[q] : make_float4(0.f, 0.f, 0.f, 0.f);
          a[u][4 * q] = v.x; a[u][4 * q + 1] = v.y; a[u][4 * q + 2] = v.z; a[u][4 * q + 3] = v.w;
        }
      }
#pragma unroll
      for (int m = 0; m < 4; ++m) {
        const int64_t kg = k0 / 8 + 4 * h + m;
        float b[8];
        const float4 *src = reinterpret_cast<const float4 *>(Wf + (kg * kJ + row) * 8);
        const float4 b0 = bcol ? src[0] : make_float4(0.f, 0.f, 0.f, 0.f);
        const float4 b1 = bcol ? src[1] : make_float4(0.f, 0.f, 0.f, 0.f);
        b[0] = b0.x; b[1] = b0.y; b[2] = b0.z; b[3] = b0.w;
        b[4] = b1.x; b[5] = b1.y; b[6] = b1.z; b[7] = b1.w;
#pragma unroll
        for (int e = 0; e < 8; ++e)
#pragma unroll
          for (int u = 0; u < kTPW; ++u)
            acc[u] = __builtin_amdgcn_mfma_f32_32x32x2f32(a[u][8 * m + e], b[e], acc[u], 0, 0, 0);
      }
#pragma unroll
      for (int u = 0; u < kTPW; ++u) {
        float s = 0.f;
#pragma unroll
        for (int e = 0; e < 32; ++e) s = fmaf(a[u][e], a[u][e], s);
        ss[u] += s;
      }
    }
#pragma unroll
    for (int u = 0; u < kTPW; ++u)
#pragma unroll
      for (int r = 0; r < 16; ++r) outer[u][r] += acc[u][r];
  }

  // accumulator layout of a 32x32 MFMA: lane (col, h), register r holds
  // row 8*(r/4) + 4*h + (r%4), column col.
#pragma unroll
  for (int u = 0; u < kTPW; ++u) {
    if (bcol) {
#pragma unroll
      for (int r = 0; r < 16; ++r) red_p[wave][32 * u + 8 * (r >> 2) + 4 * h + (r & 3)][row] = outer[u][r];
    }
    red_s[wave][32 * u + row][h] = ss[u];
  }
  __syncthreads();
  for (int idx = threadIdx.x; idx < kTB * (kJ + 1); idx += 256) {
    const int tt = idx / (kJ + 1), j = idx % (kJ + 1);
    const int64_t t = tb * kTB + tt;
    if (t >= N) continue;
    float v;
    if (j < kJ)
      v = (red_p[0][tt][j] + red_p[1][tt][j]) + (red_p[2][tt][j] + red_p[3][tt][j]);
    else
      v = ((red_s[0][tt][0] + red_s[0][tt][1]) + (red_s[1][tt][0] + red_s[1][tt][1])) +
          ((red_s[2][tt][0] + red_s[2][tt][1]) + (red_s[3][tt][0] + red_s[3][tt][1]));
    part[((int64_t)slice * N + t) * kPartStride + j] = v;
  }
}

// ------------------------------------------------------------------ partial projection, bf16 (LDS-staged)
// Workgroup = 8 waves x 32 tokens (256 tokens) on one k slice (slice =
// workgroup % 8, one per XCD).  The k range is walked in 64-k chunks through a
// 3-stage LDS ring filled with global_load_lds_dwordx4 (each instruction moves
// 1 KB: 64 lanes x 16 bytes land at consecutive LDS addresses):
//  * the W chunk (12 KB: 8 k-groups x 3 terms x 32 columns x 8) is shared by
//    all waves; waves 0..5 load 2 KB of it each;
//  * each wave loads its own 32 x 64 X tile (4 KB, 8 lanes per 128-byte row
//    segment, so every instruction reads whole cache lines).  Row r's 16-byte
//    piece p is stored in slot p ^ (r & 7) of its LDS row, which spreads the
//    column reads of the MFMA fragments over the banks.
// Two chunks are in flight while one is computed.  Each wave waits for its
// own loads (s_waitcnt vmcnt), then one workgroup barrier makes every wave's
// loads visible and guarantees the slot refilled next was read by everyone.
// A wave owns its 32 tokens over the whole slice, so its accumulators are
// the workgroup's output (no cross-wave reduction).
// With NSUB > 1 the slice's chunks form NSUB sub-slices, each with its own
// running sum, and workgroup tb starts its walk at sub-slice tb % NSUB
// (wrapping around); the sub-slice sums are added in sub-slice order at the
// end, so a token's result depends on K alone.  Where the rows are a multiple
// of 16 KB apart (C = 4096, 8192) the unstaggered walk puts the same k offset
// of every token in flight at once, which reads 15-20% slower.
constexpr int kDmaWaves = 8;
constexpr int kDmaTok = 32 * kDmaWaves;      // 256 tokens per workgroup
constexpr int kDmaStages = 3;
constexpr int kWChunk = 8 * 3 * kWcol * 8;   // bf16 elements per 64-k W chunk (12 KB)
constexpr int kXTile = 32 * 64;              // bf16 elements per wave X tile (4 KB)
constexpr int kStageElems = kWChunk + kDmaWaves * kXTile;

template <int NSUB>
__global__ __launch_bounds__(512) void proj_partial_dma_kernel(const bf16_t *__restrict__ X,
                                                               const bf16_t *__restrict__ Wp,
                                                               float *__restrict__ part, int64_t N,
                                                               int64_t K) {
  extern __shared__ __attribute__((aligned(16))) bf16_t ring[];  // kDmaStages * kStageElems
  const int slice = blockIdx.x % kSplitK;
  const int64_t tb = blockIdx.x / kSplitK;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int row = lane & 31, h = lane >> 5;
  const int64_t nch = (K + 63) / 64;
  const int64_t cps = (nch + kSplitK - 1) / kSplitK;
  const int64_t c_begin = min(nch, slice * cps);
  const int nc = (int)(min(nch, c_begin + cps) - c_begin);
  const int64_t tw = tb * kDmaTok + 32 * wave;  // this wave's first token
  // the slice's chunks fall into NSUB sub-slices of sps chunks; the walk
  // starts at sub-slice tb % NSUB and wraps around
  const int sps = (nc + NSUB - 1) / NSUB;
  const int cstart = sps * (int)(tb % NSUB) < nc ? sps * (int)(tb % NSUB) : 0;
  auto chunk = [&](int v) { return cstart + v < nc ? cstart + v : cstart + v - nc; };

  // issue the loads of walk position v into its slot
  auto issue = [&](int v) {
    bf16_t *st = ring + (v % kDmaStages) * kStageElems;
    const int64_t k0 = (c_begin + chunk(v)) * 64;
    if (wave < 6) {
      const bf16_t *wsrc = Wp + (k0 / 8) * 3 * kWcol * 8;
#pragma unroll
      for (int q = 0; q < 2; ++q) {
        const int blk = 2 * wave + q;  // 1 KB blocks of the chunk
        dma16(wsrc + blk * 512 + lane * 8, st + blk * 512);
      }
    }
    bf16_t *xs = st + kWChunk + wave * kXTile;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int rr = 8 * q + (lane >> 3);                 // row within the wave's 32
      const int p = (lane & 7) ^ (rr & 7);                // global 16-byte piece for this slot
      const int64_t t = min(tw + rr, N - 1);              // rows past N re-read row N-1 (never stored)
      int64_t k = k0 + 8 * p;
      if (k >= K) k -= 32;                                // past K: any valid address (W rows there are 0)
      dma16_nt(X + t * K + k, xs + q * 512);
    }
  };

  f32x16 outer[NSUB];  // one running sum per sub-slice
  float ss[NSUB];
#pragma unroll
  for (int q = 0; q < NSUB; ++q) {
#pragma unroll
    for (int r = 0; r < 16; ++r) outer[q][r] = 0.f;
    ss[q] = 0.f;
  }
  if (nc > 0) issue(0);
  if (nc > 1) issue(1);
  for (int v = 0; v < nc; ++v) {
    // this wave's loads of position v are complete once at most those of
    // position v+1 remain outstanding
    if (v + 1 < nc) {
      if (wave < 6) wait_vmcnt<6>(); else wait_vmcnt<4>();
    } else {
      wait_vmcnt<0>();
    }
    // a bare barrier: __syncthreads' fence would also wait for the chunk
    // still in flight.  The memory clobber keeps LDS reads below it.
    asm volatile("s_barrier" ::: "memory");
    if (v + 2 < nc) issue(v + 2);  // slot (v+2) % 3 was last read in iteration v-1
    const bf16_t *st = ring + (v % kDmaStages) * kStageElems;
    const bf16_t *xs = st + kWChunk + wave * kXTile;
    const int ci = chunk(v);
    const int64_t k0 = (c_begin + ci) * 64;
    f32x16 acc;
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[r] = 0.f;
    u32x4 a[4], b[4][3];
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      const int P = 4 * h + m;  // this lane's 16-byte piece (k = k0 + 8P .. +8)
      a[m] = *reinterpret_cast<const u32x4 *>(xs + row * 64 + 8 * (P ^ (row & 7)));
#pragma unroll
      for (int tm = 0; tm < 3; ++tm)
        b[m][tm] = *reinterpret_cast<const u32x4 *>(st + ((P * 3 + tm) * kWcol + row) * 8);
    }
#pragma unroll
    for (int m = 0; m < 4; ++m)
#pragma unroll
      for (int tm = 0; tm < 3; ++tm)
        acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a[m]),
                                                      __builtin_bit_cast(bf16x8, b[m][tm]), acc, 0, 0, 0);
    // sum of squares of this lane's 32 elements of its row.  The dwords are
    // pulled out by name: bit-casting an indexed ext-vector element (a[m][q])
    // makes hipcc reuse dword 0 for every q.
    float s = 0.f;
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      if (k0 + 8 * (4 * h + m) < K) {
        const unsigned w4[4] = {a[m].x, a[m].y, a[m].z, a[m].w};
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2;
          const bf16x2 v = __builtin_bit_cast(bf16x2, w4[q]);
          s = __builtin_amdgcn_fdot2_f32_bf16(v, v, s, false);
        }
      }
    }
    // into the running sum of the chunk's sub-slice (workgroup-uniform branch)
    const int sub = NSUB == 1 ? 0 : ci / sps;
#pragma unroll
    for (int q = 0; q < NSUB; ++q)
      if (sub == q) {
#pragma unroll
        for (int r = 0; r < 16; ++r) outer[q][r] += acc[r];
        ss[q] += s;
      }
  }
  // the sub-slice sums in sub-slice order, so a token's summation order
  // depends on K alone, not on where the walk started
  f32x16 tot = outer[0];
  float sst = ss[0];
#pragma unroll
  for (int q = 1; q < NSUB; ++q) {
#pragma unroll
    for (int r = 0; r < 16; ++r) tot[r] += outer[q][r];
    sst += ss[q];
  }
  // sum of squares: the two lane halves hold the two 32-k halves of each row
  sst += __shfl_xor(sst, 32);
  if (row < kJ) {
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int64_t t = tw + 8 * (r >> 2) + 4 * h + (r & 3);
      if (t < N) part[((int64_t)slice * N + t) * kPartStride + row] = tot[r];
    }
  }
  if (h == 0 && tw + row < N) part[((int64_t)slice * N + tw + row) * kPartStride + kJ] = sst;
}

// ------------------------------------------------------------------ partial projection, bf16 on the VALU
// The comparison point for the MFMA kernel above: the same token blocks x k
// slices and the same partial records, with x @ W as fp32 FMAs.  Thread =
// one token (256 per workgroup).  The slice's 64-k chunks of W (fp32,
// [k][24], 6 KB) pass through a two-slot LDS buffer, the next chunk's loaded
// into registers while the current one is used; every lane reads the same W
// words (LDS broadcast).  A chunk's eight 16-byte groups of the token's x
// are loaded together, then 64 x 24 FMAs accumulate into a fresh per-chunk
// sum that is added to the running one (the same two-level blocking).
constexpr int kFmaTok = 256;

__global__ __launch_bounds__(256) void proj_partial_fma_kernel(const bf16_t *__restrict__ X,
                                                               const float *__restrict__ W,
                                                               float *__restrict__ part, int64_t N,
                                                               int64_t K) {
  __shared__ float4 wl[2][64 * kJ / 4];
  const int slice = blockIdx.x % kSplitK;
  const int64_t tb = blockIdx.x / kSplitK;
  const int64_t t = tb * kFmaTok + threadIdx.x;
  const bool tv = t < N;
  const bf16_t *xr = X + (tv ? t : N - 1) * K;
  const int64_t nch = (K + 63) / 64;
  const int64_t cps = (nch + kSplitK - 1) / kSplitK;
  const int64_t c_begin = min(nch, slice * cps);
  const int nc = (int)(min(nch, c_begin + cps) - c_begin);
  // W chunk i: 64 k x 24 floats = 384 float4; thread e and e + 256 load float4 e of it
  float4 wr[2];
  auto load_w = [&](int i) {
    const int64_t k0 = (c_begin + i) * 64;
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      const int e = threadIdx.x + 256 * q;
      const int64_t k = k0 + e / 6;
      wr[q] = (e < 384 && k < K) ? reinterpret_cast<const float4 *>(W + k * kJ)[e % 6]
                                 : make_float4(0.f, 0.f, 0.f, 0.f);
    }
  };
  float outer[kJ];
#pragma unroll
  for (int j = 0; j < kJ; ++j) outer[j] = 0.f;
  float ss = 0.f;
  if (nc > 0) load_w(0);
  for (int i = 0; i < nc; ++i) {
    float4 *slot = wl[i & 1];
    slot[threadIdx.x] = wr[0];
    if (threadIdx.x < 128) slot[threadIdx.x + 256] = wr[1];
    __syncthreads();  // slot i & 1 was last read two chunks ago, before the previous barrier
    if (i + 1 < nc) load_w(i + 1);
    const int64_t k0 = (c_begin + i) * 64;
    uint4 xg[8];
#pragma unroll
    for (int g = 0; g < 8; ++g)
      xg[g] = k0 + 8 * g < K ? *reinterpret_cast<const uint4 *>(xr + k0 + 8 * g) : make_uint4(0u, 0u, 0u, 0u);
    float acc[kJ];
#pragma unroll
    for (int j = 0; j < kJ; ++j) acc[j] = 0.f;
    float s = 0.f;
#pragma unroll
    for (int g = 0; g < 8; ++g) {
      const uint32_t w4[4] = {xg[g].x, xg[g].y, xg[g].z, xg[g].w};
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float xv = (e & 1) ? bf16_hi(w4[e >> 1]) : bf16_lo(w4[e >> 1]);
        s = fmaf(xv, xv, s);
        const float4 *wrow = slot + (8 * g + e) * (kJ / 4);
#pragma unroll
        for (int q = 0; q < kJ / 4; ++q) {
          const float4 wv = wrow[q];
          acc[4 * q] = fmaf(xv, wv.x, acc[4 * q]);
          acc[4 * q + 1] = fmaf(xv, wv.y, acc[4 * q + 1]);
          acc[4 * q + 2] = fmaf(xv, wv.z, acc[4 * q + 2]);
          acc[4 * q + 3] = fmaf(xv, wv.w, acc[4 * q + 3]);
        }
      }
    }
#pragma unroll
    for (int j = 0; j < kJ; ++j) outer[j] += acc[j];
    ss += s;
  }
  if (tv) {
    float *dst = part + ((int64_t)slice * N + t) * kPartStride;
#pragma unroll
    for (int q = 0; q < kJ / 4; ++q)
      reinterpret_cast<float4 *>(dst)[q] = make_float4(outer[4 * q], outer[4 * q + 1], outer[4 * q + 2], outer[4 * q + 3]);
    dst[kJ] = ss;
  }
}

// ------------------------------------------------------------------ finalize
// Four lanes per token (quad layout of the Sinkhorn code: lane r = row r of
// H_res), 16 tokens per one-wave workgroup, so a layer's tokens make enough
// waves to spread over all CUs.  Lane r owns the columns r (PRE), 4 + r
// (POST) and 8 + 4r .. 11 + 4r (RES row r): fixed-order sum of the kSplitK
// partials, RMS, compute_h, and (when H_res != NULL) the Sinkhorn projection.
// Every value is computed as in a one-lane-per-token form, bit for bit.
__global__ __launch_bounds__(64) void proj_finalize_kernel(
    const float *__restrict__ part, const float *__restrict__ alpha, const float *__restrict__ hbias,
    float rms_eps, float *__restrict__ Hpre, float *__restrict__ Hpost, float *__restrict__ logits,
    float *__restrict__ saved, float *__restrict__ Hres, int iters, float eps, int64_t N, int64_t K) {
  const int r4 = threadIdx.x & 3;
  const int64_t t = (int64_t)blockIdx.x * 16 + (threadIdx.x >> 2);
  if (t >= N) return;  // whole quads
  // owned columns: jp = r4, jq = 4 + r4, jr = 8 + 4 r4 .. + 3; and the sum of squares
  float vp[kSplitK], vq[kSplitK], vr[kSplitK][4], vs[kSplitK];
#pragma unroll
  for (int sl = 0; sl < kSplitK; ++sl) {
    const float *row = part + ((int64_t)sl * N + t) * kPartStride;
    vp[sl] = row[r4];
    vq[sl] = row[4 + r4];
    const float4 w = reinterpret_cast<const float4 *>(row)[2 + r4];
    vr[sl][0] = w.x; vr[sl][1] = w.y; vr[sl][2] = w.z; vr[sl][3] = w.w;
    vs[sl] = row[kJ];
  }
  auto tree = [](const float v[kSplitK]) {
    return ((v[0] + v[1]) + (v[2] + v[3])) + ((v[4] + v[5]) + (v[6] + v[7]));
  };
  static_assert(kSplitK == 8, "tree");
  float p[6];
  p[0] = tree(vp);
  p[1] = tree(vq);
#pragma unroll
  for (int b = 0; b < 4; ++b) {
    float v[kSplitK];
#pragma unroll
    for (int sl = 0; sl < kSplitK; ++sl) v[sl] = vr[sl][b];
    p[2 + b] = tree(v);
  }
  const float q = sqrtf(tree(vs) / (float)K);
  const float r = 1.0f / (q + rms_eps);
  const int jcol[6] = {r4, 4 + r4, 8 + 4 * r4, 9 + 4 * r4, 10 + 4 * r4, 11 + 4 * r4};
  float z[6], zh[6];
#pragma unroll
  for (int u = 0; u < 6; ++u) {
    z[u] = r * p[u];
    const int seg = u == 0 ? 0 : (u == 1 ? 1 : 2);
    const float a = alpha ? alpha[seg] : 1.f;
    const float b = hbias ? hbias[jcol[u]] : 0.f;
    zh[u] = a * z[u] + b;
  }
  Hpre[t * 4 + r4] = 1.0f / (1.0f + expf(-zh[0]));
  Hpost[t * 4 + r4] = 2.0f / (1.0f + expf(-zh[1]));
  reinterpret_cast<float4 *>(logits + t * 16)[r4] = make_float4(zh[2], zh[3], zh[4], zh[5]);
  if (saved) {
    float *sv = saved + t * kSavedStride;
    sv[2 + r4] = z[0];
    sv[6 + r4] = z[1];
    reinterpret_cast<float2 *>(sv + 10 + 4 * r4)[0] = make_float2(z[2], z[3]);
    reinterpret_cast<float2 *>(sv + 12 + 4 * r4)[0] = make_float2(z[4], z[5]);
    if (r4 == 0) {
      reinterpret_cast<float2 *>(sv)[0] = make_float2(r, q);
      reinterpret_cast<float2 *>(sv + 26)[0] = make_float2(0.f, 0.f);
      reinterpret_cast<float4 *>(sv + 28)[0] = make_float4(0.f, 0.f, 0.f, 0.f);
    }
  }
  if (Hres) {
    float m[4];
    sk_exp4(zh + 2, m);
    sk_forward_q(m, iters, eps, r4);
    reinterpret_cast<float4 *>(Hres + t * 16)[r4] = make_float4(m[0], m[1], m[2], m[3]);
  }
}

void launch_proj_fwd(hipStream_t s, bool f32, int64_t N, int64_t C, const void *X, const float *W,
                     const float *alpha, const float *hbias, float rms_eps, float *H_pre,
                     float *H_post, float *logits, float *saved, float *H_res, int iters, float eps,
                     void *ws) {
  const int64_t K = 4 * C;
  const int64_t Kp = kpad64(K);
  char *base = (char *)ws;
  void *wpk = base;
  float *part = (float *)(base + align256(wpack_bytes(C, f32)));
  if (f32) {
    const unsigned pack_blocks = (unsigned)((Kp / 8 * kJ + 255) / 256);
    const unsigned pblocks = (unsigned)(((N + kTB - 1) / kTB) * kSplitK);
    hipLaunchKernelGGL((pack_w_kernel<true>), dim3(pack_blocks), dim3(256), 0, s, W, wpk, K, Kp);
    hipLaunchKernelGGL(proj_partial_f32_kernel, dim3(pblocks), dim3(256), 0, s, X, wpk, part, N, K);
  } else {
    const unsigned pack_blocks = (unsigned)((Kp / 8 * kWcol + 255) / 256);
    const unsigned pblocks = (unsigned)(((N + kDmaTok - 1) / kDmaTok) * kSplitK);
    const size_t lds = (size_t)kDmaStages * kStageElems * sizeof(bf16_t);
    hipLaunchKernelGGL((pack_w_kernel<false>), dim3(pack_blocks), dim3(256), 0, s, W, wpk, K, Kp);
    // rows a multiple of 16 KB apart, 32 KB or more: staggered walk starts
    // over 4 sub-slices
    if ((2 * K) % 16384 == 0 && 2 * K >= 32768)
      hipLaunchKernelGGL(proj_partial_dma_kernel<4>, dim3(pblocks), dim3(kDmaWaves * 64), lds, s,
                         (const bf16_t *)X, (const bf16_t *)wpk, part, N, K);
    else
      hipLaunchKernelGGL(proj_partial_dma_kernel<1>, dim3(pblocks), dim3(kDmaWaves * 64), lds, s,
                         (const bf16_t *)X, (const bf16_t *)wpk, part, N, K);
  }
  hipLaunchKernelGGL(proj_finalize_kernel, dim3((unsigned)((N + 15) / 16)), dim3(64), 0, s, part,
                     alpha, hbias, rms_eps, H_pre, H_post, logits, saved, H_res, iters, eps, N, K);
}

void launch_proj_fwd_fma(hipStream_t s, int64_t N, int64_t C, const void *X, const float *W, const float *alpha,
                         const float *hbias, float rms_eps, float *H_pre, float *H_post, float *logits,
                         float *saved, void *ws) {
  const int64_t K = 4 * C;
  float *part = (float *)((char *)ws + align256(wpack_bytes(C, false)));
  const unsigned pblocks = (unsigned)(((N + kFmaTok - 1) / kFmaTok) * kSplitK);
  hipLaunchKernelGGL(proj_partial_fma_kernel, dim3(pblocks), dim3(256), 0, s, (const bf16_t *)X, W, part, N, K);
  hipLaunchKernelGGL(proj_finalize_kernel, dim3((unsigned)((N + 15) / 16)), dim3(64), 0, s, part, alpha, hbias,
                     rms_eps, H_pre, H_post, logits, saved, (float *)nullptr, 0, 0.f, N, K);
}

// ================================================================== backward
// Per token (proj_bwd_token_kernel): the sigmoid / Sinkhorn backward gives
// dzh; dp = r alpha dzh and c_rms = -S r / (K q) with S = sum_j alpha dzh_j z_j
// (the RMS leg -dr r^2 x / (K q) of the reference backward, using
// dr = S / r and r (q + eps) = 1).  Then, over all tokens and k,
//   dX[t][k] (+)= H_pre[t][i] g[t][c] + c_rms[t] x[t][k] + sum_j dp[t][j] W[k][j]
//   dW[k][j]    = sum_t x[t][k] dp[t][j]
// Both contractions run on MFMA for bf16 activations:
//  * dX: bf16 MFMA on the exact three-term splits of dp (hi + mid + lo, from
//    the per-token record) and of W (split in registers), keeping the six
//    term products hh, hm, mh, hl, lh, mm; the three dropped ones are below
//    2^-24 of |dp||W|.  Two terms are not enough here: for an all-zero
//    residual row r = 1/eps amplifies dp to ~1e5 while dX entries cancel to
//    O(1).
//  * dW: bf16 MFMA.  The contraction runs over tokens, so the X tile is
//    staged in LDS and 8-token columns are read as A fragments; the B
//    fragments are 8-token columns of the dp terms gathered from the
//    records.
// fp32 activations use a VALU kernel for both contractions.
constexpr int kDpf = 32;     // fp32 per-token record: dp[24], c_rms, pad
constexpr int kDpaBytes = 160;  // bf16 per-token record: dp terms [3][24], c_rms (fp32), pad
constexpr int kTokTB = 64;      // tokens per workgroup of the per-token kernel
constexpr int kBwKW = 64;    // k per wave in the MFMA kernel
constexpr int kBwKT = 4 * kBwKW;
constexpr int kDxK = 4;      // k per thread in the fp32 VALU kernel
constexpr int kDxKT = 256 * kDxK;

static int64_t round_up(int64_t a, int64_t b) { return (a + b - 1) / b * b; }

// Tokens per block of the dX / dW kernels (a multiple of 32).  fp32: about
// 2048 workgroups.  bf16: the grid (token blocks x k tiles) is sized to fill
// whole multiples of kCUs workgroups (the kernel runs two per CU; blocks of
// 512 to 2048 tokens measured within 1% of each other); among equally full
// choices the fewest token blocks win (fewer dW partials to reduce).
constexpr int64_t kCUs = 256;
static int64_t bwd_token_block(int64_t N, int64_t K, bool f32) {
  if (f32) {
    const int64_t nkt = (K + kDxKT - 1) / kDxKT;
    const int64_t tb = (N * nkt + 2047) / 2048;
    return round_up(tb < 32 ? 32 : tb, 32);
  }
  if (N <= 0) return 32;
  const int64_t nkt = (K + kBwKT - 1) / kBwKT;
  int64_t best_tb = round_up(N, 32), best_fill = -1, best_n = 0;
  for (int64_t want = 1; want <= 64; ++want) {
    const int64_t tb = round_up((N + want - 1) / want, 32);
    const int64_t n = (N + tb - 1) / tb;
    const int64_t wgs = n * nkt;
    const int64_t fill = wgs * 100 / (round_up(wgs, kCUs));  // percent of the last round used
    if (fill > best_fill || (fill == best_fill && n < best_n)) {
      best_fill = fill;
      best_n = n;
      best_tb = tb;
    }
  }
  return best_tb;
}

struct BwdWs {
  float *dpf, *dhpre, *ppart, *dwpart;  // dpf: fp32 activations only
  char *dpA;                            // bf16 activations only
  int64_t npad, nblk, tbsz, ntb;
  size_t bytes;                         // workspace size
};

static BwdWs bwd_layout(void *ws, int64_t N, int64_t C, bool f32) {
  const int64_t K = 4 * C;
  BwdWs L{};
  L.npad = round_up(N, 32);
  L.nblk = (L.npad + kTokTB - 1) / kTokTB;  // per-token kernel workgroups
  L.tbsz = bwd_token_block(N, K, f32);
  L.ntb = (N + L.tbsz - 1) / L.tbsz;
  size_t off = 0;
  char *b = (char *)ws;
  auto take = [&](size_t bytes) { char *p = b ? b + off : nullptr; off += align256(bytes); return p; };
  if (f32) L.dpf = (float *)take((size_t)N * kDpf * 4);
  else L.dpA = take((size_t)kDpaBytes * L.npad);
  L.dhpre = (float *)take((size_t)N * 16);
  L.ppart = (float *)take((size_t)L.nblk * 32 * 4);
  L.dwpart = (float *)take((size_t)L.ntb * K * kJ * 4);
  L.bytes = off;
  return L;
}

size_t proj_bwd_ws(int64_t N, int64_t C, bool f32) { return bwd_layout(nullptr, N, C, f32).bytes; }

__device__ __forceinline__ uint16_t bf16_bits(float v) { return __builtin_bit_cast(uint16_t, (__bf16)v); }

// Four lanes per token (the quad layout of the Sinkhorn code), 64 tokens per
// 256-thread workgroup; lane r owns the columns r (PRE), 4 + r (POST) and
// 8 + 4r .. 11 + 4r (RES row r).  The grid covers npad tokens (tokens >= N
// only zero their dpA record).  Workgroup partial sums of dhbias (24) and
// dalpha (3) go to ppart.  MFMA_OUT (bf16 activations): the token's record
// for the MFMA kernel is the exact three-term bf16 split of dp, [term][j],
// then c_rms (fp32) and zero padding (kDpaBytes), staged in LDS and written
// as whole 16-byte pieces.  Otherwise dp and c_rms go to the fp32 row dpf.
template <bool MFMA_OUT>
__global__ __launch_bounds__(256) void proj_bwd_token_kernel(
    const float *__restrict__ alpha, const float *__restrict__ saved, const float *__restrict__ Hpre,
    const float *__restrict__ Hpost, const float *__restrict__ dHpre, const float *__restrict__ dHpost,
    const float *__restrict__ dL_in, const float *__restrict__ dHres, const float *__restrict__ logits,
    int iters, float eps, float *__restrict__ dpf, char *__restrict__ dpA,
    float *__restrict__ ppart, float *__restrict__ dL_out, float *__restrict__ dHpre_out, int64_t N,
    int64_t npad, int64_t K) {
  constexpr int kRec = MFMA_OUT ? kDpaBytes : kDpf * 4;  // bytes per staged token
  __shared__ float red[4][28];
  __shared__ __attribute__((aligned(16))) char stage[kTokTB * kRec];
  const int r4 = threadIdx.x & 3;
  const int tl = threadIdx.x >> 2;
  const int64_t t0 = (int64_t)blockIdx.x * kTokTB;
  const int64_t t = t0 + tl;
  char *st = stage + tl * kRec;
  float contrib[27];
#pragma unroll
  for (int e = 0; e < 27; ++e) contrib[e] = 0.f;
  if (t < N) {  // whole quads
    float g[4];
    {
      const float4 w = reinterpret_cast<const float4 *>((dL_in ? dL_in : dHres) + t * 16)[r4];
      g[0] = w.x; g[1] = w.y; g[2] = w.z; g[3] = w.w;
    }
    if (!dL_in) {
      const float4 w = reinterpret_cast<const float4 *>(logits + t * 16)[r4];
      const float l[4] = {w.x, w.y, w.z, w.w};
      sk_backward_q(l, g, iters, eps, r4);
    }
    if (dL_out) reinterpret_cast<float4 *>(dL_out + t * 16)[r4] = make_float4(g[0], g[1], g[2], g[3]);
    const float *sv = saved + t * kSavedStride;
    const float r = sv[0], q = sv[1];
    // owned columns u: 0 -> r4 (PRE), 1 -> 4 + r4 (POST), 2..5 -> 8 + 4 r4 + (u - 2) (RES)
    float z[6], dzh[6];
    z[0] = sv[2 + r4];
    z[1] = sv[6 + r4];
#pragma unroll
    for (int b = 0; b < 4; ++b) z[2 + b] = sv[10 + 4 * r4 + b];
    const float hp = Hpre[t * 4 + r4];
    const float dhp = dHpre[t * 4 + r4];
    if (dHpre_out) dHpre_out[t * 4 + r4] = dhp;
    dzh[0] = dhp * (hp * (1.f - hp));
    const float hq = Hpost[t * 4 + r4];
    dzh[1] = dHpost[t * 4 + r4] * (hq * (1.f - 0.5f * hq));
#pragma unroll
    for (int b = 0; b < 4; ++b) dzh[2 + b] = g[b];
    float a3[3] = {1.f, 1.f, 1.f};
    if (alpha) { a3[0] = alpha[0]; a3[1] = alpha[1]; a3[2] = alpha[2]; }
    float Sp = 0.f, dp[6];
#pragma unroll
    for (int u = 0; u < 6; ++u) {
      const int seg = u == 0 ? 0 : (u == 1 ? 1 : 2);
      contrib[kJ + seg] += dzh[u] * z[u];
      const float dz = a3[seg] * dzh[u];
      Sp += dz * z[u];
      dp[u] = r * dz;
    }
    // dhbias contributions of the owned columns (compile-time slots, lane-selected)
#pragma unroll
    for (int j = 0; j < kJ; ++j) {
      const int owner = j < 4 ? j : (j < 8 ? j - 4 : (j - 8) >> 2);
      const int u = j < 4 ? 0 : (j < 8 ? 1 : 2 + ((j - 8) & 3));
      contrib[j] = r4 == owner ? dzh[u] : 0.f;
    }
    const float S = quad_sum(Sp);
    const float crms = q > 0.f ? -S * r / ((float)K * q) : 0.f;
    if (MFMA_OUT) {
      // terms [3][24] bf16 at byte 48 * term + 2 * j, then c_rms at byte 144
      uint16_t hb[3][6];
#pragma unroll
      for (int u = 0; u < 6; ++u) {
        const float h = bf16_round(dp[u]);
        const float r1 = dp[u] - h;
        const float m = bf16_round(r1);
        hb[0][u] = bf16_bits(h);
        hb[1][u] = bf16_bits(m);
        hb[2][u] = bf16_bits(r1 - m);
      }
#pragma unroll
      for (int tm = 0; tm < 3; ++tm) {
        uint16_t *row = reinterpret_cast<uint16_t *>(st + 48 * tm);
        row[r4] = hb[tm][0];
        row[4 + r4] = hb[tm][1];
        *reinterpret_cast<uint2 *>(row + 8 + 4 * r4) =
            make_uint2((uint32_t)hb[tm][2] | ((uint32_t)hb[tm][3] << 16), (uint32_t)hb[tm][4] | ((uint32_t)hb[tm][5] << 16));
      }
      if (r4 == 0) *reinterpret_cast<uint4 *>(st + 144) = make_uint4(__float_as_uint(crms), 0u, 0u, 0u);
    } else {
      float *row = reinterpret_cast<float *>(st);
      row[r4] = dp[0];
      row[4 + r4] = dp[1];
      *reinterpret_cast<float4 *>(row + 8 + 4 * r4) = make_float4(dp[2], dp[3], dp[4], dp[5]);
      if (r4 == 0) {
        *reinterpret_cast<float4 *>(row + 24) = make_float4(crms, 0.f, 0.f, 0.f);
        *reinterpret_cast<float4 *>(row + 28) = make_float4(0.f, 0.f, 0.f, 0.f);
      }
    }
  } else if (MFMA_OUT && t < npad) {  // padding token: a zero record
    reinterpret_cast<uint4 *>(st)[r4] = make_uint4(0u, 0u, 0u, 0u);
    reinterpret_cast<uint4 *>(st)[4 + r4] = make_uint4(0u, 0u, 0u, 0u);
    if (r4 < 2) reinterpret_cast<uint4 *>(st)[8 + r4] = make_uint4(0u, 0u, 0u, 0u);
  }
  __syncthreads();
  // staged records -> global, whole 16-byte pieces
  const int64_t nt = min<int64_t>(kTokTB, (MFMA_OUT ? npad : N) - t0);
  if (nt > 0) {
    const uint4 *src = reinterpret_cast<const uint4 *>(stage);
    uint4 *dst = reinterpret_cast<uint4 *>(MFMA_OUT ? dpA + t0 * kDpaBytes : reinterpret_cast<char *>(dpf + t0 * kDpf));
    for (int i = threadIdx.x; i < nt * (kRec / 16); i += 256) dst[i] = src[i];
  }
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
#pragma unroll
  for (int e = 0; e < 27; ++e) {
    const float s = wave_sum(contrib[e]);
    if (lane == 0) red[wave][e] = s;
  }
  __syncthreads();
  if (threadIdx.x < 27)
    ppart[blockIdx.x * 32 + threadIdx.x] =
        (red[0][threadIdx.x] + red[1][threadIdx.x]) + (red[2][threadIdx.x] + red[3][threadIdx.x]);
}

// dhbias / dalpha: 32 lanes per value stride the per-block partials (four
// loads in flight each), then the 32 partial sums are added in a fixed
// pairwise tree (deterministic).
__global__ __launch_bounds__(1024) void param_final_kernel(const float *__restrict__ ppart, int64_t nblk,
                                                           float *__restrict__ dalpha,
                                                           float *__restrict__ dhbias) {
  __shared__ float red[32][32];
  const int e = threadIdx.x & 31, part = threadIdx.x >> 5;
  float s = 0.f;
#pragma unroll 4
  for (int64_t b = part; b < nblk; b += 32) s += ppart[b * 32 + e];
  red[part][e] = s;
  __syncthreads();
  for (int w = 16; w > 0; w >>= 1) {
    if (part < w) red[part][e] += red[part + w][e];
    __syncthreads();
  }
  if (threadIdx.x >= 27) return;
  const float tot = red[0][e];
  if (e < kJ) {
    if (dhbias) dhbias[e] = tot;
  } else if (dalpha) {
    dalpha[e - kJ] = tot;
  }
}

// ------------------------------------------------------------------ MFMA dX / dW kernel
// Workgroup = 8 waves on one token block and one k tile of four 64-k
// quarters, walked in 16-token sub-tiles through a 3-stage LDS ring:
//  * waves 4..7 (loaders) fill each stage with global_load_lds_dwordx4: the X
//    tile, the g tile, the h_post_bda upstream gradient G (POST) and the 16
//    per-token dp records of the sub-tile, two sub-tiles ahead.  With dW they
//    then run x^T dp on MFMA (32x32x16 with the 16 tokens as the
//    contraction; loader w-4 owns quarter w-4; A = 8 tokens of an X column
//    read from LDS, B = the same 8 tokens of a dp term's column);
//  * waves 0..3 own one quarter each: dp W^T on v_mfma_f32_16x16x32_bf16,
//    one 16 x 16 block per 16 channels; the contraction runs over j (24,
//    padded to 32) once per kept pair of exact bf16 terms (hh, hm, mh, hl,
//    lh, mm: the products above 2^-24 relative), A = a dp term's 8 j of one
//    token (one 16-byte record piece; lane group 3 holds zeros), B = a W
//    term's 8 j of one channel.  Each W term is held once in registers (3 x 4
//    per 16 channels) and serves every pair it appears in.  The 16 x 64
//    result goes through a private LDS area, then the dX epilogue with dX_in,
//    H_pre and H_res rows loaded one sub-tile ahead into registers.
// The ring (20,992 bytes a stage with the h_post_bda term) and the
// accumulator tiles take at most 80,384 bytes and every wave stays within
// 128 registers, so two workgroups share a CU.
// One barrier per sub-tile: loaders first wait for their own loads of the
// sub-tile (s_waitcnt vmcnt), so the barrier both publishes the stage and
// guarantees that the slot refilled next has been read by every wave.  The
// loaders issue no other global memory instructions inside the loop, which
// keeps their vmcnt arithmetic exact; dX waves never issue DMA, so their LDS
// reads need no wait on vmcnt.
// In every 128-byte LDS row (64 bf16 of X, g or G) the 16-byte piece p of
// row r sits in slot p ^ (r & 7): the DMA lanes of an instruction cover 8
// rows x 8 slots, and the row-wise and column-wise reads below spread over
// the banks.  The 16 dp records (160 bytes each) are copied as they are
// (2.5 KB: loaders 0-2, half a copy on loader 2).
// Channel tiles: without the h_post_bda term, 256 consecutive k (g pieces
// addressed per piece; when C is a multiple of 256 the four tiles that read
// the same g tile run back to back on one XCD).  With it (POST), one
// 64-channel range c0 for all 4 streams (quarter i = stream i): the g tile
// (16 x 64) and the G tile (4 x 16 x 64) are then loaded once and shared by
// the four dX waves, which each need all four streams of G; these tiles are
// walked in XCD-contiguous order, so an XCD's CUs read neighbouring row
// pieces of the same tokens together.
constexpr int kB3Stages = 3;
constexpr int kB3Quarter = 16 * 128;  // bytes of one 16 x 64 bf16 tile
constexpr int kB3AccRow = 68;         // floats per row of a wave's 16 x 64 accumulator tile

template <bool HAS_G, bool POST>
struct B3Lay {
  static constexpr int X = 0;
  static constexpr int G = 4 * kB3Quarter;                               // g
  static constexpr int Q = G + (HAS_G ? (POST ? 1 : 4) * kB3Quarter : 0);  // G of h_post_bda
  static constexpr int P = Q + (POST ? 4 * kB3Quarter : 0);              // 16 dp records
  static constexpr int stage = P + 16 * kDpaBytes;
  static constexpr int acc = kB3Stages * stage;
  static constexpr int total = acc + 4 * 16 * kB3AccRow * 4;
  static_assert(2 * total <= 160 * 1024, "two workgroups' LDS on one CU");
};

typedef __attribute__((ext_vector_type(4))) float f32x4;

// Per-lane inputs of one sub-tile's dX epilogue, for rows er + 8q: dX_in,
// H_pre and the row's H_res row.
struct DxPre16 {
  u32x4 d[2];
  float hp[2];
  float4 hr[2];
};

template <bool ACCUM, bool HAS_G, bool DW, bool POST>
__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(4, 4))) void proj_bwd_mfma16_kernel(
    const bf16_t *__restrict__ X, const float *__restrict__ W, const char *__restrict__ dpA,
    const float *__restrict__ Hpre, const bf16_t *__restrict__ gr, const bf16_t *__restrict__ Gp,
    const float *__restrict__ Hres, bf16_t *__restrict__ dX, float *__restrict__ dWpart, int64_t N, int64_t C,
    int64_t tbsz, int group4) {
  constexpr bool SPW = POST;  // stream-per-wave channel tiles
  using L = B3Lay<HAS_G, POST>;
  extern __shared__ __attribute__((aligned(16))) char b3lds[];
  const int64_t K = 4 * C;
  const int64_t nkt = SPW ? (C + kBwKW - 1) / kBwKW : (K + 4 * kBwKW - 1) / (4 * kBwKW);
  const int64_t ntb = (N + tbsz - 1) / tbsz;
  int64_t kt, tbi;
  if (SPW) {  // XCD-contiguous tile order
    const int64_t T = nkt * ntb, per = (T + 7) / 8;
    const int64_t tile = (int64_t)(blockIdx.x % 8) * per + blockIdx.x / 8;
    if (tile >= T) return;  // grid padding to a multiple of 8 (whole workgroup)
    tbi = tile / nkt;
    kt = tile % nkt;
  } else if (group4) {  // the four k tiles that read the same g tile on one XCD, back to back
    const int64_t b = blockIdx.x, nct = C / (4 * kBwKW);
    const int64_t pidx = (b / 32) * 8 + (b % 8);
    if (pidx >= ntb * nct) return;  // grid padding to a multiple of 32 (whole workgroup)
    tbi = pidx / nct;
    kt = ((b / 8) % 4) * nct + pidx % nct;
  } else {
    tbi = blockIdx.x / nkt;
    kt = blockIdx.x % nkt;
  }
  const int64_t tb = ntb - 1 - tbi;  // token blocks from the last down
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const bool loader = wave >= 4;
  const int kq = wave & 3;  // quarter of this wave
  // k of the quarter's first column and the number of its real columns
  const int64_t c0 = SPW ? kt * kBwKW : 0;
  const int64_t kbase = SPW ? kq * C + c0 : kt * 4 * kBwKW + kq * kBwKW;
  const int64_t nvalid = SPW ? min<int64_t>(kBwKW, C - c0) : max<int64_t>(0, min<int64_t>(kBwKW, K - kbase));
  const int64_t ksafe = SPW ? kbase : kt * 4 * kBwKW;  // a real k of the tile (redirect target)

  const int64_t t_begin = tb * tbsz;
  const int64_t t_end = min(N, t_begin + tbsz);
  const int nsub = (int)((t_end - t_begin + 15) / 16);

  // ---- loader geometry: lane -> (row in its 8-row group, 16-byte piece)
  const int drow = lane >> 3;
  const int dpiece = (lane & 7) ^ drow;
  const bool dvalid = 8 * dpiece < nvalid;
  const int64_t xk = dvalid ? kbase + 8 * dpiece : ksafe;
  // channel of the lane's piece (g and G tiles); a real channel when the
  // piece lies past the tile
  const int64_t gcol = SPW ? (dvalid ? c0 + 8 * dpiece : c0) : xk - (xk / C) * C;
  const int nload = 2 + (HAS_G ? (SPW ? (kq < 2 ? 1 : 0) : 2) : 0) + (POST ? 2 : 0) + (kq < 3 ? 1 : 0);

  auto issue = [&](int i) {
    char *st = b3lds + (i % kB3Stages) * L::stage;
    const int64_t t0 = t_begin + 16 * (int64_t)i;
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      const int64_t t = min(t0 + 8 * q + drow, N - 1);
      dma16(X + t * K + xk, st + L::X + kq * kB3Quarter + q * 1024);
      if (HAS_G && !SPW) dma16(gr + t * C + gcol, st + L::G + kq * kB3Quarter + q * 1024);
      if (POST) dma16(Gp + (t * 4 + kq) * C + gcol, st + L::Q + kq * kB3Quarter + q * 1024);
    }
    if (HAS_G && SPW && kq < 2) {
      const int64_t t = min(t0 + 8 * kq + drow, N - 1);
      dma16(gr + t * C + gcol, st + L::G + kq * 1024);
    }
    // the sub-tile's 16 records are contiguous (they exist up to the
    // 32-token padding): 2.5 KB, the last half copy on lanes 0..31
    const char *rs = dpA + t0 * kDpaBytes;
    if (kq < 2) dma16(rs + kq * 1024 + lane * 16, st + L::P + kq * 1024);
    if (kq == 2 && lane < 32) dma16(rs + 2048 + lane * 16, st + L::P + 2048);
  };

  // ---- dX geometry: lane -> token rows er + 8q (q = 0, 1) and 8 channels
  // at ek of the wave's 64, so eight lanes store one row's 128-byte line
  const int er = lane >> 3;
  const int ek = (lane & 7) * 8;
  const bool ekv = ek < nvalid;
  const int64_t kx = kbase + ek;
  const int si_x = SPW ? kq : (int)(min<int64_t>(kx, K - 1) / C);  // stream of the lane's k

  auto prefetch = [&](DxPre16 &P, int i) {
    const int64_t t0 = t_begin + 16 * (int64_t)i;
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      const int64_t tt = t0 + er + 8 * q;
      const bool v = tt < N && ekv;
      if (ACCUM) P.d[q] = v ? *reinterpret_cast<const u32x4 *>(dX + tt * K + kx) : u32x4{0u, 0u, 0u, 0u};
      if (HAS_G) P.hp[q] = v ? Hpre[tt * 4 + si_x] : 0.f;
      if (POST)
        P.hr[q] = tt < N ? *reinterpret_cast<const float4 *>(Hres + tt * 16 + kq * 4) : make_float4(0.f, 0.f, 0.f, 0.f);
    }
  };

  // 16x16x32 layout: lane (n = lane & 15, group gq = lane >> 4); A holds row
  // n's k = 8 gq .. 8 gq + 7, B column n's same k, D rows 4 gq + r, column n
  const int n16 = lane & 15, gq = lane >> 4;
  // B fragments: W term m of channel 16 bi + n16, j = 8 gq .. + 7 (zero for gq = 3)
  u32x4 wt[4][3];
  f32x4 accX[4];
  f32x16 accW[2];
  if (!loader) {
#pragma unroll
    for (int bi = 0; bi < 4; ++bi) {
      const bool kv = 16 * bi + n16 < nvalid && gq < 3;
      const float *wr = W + (kbase + 16 * bi + n16) * kJ + 8 * gq;
      const float4 v0 = kv ? *reinterpret_cast<const float4 *>(wr) : make_float4(0.f, 0.f, 0.f, 0.f);
      const float4 v1 = kv ? *reinterpret_cast<const float4 *>(wr + 4) : make_float4(0.f, 0.f, 0.f, 0.f);
      const float w8[8] = {v0.x, v0.y, v0.z, v0.w, v1.x, v1.y, v1.z, v1.w};
      float th[8], tmid[8], tl[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        th[e] = bf16_round(w8[e]);
        const float r1 = w8[e] - th[e];
        tmid[e] = bf16_round(r1);
        tl[e] = r1 - tmid[e];
      }
      wt[bi][0] = u32x4{pack_bf16x2(th[0], th[1]), pack_bf16x2(th[2], th[3]), pack_bf16x2(th[4], th[5]),
                        pack_bf16x2(th[6], th[7])};
      wt[bi][1] = u32x4{pack_bf16x2(tmid[0], tmid[1]), pack_bf16x2(tmid[2], tmid[3]), pack_bf16x2(tmid[4], tmid[5]),
                        pack_bf16x2(tmid[6], tmid[7])};
      wt[bi][2] = u32x4{pack_bf16x2(tl[0], tl[1]), pack_bf16x2(tl[2], tl[3]), pack_bf16x2(tl[4], tl[5]),
                        pack_bf16x2(tl[6], tl[7])};
    }
  }
#pragma unroll
  for (int rt = 0; rt < 2; ++rt)
#pragma unroll
    for (int r = 0; r < 16; ++r) accW[rt][r] = 0.f;

  float *acc_t = reinterpret_cast<float *>(b3lds + L::acc) + kq * 16 * kB3AccRow;

  // The two roles run separate loops with the same barrier sequence: a dX
  // wave never issues an LDS DMA, so its LDS reads need no wait on vmcnt.
  if (loader) {
    const int col = lane & 31, h = lane >> 5;
    issue(0);
    if (nsub > 1) issue(1);
    for (int i = 0; i < nsub; ++i) {
      if (i + 1 < nsub) wait_vmcnt_le(nload); else wait_vmcnt<0>();
      lds_barrier();
      const char *st = b3lds + (i % kB3Stages) * L::stage;
      if (i + 2 < nsub) issue(i + 2);
      if (DW) {
        // dW += X^T dp: A = 8 tokens (8h .. 8h + 7) of X column k = 32 rt + col,
        // B = the same 8 tokens of dp term tm at j = col
        const bf16_t *xs = reinterpret_cast<const bf16_t *>(st + L::X + kq * kB3Quarter);
        u32x4 xa[2];
#pragma unroll
        for (int rt = 0; rt < 2; ++rt) {
          uint32_t w4[4];
          const int kk = 32 * rt + col;
#pragma unroll
          for (int p = 0; p < 4; ++p) {
            const int r0 = 8 * h + 2 * p;
            const uint32_t lo16 = xs[r0 * 64 + 8 * ((kk >> 3) ^ (r0 & 7)) + (kk & 7)];
            const uint32_t hi16 = xs[(r0 + 1) * 64 + 8 * ((kk >> 3) ^ ((r0 + 1) & 7)) + (kk & 7)];
            w4[p] = lo16 | (hi16 << 16);
          }
          xa[rt] = u32x4{w4[0], w4[1], w4[2], w4[3]};
        }
        const char *ps = st + L::P;
#pragma unroll
        for (int tm = 0; tm < 3; ++tm) {
          uint32_t w4[4] = {0u, 0u, 0u, 0u};
          if (col < kJ) {
#pragma unroll
            for (int p = 0; p < 4; ++p) {
              const int r0 = 8 * h + 2 * p;
              const int off = (tm * 3 + (col >> 3)) * 16 + (col & 7) * 2;
              const uint32_t lo16 = *reinterpret_cast<const uint16_t *>(ps + r0 * kDpaBytes + off);
              const uint32_t hi16 = *reinterpret_cast<const uint16_t *>(ps + (r0 + 1) * kDpaBytes + off);
              w4[p] = lo16 | (hi16 << 16);
            }
          }
          const u32x4 bfr = u32x4{w4[0], w4[1], w4[2], w4[3]};
#pragma unroll
          for (int rt = 0; rt < 2; ++rt)
            accW[rt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, xa[rt]),
                                                               __builtin_bit_cast(bf16x8, bfr), accW[rt], 0, 0, 0);
        }
      }
    }
    if (DW && col < kJ) {
#pragma unroll
      for (int rt = 0; rt < 2; ++rt)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int e = 32 * rt + 8 * (r >> 2) + 4 * h + (r & 3);
          if (e < nvalid) dWpart[(tb * K + kbase + e) * kJ + col] = accW[rt][r];
        }
    }
  } else {
    wait_vmcnt<0>();  // W in registers: only the prefetches are pending inside the loop
    DxPre16 cur;
    prefetch(cur, 0);
    for (int i = 0; i < nsub; ++i) {
      lds_barrier();
      const char *st = b3lds + (i % kB3Stages) * L::stage;
      const int64_t t0 = t_begin + 16 * (int64_t)i;
      // (a) dp W^T for 16 tokens x 64 channels: A fragments (token t0 + n16,
      // dp term s, j = 8 gq ..) from the records, 4 blocks x 6 term pairs
      const char *ps = st + L::P;
      u32x4 af[3];
#pragma unroll
      for (int sdp = 0; sdp < 3; ++sdp)
        af[sdp] = gq < 3 ? *reinterpret_cast<const u32x4 *>(ps + n16 * kDpaBytes + (sdp * 3 + gq) * 16)
                         : u32x4{0u, 0u, 0u, 0u};
#pragma unroll
      for (int bi = 0; bi < 4; ++bi) {
        f32x4 a4 = f32x4{0.f, 0.f, 0.f, 0.f};
        // pairs (dp term, W term): hh, hm, mh, hl, lh, mm
        a4 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, af[0]),
                                                     __builtin_bit_cast(bf16x8, wt[bi][0]), a4, 0, 0, 0);
        a4 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, af[0]),
                                                     __builtin_bit_cast(bf16x8, wt[bi][1]), a4, 0, 0, 0);
        a4 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, af[1]),
                                                     __builtin_bit_cast(bf16x8, wt[bi][0]), a4, 0, 0, 0);
        a4 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, af[0]),
                                                     __builtin_bit_cast(bf16x8, wt[bi][2]), a4, 0, 0, 0);
        a4 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, af[2]),
                                                     __builtin_bit_cast(bf16x8, wt[bi][0]), a4, 0, 0, 0);
        a4 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, af[1]),
                                                     __builtin_bit_cast(bf16x8, wt[bi][1]), a4, 0, 0, 0);
        accX[bi] = a4;
      }
      // (b) dX = dp W^T + c_rms x + H_pre g + sum_i H_res[j][i] G[i] + dX_in,
      // through the wave's LDS accumulator tile
      __builtin_amdgcn_sched_barrier(0);
      wait_vmcnt<0>();
      const char *xs = st + L::X + kq * kB3Quarter;
      const char *gs = st + L::G + (SPW ? 0 : kq * kB3Quarter);
      const char *qs = st + L::Q;
#pragma unroll
      for (int bi = 0; bi < 4; ++bi)
#pragma unroll
        for (int r = 0; r < 4; ++r) acc_t[(4 * gq + r) * kB3AccRow + 16 * bi + n16] = accX[bi][r];
      wave_lds_sync();
#pragma unroll
      for (int q = 0; q < 2; ++q) {
        const int row = er + 8 * q;
        const int64_t tt = t0 + row;
        if (!(tt < N && ekv)) continue;
        const int slot = (ek >> 3) ^ (row & 7);
        const float4 a0 = *reinterpret_cast<const float4 *>(&acc_t[row * kB3AccRow + ek]);
        const float4 a1 = *reinterpret_cast<const float4 *>(&acc_t[row * kB3AccRow + ek + 4]);
        const float acc8[8] = {a0.x, a0.y, a0.z, a0.w, a1.x, a1.y, a1.z, a1.w};
        const float crms = *reinterpret_cast<const float *>(ps + row * kDpaBytes + 9 * 16);
        const u32x4 xv = *reinterpret_cast<const u32x4 *>(xs + row * 128 + 16 * slot);
        const uint32_t xw[4] = {xv.x, xv.y, xv.z, xv.w};
        float o[8];
#pragma unroll
        for (int p = 0; p < 4; ++p) {
          o[2 * p] = acc8[2 * p] + crms * bf16_lo(xw[p]);
          o[2 * p + 1] = acc8[2 * p + 1] + crms * bf16_hi(xw[p]);
        }
        if (HAS_G) {
          const u32x4 gv = *reinterpret_cast<const u32x4 *>(gs + row * 128 + 16 * slot);
          const uint32_t gw[4] = {gv.x, gv.y, gv.z, gv.w};
          const float hp = cur.hp[q];
#pragma unroll
          for (int p = 0; p < 4; ++p) {
            o[2 * p] += hp * bf16_lo(gw[p]);
            o[2 * p + 1] += hp * bf16_hi(gw[p]);
          }
        }
        if (POST) {  // h_post_bda term: sum_i H_res[j][i] G[i], j = this wave's stream
          const float4 hr = cur.hr[q];
          uint32_t gw[4][4];
#pragma unroll
          for (int si = 0; si < 4; ++si) {
            const u32x4 v = *reinterpret_cast<const u32x4 *>(qs + si * kB3Quarter + row * 128 + 16 * slot);
            gw[si][0] = v.x; gw[si][1] = v.y; gw[si][2] = v.z; gw[si][3] = v.w;
          }
#pragma unroll
          for (int p = 0; p < 4; ++p) {
            o[2 * p] += (hr.x * bf16_lo(gw[0][p]) + hr.y * bf16_lo(gw[1][p])) +
                        (hr.z * bf16_lo(gw[2][p]) + hr.w * bf16_lo(gw[3][p]));
            o[2 * p + 1] += (hr.x * bf16_hi(gw[0][p]) + hr.y * bf16_hi(gw[1][p])) +
                            (hr.z * bf16_hi(gw[2][p]) + hr.w * bf16_hi(gw[3][p]));
          }
        }
        if (ACCUM) {
          const uint32_t dw4[4] = {cur.d[q].x, cur.d[q].y, cur.d[q].z, cur.d[q].w};
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
        *reinterpret_cast<uint4 *>(dX + tt * K + kx) = ow;
      }
      wave_lds_sync();  // the reads of the accumulator area precede the next sub-tile's writes
      if (i + 1 < nsub) prefetch(cur, i + 1);
    }
  }
}

// ------------------------------------------------------------------ fp32 VALU dX / dW kernel
template <bool ACCUM, bool HAS_G, bool DW>
__global__ __launch_bounds__(256) void proj_bwd_dx_f32_kernel(
    const float *__restrict__ X, const float *__restrict__ W, const float *__restrict__ dpf,
    const float *__restrict__ Hpre, const float *__restrict__ gr, const float *__restrict__ Gp,
    const float *__restrict__ Hres, float *__restrict__ dX, float *__restrict__ dWpart, int64_t N, int64_t C,
    int64_t tbsz) {
  const int64_t K = 4 * C;
  const int64_t nkt = (K + kDxKT - 1) / kDxKT;
  const int64_t kt = blockIdx.x % nkt;
  const int64_t tb = blockIdx.x / nkt;
  const int64_t k = kt * kDxKT + kDxK * threadIdx.x;
  const bool kv = k < K;
  const int64_t si = k / C;
  const int64_t c = k - si * C;
  float w[kDxK][kJ], dw[kDxK][kJ];
#pragma unroll
  for (int e = 0; e < kDxK; ++e)
#pragma unroll
    for (int j = 0; j < kJ; ++j) {
      w[e][j] = kv ? W[(k + e) * kJ + j] : 0.f;
      dw[e][j] = 0.f;
    }
  const int64_t t_end = min(N, (tb + 1) * tbsz);
  for (int64_t t = tb * tbsz; t < t_end; ++t) {
    const float *rt = dpf + t * kDpf;
    float dp[kJ];
#pragma unroll
    for (int j = 0; j < kJ; ++j) dp[j] = rt[j];
    const float crms = rt[kJ];
    if (!kv) continue;
    const float4 x4 = *reinterpret_cast<const float4 *>(X + t * K + k);
    const float xv[kDxK] = {x4.x, x4.y, x4.z, x4.w};
    float o[kDxK] = {0.f, 0.f, 0.f, 0.f};
    if (ACCUM) {
      const float4 d4 = *reinterpret_cast<const float4 *>(dX + t * K + k);
      o[0] = d4.x; o[1] = d4.y; o[2] = d4.z; o[3] = d4.w;
    }
    if (HAS_G) {
      const float hpi = Hpre[t * 4 + si];
      const float4 g4 = *reinterpret_cast<const float4 *>(gr + t * C + c);
      o[0] += hpi * g4.x; o[1] += hpi * g4.y; o[2] += hpi * g4.z; o[3] += hpi * g4.w;
    }
    if (Gp) {  // h_post_bda term: sum_i H_res[si][i] G[i]
      const float4 hr = *reinterpret_cast<const float4 *>(Hres + t * 16 + si * 4);
      float4 gv[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) gv[i] = *reinterpret_cast<const float4 *>(Gp + (t * 4 + i) * C + c);
      o[0] += (hr.x * gv[0].x + hr.y * gv[1].x) + (hr.z * gv[2].x + hr.w * gv[3].x);
      o[1] += (hr.x * gv[0].y + hr.y * gv[1].y) + (hr.z * gv[2].y + hr.w * gv[3].y);
      o[2] += (hr.x * gv[0].z + hr.y * gv[1].z) + (hr.z * gv[2].z + hr.w * gv[3].z);
      o[3] += (hr.x * gv[0].w + hr.y * gv[1].w) + (hr.z * gv[2].w + hr.w * gv[3].w);
    }
#pragma unroll
    for (int e = 0; e < kDxK; ++e) {
      float acc = crms * xv[e];
#pragma unroll
      for (int j = 0; j < kJ; ++j) acc = fmaf(dp[j], w[e][j], acc);
      o[e] += acc;
      if (DW) {
#pragma unroll
        for (int j = 0; j < kJ; ++j) dw[e][j] = fmaf(xv[e], dp[j], dw[e][j]);
      }
    }
    *reinterpret_cast<float4 *>(dX + t * K + k) = make_float4(o[0], o[1], o[2], o[3]);
  }
  if (DW && kv) {
    float *dst = dWpart + (tb * K + k) * kJ;
#pragma unroll
    for (int e = 0; e < kDxK; ++e)
#pragma unroll
      for (int jq = 0; jq < kJ / 4; ++jq)
        reinterpret_cast<float4 *>(dst + e * kJ)[jq] =
            make_float4(dw[e][4 * jq], dw[e][4 * jq + 1], dw[e][4 * jq + 2], dw[e][4 * jq + 3]);
  }
}

// dW[k][j] = sum over token blocks of the partials, in block order; four
// consecutive entries per thread (K * 24 is a multiple of 4), the partials
// read once with non-temporal loads.
__global__ __launch_bounds__(256) void dw_reduce_kernel(const float *__restrict__ part,
                                                        float *__restrict__ dW, int64_t ntb,
                                                        int64_t KJ) {
  const int64_t i4 = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (4 * i4 >= KJ) return;
  const nt_f32x4 *p = reinterpret_cast<const nt_f32x4 *>(part) + i4;
  const int64_t stride = KJ / 4;
  nt_f32x4 s = {0.f, 0.f, 0.f, 0.f};
#pragma unroll 4
  for (int64_t b = 0; b < ntb; ++b) s += __builtin_nontemporal_load(p + b * stride);
  reinterpret_cast<nt_f32x4 *>(dW)[i4] = s;
}

template <bool ACCUM, bool HAS_G, bool DW, bool POST>
static void launch_b3(hipStream_t s, const ProjBwdArgs &a, const BwdWs &L) {
  const int64_t K = 4 * a.C;
  const int64_t nkt = POST ? (a.C + kBwKW - 1) / kBwKW : (K + 4 * kBwKW - 1) / (4 * kBwKW);
  const int group4 = (!POST && a.C % (4 * kBwKW) == 0) ? 1 : 0;
  const int64_t blocks = POST ? round_up(nkt * L.ntb, 8) : group4 ? round_up(nkt * L.ntb, 32) : nkt * L.ntb;
  const size_t lds = (size_t)B3Lay<HAS_G, POST>::total;
  hipLaunchKernelGGL((proj_bwd_mfma16_kernel<ACCUM, HAS_G, DW, POST>), dim3((unsigned)blocks), dim3(512), lds, s,
                     (const bf16_t *)a.X, a.W, (const char *)L.dpA, a.H_pre, (const bf16_t *)a.g,
                     (const bf16_t *)a.post_G, a.post_H_res, (bf16_t *)a.dX, L.dwpart, a.N, a.C, L.tbsz, group4);
}

template <bool ACCUM, bool HAS_G>
static void launch_b2(hipStream_t s, const ProjBwdArgs &a, const BwdWs &L) {
  if (HAS_G && a.post_G) {  // the fused pre backward with the h_post_bda term
    if (a.dW) launch_b3<ACCUM, true, true, true>(s, a, L);
    else launch_b3<ACCUM, true, false, true>(s, a, L);
  } else {
    if (a.dW) launch_b3<ACCUM, HAS_G, true, false>(s, a, L);
    else launch_b3<ACCUM, HAS_G, false, false>(s, a, L);
  }
}

template <bool ACCUM, bool HAS_G>
static void launch_dx_kernel(hipStream_t s, const ProjBwdArgs &a, const BwdWs &L) {
  const int64_t K = 4 * a.C;
  if (a.f32) {
    const unsigned blocks = (unsigned)(((K + kDxKT - 1) / kDxKT) * L.ntb);
    if (a.dW)
      hipLaunchKernelGGL((proj_bwd_dx_f32_kernel<ACCUM, HAS_G, true>), dim3(blocks), dim3(256), 0, s,
                         (const float *)a.X, a.W, L.dpf, a.H_pre, (const float *)a.g, (const float *)a.post_G,
                         a.post_H_res, (float *)a.dX, L.dwpart, a.N, a.C, L.tbsz);
    else
      hipLaunchKernelGGL((proj_bwd_dx_f32_kernel<ACCUM, HAS_G, false>), dim3(blocks), dim3(256), 0, s,
                         (const float *)a.X, a.W, L.dpf, a.H_pre, (const float *)a.g, (const float *)a.post_G,
                         a.post_H_res, (float *)a.dX, L.dwpart, a.N, a.C, L.tbsz);
  } else {
    launch_b2<ACCUM, HAS_G>(s, a, L);
  }
}

template <bool ACCUM, bool HAS_G>
static void launch_dx(hipStream_t s, const ProjBwdArgs &a, const BwdWs &L) {
  kernel_event(kKernelProjBwdDxDw, s, true);
  launch_dx_kernel<ACCUM, HAS_G>(s, a, L);
  kernel_event(kKernelProjBwdDxDw, s, false);
}

void launch_proj_bwd(hipStream_t s, const ProjBwdArgs &a) {
  const int64_t N = a.N, K = 4 * a.C;
  const BwdWs L = bwd_layout(a.ws, N, a.C, a.f32);
  const float *dHpre = a.dH_pre;
  if (a.g) {  // fused pre backward: dH_pre = g . X per stream
    launch_h_aggregate_bwd(s, a.f32, N, a.C, a.g, a.X, a.H_pre, nullptr, false, L.dhpre);
    dHpre = L.dhpre;
  }
  if (a.f32)
    hipLaunchKernelGGL((proj_bwd_token_kernel<false>), dim3((unsigned)L.nblk), dim3(256), 0, s, a.alpha, a.saved,
                       a.H_pre, a.H_post, dHpre, a.dH_post, a.dL, a.dH_res, a.logits, a.iters, a.eps, L.dpf,
                       L.dpA, L.ppart, a.dL_out, a.dH_pre_out, N, L.npad, K);
  else
    hipLaunchKernelGGL((proj_bwd_token_kernel<true>), dim3((unsigned)L.nblk), dim3(256), 0, s, a.alpha, a.saved,
                       a.H_pre, a.H_post, dHpre, a.dH_post, a.dL, a.dH_res, a.logits, a.iters, a.eps, L.dpf,
                       L.dpA, L.ppart, a.dL_out, a.dH_pre_out, N, L.npad, K);
  const bool hg = a.g != nullptr;
  if (a.accumulate) {
    if (hg) launch_dx<true, true>(s, a, L);
    else launch_dx<true, false>(s, a, L);
  } else {
    if (hg) launch_dx<false, true>(s, a, L);
    else launch_dx<false, false>(s, a, L);
  }
  if (a.dW)
    hipLaunchKernelGGL(dw_reduce_kernel, dim3((unsigned)((K * kJ / 4 + 255) / 256)), dim3(256), 0, s, L.dwpart,
                       a.dW, L.ntb, K * kJ);
  if (a.dalpha || a.dhbias)
    hipLaunchKernelGGL(param_final_kernel, dim3(1), dim3(1024), 0, s, L.ppart, L.nblk, a.dalpha, a.dhbias);
}

}  // namespace mhc
