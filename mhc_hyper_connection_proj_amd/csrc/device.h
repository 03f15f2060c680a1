// device.h -- shared gfx950 device helpers for libmhc kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mhc {

typedef uint16_t bf16_t;  // bf16 storage: the upper half of an fp32 bit pattern

// ---------------------------------------------------------------- conversions
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// Two fp32 -> two bf16 (round to nearest even) packed low|high.  Converted as
// one two-element vector, so the pair is a single v_cvt_pk_bf16_f32 (two
// scalar conversions compile to two of them plus a shift and an or).
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  typedef __attribute__((ext_vector_type(2))) float f32x2_t;
  typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2_t;
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2_t{a, b}, bf16x2_t));
}

// ---------------------------------------------------------------- 8-wide activation I/O
// Activations move in groups of 8 channels: one 128-bit access for bf16,
// two for fp32.  Callers guarantee 16-byte alignment (C % 8 == 0 and
// 16-byte aligned base pointers are checked on the host).
template <typename T> struct Io8;

typedef __attribute__((ext_vector_type(4))) unsigned int nt_u32x4;
typedef __attribute__((ext_vector_type(4))) float nt_f32x4;

// load: cached, converted.  ld_nt + cvt: non-temporal raw load (streamed
// once; the line is not kept in the caches), for tensors a kernel reads
// exactly once in whole lines, converted where the values are used.
template <> struct Io8<bf16_t> {
  static __device__ __forceinline__ void load(const bf16_t *p, float v[8]) {
    const uint4 w = *reinterpret_cast<const uint4 *>(p);
    v[0] = bf16_lo(w.x); v[1] = bf16_hi(w.x);
    v[2] = bf16_lo(w.y); v[3] = bf16_hi(w.y);
    v[4] = bf16_lo(w.z); v[5] = bf16_hi(w.z);
    v[6] = bf16_lo(w.w); v[7] = bf16_hi(w.w);
  }
  // raw 16 bytes (8 values), loaded non-temporally, converted later
  typedef nt_u32x4 raw_t;
  static __device__ __forceinline__ raw_t ld_nt(const bf16_t *p) {
    return __builtin_nontemporal_load(reinterpret_cast<const nt_u32x4 *>(p));
  }
  static __device__ __forceinline__ void cvt(raw_t w, float v[8]) {
    // components taken by name: bit-casting an indexed ext-vector element
    // makes hipcc reuse dword 0 for every index
    const unsigned a = w.x, b = w.y, c = w.z, d = w.w;
    v[0] = bf16_lo(a); v[1] = bf16_hi(a);
    v[2] = bf16_lo(b); v[3] = bf16_hi(b);
    v[4] = bf16_lo(c); v[5] = bf16_hi(c);
    v[6] = bf16_lo(d); v[7] = bf16_hi(d);
  }
  static __device__ __forceinline__ void load_nt(const bf16_t *p, float v[8]) { cvt(ld_nt(p), v); }
  // values 2p and 2p+1 (p a compile-time constant in unrolled loops)
  static __device__ __forceinline__ void pair(raw_t w, int p, float &lo, float &hi) {
    const unsigned d = p == 0 ? w.x : p == 1 ? w.y : p == 2 ? w.z : w.w;
    lo = bf16_lo(d);
    hi = bf16_hi(d);
  }
  // two values packed back into the storage type (one dword of a raw_t)
  typedef uint32_t pair_t;
  static __device__ __forceinline__ pair_t pack(float lo, float hi) { return pack_bf16x2(lo, hi); }
  static __device__ __forceinline__ void store_pairs(bf16_t *p, const pair_t q[4]) {
    *reinterpret_cast<uint4 *>(p) = make_uint4(q[0], q[1], q[2], q[3]);
  }
  static __device__ __forceinline__ void store(bf16_t *p, const float v[8]) {
    uint4 w;
    w.x = pack_bf16x2(v[0], v[1]);
    w.y = pack_bf16x2(v[2], v[3]);
    w.z = pack_bf16x2(v[4], v[5]);
    w.w = pack_bf16x2(v[6], v[7]);
    *reinterpret_cast<uint4 *>(p) = w;
  }
  // non-temporal store, for outputs that no later kernel of the pass reads
  static __device__ __forceinline__ void store_nt(bf16_t *p, const float v[8]) {
    nt_u32x4 w;
    w.x = pack_bf16x2(v[0], v[1]);
    w.y = pack_bf16x2(v[2], v[3]);
    w.z = pack_bf16x2(v[4], v[5]);
    w.w = pack_bf16x2(v[6], v[7]);
    __builtin_nontemporal_store(w, reinterpret_cast<nt_u32x4 *>(p));
  }
};

template <> struct Io8<float> {
  static __device__ __forceinline__ void load(const float *p, float v[8]) {
    const float4 a = *reinterpret_cast<const float4 *>(p);
    const float4 b = *reinterpret_cast<const float4 *>(p + 4);
    v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
    v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
  }
  struct raw_t {
    nt_f32x4 a, b;
  };
  static __device__ __forceinline__ raw_t ld_nt(const float *p) {
    return {__builtin_nontemporal_load(reinterpret_cast<const nt_f32x4 *>(p)),
            __builtin_nontemporal_load(reinterpret_cast<const nt_f32x4 *>(p + 4))};
  }
  static __device__ __forceinline__ void cvt(const raw_t &r, float v[8]) {
    v[0] = r.a.x; v[1] = r.a.y; v[2] = r.a.z; v[3] = r.a.w;
    v[4] = r.b.x; v[5] = r.b.y; v[6] = r.b.z; v[7] = r.b.w;
  }
  static __device__ __forceinline__ void load_nt(const float *p, float v[8]) { cvt(ld_nt(p), v); }
  static __device__ __forceinline__ void pair(const raw_t &r, int p, float &lo, float &hi) {
    lo = p == 0 ? r.a.x : p == 1 ? r.a.z : p == 2 ? r.b.x : r.b.z;
    hi = p == 0 ? r.a.y : p == 1 ? r.a.w : p == 2 ? r.b.y : r.b.w;
  }
  typedef float2 pair_t;
  static __device__ __forceinline__ pair_t pack(float lo, float hi) { return make_float2(lo, hi); }
  static __device__ __forceinline__ void store_pairs(float *p, const pair_t q[4]) {
    *reinterpret_cast<float4 *>(p) = make_float4(q[0].x, q[0].y, q[1].x, q[1].y);
    *reinterpret_cast<float4 *>(p + 4) = make_float4(q[2].x, q[2].y, q[3].x, q[3].y);
  }
  static __device__ __forceinline__ void store(float *p, const float v[8]) {
    *reinterpret_cast<float4 *>(p) = make_float4(v[0], v[1], v[2], v[3]);
    *reinterpret_cast<float4 *>(p + 4) = make_float4(v[4], v[5], v[6], v[7]);
  }
  static __device__ __forceinline__ void store_nt(float *p, const float v[8]) {
    __builtin_nontemporal_store(nt_f32x4{v[0], v[1], v[2], v[3]}, reinterpret_cast<nt_f32x4 *>(p));
    __builtin_nontemporal_store(nt_f32x4{v[4], v[5], v[6], v[7]}, reinterpret_cast<nt_f32x4 *>(p + 4));
  }
};

// ---------------------------------------------------------------- wave64 reductions
// DPP control words (GFX9 encoding).
enum : int {
  DPP_QUAD_1032 = 0xb1,  // quad_perm [1,0,3,2]
  DPP_QUAD_2301 = 0x4e,  // quad_perm [2,3,0,1]
  DPP_ROW_ROR4 = 0x124,
  DPP_ROW_ROR8 = 0x128,
  DPP_ROW_BCAST15 = 0x142,
  DPP_ROW_BCAST31 = 0x143,
};

template <int CTRL, int ROW_MASK = 0xf>
__device__ __forceinline__ float dpp(float v) {
  return __int_as_float(
      __builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, ROW_MASK, 0xf, false));
}

// Sum over the 64 lanes of a wave; the total is returned to every lane.
// Fixed association order, so the result is deterministic.
__device__ __forceinline__ float wave_sum(float v) {
  v += dpp<DPP_QUAD_1032>(v);
  v += dpp<DPP_QUAD_2301>(v);
  v += dpp<DPP_ROW_ROR4>(v);
  v += dpp<DPP_ROW_ROR8>(v);           // every lane holds its 16-lane row sum
  v += dpp<DPP_ROW_BCAST15, 0xa>(v);   // rows 1, 3 += rows 0, 2
  v += dpp<DPP_ROW_BCAST31, 0xc>(v);   // rows 2, 3 += row 1 (now rows 0+1)
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 63));
}

__device__ __forceinline__ float fast_rcp(float x) { return __builtin_amdgcn_rcpf(x); }

}  // namespace mhc
