// probe.hip -- bandwidth probes: the practical read and copy rates of the
// device, reported beside the HBM peak (nothing of the mHC path is computed).
//
// Workgroup b streams one contiguous share of the buffer, its 256 threads
// reading 16-byte words four 4 KB steps at a time (the four loads issued
// together).  8192 workgroups of 256 threads (32 per CU).  Read mode folds
// the words into a checksum per workgroup (so the loads are kept) and
// stores it to a 4 KB sink; copy mode stores every word to dst.  Measured
// against grid-stride variants and 1024-8192 workgroups with 4-16 loads in
// flight, this form read and copied fastest.
#include "device.h"
#include "internal.h"

namespace mhc {

namespace {

constexpr int kProbeBlocks = 8192;

template <bool COPY, bool NT>
__global__ __launch_bounds__(256) void bandwidth_probe_kernel(const nt_u32x4 *__restrict__ src,
                                                              nt_u32x4 *__restrict__ dst, int64_t n16) {
  const int64_t per = (n16 + gridDim.x - 1) / gridDim.x;
  const int64_t b0 = (int64_t)blockIdx.x * per, b1 = min(n16, b0 + per);
  unsigned acc = 0;
  int64_t i = b0 + threadIdx.x;
  for (; i + 3 * 256 < b1; i += 4 * 256) {
    nt_u32x4 v[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) v[q] = NT ? __builtin_nontemporal_load(src + i + q * 256) : src[i + q * 256];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      if (COPY) {
        if (NT) __builtin_nontemporal_store(v[q], dst + i + q * 256);
        else dst[i + q * 256] = v[q];
      } else {
        acc ^= (v[q].x ^ v[q].y) ^ (v[q].z ^ v[q].w);
      }
    }
  }
  for (; i < b1; i += 256) {
    const nt_u32x4 v = NT ? __builtin_nontemporal_load(src + i) : src[i];
    if (COPY) dst[i] = v;
    else acc ^= (v.x ^ v.y) ^ (v.z ^ v.w);
  }
  if (!COPY) {
    __shared__ unsigned red[4];
    for (int o = 32; o > 0; o >>= 1) acc ^= __shfl_xor(acc, o);
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = acc;
    __syncthreads();
    // the sink holds kProbeSinkWords words; workgroups share them (the value is an unspecified checksum)
    if (threadIdx.x == 0)
      reinterpret_cast<unsigned *>(dst)[blockIdx.x % kProbeSinkWords] = (red[0] ^ red[1]) ^ (red[2] ^ red[3]);
  }
}

}  // namespace

void launch_bandwidth_probe(hipStream_t s, bool copy, bool nt, const void *src, void *dst, int64_t bytes) {
  const int64_t n16 = bytes / 16;
  const nt_u32x4 *a = reinterpret_cast<const nt_u32x4 *>(src);
  nt_u32x4 *b = reinterpret_cast<nt_u32x4 *>(dst);
  const dim3 g(kProbeBlocks), t(256);
  if (copy) {
    if (nt) hipLaunchKernelGGL((bandwidth_probe_kernel<true, true>), g, t, 0, s, a, b, n16);
    else hipLaunchKernelGGL((bandwidth_probe_kernel<true, false>), g, t, 0, s, a, b, n16);
  } else {
    if (nt) hipLaunchKernelGGL((bandwidth_probe_kernel<false, true>), g, t, 0, s, a, b, n16);
    else hipLaunchKernelGGL((bandwidth_probe_kernel<false, false>), g, t, 0, s, a, b, n16);
  }
}

}  // namespace mhc
