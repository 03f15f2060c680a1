// reduce.hip -- fixed-order sums over rows of per-workgroup partials.
//
// out[c] = sum over r < R of part[r][c] (fp32 partials, C % 8 == 0), in two
// stages so that the sum is spread over the chip: stage 1 sums rows
// [s R / S, (s+1) R / S) of slice s into mid[s][C] (grid: column blocks x S
// slices; four consecutive channels per thread, the loads of a slice issued
// together, non-temporal since the partials are read once), stage 2 sums the
// S slice rows in slice order and stores to the output type.  The partition
// and both orders are fixed, so the result is bitwise reproducible.  A
// single thread per column walking 1024 rows had run ~100x slower than the
// stream that produced the partials.
#include "device.h"
#include "internal.h"

namespace mhc {

namespace {

__global__ __launch_bounds__(256) void rows_slice_sum_kernel(const float *__restrict__ part,
                                                             float *__restrict__ mid, int64_t R,
                                                             int64_t C) {
  const int64_t c4 = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (4 * c4 >= C) return;
  const int64_t s = blockIdx.y;
  const int64_t r0 = s * R / kRowSumSlices, r1 = (s + 1) * R / kRowSumSlices;
  const nt_f32x4 *p = reinterpret_cast<const nt_f32x4 *>(part) + c4;
  const int64_t stride = C / 4;
  nt_f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll 8
  for (int64_t r = r0; r < r1; ++r) acc += __builtin_nontemporal_load(p + r * stride);
  reinterpret_cast<nt_f32x4 *>(mid)[s * stride + c4] = acc;
}

template <typename T>
__global__ __launch_bounds__(256) void rows_final_sum_kernel(const float *__restrict__ mid,
                                                             T *__restrict__ out, int64_t C) {
  const int64_t c4 = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (4 * c4 >= C) return;
  const nt_f32x4 *p = reinterpret_cast<const nt_f32x4 *>(mid) + c4;
  const int64_t stride = C / 4;
  nt_f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int s = 0; s < kRowSumSlices; ++s) acc += p[s * stride];
  if constexpr (sizeof(T) == 2) {
    uint2 w;
    w.x = pack_bf16x2(acc.x, acc.y);
    w.y = pack_bf16x2(acc.z, acc.w);
    reinterpret_cast<uint2 *>(out)[c4] = w;
  } else {
    reinterpret_cast<nt_f32x4 *>(out)[c4] = acc;
  }
}

}  // namespace

void launch_rows_sum(hipStream_t s, const float *part, int64_t R, int64_t C, float *mid, void *out,
                     bool out_bf16) {
  const unsigned cb = (unsigned)((C / 4 + 255) / 256);
  hipLaunchKernelGGL(rows_slice_sum_kernel, dim3(cb, kRowSumSlices), dim3(256), 0, s, part, mid, R, C);
  if (out_bf16)
    hipLaunchKernelGGL((rows_final_sum_kernel<bf16_t>), dim3(cb), dim3(256), 0, s, mid, (bf16_t *)out, C);
  else
    hipLaunchKernelGGL((rows_final_sum_kernel<float>), dim3(cb), dim3(256), 0, s, mid, (float *)out, C);
}

}  // namespace mhc
