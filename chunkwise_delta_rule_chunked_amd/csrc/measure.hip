// A plain streaming copy, the measured ceiling of a kernel that reads and writes HBM once with
// nothing else to do, and a kernel of known traffic for scaling the HBM byte counters.  Not a
// step of the delta rule.
//
// Each lane moves 16-byte pieces; a workgroup of 256 lanes issues `U` pieces per lane before
// storing any, and the grid strides over the buffer.  Optional non-temporal accesses.
#include "../../include/delta_measure.h"
#include "common.h"

namespace delta {

template <int U, bool NT>
__global__ __launch_bounds__(256) void copy_kernel(const u32x4* __restrict__ src, u32x4* __restrict__ dst, long n) {
  const long stride = (long)gridDim.x * 256 * U;
  for (long base = (long)blockIdx.x * 256 * U + threadIdx.x; base < n; base += stride) {
    u32x4 x[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const long i = base + 256L * u;
      if (i < n) x[u] = NT ? __builtin_nontemporal_load(src + i) : src[i];
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const long i = base + 256L * u;
      if (i < n) {
        if (NT) __builtin_nontemporal_store(x[u], dst + i);
        else dst[i] = x[u];
      }
    }
  }
}

template <bool NT>
static hipError_t copy_by_u(const u32x4* s, u32x4* d, long n, int unroll, int blocks, hipStream_t st) {
  switch (unroll) {
    case 1: hipLaunchKernelGGL((copy_kernel<1, NT>), dim3(blocks), dim3(256), 0, st, s, d, n); break;
    case 2: hipLaunchKernelGGL((copy_kernel<2, NT>), dim3(blocks), dim3(256), 0, st, s, d, n); break;
    case 4: hipLaunchKernelGGL((copy_kernel<4, NT>), dim3(blocks), dim3(256), 0, st, s, d, n); break;
    case 8: hipLaunchKernelGGL((copy_kernel<8, NT>), dim3(blocks), dim3(256), 0, st, s, d, n); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace delta

extern "C" int delta_measure_copy(const void* src, void* dst, size_t bytes, int32_t unroll, int32_t blocks,
                                  int32_t nontemporal, void* stream) {
  if (bytes == 0) return 0;
  if (!src || !dst) return -1;
  if (bytes % 16 || (reinterpret_cast<uintptr_t>(src) | reinterpret_cast<uintptr_t>(dst)) % 16) return -4;
  if ((unroll != 1 && unroll != 2 && unroll != 4 && unroll != 8) || blocks < 1 || blocks > (1 << 20)) return -3;
  const uintptr_t s = reinterpret_cast<uintptr_t>(src), d = reinterpret_cast<uintptr_t>(dst);
  if (s < d + bytes && d < s + bytes) return -6;
  const auto* sp = static_cast<const delta::u32x4*>(src);
  auto* dp = static_cast<delta::u32x4*>(dst);
  const long n = (long)(bytes / 16);
  hipStream_t st = static_cast<hipStream_t>(stream);
  const hipError_t e = nontemporal ? delta::copy_by_u<true>(sp, dp, n, unroll, blocks, st)
                                   : delta::copy_by_u<false>(sp, dp, n, unroll, blocks, st);
  return e == hipSuccess ? 0 : -7;
}
