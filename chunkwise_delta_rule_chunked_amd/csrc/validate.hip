// Opt-in input check of the forward and backward passes (DELTA_VALIDATE=1): the write strengths
// must be finite, and each log gate either finite or -inf.  -inf is the hard reset g = 0 that the
// DeltaProduct notes (section 3.3) use to clear the state; NaN and +inf have no reading.
//
// One flag word per workgroup (1: some value it scanned is outside that range), so the pass needs
// no atomics and no prior clearing; the host reads the words back and ORs them.
#include "common.h"
#include "kernels.h"

namespace delta {

__global__ __launch_bounds__(256) void validate_kernel(const float* beta, long nbeta, const float* glog, long ngate,
                                                      unsigned* flags) {
  bool bad = false;
  const long stride = (long)gridDim.x * blockDim.x;
  for (long i = (long)blockIdx.x * blockDim.x + threadIdx.x; i < nbeta; i += stride)
    bad |= !__builtin_isfinite(beta[i]);
  for (long i = (long)blockIdx.x * blockDim.x + threadIdx.x; i < ngate; i += stride) {
    const float x = glog[i];
    bad |= (x != x) || (x == __builtin_inff());
  }
  bad = __syncthreads_or(bad);
  if (threadIdx.x == 0) flags[blockIdx.x] = bad ? 1u : 0u;
}

hipError_t launch_validate(const float* beta, long nbeta, const float* glog, long ngate, unsigned* flags,
                           hipStream_t st) {
  hipLaunchKernelGGL(validate_kernel, dim3(VALIDATE_BLOCKS), dim3(256), 0, st, beta, nbeta, glog, ngate, flags);
  return hipGetLastError();
}

}  // namespace delta
