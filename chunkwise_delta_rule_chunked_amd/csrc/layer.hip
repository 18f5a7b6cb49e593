// The layer steps on either side of the token mixer ("08 linear delta rule & DPLR" page, the
// Gated DeltaNet layer-design figure after section 3): after the q/k/v projections a causal
// depthwise short convolution along time, SiLU, and for q and k an L2 norm over each head's
// channels; after the mixer an RMS norm over each head's d_v channels scaled by a per-channel
// weight and multiplied by SiLU of the gate projection.
//
// One wave per (token, head) row; lane l owns channels l, l + 64, ... of the row.  The row's
// earlier taps are the same channels of the preceding tokens' rows, which neighbouring waves
// read too, so HBM sees each input about once.  Arithmetic in float32; outputs rounded to the
// element type.
#include <hip/hip_runtime.h>

#include "common.h"
#include "kernels.h"

namespace delta {
namespace {

constexpr int ROWS_PER_WG = 4;  // waves per workgroup, one row each
constexpr int MAXJ = 4;         // channels per lane: d <= 256

__device__ inline float silu(float x) { return x / (1.f + expf(-x)); }

__device__ inline float wave_sum(float x) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) x += __shfl_xor(x, o, WAVE);
  return x;
}

// x, y [B, T, H, d]; w [H * d, width].  NORM: divide each row by sqrt(sum of squares + eps).
template <typename E, bool NORM>
__global__ __launch_bounds__(WAVE * ROWS_PER_WG) void conv_act_kernel(const E* __restrict__ x,
                                                                    const float* __restrict__ w,
                                                                    E* __restrict__ y, long rows, int T,
                                                                    int H, int d, int width, float eps) {
  const long row = (long)blockIdx.x * ROWS_PER_WG + threadIdx.x / WAVE;
  const int lane = threadIdx.x % WAVE;
  if (row >= rows) return;
  const int h = (int)(row % H);
  const long bt = row / H;
  const int t = (int)(bt % T);
  const long base = row * d;            // this row's first element
  const long step = (long)H * d;        // one token back
  float a[MAXJ];
  float ss = 0.f;
#pragma unroll
  for (int j = 0; j < MAXJ; ++j) {
    const int i = lane + WAVE * j;
    a[j] = 0.f;
    if (i < d) {
      const float* wc = w + ((long)h * d + i) * width;
      float acc = 0.f;
      for (int s = 0; s < width; ++s) {
        const int lag = width - 1 - s;
        if (lag <= t) acc += wc[s] * to_float(x[base - lag * step + i]);
      }
      a[j] = silu(acc);
      ss += a[j] * a[j];
    }
  }
  float scale = 1.f;
  if (NORM) scale = rsqrtf(wave_sum(ss) + eps);
#pragma unroll
  for (int j = 0; j < MAXJ; ++j) {
    const int i = lane + WAVE * j;
    if (i < d) y[base + i] = to_elem<E>(a[j] * scale);
  }
}

// o, g, y [rows, d]; weight [d].  y = o / sqrt(mean(o^2) + eps) * weight * SiLU(g).
template <typename E>
__global__ __launch_bounds__(WAVE * ROWS_PER_WG) void norm_gate_kernel(const E* o, const E* __restrict__ g,
                                                                     const float* __restrict__ weight, E* y,
                                                                     long rows, int d, float eps) {
  const long row = (long)blockIdx.x * ROWS_PER_WG + threadIdx.x / WAVE;
  const int lane = threadIdx.x % WAVE;
  if (row >= rows) return;
  const long base = row * d;
  float a[MAXJ], ss = 0.f;
#pragma unroll
  for (int j = 0; j < MAXJ; ++j) {
    const int i = lane + WAVE * j;
    a[j] = i < d ? to_float(o[base + i]) : 0.f;
    ss += a[j] * a[j];
  }
  const float r = rsqrtf(wave_sum(ss) / d + eps);
#pragma unroll
  for (int j = 0; j < MAXJ; ++j) {
    const int i = lane + WAVE * j;
    if (i < d) y[base + i] = to_elem<E>(a[j] * r * weight[i] * silu(to_float(g[base + i])));
  }
}

template <typename E>
hipError_t prologue_t(const LayerParams& p, hipStream_t st) {
  const dim3 block(WAVE * ROWS_PER_WG);
  const long rq = (long)p.B * p.L * p.H, rkv = (long)p.B * p.Lx * p.H;
  auto blocks = [](long rows) { return dim3((unsigned)((rows + ROWS_PER_WG - 1) / ROWS_PER_WG)); };
  if (rq > 0)
    hipLaunchKernelGGL((conv_act_kernel<E, true>), blocks(rq), block, 0, st, static_cast<const E*>(p.xq), p.wq,
                       static_cast<E*>(p.q), rq, p.L, p.H, p.DK, p.width, p.eps);
  if (rkv > 0) {
    hipLaunchKernelGGL((conv_act_kernel<E, true>), blocks(rkv), block, 0, st, static_cast<const E*>(p.xk), p.wk,
                       static_cast<E*>(p.k), rkv, p.Lx, p.H, p.DK, p.width, p.eps);
    hipLaunchKernelGGL((conv_act_kernel<E, false>), blocks(rkv), block, 0, st, static_cast<const E*>(p.xv), p.wv,
                       static_cast<E*>(p.v), rkv, p.Lx, p.H, p.DV, p.width, p.eps);
  }
  return hipGetLastError();
}

template <typename E>
hipError_t epilogue_t(const LayerParams& p, hipStream_t st) {
  const long rows = (long)p.B * p.L * p.H;
  if (rows > 0)
    hipLaunchKernelGGL((norm_gate_kernel<E>), dim3((unsigned)((rows + ROWS_PER_WG - 1) / ROWS_PER_WG)),
                       dim3(WAVE * ROWS_PER_WG), 0, st, static_cast<const E*>(p.o), static_cast<const E*>(p.g),
                       p.weight, static_cast<E*>(p.y), rows, p.DV, p.eps);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_layer_prologue(const LayerParams& p, bool bf16_in, hipStream_t st) {
  return bf16_in ? prologue_t<bf16>(p, st) : prologue_t<float>(p, st);
}

hipError_t launch_layer_epilogue(const LayerParams& p, bool bf16_in, hipStream_t st) {
  return bf16_in ? epilogue_t<bf16>(p, st) : epilogue_t<float>(p, st);
}

}  // namespace delta
