// The layer steps on either side of the token mixer ("08 linear delta rule & DPLR" page, the
// Gated DeltaNet layer-design figure after section 3): after the q/k/v projections a causal
// depthwise short convolution along time, SiLU, and for q and k an L2 norm over each head's
// channels; after the mixer an RMS norm over each head's d_v channels scaled by a per-channel
// weight and multiplied by SiLU of the gate projection.
//
// Rows of d elements whose 16-byte vectors number a power of two are split over that many
// lanes (conv_act_vec_kernel, norm_gate_vec_kernel); other widths take one wave per
// (token, head) row, lane l owning channels l, l + 64, ... .  The row's
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

// 16-byte vectors of E as floats, and back (rounded to nearest even for bf16).
template <typename E>
__device__ inline void unpack(u32x4 r, float* x) {
  const E* e = reinterpret_cast<const E*>(&r);
#pragma unroll
  for (int i = 0; i < 16 / (int)sizeof(E); ++i) x[i] = to_float(e[i]);
}
template <typename E>
__device__ inline u32x4 pack(const float* x) {
  E e[16 / sizeof(E)];
#pragma unroll
  for (int i = 0; i < 16 / (int)sizeof(E); ++i) e[i] = to_elem<E>(x[i]);
  u32x4 r;
  __builtin_memcpy(&r, e, 16);
  return r;
}

// Vector form of conv_act_kernel for four-tap filters and rows of LPR 16-byte vectors (LPR a
// power of two): LPR lanes share a row, each owning VE consecutive channels.  A workgroup takes
// NR runs of RPB consecutive tokens of one (sequence, head); each lane has its NR rows' tap
// loads (and its channels' filters, loaded once) in flight together, and the earlier taps of
// the workgroup's rows are rows it reads itself, so they come from this compute unit's caches.
constexpr int NR = 4;

template <typename E, bool NORM, int LPR>
__global__ __launch_bounds__(256) void conv_act_vec_kernel(const E* __restrict__ x, const float* __restrict__ w,
                                                          E* __restrict__ y, int T, int H, int d, float eps) {
  constexpr int VE = 16 / (int)sizeof(E), RPW = WAVE / LPR, RPB = 256 / LPR;
  const int lane = threadIdx.x % WAVE;
  const int TB = (T + RPB * NR - 1) / (RPB * NR);
  const long bh = (long)blockIdx.x / TB;
  const int h = (int)(bh % H);
  const int t0 = (int)(blockIdx.x % TB) * RPB * NR + (int)(threadIdx.x / WAVE) * RPW + lane / LPR;
  const int i0 = (lane % LPR) * VE;
  const long step = (long)H * d;
  const long row0 = ((bh / H) * T + t0) * H + h;  // row of token t0; token t0 + j is j * H rows on
  u32x4 xs[NR][4];
#pragma unroll
  for (int r = 0; r < NR; ++r) {
    const int t = t0 + r * RPB;
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const int lag = 3 - s;
      xs[r][s] = t < T && lag <= t ? *reinterpret_cast<const u32x4*>(x + (row0 + (long)(r * RPB - lag) * H) * d + i0)
                                   : u32x4{0, 0, 0, 0};
    }
  }
  const float* wc = w + ((long)h * d + i0) * 4;  // each channel's four taps: one 16-byte vector
  float4 wv[VE];
#pragma unroll
  for (int e = 0; e < VE; ++e) wv[e] = *reinterpret_cast<const float4*>(wc + 4 * e);
#pragma unroll
  for (int r = 0; r < NR; ++r) {
    float xv[4][VE], a[VE], ss = 0.f;
#pragma unroll
    for (int s = 0; s < 4; ++s) unpack<E>(xs[r][s], xv[s]);
#pragma unroll
    for (int e = 0; e < VE; ++e) {
      a[e] = silu(wv[e].x * xv[0][e] + wv[e].y * xv[1][e] + wv[e].z * xv[2][e] + wv[e].w * xv[3][e]);
      ss += a[e] * a[e];
    }
    float scale = 1.f;
    if (NORM) {
#pragma unroll
      for (int o = LPR / 2; o > 0; o >>= 1) ss += __shfl_xor(ss, o, WAVE);
      scale = rsqrtf(ss + eps);
    }
    if (t0 + r * RPB < T) {
#pragma unroll
      for (int e = 0; e < VE; ++e) a[e] *= scale;
      *reinterpret_cast<u32x4*>(y + (row0 + (long)r * RPB * H) * d + i0) = pack<E>(a);
    }
  }
}

// Vector form of norm_gate_kernel, same row split.
template <typename E, int LPR>
__global__ __launch_bounds__(256) void norm_gate_vec_kernel(const E* o, const E* __restrict__ g,
                                                           const float* __restrict__ weight, E* y, long rows,
                                                           int d, float eps) {
  constexpr int VE = 16 / (int)sizeof(E), RPW = WAVE / LPR;
  const int lane = threadIdx.x % WAVE;
  const long row = ((long)blockIdx.x * (256 / WAVE) + threadIdx.x / WAVE) * RPW + lane / LPR;
  const int i0 = (lane % LPR) * VE;
  const bool ok = row < rows;
  float a[VE], gv[VE], ss = 0.f;
#pragma unroll
  for (int e = 0; e < VE; ++e) a[e] = gv[e] = 0.f;
  if (ok) {
    unpack<E>(*reinterpret_cast<const u32x4*>(o + row * d + i0), a);
    unpack<E>(*reinterpret_cast<const u32x4*>(g + row * d + i0), gv);
#pragma unroll
    for (int e = 0; e < VE; ++e) ss += a[e] * a[e];
  }
#pragma unroll
  for (int s = LPR / 2; s > 0; s >>= 1) ss += __shfl_xor(ss, s, WAVE);
  const float r = rsqrtf(ss / d + eps);
  if (ok) {
#pragma unroll
    for (int e = 0; e < VE; ++e) a[e] = a[e] * r * weight[i0 + e] * silu(gv[e]);
    *reinterpret_cast<u32x4*>(y + row * d + i0) = pack<E>(a);
  }
}

// Rows of d elements as 16-byte vectors: lanes per row when that is a power of two, else 0.
template <typename E>
int lanes_per_row(int d) {
  const int l = d * (int)sizeof(E) / 16;
  return (l & (l - 1)) == 0 && l >= 1 && l <= WAVE ? l : 0;
}

template <typename E, bool NORM>
void launch_conv(const E* x, const float* w, E* y, long rows, int T, int H, int d, int width, float eps,
                 hipStream_t st) {
  int lpr = width == 4 ? lanes_per_row<E>(d) : 0;
  const long run = lpr ? 256 / lpr * NR : 1, nblk = rows / T * ((T + run - 1) / run);  // rows / T sequence-heads
  if (nblk > 0x7fffffffL) lpr = 0;
  if (lpr == 0) {
    hipLaunchKernelGGL((conv_act_kernel<E, NORM>), dim3((unsigned)((rows + ROWS_PER_WG - 1) / ROWS_PER_WG)),
                       dim3(WAVE * ROWS_PER_WG), 0, st, x, w, y, rows, T, H, d, width, eps);
    return;
  }
  const dim3 grid((unsigned)nblk), block(256);
  switch (lpr) {
#define DELTA_CONV_CASE(N) \
  case N: hipLaunchKernelGGL((conv_act_vec_kernel<E, NORM, N>), grid, block, 0, st, x, w, y, T, H, d, eps); break;
    DELTA_CONV_CASE(1) DELTA_CONV_CASE(2) DELTA_CONV_CASE(4) DELTA_CONV_CASE(8) DELTA_CONV_CASE(16)
    DELTA_CONV_CASE(32) DELTA_CONV_CASE(64)
#undef DELTA_CONV_CASE
  }
}

template <typename E>
hipError_t prologue_t(const LayerParams& p, hipStream_t st) {
  const long rq = (long)p.B * p.L * p.H, rkv = (long)p.B * p.Lx * p.H;
  if (rq > 0)
    launch_conv<E, true>(static_cast<const E*>(p.xq), p.wq, static_cast<E*>(p.q), rq, p.L, p.H, p.DK, p.width,
                         p.eps, st);
  if (rkv > 0) {
    launch_conv<E, true>(static_cast<const E*>(p.xk), p.wk, static_cast<E*>(p.k), rkv, p.Lx, p.H, p.DK, p.width,
                         p.eps, st);
    launch_conv<E, false>(static_cast<const E*>(p.xv), p.wv, static_cast<E*>(p.v), rkv, p.Lx, p.H, p.DV, p.width,
                          p.eps, st);
  }
  return hipGetLastError();
}

template <typename E>
hipError_t epilogue_t(const LayerParams& p, hipStream_t st) {
  const long rows = (long)p.B * p.L * p.H;
  if (rows == 0) return hipSuccess;
  const E* o = static_cast<const E*>(p.o);
  const E* g = static_cast<const E*>(p.g);
  E* y = static_cast<E*>(p.y);
  const int lpr = lanes_per_row<E>(p.DV);
  if (lpr == 0) {
    hipLaunchKernelGGL((norm_gate_kernel<E>), dim3((unsigned)((rows + ROWS_PER_WG - 1) / ROWS_PER_WG)),
                       dim3(WAVE * ROWS_PER_WG), 0, st, o, g, p.weight, y, rows, p.DV, p.eps);
    return hipGetLastError();
  }
  const long per_block = 256 / lpr;
  const dim3 grid((unsigned)((rows + per_block - 1) / per_block)), block(256);
  switch (lpr) {
#define DELTA_NG_CASE(N) \
  case N: hipLaunchKernelGGL((norm_gate_vec_kernel<E, N>), grid, block, 0, st, o, g, p.weight, y, rows, p.DV, p.eps); break;
    DELTA_NG_CASE(1) DELTA_NG_CASE(2) DELTA_NG_CASE(4) DELTA_NG_CASE(8) DELTA_NG_CASE(16)
    DELTA_NG_CASE(32) DELTA_NG_CASE(64)
#undef DELTA_NG_CASE
  }
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
