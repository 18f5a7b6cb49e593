// The layer steps on either side of the token mixer ("08 linear delta rule & DPLR" page, the
// Gated DeltaNet layer-design figure after section 3): after the q/k/v projections a causal
// depthwise short convolution along time, SiLU, and for q and k an L2 norm over each head's
// channels; after the mixer an RMS norm over each head's d_v channels scaled by a per-channel
// weight and multiplied by SiLU of the gate projection.
//
// Rows of d elements whose 16-byte vectors number a power of two are split over that many
// lanes: the prologue's three tensors in one launch (prologue_fused_kernel, below), the epilogue
// in norm_gate_vec_kernel.  Other widths take one wave per (token, head) row, lane l owning
// channels l, l + 64, ... (conv_act_kernel once per tensor, norm_gate_kernel).  Arithmetic in
// float32; outputs rounded to the element type.
#include <hip/hip_runtime.h>

#include "common.h"
#include "kernels.h"

namespace delta {
namespace {

constexpr int ROWS_PER_WG = 4;  // waves per workgroup, one row each
constexpr int MAXJ = 4;         // channels per lane: d <= 256

// SiLU(x) = x sigmoid(x) with the hardware exp2 and reciprocal (each within 1 ulp): the
// full-precision exp and IEEE division took ~30 instructions per element and made the prologue
// bound by its arithmetic rather than by its memory traffic.
__device__ inline float silu(float x) { return x * __builtin_amdgcn_rcpf(1.f + gate_exp(-x)); }

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

// Sum over groups of 2^lg consecutive lanes (lg <= 6, wave-uniform), every lane of a group
// receiving its group's total: DPP steps inside a 16-lane row (quad permutations xor 1 and xor 2,
// then the half-mirror and mirror of the row), lane shuffles across rows.
template <int CTRL>
__device__ inline float dpp_mov(float x) {
  return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x), CTRL, 0xF, 0xF, false));
}
__device__ inline float group_sum(float x, int lg) {
  if (lg >= 1) x += dpp_mov<0xB1>(x);
  if (lg >= 2) x += dpp_mov<0x4E>(x);
  if (lg >= 3) x += dpp_mov<0x141>(x);
  if (lg >= 4) x += dpp_mov<0x140>(x);
  if (lg >= 5) x += __shfl_xor(x, 16, WAVE);
  if (lg >= 6) x += __shfl_xor(x, 32, WAVE);
  return x;
}

// The whole prologue in one launch: q, k and v, each a sequence of rows [B, T, H, d] filtered
// along T by a causal depthwise filter of W taps, then SiLU, then (q, k) divided by the row's
// L2 norm.  A lane walks RUN consecutive tokens of one (sequence, head) over one 16-byte vector
// of channels (2^lg lanes per row), keeping the previous W - 1 rows in registers, so every input
// byte is read once (plus W - 1 rows per run).  Rows come in batches of UNR, the next batch's
// loads in flight while the current one is computed; loads past the sequence are clamped to its
// last row (the results are not stored), so the loop has no branches.  The runs of a wavefront
// are consecutive heads at the same tokens, so each load instruction covers 64 x 16 contiguous
// bytes; the L2 norm is a lane-group sum.  Workgroups [0, nq) filter q, [nq, nq + nk) k, the rest
// v (a uniform choice per workgroup).
constexpr int RUN = 32, UNR = 4;

struct FusedSeg {
  const void* x;
  const float* w;
  void* y;
  int T, d, lg;   // lg: log2 of the lanes per row
};

template <typename E, int W, bool NORM>
__device__ inline void conv_run(const FusedSeg& sg, int B, int H, float eps, int wg) {
  constexpr int VE = 16 / (int)sizeof(E);
  const int tid = threadIdx.x;
  const int run = wg * (256 >> sg.lg) + (tid >> sg.lg);   // run index: head fastest
  const int i0 = (tid & ((1 << sg.lg) - 1)) * VE;
  const int nb = (sg.T + RUN - 1) / RUN;
  const int h = run % H, bt = run / H;
  const bool live = bt / nb < B;
  const int b = live ? bt / nb : B - 1, t0 = (bt % nb) * RUN;
  const E* x = static_cast<const E*>(sg.x) + (((long)b * sg.T) * H + h) * sg.d + i0;
  E* y = static_cast<E*>(sg.y) + (((long)b * sg.T) * H + h) * sg.d + i0;
  const long step = (long)H * sg.d;                       // one token along T
  // inputs are read once: non-temporal loads (measured 71.8 against 81.8 us for q, k and v of
  // the 32-head 8K-token shape; non-temporal stores of the outputs, which the forward pass reads
  // next, were slower)
  auto row = [&](int t) {
    return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(x + min(max(t, 0), sg.T - 1) * step));
  };
  float wv[VE][W];
  {
    const float* wc = sg.w + ((long)h * sg.d + i0) * W;
#pragma unroll
    for (int e = 0; e < VE; ++e)
#pragma unroll
      for (int s = 0; s < W; ++s) wv[e][s] = wc[e * W + s];
  }
  // win[s]: the input row s + 1 tokens back (zeros before the sequence)
  float win[W > 1 ? W - 1 : 1][VE];
#pragma unroll
  for (int s = 0; s < W - 1; ++s) {
    float f[VE];
    unpack<E>(row(t0 - 1 - s), f);
#pragma unroll
    for (int e = 0; e < VE; ++e) win[s][e] = t0 - 1 - s >= 0 ? f[e] : 0.f;
  }
  u32x4 nxt[UNR];
#pragma unroll
  for (int u = 0; u < UNR; ++u) nxt[u] = row(t0 + u);
  for (int tb = t0; tb < t0 + RUN; tb += UNR) {
    u32x4 cur[UNR];
#pragma unroll
    for (int u = 0; u < UNR; ++u) cur[u] = nxt[u];
    if (tb + UNR < t0 + RUN) {
#pragma unroll
      for (int u = 0; u < UNR; ++u) nxt[u] = row(tb + UNR + u);
    }
#pragma unroll
    for (int u = 0; u < UNR; ++u) {
      float xt[VE], a[VE], ss = 0.f;
      unpack<E>(cur[u], xt);
#pragma unroll
      for (int e = 0; e < VE; ++e) {
        float acc = wv[e][W - 1] * xt[e];  // tap W-1: the current token
#pragma unroll
        for (int s = 0; s < W - 1; ++s) acc += wv[e][W - 2 - s] * win[s][e];
        a[e] = silu(acc);
        ss += a[e] * a[e];
      }
      if constexpr (NORM) {
        const float r = rsqrtf(group_sum(ss, sg.lg) + eps);
#pragma unroll
        for (int e = 0; e < VE; ++e) a[e] *= r;
      }
      if (live && tb + u < sg.T) *reinterpret_cast<u32x4*>(y + (tb + u) * step) = pack<E>(a);
#pragma unroll
      for (int s = W - 2; s > 0; --s)
#pragma unroll
        for (int e = 0; e < VE; ++e) win[s][e] = win[s - 1][e];
      if constexpr (W > 1) {
#pragma unroll
        for (int e = 0; e < VE; ++e) win[0][e] = xt[e];
      }
    }
  }
}

template <typename E, int W>
__global__ __launch_bounds__(256) void prologue_fused_kernel(FusedSeg sq, FusedSeg sk, FusedSeg sv, int B, int H,
                                                            float eps, int nq, int nk) {
  const int wg = blockIdx.x;
  if (wg < nq) conv_run<E, W, true>(sq, B, H, eps, wg);
  else if (wg < nq + nk) conv_run<E, W, true>(sk, B, H, eps, wg - nq);
  else conv_run<E, W, false>(sv, B, H, eps, wg - nq - nk);
}

// Workgroups that cover B x H x ceil(T / RUN) runs at 256 / LPR runs each.
inline long fused_blocks(int B, int H, int T, int lpr) {
  const long runs = (long)B * H * ((T + RUN - 1) / RUN);
  const long per = 256 / lpr;
  return (runs + per - 1) / per;
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
  hipLaunchKernelGGL((conv_act_kernel<E, NORM>), dim3((unsigned)((rows + ROWS_PER_WG - 1) / ROWS_PER_WG)),
                     dim3(WAVE * ROWS_PER_WG), 0, st, x, w, y, rows, T, H, d, width, eps);
}

// One launch when both row widths split into a power of two of 16-byte lanes: returns false
// otherwise (then one per-row launch per tensor).
template <typename E>
bool prologue_fused(const LayerParams& p, hipStream_t st) {
  const int lqk = lanes_per_row<E>(p.DK), lv = lanes_per_row<E>(p.DV);
  if (lqk == 0 || lv == 0) return false;
  const long nq = p.L > 0 ? fused_blocks(p.B, p.H, p.L, lqk) : 0;
  const long nk = fused_blocks(p.B, p.H, p.Lx, lqk), nv = fused_blocks(p.B, p.H, p.Lx, lv);
  if (nq + nk + nv > 0x7fffffffL) return false;
  const FusedSeg sq{p.xq, p.wq, p.q, p.L, p.DK, __builtin_ctz(lqk)}, sk{p.xk, p.wk, p.k, p.Lx, p.DK, __builtin_ctz(lqk)},
      sv{p.xv, p.wv, p.v, p.Lx, p.DV, __builtin_ctz(lv)};
  const dim3 grid((unsigned)(nq + nk + nv)), block(256);
  switch (p.width) {
#define DELTA_FUSED_W(W)                                                                                        \
  case W:                                                                                                       \
    hipLaunchKernelGGL((prologue_fused_kernel<E, W>), grid, block, 0, st, sq, sk, sv, p.B, p.H, p.eps, (int)nq, \
                       (int)nk);                                                                                \
    break;
    DELTA_FUSED_W(1) DELTA_FUSED_W(2) DELTA_FUSED_W(3) DELTA_FUSED_W(4)
#undef DELTA_FUSED_W
    default: return false;
  }
  return true;
}

template <typename E>
hipError_t prologue_t(const LayerParams& p, hipStream_t st) {
  if (prologue_fused<E>(p, st)) return hipGetLastError();
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

// One decode token through the prologue, the filters' inputs carried in a state: per (sequence,
// head) the row of q, and the n_h rows of k and of v in order (a DeltaProduct token's sub-steps
// are consecutive steps of the filter).  For each row x_t,
//     y = sum_{s < W-1} w[c][s] state[s] + w[c][W-1] x_t,   then state <- (state[1 ..], x_t),
// the state holding the W - 1 previous inputs oldest first, then SiLU and, for q and k, the L2
// norm.  One wave per (sequence, head, tensor); lane l owns channels l, l + 64, ... (d <= 256).
template <typename E, int W>
__global__ __launch_bounds__(WAVE * ROWS_PER_WG) void prologue_step_kernel(LayerParams p) {
  const long idx = (long)blockIdx.x * ROWS_PER_WG + threadIdx.x / WAVE;
  const int lane = threadIdx.x % WAVE;
  if (idx >= 3L * p.B * p.H) return;
  const int which = (int)(idx % 3);             // 0 q, 1 k, 2 v
  const long bh = idx / 3;
  const int b = (int)(bh / p.H), h = (int)(bh % p.H);
  const int d = which == 2 ? p.DV : p.DK, rows = which == 0 ? 1 : p.Lx;  // Lx = n_h rows per token
  const E* x = static_cast<const E*>(which == 0 ? p.xq : which == 1 ? p.xk : p.xv);
  const float* w = which == 0 ? p.wq : which == 1 ? p.wk : p.wv;
  E* cs = static_cast<E*>(which == 0 ? p.cq : which == 1 ? p.ck : p.cv);
  E* y = static_cast<E*>(which == 0 ? p.q : which == 1 ? p.k : p.v);
  float st[W > 1 ? W - 1 : 1][MAXJ], wv[MAXJ][W];
#pragma unroll
  for (int j = 0; j < MAXJ; ++j) {
    const int i = lane + WAVE * j;
#pragma unroll
    for (int s = 0; s < W - 1; ++s) st[s][j] = i < d ? to_float(cs[(((long)b * (W - 1) + s) * p.H + h) * d + i]) : 0.f;
#pragma unroll
    for (int s = 0; s < W; ++s) wv[j][s] = i < d ? w[((long)h * d + i) * W + s] : 0.f;
  }
  for (int r = 0; r < rows; ++r) {
    const long row = ((long)b * rows + r) * p.H + h;
    float a[MAXJ], ss = 0.f;
#pragma unroll
    for (int j = 0; j < MAXJ; ++j) {
      const int i = lane + WAVE * j;
      const float xt = i < d ? to_float(x[row * d + i]) : 0.f;
      float acc = wv[j][W - 1] * xt;
#pragma unroll
      for (int s = 0; s < W - 1; ++s) acc += wv[j][s] * st[s][j];
#pragma unroll
      for (int s = 0; s + 1 < W - 1; ++s) st[s][j] = st[s + 1][j];
      if constexpr (W > 1) st[W - 2][j] = xt;
      a[j] = i < d ? silu(acc) : 0.f;
      ss += a[j] * a[j];
    }
    const float scale = which < 2 ? rsqrtf(wave_sum(ss) + p.eps) : 1.f;
#pragma unroll
    for (int j = 0; j < MAXJ; ++j) {
      const int i = lane + WAVE * j;
      if (i < d) y[row * d + i] = to_elem<E>(a[j] * scale);
    }
  }
#pragma unroll
  for (int j = 0; j < MAXJ; ++j) {
    const int i = lane + WAVE * j;
#pragma unroll
    for (int s = 0; s < W - 1; ++s)
      if (i < d) cs[(((long)b * (W - 1) + s) * p.H + h) * d + i] = to_elem<E>(st[s][j]);
  }
}

template <typename E>
hipError_t prologue_step_t(const LayerParams& p, hipStream_t st) {
  const dim3 grid((unsigned)((3L * p.B * p.H + ROWS_PER_WG - 1) / ROWS_PER_WG)), block(WAVE * ROWS_PER_WG);
  switch (p.width) {
    case 1: hipLaunchKernelGGL((prologue_step_kernel<E, 1>), grid, block, 0, st, p); break;
    case 2: hipLaunchKernelGGL((prologue_step_kernel<E, 2>), grid, block, 0, st, p); break;
    case 3: hipLaunchKernelGGL((prologue_step_kernel<E, 3>), grid, block, 0, st, p); break;
    case 4: hipLaunchKernelGGL((prologue_step_kernel<E, 4>), grid, block, 0, st, p); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_layer_prologue_step(const LayerParams& p, bool bf16_in, hipStream_t st) {
  return bf16_in ? prologue_step_t<bf16>(p, st) : prologue_step_t<float>(p, st);
}

hipError_t launch_layer_prologue(const LayerParams& p, bool bf16_in, hipStream_t st) {
  return bf16_in ? prologue_t<bf16>(p, st) : prologue_t<float>(p, st);
}

hipError_t launch_layer_epilogue(const LayerParams& p, bool bf16_in, hipStream_t st) {
  return bf16_in ? epilogue_t<bf16>(p, st) : epilogue_t<float>(p, st);
}

}  // namespace delta
