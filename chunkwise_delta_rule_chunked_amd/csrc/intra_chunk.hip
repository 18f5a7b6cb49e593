// Intra-chunk kernel: per (b, h, chunk) tile, the gate prefix, the Gram matrix K K^T on
// MFMA and the UT transform T = (I + strictLower(diag(beta) (Gamma * K K^T)))^-1 diag(beta)
// by forward substitution.
//
// Sources: "08 linear delta rule & DPLR" page, section 2.2 (UT transform, triangular
// inverse by forward substitution, small enough to stay on chip at C = 64) and section 3
// (gated chunk form: in-chunk cumulative log decay restarting every chunk, Gram matrix
// weighted by Gamma_ij = gamma_i / gamma_j).  DeltaProduct notes, section 4.1: on the
// expanded sequence the token's log gate sits at its first sub-step, 0 at the others.
//
// One wavefront per tile.  The tile's keys are staged in LDS; the lower-triangular
// 16x16 blocks of K K^T come from MFMA (fp32 accumulation) and are kept in registers
// until the key tile is dead, then the scaled strictly-lower matrix A replaces it in LDS.
// Lane c then solves column c of N = (I + A)^-1 by forward substitution with the column
// in registers (rows of A are LDS broadcasts), and T = N diag(beta) is written row-major.
#include "common.h"
#include "kernels.h"

namespace delta {

template <typename E, int DK, int C>
struct IntraLds {
  static constexpr int PAD = 16 / sizeof(E);
  static constexpr int LDK = DK + PAD;  // key row stride (elements)
  static constexpr int LDA = C + 4;     // A row stride (floats), keeps 16-byte rows
  static constexpr int KBYTES = C * LDK * (int)sizeof(E);
  static constexpr int ABYTES = C * LDA * 4;
  static constexpr int BYTES = KBYTES > ABYTES ? KBYTES : ABYTES;
};

template <typename E, typename TO, int DK, int C>
__global__ __launch_bounds__(64) void intra_chunk_kernel(FwdParams p) {
  using Lds = IntraLds<E, DK, C>;
  constexpr int LDK = Lds::LDK, LDA = Lds::LDA, NB = C / 16;
  __shared__ __attribute__((aligned(16))) unsigned char smem[Lds::BYTES];
  __shared__ float gcs[C], bs[C];
  E* Ks = reinterpret_cast<E*>(smem);
  float* As = reinterpret_cast<float*>(smem);

  const int lane = threadIdx.x;
  const int n = blockIdx.x % p.NT;
  const int bh = blockIdx.x / p.NT;
  const int b = bh / p.H, h = bh % p.H;
  const long P0 = (long)n * C;

  // beta and log gate of position `lane`; padded positions carry beta = 0, log g = 0
  float beta_i = 0.f, lg = 0.f;
  if (lane < C) {
    const long pos = P0 + lane;
    if (pos < p.Lx) {
      beta_i = p.beta[((long)b * p.Lx + pos) * p.H + h];
      if (p.g_log && (pos % p.nh) == 0) lg = p.g_log[((long)b * p.L + pos / p.nh) * p.H + h];
    }
  }
  const float gc = wave_inclusive_scan(lane < C ? lg : 0.f, lane);
  if (lane < C) {
    gcs[lane] = gc;
    bs[lane] = beta_i;
  }

  // stage the key tile [C][DK] (zero rows past the end of the sequence)
  constexpr int VEC = 16 / sizeof(E);
  constexpr int PER_ROW = DK / VEC;
  const E* kbase = reinterpret_cast<const E*>(p.k);
  for (int idx = lane; idx < C * PER_ROW; idx += WAVE) {
    const int r = idx / PER_ROW, c = (idx % PER_ROW) * VEC;
    const long pos = P0 + r;
    u32x4 val = {0u, 0u, 0u, 0u};
    if (pos < p.Lx) val = *reinterpret_cast<const u32x4*>(kbase + (((long)b * p.Lx + pos) * p.H + h) * DK + c);
    *reinterpret_cast<u32x4*>(Ks + r * LDK + c) = val;
  }
  __syncthreads();

  // lower-triangular blocks of K K^T (block row i >= block column j)
  floatx4 G[NB * (NB + 1) / 2];
#pragma unroll
  for (int i = 0, t = 0; i < NB; ++i)
#pragma unroll
    for (int j = 0; j <= i; ++j, ++t) {
      floatx4 acc = {0.f, 0.f, 0.f, 0.f};
      G[t] = mma_tile<E>(acc, Ks + 16 * i * LDK, LDK, Ks + 16 * j * LDK, LDK, DK, lane);
    }
  __syncthreads();  // the key tile is dead: A overwrites it

  // A_rc = beta_r exp(gc_r - gc_c) (K K^T)_rc for r > c
#pragma unroll
  for (int i = 0, t = 0; i < NB; ++i)
#pragma unroll
    for (int j = 0; j <= i; ++j, ++t) {
      const int col = 16 * j + (lane & 15);
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int row = 16 * i + 4 * (lane >> 4) + r;
        float a = 0.f;
        if (row > col) a = bs[row] * expf(gcs[row] - gcs[col]) * G[t][r];
        As[row * LDA + col] = a;
      }
    }
  __syncthreads();

  // forward substitution, lane c owns column c of N = (I + A)^-1:
  //   N_ic = delta_ic - sum_{j<i} A_ij N_jc
  float x[C];
#pragma unroll
  for (int i = 0; i < C; ++i) {
    float acc = (i == lane) ? 1.f : 0.f;
    const float* Ai = As + i * LDA;
#pragma unroll
    for (int j = 0; j < i; ++j) acc -= Ai[j] * x[j];
    x[i] = acc;
  }

  // T = N diag(beta): column c scaled by beta_c; rows written coalesced across lanes
  if (lane < C) {
    const float bc = bs[lane];
    TO* Tout = reinterpret_cast<TO*>(p.T) + ((long)bh * p.NT + n) * C * C;
#pragma unroll
    for (int i = 0; i < C; ++i) Tout[i * C + lane] = to_elem<TO>(x[i] * bc);
    p.gc[((long)bh * p.NT + n) * C + lane] = gc;
  }
}

// Inspection only: W = T (exp(gc) * K), U = T V from the fp32 T written above.
template <typename E, int DK>
__global__ __launch_bounds__(64) void wy_factors_kernel(FwdParams p) {
  const int lane = threadIdx.x;
  const int C = p.C;
  const int n = blockIdx.x % p.NT;
  const int bh = blockIdx.x / p.NT;
  const int b = bh / p.H, h = bh % p.H;
  const long P0 = (long)n * C;
  const float* T = reinterpret_cast<const float*>(p.T) + ((long)bh * p.NT + n) * C * C;
  const float* gc = p.gc + ((long)bh * p.NT + n) * C;
  const E* kb = reinterpret_cast<const E*>(p.k);
  const E* vb = reinterpret_cast<const E*>(p.v);
  if (p.W) {
    float* W = p.W + ((long)bh * p.NT + n) * C * DK;
    for (int idx = lane; idx < C * DK; idx += WAVE) {
      const int i = idx / DK, d = idx % DK;
      float acc = 0.f;
      for (int j = 0; j <= i; ++j) {
        const long pos = P0 + j;
        if (pos >= p.Lx) break;
        acc += T[i * C + j] * expf(gc[j]) * to_float(kb[(((long)b * p.Lx + pos) * p.H + h) * DK + d]);
      }
      W[idx] = acc;
    }
  }
  if (p.U) {
    const int DV = p.DV;
    float* U = p.U + ((long)bh * p.NT + n) * C * DV;
    for (int idx = lane; idx < C * DV; idx += WAVE) {
      const int i = idx / DV, c = idx % DV;
      float acc = 0.f;
      for (int j = 0; j <= i; ++j) {
        const long pos = P0 + j;
        if (pos >= p.Lx) break;
        acc += T[i * C + j] * to_float(vb[(((long)b * p.Lx + pos) * p.H + h) * DV + c]);
      }
      U[idx] = acc;
    }
  }
}

template <typename E, typename TO, int DK>
static hipError_t intra_by_c(const FwdParams& p, hipStream_t st) {
  const dim3 grid((unsigned)(p.B * p.H * p.NT)), block(WAVE);
  switch (p.C) {
    case 16: hipLaunchKernelGGL((intra_chunk_kernel<E, TO, DK, 16>), grid, block, 0, st, p); break;
    case 32: hipLaunchKernelGGL((intra_chunk_kernel<E, TO, DK, 32>), grid, block, 0, st, p); break;
    case 48: hipLaunchKernelGGL((intra_chunk_kernel<E, TO, DK, 48>), grid, block, 0, st, p); break;
    case 64: hipLaunchKernelGGL((intra_chunk_kernel<E, TO, DK, 64>), grid, block, 0, st, p); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

template <typename E, typename TO>
static hipError_t intra_by_dk(const FwdParams& p, hipStream_t st) {
  switch (p.DK) {
    case 16: return intra_by_c<E, TO, 16>(p, st);
    case 32: return intra_by_c<E, TO, 32>(p, st);
    case 64: return intra_by_c<E, TO, 64>(p, st);
    case 128: return intra_by_c<E, TO, 128>(p, st);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_intra_chunk(const FwdParams& p, bool bf16_in, bool t_as_float, hipStream_t st) {
  if (bf16_in) return t_as_float ? intra_by_dk<bf16, float>(p, st) : intra_by_dk<bf16, bf16>(p, st);
  return intra_by_dk<float, float>(p, st);
}

template <typename E>
static hipError_t wy_by_dk(const FwdParams& p, hipStream_t st) {
  const dim3 grid((unsigned)(p.B * p.H * p.NT)), block(WAVE);
  switch (p.DK) {
    case 16: hipLaunchKernelGGL((wy_factors_kernel<E, 16>), grid, block, 0, st, p); break;
    case 32: hipLaunchKernelGGL((wy_factors_kernel<E, 32>), grid, block, 0, st, p); break;
    case 64: hipLaunchKernelGGL((wy_factors_kernel<E, 64>), grid, block, 0, st, p); break;
    case 128: hipLaunchKernelGGL((wy_factors_kernel<E, 128>), grid, block, 0, st, p); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_wy_factors(const FwdParams& p, bool bf16_in, hipStream_t st) {
  return bf16_in ? wy_by_dk<bf16>(p, st) : wy_by_dk<float>(p, st);
}

}  // namespace delta
