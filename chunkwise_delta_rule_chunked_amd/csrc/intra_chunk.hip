// Intra-chunk kernel: per (b, h, chunk) tile, the gate prefix, the Gram matrix K K^T on
// MFMA and the UT transform T = (I + strictLower(diag(beta) (Gamma * K K^T)))^-1 diag(beta).
//
// Sources: "08 linear delta rule & DPLR" page, section 2.2 (UT transform; the triangular
// inverse by forward substitution fits on chip at C = 64; prior art blocks it as 16 x 16
// diagonal blocks merged exactly) and section 3 (gated chunk form: in-chunk cumulative log
// decay restarting every chunk, Gram matrix weighted by Gamma_ij = gamma_i / gamma_j).
// DeltaProduct notes, section 4.1: on the expanded sequence the token's log gate sits at its
// first sub-step, 0 at the others.
//
// One workgroup of 4 wavefronts per tile.  Keys are staged in LDS; the lower 16 x 16 blocks
// of K K^T come from MFMA (fp32 accumulation).  (The gated causal Q K^T is formed where it is
// used, in the outputs launch of the inter-chunk pass.)
//
// The unit-lower-triangular inverse N = (I + A)^-1 and T = N diag(beta): ut_solve.h.
#include "common.h"
#include "kernels.h"
#include "ut_solve.h"

namespace delta {

// The key tile, then (once it is dead) the A / N block slots of ut_solve.h in the same bytes.
template <typename E, int DK, int C>
struct IntraLds {
  static constexpr int NB = C / 16;
  static constexpr int LDK = TileLayout<E, DK>::LD;  // key row stride (elements)
  static constexpr int LDB = UtSlots<C>::LDB, BLK = UtSlots<C>::BLK, NBLK = UtSlots<C>::NBLK;
  static constexpr int KBYTES = C * LDK * (int)sizeof(E);
  static constexpr int ANBYTES = UtSlots<C>::BYTES;  // A and N
  static constexpr int BYTES = KBYTES > ANBYTES ? KBYTES : ANBYTES;
};

template <typename E, typename TO, int DK, int C>
__global__ __launch_bounds__(256) void intra_chunk_kernel(FwdParams p) {
  using Lds = IntraLds<E, DK, C>;
  constexpr int LDB = Lds::LDB, BLK = Lds::BLK;
  constexpr int NBLK = Lds::NBLK;  // lower blocks of K K^T
  __shared__ __attribute__((aligned(16))) unsigned char smem[Lds::BYTES];
  __shared__ float gcs[C], bs[C];
  const Tile<E> Kt = make_tile<E, DK>(reinterpret_cast<E*>(smem));
  float* As = reinterpret_cast<float*>(smem);   // after the key tile is dead
  auto ablk = [&](int i, int j) { return As + lower_block(i, j) * BLK; };

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int col = lane & 15, rq = 4 * (lane >> 4);
  const int n = blockIdx.x % p.NT;
  const int bh = blockIdx.x / p.NT;
  const int b = bh / p.H, h = bh % p.H;
  const long P0 = (long)n * C;
  const int nh = p.nh;
  const int valid = (int)min((long)C, p.Lx - P0);   // positions of this chunk inside the sequence

  // stage the key tile [C][DK]: rows past the sequence fall outside the buffer range and read 0
  constexpr int VEC = 16 / sizeof(E);
  constexpr int PER_ROW = DK / VEC;
  const int HDK = p.H * DK;
  const __amdgpu_buffer_rsrc_t krs = buffer_rsrc(
      const_cast<E*>(reinterpret_cast<const E*>(p.k)) + (((long)b * p.Lx + P0) * p.H + h) * DK,
      valid * HDK * (int)sizeof(E));
  // every thread issues all of its loads before its first LDS store, so their latencies overlap
  constexpr int NLD = (C * PER_ROW + 255) / 256;
  constexpr bool WHOLE = (C * PER_ROW) % 256 == 0;   // every thread's copies fall inside the tile
  u32x4 kv[NLD];
#pragma unroll
  for (int u = 0; u < NLD; ++u) {
    const int idx = tid + 256 * u;
    const int r = idx / PER_ROW, c = (idx % PER_ROW) * VEC;
    kv[u] = buffer_load16(krs, (r * HDK + c) * (int)sizeof(E));
  }
  // beta and log gate of position `lane` (wave 0); padded positions carry beta = 0, log g = 0
  if (wave == 0) {
    const __amdgpu_buffer_rsrc_t brs = buffer_rsrc(const_cast<float*>(p.beta) + ((long)b * p.Lx + P0) * p.H + h,
                                                   valid * p.H * 4);
    const float beta_i = buffer_load4(brs, lane < C ? lane * p.H * 4 : valid * p.H * 4);
    float lg = 0.f;
    if (p.g_log) {
      // the token's log gate sits at its first sub-step (P0 is a multiple of n_h)
      const int tok0 = (int)(P0 / nh), ntok = (valid + nh - 1) / nh;
      const __amdgpu_buffer_rsrc_t grs = buffer_rsrc(const_cast<float*>(p.g_log) + ((long)b * p.L + tok0) * p.H + h,
                                                     ntok * p.H * 4);
      const bool first = lane < C && lane % nh == 0;
      lg = buffer_load4(grs, first ? (lane / nh) * p.H * 4 : ntok * p.H * 4);
      // g = 0 (log g = -inf) is a hard reset (DeltaProduct notes, section 3.3).  Taken as the
      // finite LOG_GATE_FLOOR it makes every decay that spans the position underflow to exactly 0
      // in float32 (gamma, Gamma_ij, gamma_C / gamma), which erases the state as g = 0 does,
      // while differences of prefix sums on one side of it stay finite (-inf - (-inf) would be
      // NaN).  NaN fails the comparison and passes through.
      lg = lg < LOG_GATE_FLOOR ? LOG_GATE_FLOOR : lg;
    }
    const float gc = wave_inclusive_scan(lg, lane);
    if (lane < C) {
      gcs[lane] = gc;
      bs[lane] = beta_i;
      p.gc[((long)bh * p.NT + n) * C + lane] = gc;
    }
  }

#pragma unroll
  for (int u = 0; u < NLD; ++u) {
    const int idx = tid + 256 * u;
    const int r = idx / PER_ROW, c = (idx % PER_ROW) * VEC;
    if (WHOLE || idx < C * PER_ROW) *reinterpret_cast<u32x4*>(Kt.at(r, c)) = kv[u];
  }
  __syncthreads();

  // lower-triangular blocks of K K^T, block t = (i, j) with i >= j, dealt round-robin to waves
  floatx4 G[(NBLK + 3) / 4];
#pragma unroll
  for (int u = 0; u < (NBLK + 3) / 4; ++u) {
    const int t = wave + 4 * u;
    G[u] = floatx4{0.f, 0.f, 0.f, 0.f};
    if (t < NBLK) {
      int i = 0;
      while ((i + 1) * (i + 2) / 2 <= t) ++i;
      const int j = t - i * (i + 1) / 2;
      G[u] = mma_tile<E>(G[u], Kt, 16 * i, Kt, 16 * j, DK, lane);
    }
  }

  __syncthreads();  // the key tile is dead: A and N overwrite it

  // A_rc = beta_r exp(gc_r - gc_c) (K K^T)_rc for r > c (0 on and above the diagonal)
#pragma unroll
  for (int u = 0; u < (NBLK + 3) / 4; ++u) {
    const int t = wave + 4 * u;
    if (t < NBLK) {
      int i = 0;
      while ((i + 1) * (i + 2) / 2 <= t) ++i;
      const int j = t - i * (i + 1) / 2;
      const int c = 16 * j + col, row0 = 16 * i + rq;
      const floatx4 br = *reinterpret_cast<const floatx4*>(bs + row0);
      const floatx4 gr = *reinterpret_cast<const floatx4*>(gcs + row0);
      const float gcc = gcs[c];
      float* Ab = ablk(i, j) + rq * LDB + col;
#pragma unroll
      for (int r = 0; r < 4; ++r)
        Ab[r * LDB] = (row0 + r > c) ? br[r] * gate_exp(gr[r] - gcc) * G[u][r] : 0.f;
    }
  }
  // N starts as zero above the block diagonal (never read there) -- only the computed tiles
  // are read, so no clearing is needed.
  __syncthreads();
  ut_solve_store<C>(As, bs, reinterpret_cast<TO*>(p.T) + ((long)bh * p.NT + n) * C * C,
                    p.N ? p.N + ((long)bh * p.NT + n) * C * C : nullptr, tid);
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
  const dim3 grid((unsigned)(p.B * p.H * p.NT)), block(256);
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
