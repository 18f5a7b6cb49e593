// The UT transform of a chunk ("08 linear delta rule & DPLR" page, section 2.2): from the
// strictly lower C x C matrix A (float32, in 16 x 16 blocks in LDS) the unit-lower-triangular
// inverse N = (I + A)^-1, and T = N diag(beta) written row-major.  Shared by the intra-chunk
// kernels of the scalar-gated (intra_chunk.hip) and per-channel-decayed (kda_chunk.hip) forms,
// which differ only in how they weight the Gram matrix.
//
// A and N are lower triangular: only their blocks of 16 x 16 on and below the diagonal are
// stored, rows padded to LDB floats, in slots of one array.  A block (i, j) is in slot
// lower_block(i, j).  N's diagonal blocks take the slots of A's (a diagonal A block is read only
// by the substitution that turns it into the N block, in the same wavefront); N's blocks below
// the diagonal follow A's, except at C = 64, where N_20 and N_30 take the slots of A_10 and A_21,
// which are no longer read once those are formed (A_10 only feeds N_10, A_21 only N_21 and
// N_20).  Fewer LDS bytes per tile let more workgroups share a compute unit.
//
// The diagonal blocks are inverted by forward substitution (lane c owns column c), then the
// blocks below the diagonal follow diagonal by diagonal from the exact identity
//     N_ij = -N_ii * sum_{k=j}^{i-1} A_ik N_kj          (i > j),
// with the 16 x 16 products on the fp32 MFMA.
#pragma once

#include "common.h"

namespace delta {

__host__ __device__ constexpr int lower_block(int i, int j) { return i * (i + 1) / 2 + j; }
template <int NB>
__host__ __device__ constexpr int n_slot(int i, int j) {
  constexpr int NBLK = NB * (NB + 1) / 2;
  if (i == j) return lower_block(i, i);
  if (NB == 4) {
    if (i == 2 && j == 0) return lower_block(1, 0);
    if (i == 3 && j == 0) return lower_block(2, 1);
    return NBLK + (i == 1 ? 0 : i == 2 ? 1 : j + 1);  // N_10, N_21, N_31, N_32
  }
  return NBLK + i * (i - 1) / 2 + j;
}

template <int C>
struct UtSlots {
  static constexpr int NB = C / 16;
  static constexpr int LDB = 20;                      // fp32 row stride inside a 16 x 16 block
  static constexpr int BLK = 16 * LDB;                // floats per block
  static constexpr int NBLK = NB * (NB + 1) / 2;
  static constexpr int NSLOT = NBLK + (NB == 4 ? 4 : NB * (NB - 1) / 2);
  static constexpr int BYTES = NSLOT * BLK * 4;       // A and N
};

// With A's lower blocks in the slots at As (4 wavefronts of 256 threads, A written and published
// by a barrier before the call): N into the slots, then T = N diag(bs) to Tout (and, if Nout,
// N itself in float32) as C x C row-major, zero above the diagonal.  Ends with the workgroup past
// its last barrier; the slots hold N afterwards.
template <int C, typename TO>
__device__ __forceinline__ void ut_solve_store(float* As, const float* bs, TO* Tout, float* Nout, int tid) {
  using U = UtSlots<C>;
  constexpr int NB = U::NB, LDB = U::LDB, BLK = U::BLK;
  auto ablk = [&](int i, int j) { return As + lower_block(i, j) * BLK; };
  auto nblk = [&](int i, int j) { return As + n_slot<NB>(i, j) * BLK; };
  const int lane = tid & 63, wave = tid >> 6;
  const int col = lane & 15, rq = 4 * (lane >> 4);

  // diagonal tiles by forward substitution, all in wave 0: lane 16 t + c owns column c of tile t
  // (x_i = e_i - sum_{j<i} A_ij x_j), rows of A read 4 at a time
  if (wave == 0 && lane < 16 * NB) {
    const int t = lane >> 4;
    float x[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      float a0 = (i == col) ? 1.f : 0.f, a1 = 0.f;
      const float* Ai = ablk(t, t) + i * LDB;
#pragma unroll
      for (int j4 = 0; j4 < i; j4 += 4) {
        const floatx4 a = *reinterpret_cast<const floatx4*>(Ai + j4);
#pragma unroll
        for (int e = 0; e < 4; ++e)
          if (j4 + e < i) {
            if (e & 1) a1 -= a[e] * x[j4 + e];
            else a0 -= a[e] * x[j4 + e];
          }
      }
      x[i] = a0 + a1;
    }
#pragma unroll
    for (int i = 0; i < 16; ++i) nblk(t, t)[i * LDB + col] = x[i];
  }
  __syncthreads();

  // tiles below the diagonal, one block diagonal d at a time:
  //   P = sum_{k=j}^{i-1} A_ik N_kj,  N_ij = -N_ii P
  // P stays in the accumulator registers: lane (g, n) holds P[4g + r][n], r < 4, which is the B
  // operand of step r of the second product when its contraction index is taken as 4g + r (the
  // A operand N_ii[m][4g + r] is read to match).  P being the wave's own, one barrier per block
  // diagonal orders the N tiles between the waves.
  for (int d = 1; d < NB; ++d) {
    const int i = wave + d, j = wave;   // wave w owns tile (w + d, w)
    if (i < NB) {
      floatx4 acc = {0.f, 0.f, 0.f, 0.f};
      for (int k = j; k < i; ++k) {
        // A operand: rows of A_ik; B operand B[kk][n] = N[16k + kk][16j + n] read column-wise
#pragma unroll
        for (int k0 = 0; k0 < 16; k0 += 4) {
          const int kk = k0 + (lane >> 4);
          acc = Mfma<float>::mma(ablk(i, k)[col * LDB + kk], nblk(k, j)[kk * LDB + col], acc);
        }
      }
      floatx4 nij = {0.f, 0.f, 0.f, 0.f};
      const float* Nii = nblk(i, i) + col * LDB + rq;
#pragma unroll
      for (int r = 0; r < 4; ++r) nij = Mfma<float>::mma(Nii[r], acc[r], nij);
#pragma unroll
      for (int r = 0; r < 4; ++r) nblk(i, j)[(rq + r) * LDB + col] = -nij[r];
    }
    __syncthreads();
  }

  // T = N diag(beta), row-major, zero above the diagonal; 4 consecutive elements per store
#pragma unroll
  for (int idx = 4 * tid; idx < C * C; idx += 4 * 256) {
    const int r = idx / C, c = idx % C;
    // blocks above the diagonal are not stored: read the row's diagonal block, the select drops it
    const floatx4 nv = *reinterpret_cast<const floatx4*>(nblk(r >> 4, min(c >> 4, r >> 4)) + (r & 15) * LDB + (c & 15));
    const floatx4 bv = *reinterpret_cast<const floatx4*>(bs + c);
    float x[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) x[e] = c + e <= r ? nv[e] * bv[e] : 0.f;
    store4<TO>(Tout + idx, x[0], x[1], x[2], x[3]);
    if (Nout) {  // the backward also takes N itself (beta may be 0, so T does not determine it)
#pragma unroll
      for (int e = 0; e < 4; ++e) x[e] = c + e <= r ? nv[e] : 0.f;
      store4<float>(Nout + idx, x[0], x[1], x[2], x[3]);
    }
  }
}

}  // namespace delta
