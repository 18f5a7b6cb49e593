// Recurrent decode kernel: one token per (b, h), state updated in place.
//
// Sources: "08 linear delta rule & DPLR" page, recurrent reference after section 2.3
// (read v_old = S^T k, write beta k (v - v_old)^T, output S^T q), section 3 (scalar
// gate applied to the state first) and sections 1.4 / 5 (KDA: a decay per key channel,
// Diag(alpha) applied to the state's rows before the write); DeltaProduct notes, section 2.6
// pseudocode (gate, then n_h ordered residual writes, then the readout).
//
// The step is bound by HBM traffic: the d_k x d_v fp32 state is read once and written
// once.  One workgroup owns a d_k x SW column slab of one head's state (columns are
// independent), held in registers as 4 rows x 4 columns per thread with 16-byte,
// row-coalesced loads and stores.  The two reductions over d_k of the last sub-step,
// S^T k and S^T q, share one pass: with e = v - S^T k,
//   o = scale * S'^T q = scale * (S^T q + beta (k . q) e),   S' = S + beta k e^T.
#include "common.h"
#include "kernels.h"

namespace delta {

// Barrier that waits only for this wave's LDS operations.
__device__ inline void lds_barrier() {
  __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
  asm volatile("s_barrier" ::: "memory");
}

// Sum NV per-thread values over all threads of the block that share column quad cq;
// every thread receives the sums for its cq.
template <int NTH, int CQ, int NV>
__device__ inline void reduce_rows(float (&x)[NV], float* red, int tid) {
  const int lane = tid & 63, wave = tid >> 6;
  constexpr int WSPAN = NTH < 64 ? NTH : 64;
#pragma unroll
  for (int off = CQ; off < WSPAN; off <<= 1)
#pragma unroll
    for (int i = 0; i < NV; ++i) x[i] += __shfl_xor(x[i], off, 64);
  constexpr int NW = (NTH + 63) / 64;
  if constexpr (NW > 1) {
    if (lane < CQ)
#pragma unroll
      for (int i = 0; i < NV; ++i) red[(wave * NV + i) * CQ + lane] = x[i];
    lds_barrier();
    const int cq = tid % CQ;
#pragma unroll
    for (int i = 0; i < NV; ++i) {
      float s = 0.f;
#pragma unroll
      for (int w = 0; w < NW; ++w) s += red[(w * NV + i) * CQ + cq];
      x[i] = s;
    }
    lds_barrier();
  }
}

// 4 consecutive elements of E as floats (one 8- or 16-byte load), and back.
template <typename E>
__device__ inline void load4(float (&x)[4], const E* src) {
  if constexpr (sizeof(E) == 2) {
    const bf16x4 v = *reinterpret_cast<const bf16x4*>(src);
#pragma unroll
    for (int i = 0; i < 4; ++i) x[i] = (float)v[i];
  } else {
    const floatx4 v = *reinterpret_cast<const floatx4*>(src);
#pragma unroll
    for (int i = 0; i < 4; ++i) x[i] = v[i];
  }
}
template <typename E>
__device__ inline void store4(E* dst, const float (&x)[4]) {
  if constexpr (sizeof(E) == 2) *reinterpret_cast<bf16x4*>(dst) = bf16x4{(bf16)x[0], (bf16)x[1], (bf16)x[2], (bf16)x[3]};
  else *reinterpret_cast<floatx4*>(dst) = floatx4{x[0], x[1], x[2], x[3]};
}

// One workgroup per (sequence, head, SW columns); thread (rg, cq) owns rows 4 rg .. 4 rg + 3 and
// columns 4 cq .. 4 cq + 3 of the slab, so its rows of q and k, its value quad and its output
// quad are single vector accesses.  The state is read and written with non-temporal accesses
// (each byte is touched once per step).
template <typename E, int DK, int SW>
__global__ __launch_bounds__(DK * SW / 16) void decode_kernel(DecodeParams p) {
  constexpr int CQ = SW / 4;          // column quads per slab
  constexpr int RG = DK / 4;          // row groups of 4 consecutive rows
  constexpr int NTH = RG * CQ;
  constexpr int NW = (NTH + 63) / 64;
  __shared__ float red[NW * 9 * CQ];

  const int tid = threadIdx.x;
  const int cq = tid % CQ, rg = tid / CQ;
  const int r0 = 4 * rg;
  const int nsl = p.DV / SW;
  const int head = blockIdx.x / nsl, slab = blockIdx.x % nsl;
  const int b = head / p.H, h = head % p.H;
  const E* qg = reinterpret_cast<const E*>(p.q);
  const E* kg = reinterpret_cast<const E*>(p.k);
  const E* vg = reinterpret_cast<const E*>(p.v);

  float* Sg = p.S + (long)head * DK * p.DV + slab * SW + cq * 4;
  floatx4 s[4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
    s[i] = __builtin_nontemporal_load(reinterpret_cast<const floatx4*>(Sg + (long)(r0 + i) * p.DV));
  float qr[4];
  load4<E>(qr, qg + ((long)b * p.H + h) * DK + r0);
  float dec[4] = {0.f, 0.f, 0.f, 0.f};
  if (p.a_log) {  // KDA: each key channel (row of S) decays by its own factor before the write
    const floatx4 a = *reinterpret_cast<const floatx4*>(p.a_log + ((long)b * p.H + h) * DK + r0);
#pragma unroll
    for (int i = 0; i < 4; ++i) dec[i] = a[i];
  } else if (p.g_log) {
    const float g = p.g_log[(long)b * p.H + h];
#pragma unroll
    for (int i = 0; i < 4; ++i) dec[i] = g;
  }
  if (p.a_log || p.g_log) {
#pragma unroll
    for (int i = 0; i < 4; ++i) s[i] *= expf(dec[i]);
  }

  for (int j = 0; j < p.nh; ++j) {
    const long tj = ((long)b * p.nh + j) * p.H + h;
    float kr[4], vj[4];
    load4<E>(kr, kg + tj * DK + r0);
    load4<E>(vj, vg + tj * p.DV + slab * SW + cq * 4);
    const float bj = p.beta[tj];
    const bool last = (j == p.nh - 1);
    float red_in[9];
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      float a = 0.f, q = 0.f;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        a += s[i][c] * kr[i];
        q += s[i][c] * qr[i];
      }
      red_in[c] = a;
      red_in[4 + c] = last ? q : 0.f;
    }
    float kq = 0.f;
#pragma unroll
    for (int i = 0; i < 4; ++i) kq += kr[i] * qr[i];
    red_in[8] = last ? kq : 0.f;
    reduce_rows<NTH, CQ, 9>(red_in, red, tid);
    float e[4];
#pragma unroll
    for (int c = 0; c < 4; ++c) e[c] = vj[c] - red_in[c];
    if (last && rg == 0) {
      float o[4];
#pragma unroll
      for (int c = 0; c < 4; ++c) o[c] = p.scale * (red_in[4 + c] + bj * red_in[8] * e[c]);
      store4<E>(reinterpret_cast<E*>(p.O) + ((long)b * p.H + h) * p.DV + slab * SW + cq * 4, o);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float a = bj * kr[i];
#pragma unroll
      for (int c = 0; c < 4; ++c) s[i][c] += a * e[c];
    }
  }

#pragma unroll
  for (int i = 0; i < 4; ++i)
    __builtin_nontemporal_store(s[i], reinterpret_cast<floatx4*>(Sg + (long)(r0 + i) * p.DV));
}

// 32-column slabs where d_v allows (one workgroup of 256 threads per slab at d_k = 128); a sweep
// of slab widths 16 / 32 / 64 and of grid-stride variants that prefetch the next slab measured
// 42 / 25.5 / 32 us per step and no gain from the prefetch at batch 64, 16 heads.
template <typename E, int DK>
static hipError_t decode_by_sw(const DecodeParams& p, hipStream_t st) {
  if (p.DV % 32 == 0) {
    const dim3 grid((unsigned)(p.B * p.H * (p.DV / 32))), block(DK * 32 / 16);
    hipLaunchKernelGGL((decode_kernel<E, DK, 32>), grid, block, 0, st, p);
  } else {
    const dim3 grid((unsigned)(p.B * p.H * (p.DV / 16))), block(DK * 16 / 16);
    hipLaunchKernelGGL((decode_kernel<E, DK, 16>), grid, block, 0, st, p);
  }
  return hipGetLastError();
}

template <typename E>
static hipError_t decode_by_dk(const DecodeParams& p, hipStream_t st) {
  switch (p.DK) {
    case 16: return decode_by_sw<E, 16>(p, st);
    case 32: return decode_by_sw<E, 32>(p, st);
    case 64: return decode_by_sw<E, 64>(p, st);
    case 128: return decode_by_sw<E, 128>(p, st);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_decode(const DecodeParams& p, bool bf16_in, hipStream_t st) {
  return bf16_in ? decode_by_dk<bf16>(p, st) : decode_by_dk<float>(p, st);
}

}  // namespace delta
