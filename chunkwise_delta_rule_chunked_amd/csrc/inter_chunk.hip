// Inter-chunk kernel: carries the state across chunks and produces the outputs.
//
// Sources: "08 linear delta rule & DPLR" page, section 2.3 (chunkwise algorithm:
// pseudo-values V~ = U - W S, O = Q S + (Q K^T * M) V~, S <- S + K^T V~), section 2.5
// (V~ contracts over all of d_k, so the key dimension cannot be split across
// workgroups) and section 3 (gated form: queries decayed to the chunk start, keys to
// the chunk end, S <- gamma_C S + (K * gamma_C / gamma)^T V~, Gamma-weighted Q K^T).
// DeltaProduct notes, section 4.1: on the expanded sequence only each token's last
// sub-step produces an output.
//
// Work split: one workgroup (4 wavefronts) per (b, h, 16-column slab of d_v).  State
// columns are independent, so slabs need no communication; each slab keeps its
// d_k x 16 fp32 state in MFMA accumulators for the whole sequence.
//
// Per chunk, with T from the intra-chunk kernel and gamma_r = exp(gc_r):
//   Y   = V - gamma * (K S)                    (the residual the writes must correct)
//   V~  = T Y                                  (= U - W S with U = T V, W = T (gamma K))
//   O   = scale * (gamma_p * (Q S) + A V~),    A = Q K^T weighted by Gamma, causal
//   S  <- gamma_C S + K^T (gamma_C / gamma * V~)
// Forming V~ as T (V - gamma K S) instead of materialising W = T (gamma K) (C x d_k per
// chunk) saves a C x C x d_k contraction per slab; both are the same product.
//
// MFMA operands live in LDS in K-contiguous rows: K and Q row-major (A operands, and B
// operands of K Q^T), K^T (A operand of the state update), T row-major, and S^T, Y^T,
// V~^T, (gamma_C/gamma V~)^T as B operands.  Products with bf16 inputs round the
// operands to bf16 and accumulate in fp32; the master state stays fp32.
#include "common.h"
#include "kernels.h"

namespace delta {

template <typename E, int DK, int C>
struct InterLds {
  static constexpr int PAD = 16 / sizeof(E);
  static constexpr int LDK = DK + PAD;  // stride of K, Q, S^T rows
  static constexpr int LDC = C + PAD;   // stride of K^T, T, Y^T, V~^T, A rows
  static constexpr int KS = C * LDK, QS = C * LDK, KTS = DK * LDC, TS = C * LDC, VS = C * 16,
                       STS = 16 * LDK, YTS = 16 * LDC, AQS = C * LDC;
  static constexpr int ELEMS = KS + QS + KTS + TS + VS + STS + 3 * YTS + AQS;
  static constexpr int BYTES = ELEMS * (int)sizeof(E) + C * 4;
};

__device__ inline int round_up(int x, int m) { return (x + m - 1) / m * m; }

template <typename E, int DK, int C>
__global__ __launch_bounds__(256) void inter_chunk_kernel(FwdParams p) {
  using Lds = InterLds<E, DK, C>;
  constexpr int LDK = Lds::LDK, LDC = Lds::LDC;
  constexpr int NBC = C / 16;          // position blocks per chunk
  constexpr int NTS = DK / 16;         // state row tiles
  constexpr int SLOTS = (NTS + 3) / 4; // state tiles per wave
  constexpr int VEC = 16 / sizeof(E);  // elements per 16-byte copy
  constexpr int KSTEP = Mfma<E>::KSTEP;

  __shared__ __attribute__((aligned(16))) E smem[Lds::ELEMS];
  __shared__ float gcs[C];
  E* Ks = smem;
  E* Qs = Ks + Lds::KS;
  E* KTs = Qs + Lds::QS;
  E* Ts = KTs + Lds::KTS;
  E* Vs = Ts + Lds::TS;
  E* StS = Vs + Lds::VS;
  E* YTs = StS + Lds::STS;
  E* VtTs = YTs + Lds::YTS;
  E* DVtTs = VtTs + Lds::YTS;
  E* Aqs = DVtTs + Lds::YTS;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int NSL = p.DV / 16;
  const int BH = p.B * p.H;

  // workgroup -> (head, slab).  Workgroups are dispatched round-robin over the 8 XCDs;
  // place all slabs of one head on the same XCD so their shared K/Q/T reads hit one L2.
  int head, slab;
  {
    const int i = blockIdx.x;
    if (BH % 8 == 0) {
      const int x = i % 8, j = i / 8;
      head = x + 8 * (j / NSL);
      slab = j % NSL;
    } else {
      head = i / NSL;
      slab = i % NSL;
    }
  }
  const int b = head / p.H, h = head % p.H;
  const int nh = p.nh;
  const int QR = C / nh;                 // tokens per chunk
  const int NQT = (QR + 15) / 16;        // token row tiles
  const int col = lane & 15;             // this lane's state column within the slab
  const int rq = 4 * (lane >> 4);        // first of this lane's 4 accumulator rows

  const E* qg = reinterpret_cast<const E*>(p.q);
  const E* kg = reinterpret_cast<const E*>(p.k);
  const E* vg = reinterpret_cast<const E*>(p.v);
  const E* Tg = reinterpret_cast<const E*>(p.T);
  E* Og = reinterpret_cast<E*>(p.O);

  // ---- initial state: S[16 t + rq + r][col] for tiles t = wave + 4 s
  floatx4 S[SLOTS];
#pragma unroll
  for (int s = 0; s < SLOTS; ++s) {
    const int t = wave + 4 * s;
    S[s] = floatx4{0.f, 0.f, 0.f, 0.f};
    if (t < NTS && p.S0) {
#pragma unroll
      for (int r = 0; r < 4; ++r)
        S[s][r] = p.S0[((long)head * DK + 16 * t + rq + r) * p.DV + slab * 16 + col];
    }
    if (t < NTS) store4<E>(StS + col * LDK + 16 * t + rq, S[s][0], S[s][1], S[s][2], S[s][3]);
  }

  for (int n = 0; n < p.NT; ++n) {
    const long P0 = (long)n * C;
    // ---------------- stage the chunk: K (and K^T), Q, T, V slab, gc
    for (int idx = tid; idx < C * (DK / VEC); idx += 256) {
      const int r = idx / (DK / VEC), c = (idx % (DK / VEC)) * VEC;
      const long pos = P0 + r;
      u32x4 val = {0u, 0u, 0u, 0u};
      if (pos < p.Lx) val = *reinterpret_cast<const u32x4*>(kg + (((long)b * p.Lx + pos) * p.H + h) * DK + c);
      *reinterpret_cast<u32x4*>(Ks + r * LDK + c) = val;
      const E* ve = reinterpret_cast<const E*>(&val);
#pragma unroll
      for (int e = 0; e < VEC; ++e) KTs[(c + e) * LDC + r] = ve[e];
    }
    for (int idx = tid; idx < 16 * NQT * (DK / VEC); idx += 256) {
      const int r = idx / (DK / VEC), c = (idx % (DK / VEC)) * VEC;
      const long tok = (long)n * QR + r;
      u32x4 val = {0u, 0u, 0u, 0u};
      if (r < QR && tok < p.L) val = *reinterpret_cast<const u32x4*>(qg + (((long)b * p.L + tok) * p.H + h) * DK + c);
      *reinterpret_cast<u32x4*>(Qs + r * LDK + c) = val;
    }
    {
      const E* Tc = Tg + ((long)head * p.NT + n) * C * C;
      for (int idx = tid; idx < C * (C / VEC); idx += 256) {
        const int r = idx / (C / VEC), c = (idx % (C / VEC)) * VEC;
        *reinterpret_cast<u32x4*>(Ts + r * LDC + c) = *reinterpret_cast<const u32x4*>(Tc + r * C + c);
      }
    }
    for (int idx = tid; idx < C * (16 / VEC); idx += 256) {
      const int r = idx / (16 / VEC), c = (idx % (16 / VEC)) * VEC;
      const long pos = P0 + r;
      u32x4 val = {0u, 0u, 0u, 0u};
      if (pos < p.Lx) val = *reinterpret_cast<const u32x4*>(vg + (((long)b * p.Lx + pos) * p.H + h) * p.DV + slab * 16 + c);
      *reinterpret_cast<u32x4*>(Vs + r * 16 + c) = val;
    }
    if (tid < C) gcs[tid] = p.gc[((long)head * p.NT + n) * C + tid];
    __syncthreads();

    // ---------------- phase 1: Y = V - gamma (K S); O1 = Q S; A = Gamma-weighted causal Q K^T
    if (wave < NBC) {
      floatx4 x = {0.f, 0.f, 0.f, 0.f};
      x = mma_tile<E>(x, Ks + 16 * wave * LDK, LDK, StS, LDK, DK, lane);
      const int r0 = 16 * wave + rq;
      float y[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) y[r] = to_float(Vs[(r0 + r) * 16 + col]) - expf(gcs[r0 + r]) * x[r];
      store4<E>(YTs + col * LDC + r0, y[0], y[1], y[2], y[3]);
    }
    floatx4 o1 = {0.f, 0.f, 0.f, 0.f};
    int jmax = 0;
    if (wave < NQT) {
      o1 = mma_tile<E>(o1, Qs + 16 * wave * LDK, LDK, StS, LDK, DK, lane);
      // last position any token of this tile reads
      const int tlast = min(16 * wave + 15, QR - 1);
      jmax = (tlast * nh + nh - 1) / 16;
      // block (j, tile) of K Q^T holds A^T: lane's D[m][n] = A[16 wave + n][16 j + m]
      const int trow = 16 * wave + col;
      const int ptok = trow * nh + nh - 1;
      for (int j = 0; j < NBC; ++j) {
        float a[4] = {0.f, 0.f, 0.f, 0.f};
        if (j <= jmax) {
          floatx4 d = {0.f, 0.f, 0.f, 0.f};
          d = mma_tile<E>(d, Ks + 16 * j * LDK, LDK, Qs + 16 * wave * LDK, LDK, DK, lane);
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int pc = 16 * j + rq + r;
            if (trow < QR && pc <= ptok) a[r] = d[r] * expf(gcs[ptok] - gcs[pc]);
          }
        }
        store4<E>(Aqs + trow * LDC + 16 * j + rq, a[0], a[1], a[2], a[3]);
      }
    }
    __syncthreads();

    // ---------------- phase 2: V~ = T Y (T lower triangular: k up to the row block's end)
    if (wave < NBC) {
      floatx4 vt = {0.f, 0.f, 0.f, 0.f};
      const int K2 = min(round_up(16 * (wave + 1), KSTEP), C);
      vt = mma_tile<E>(vt, Ts + 16 * wave * LDC, LDC, YTs, LDC, K2, lane);
      const int r0 = 16 * wave + rq;
      store4<E>(VtTs + col * LDC + r0, vt[0], vt[1], vt[2], vt[3]);
      const float gl = gcs[C - 1];
      float dv[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) dv[r] = vt[r] * expf(gl - gcs[r0 + r]);
      store4<E>(DVtTs + col * LDC + r0, dv[0], dv[1], dv[2], dv[3]);
    }
    __syncthreads();

    // ---------------- phase 3: outputs, then the state update
    if (wave < NQT) {
      floatx4 o2 = {0.f, 0.f, 0.f, 0.f};
      const int K3 = min(round_up(16 * (jmax + 1), KSTEP), C);
      o2 = mma_tile<E>(o2, Aqs + 16 * wave * LDC, LDC, VtTs, LDC, K3, lane);
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int trow = 16 * wave + rq + r;
        const long tok = (long)n * QR + trow;
        if (trow < QR && tok < p.L) {
          const float gq = expf(gcs[trow * nh + nh - 1]);
          Og[(((long)b * p.L + tok) * p.H + h) * p.DV + slab * 16 + col] =
              to_elem<E>(p.scale * (gq * o1[r] + o2[r]));
        }
      }
    }
    {
      const float gC = expf(gcs[C - 1]);
#pragma unroll
      for (int s = 0; s < SLOTS; ++s) {
        const int t = wave + 4 * s;
        if (t < NTS) {
          floatx4 acc = S[s] * gC;
          acc = mma_tile<E>(acc, KTs + 16 * t * LDC, LDC, DVtTs, LDC, C, lane);
          S[s] = acc;
          store4<E>(StS + col * LDK + 16 * t + rq, acc[0], acc[1], acc[2], acc[3]);
        }
      }
    }
    __syncthreads();
  }

  if (p.S_final) {
#pragma unroll
    for (int s = 0; s < SLOTS; ++s) {
      const int t = wave + 4 * s;
      if (t < NTS) {
#pragma unroll
        for (int r = 0; r < 4; ++r)
          p.S_final[((long)head * DK + 16 * t + rq + r) * p.DV + slab * 16 + col] = S[s][r];
      }
    }
  }
}

template <typename E, int DK>
static hipError_t inter_by_c(const FwdParams& p, hipStream_t st) {
  const dim3 grid((unsigned)(p.B * p.H * (p.DV / 16))), block(256);
  switch (p.C) {
    case 16: hipLaunchKernelGGL((inter_chunk_kernel<E, DK, 16>), grid, block, 0, st, p); break;
    case 32: hipLaunchKernelGGL((inter_chunk_kernel<E, DK, 32>), grid, block, 0, st, p); break;
    case 48: hipLaunchKernelGGL((inter_chunk_kernel<E, DK, 48>), grid, block, 0, st, p); break;
    case 64: hipLaunchKernelGGL((inter_chunk_kernel<E, DK, 64>), grid, block, 0, st, p); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

template <typename E>
static hipError_t inter_by_dk(const FwdParams& p, hipStream_t st) {
  switch (p.DK) {
    case 16: return inter_by_c<E, 16>(p, st);
    case 32: return inter_by_c<E, 32>(p, st);
    case 64: return inter_by_c<E, 64>(p, st);
    case 128: return inter_by_c<E, 128>(p, st);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_inter_chunk(const FwdParams& p, bool bf16_in, hipStream_t st) {
  return bf16_in ? inter_by_dk<bf16>(p, st) : inter_by_dk<float>(p, st);
}

}  // namespace delta
