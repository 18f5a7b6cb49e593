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
// T and A depend only on the chunk's own inputs; the intra-chunk kernel forms them once per
// chunk and this kernel reads them (8 slabs of a head read each chunk's T and A from L2).
// Forming V~ as T (V - gamma K S) instead of materialising W = T (gamma K) (C x d_k per
// chunk) saves a C x C x d_k contraction per slab; both are the same product.
//
// Schedule per chunk (3 workgroup barriers; only the state chain S -> K S -> T Y ->
// K^T V~ -> S is sequential across chunks):
//   phase 1  X = K S (row block per wave) -> Y^T;  O1 = Q S (token block per wave);
//            the next chunk's global loads are issued here into registers
//   phase 2  V~ = T Y -> V~^T, (gamma_C/gamma V~)^T
//   phase 3  S update -> S^T;  O = gamma O1 + A V~ -> HBM;  prefetched chunk -> LDS
// bf16 inputs double-buffer the staged chunk in LDS, so phase 3 can write the next
// chunk while the current one is still read; fp32 inputs (twice the bytes) use one
// buffer and an extra barrier.
//
// MFMA operands live in LDS in K-contiguous rows: K and Q row-major (A operands, and B
// operands of K Q^T), K^T (A operand of the state update; bf16 only -- fp32 fragments
// are single elements and read K column-wise directly), T row-major, and S^T, Y^T,
// V~^T, (gamma_C/gamma V~)^T as B operands.  Products with bf16 inputs round the
// operands to bf16 and accumulate in fp32; the master state stays fp32.
#include "common.h"
#include "kernels.h"

namespace delta {

template <typename E, int DK, int C>
struct InterCfg {
  static constexpr bool BF = sizeof(E) == 2;
  static constexpr int PAD = 16 / sizeof(E);
  static constexpr int VEC = 16 / sizeof(E);   // elements per 16-byte copy
  static constexpr int LDK = DK + PAD;          // stride of K, Q, S^T rows
  static constexpr int LDC = C + PAD;           // stride of K^T, T, Y^T, V~^T, A rows
  static constexpr int NBUF = BF ? 2 : 1;       // staged-chunk buffers
  // one staged chunk: K, Q (up to C token rows), K^T (bf16 only), T, A, V slab
  static constexpr int KS = C * LDK, QS = C * LDK, KTS = BF ? DK * LDC : 0, TS = C * LDC, AS = C * LDC,
                       VS = C * 16;
  static constexpr int IN = KS + QS + KTS + TS + AS + VS;
  // per-workgroup work area: S^T, Y^T, V~^T, (D V~)^T
  static constexpr int STS = 16 * LDK, YTS = 16 * LDC;
  static constexpr int WORK = STS + 3 * YTS;
  static constexpr int ELEMS = NBUF * IN + WORK;
  // prefetch slots per thread (256 threads)
  static constexpr int KITEMS = (C / 2) * (DK / VEC);   // pairs of key rows x 16-byte columns
  static constexpr int NK = (KITEMS + 255) / 256;
  static constexpr int QITEMS = C * (DK / VEC);
  static constexpr int NQ = (QITEMS + 255) / 256;
  static constexpr int TITEMS = C * (C / VEC);
  static constexpr int NT = (TITEMS + 255) / 256;
  static constexpr int VITEMS = C * (16 / VEC);          // <= 256
};

__device__ inline int round_up(int x, int m) { return (x + m - 1) / m * m; }

template <typename E, int DK, int C>
struct Staged {
  using Cfg = InterCfg<E, DK, C>;
  u32x4 k[Cfg::NK][2];
  u32x4 q[Cfg::NQ];
  u32x4 t[Cfg::NT];
  u32x4 a[Cfg::NT];
  u32x4 v;
  float gc;
};

template <typename E, int DK, int C>
__global__ __launch_bounds__(256) void inter_chunk_kernel(FwdParams p) {
  using Cfg = InterCfg<E, DK, C>;
  constexpr int LDK = Cfg::LDK, LDC = Cfg::LDC, VEC = Cfg::VEC, NBUF = Cfg::NBUF;
  constexpr int NBC = C / 16;          // position blocks per chunk
  constexpr int NTS = DK / 16;         // state row tiles
  constexpr int SLOTS = (NTS + 3) / 4; // state tiles per wave
  constexpr int KSTEP = Mfma<E>::KSTEP;

  __shared__ __attribute__((aligned(16))) E smem[Cfg::ELEMS];
  __shared__ float egs[NBUF][C], eds[NBUF][C];  // exp(gc), exp(gc_last - gc)

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
  const E* Ag = reinterpret_cast<const E*>(p.A);
  E* Og = reinterpret_cast<E*>(p.O);

  // staged-chunk buffers are addressed as smem + buf * IN (plain arithmetic on the LDS array,
  // so every access stays an LDS access)
  E* StS = smem + NBUF * Cfg::IN;
  E* YTs = StS + Cfg::STS;
  E* VtTs = YTs + Cfg::YTS;
  E* DVtTs = VtTs + Cfg::YTS;

  // ---------------- global -> registers for chunk n (all loads issued, none waited on)
  auto load_chunk = [&](int n, Staged<E, DK, C>& st) {
    const long P0 = (long)n * C;
#pragma unroll
    for (int i = 0; i < Cfg::NK; ++i) {
      const int it = tid + 256 * i;
      const int rp = it % (C / 2), cc = it / (C / 2);
#pragma unroll
      for (int s = 0; s < 2; ++s) {
        const long pos = P0 + 2 * rp + s;
        u32x4 val = {0u, 0u, 0u, 0u};
        if (it < Cfg::KITEMS && pos < p.Lx)
          val = *reinterpret_cast<const u32x4*>(kg + (((long)b * p.Lx + pos) * p.H + h) * DK + cc * VEC);
        st.k[i][s] = val;
      }
    }
#pragma unroll
    for (int i = 0; i < Cfg::NQ; ++i) {
      const int it = tid + 256 * i;
      const int r = it / (DK / VEC), c = (it % (DK / VEC)) * VEC;
      const long tok = (long)n * QR + r;
      u32x4 val = {0u, 0u, 0u, 0u};
      if (it < Cfg::QITEMS && r < QR && tok < p.L)
        val = *reinterpret_cast<const u32x4*>(qg + (((long)b * p.L + tok) * p.H + h) * DK + c);
      st.q[i] = val;
    }
    const E* Tc = Tg + ((long)head * p.NT + n) * C * C;
    const E* Ac = Ag + ((long)head * p.NT + n) * C * C;
#pragma unroll
    for (int i = 0; i < Cfg::NT; ++i) {
      const int it = tid + 256 * i;
      u32x4 tv = {0u, 0u, 0u, 0u}, av = {0u, 0u, 0u, 0u};
      if (it < Cfg::TITEMS) {
        tv = *reinterpret_cast<const u32x4*>(Tc + it * VEC);
        av = *reinterpret_cast<const u32x4*>(Ac + it * VEC);
      }
      st.t[i] = tv;
      st.a[i] = av;
    }
    {
      const int r = tid / (16 / VEC), c = (tid % (16 / VEC)) * VEC;
      const long pos = P0 + r;
      u32x4 val = {0u, 0u, 0u, 0u};
      if (tid < Cfg::VITEMS && pos < p.Lx)
        val = *reinterpret_cast<const u32x4*>(vg + (((long)b * p.Lx + pos) * p.H + h) * p.DV + slab * 16 + c);
      st.v = val;
    }
    st.gc = (tid < C) ? p.gc[((long)head * p.NT + n) * C + tid] : 0.f;
  };

  // ---------------- registers -> LDS buffer `buf`
  auto store_chunk = [&](const Staged<E, DK, C>& st, int buf) {
    E* Ks = smem + buf * Cfg::IN;
    E* Qs = Ks + Cfg::KS;
    E* KTs = Qs + Cfg::QS;
    E* Ts = KTs + Cfg::KTS;
    E* As = Ts + Cfg::TS;
    E* Vs = As + Cfg::AS;
#pragma unroll
    for (int i = 0; i < Cfg::NK; ++i) {
      const int it = tid + 256 * i;
      if (it < Cfg::KITEMS) {
        const int rp = it % (C / 2), cc = it / (C / 2);
        *reinterpret_cast<u32x4*>(Ks + (2 * rp) * LDK + cc * VEC) = st.k[i][0];
        *reinterpret_cast<u32x4*>(Ks + (2 * rp + 1) * LDK + cc * VEC) = st.k[i][1];
        if constexpr (Cfg::BF) {
          // K^T rows: the two key rows of this pair are adjacent, so each K^T element pair is
          // one packed 4-byte write.  Dword w of a row holds elements 2w (low) and 2w+1 (high).
#pragma unroll
          for (int w = 0; w < 4; ++w) {
            const uint32_t a = st.k[i][0][w], c = st.k[i][1][w];
            *reinterpret_cast<uint32_t*>(KTs + (cc * VEC + 2 * w) * LDC + 2 * rp) = (a & 0xFFFFu) | (c << 16);
            *reinterpret_cast<uint32_t*>(KTs + (cc * VEC + 2 * w + 1) * LDC + 2 * rp) = (a >> 16) | (c & 0xFFFF0000u);
          }
        }
      }
    }
#pragma unroll
    for (int i = 0; i < Cfg::NQ; ++i) {
      const int it = tid + 256 * i;
      if (it < Cfg::QITEMS) {
        const int r = it / (DK / VEC), c = (it % (DK / VEC)) * VEC;
        *reinterpret_cast<u32x4*>(Qs + r * LDK + c) = st.q[i];
      }
    }
#pragma unroll
    for (int i = 0; i < Cfg::NT; ++i) {
      const int it = tid + 256 * i;
      if (it < Cfg::TITEMS) {
        const int r = (it * VEC) / C, c = (it * VEC) % C;
        *reinterpret_cast<u32x4*>(Ts + r * LDC + c) = st.t[i];
        *reinterpret_cast<u32x4*>(As + r * LDC + c) = st.a[i];
      }
    }
    if (tid < Cfg::VITEMS) {
      const int r = tid / (16 / VEC), c = (tid % (16 / VEC)) * VEC;
      *reinterpret_cast<u32x4*>(Vs + r * 16 + c) = st.v;
    }
    if (tid < 64) {  // C <= 64: wave 0 owns the gate arrays
      const float gl = __shfl(st.gc, C - 1, 64);
      if (tid < C) {
        egs[buf][tid] = expf(st.gc);
        eds[buf][tid] = expf(gl - st.gc);
      }
    }
  };

  // ---------------- initial state and the static zeros of A
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
  if (p.NT > 0) {
    Staged<E, DK, C> st;
    load_chunk(0, st);
    store_chunk(st, 0);
  }
  __syncthreads();

  // last position block a token row of tile t may read
  auto jmax_of = [&](int t) { return (min(16 * t + 15, QR - 1) * nh + nh - 1) / 16; };

  for (int n = 0; n < p.NT; ++n) {
    const int cur = (NBUF == 2) ? (n & 1) : 0;
    E* Ks = smem + cur * Cfg::IN;
    E* Qs = Ks + Cfg::KS;
    E* KTs = Qs + Cfg::QS;
    E* Ts = KTs + Cfg::KTS;
    E* Aqs = Ts + Cfg::TS;
    E* Vs = Aqs + Cfg::AS;
    const float* eg = egs[cur];
    const float* ed = eds[cur];

    Staged<E, DK, C> st;
    const bool more = n + 1 < p.NT;
    if (more) load_chunk(n + 1, st);

    // ---------------- phase 1: Y = V - gamma (K S); O1 = Q S
    if (wave < NBC) {
      floatx4 x = {0.f, 0.f, 0.f, 0.f};
      x = mma_tile<E>(x, Ks + 16 * wave * LDK, LDK, StS, LDK, DK, lane);
      const int r0 = 16 * wave + rq;
      float y[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) y[r] = to_float(Vs[(r0 + r) * 16 + col]) - eg[r0 + r] * x[r];
      store4<E>(YTs + col * LDC + r0, y[0], y[1], y[2], y[3]);
    }
    floatx4 o1 = {0.f, 0.f, 0.f, 0.f};
    if (wave < NQT) o1 = mma_tile<E>(o1, Qs + 16 * wave * LDK, LDK, StS, LDK, DK, lane);
    __syncthreads();

    // ---------------- phase 2: V~ = T Y (T lower triangular: k up to the row block's end)
    if (wave < NBC) {
      floatx4 vt = {0.f, 0.f, 0.f, 0.f};
      const int K2 = min(round_up(16 * (wave + 1), KSTEP), C);
      vt = mma_tile<E>(vt, Ts + 16 * wave * LDC, LDC, YTs, LDC, K2, lane);
      const int r0 = 16 * wave + rq;
      store4<E>(VtTs + col * LDC + r0, vt[0], vt[1], vt[2], vt[3]);
      store4<E>(DVtTs + col * LDC + r0, vt[0] * ed[r0], vt[1] * ed[r0 + 1], vt[2] * ed[r0 + 2],
                vt[3] * ed[r0 + 3]);
    }
    __syncthreads();

    // ---------------- phase 3: state update, outputs, next chunk into LDS
    {
      const float gC = eg[C - 1];
#pragma unroll
      for (int s = 0; s < SLOTS; ++s) {
        const int t = wave + 4 * s;
        if (t < NTS) {
          floatx4 acc = S[s] * gC;
          if constexpr (Cfg::BF) {
            acc = mma_tile<E>(acc, KTs + 16 * t * LDC, LDC, DVtTs, LDC, C, lane);
          } else {
            // fp32: A[d][r] = K[r][d] read column-wise from the row-major key tile
            const E* bcol = DVtTs + col * LDC;
#pragma unroll 4
            for (int k0 = 0; k0 < C; k0 += 4) {
              const int r = k0 + (lane >> 4);
              acc = Mfma<E>::mma(Ks[r * LDK + 16 * t + col], bcol[r], acc);
            }
          }
          S[s] = acc;
          store4<E>(StS + col * LDK + 16 * t + rq, acc[0], acc[1], acc[2], acc[3]);
        }
      }
    }
    if (wave < NQT) {
      floatx4 o2 = {0.f, 0.f, 0.f, 0.f};
      const int K3 = min(round_up(16 * (jmax_of(wave) + 1), KSTEP), C);
      o2 = mma_tile<E>(o2, Aqs + 16 * wave * LDC, LDC, VtTs, LDC, K3, lane);
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int trow = 16 * wave + rq + r;
        const long tok = (long)n * QR + trow;
        if (trow < QR && tok < p.L)
          Og[(((long)b * p.L + tok) * p.H + h) * p.DV + slab * 16 + col] =
              to_elem<E>(p.scale * (eg[trow * nh + nh - 1] * o1[r] + o2[r]));
      }
    }
    if constexpr (NBUF == 1) __syncthreads();  // the single staging buffer is still being read
    if (more) store_chunk(st, NBUF == 2 ? cur ^ 1 : 0);
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
