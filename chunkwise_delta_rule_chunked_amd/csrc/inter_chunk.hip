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
// Schedule: 8 wavefronts per workgroup.  Waves 0-3 compute and never touch global memory
// inside the chunk loop; waves 4-7 move data: while the compute waves work on chunk n they
// issue the loads of chunk n+2 into one register set, write chunk n+1 (loaded during the
// previous chunk into the other set) into the other half of a double-buffered LDS stage, and
// store the previous chunk's outputs from an LDS staging tile with 16-byte stores.  (With loads and compute in the same waves, the compiler's wait
// placement stalled the compute on the prefetch.)  Per chunk, 3 workgroup barriers:
//   phase 1  X = K S (row block per wave) -> Y^T;  O1 = Q S (token block per wave)
//   phase 2  V~ = T Y -> V~^T, (gamma_C/gamma V~)^T
//   phase 3  S update -> S^T;  O = scale (gamma O1 + A V~) -> LDS staging
// Only the state chain S -> K S -> T Y -> K^T V~ -> S is sequential across chunks.
// fp32 inputs (twice the bytes) use one staging buffer and an extra barrier.
//
// MFMA operands live in LDS in K-contiguous rows: K and Q row-major (A operands), K^T (A
// operand of the state update; bf16 only -- fp32 fragments are single elements and read K
// column-wise directly), T and A row-major, and S^T, Y^T, V~^T, (gamma_C/gamma V~)^T as B
// operands.  Rows of 128 or 256 bytes use XOR-swizzled 16-byte chunks, other lengths padding
// (see Tile in common.h), so fragment reads are free of bank conflicts.  Products with bf16
// inputs round the operands to bf16 and accumulate in fp32; the master state stays fp32.
#include "common.h"
#include "kernels.h"

namespace delta {

template <typename E, int DK, int C>
struct InterCfg {
  static constexpr bool BF = sizeof(E) == 2;
  static constexpr int VEC = 16 / sizeof(E);   // elements per 16-byte copy
  static constexpr int NBUF = BF ? 2 : 1;       // staged-chunk buffers
  using RowDK = TileLayout<E, DK>;              // rows of K, Q, S^T
  using RowC = TileLayout<E, C>;                // rows of K^T, T, A, Y^T, V~^T
  using Row16 = TileLayout<E, 16>;              // rows of the V slab
  static constexpr int OLD = BF ? 24 : 20;      // output staging row stride (conflict-free stores)
  // one staged chunk: K, Q (up to C token rows), K^T (bf16 only), T, A, V slab
  static constexpr int KS = C * RowDK::LD, QS = C * RowDK::LD, KTS = BF ? DK * RowC::LD : 0,
                       TS = C * RowC::LD, AS = C * RowC::LD, VS = C * Row16::LD;
  static constexpr int IN = KS + QS + KTS + TS + AS + VS;
  // per-workgroup work area: S^T, Y^T, V~^T, (D V~)^T, output staging [C][OLD]
  static constexpr int STS = 16 * RowDK::LD, YTS = 16 * RowC::LD, OS = C * OLD;
  static constexpr int WORK = STS + 3 * YTS + OS;
  static constexpr int ELEMS = NBUF * IN + WORK;
  // loader slots per loader thread (256 loader threads)
  static constexpr int KITEMS = (C / 2) * (DK / VEC);   // pairs of key rows x 16-byte columns
  static constexpr int NK = (KITEMS + 255) / 256;
  static constexpr int QITEMS = C * (DK / VEC);
  static constexpr int NQ = (QITEMS + 255) / 256;
  static constexpr int TITEMS = C * (C / VEC);
  static constexpr int NT = (TITEMS + 255) / 256;
  static constexpr int VITEMS = C * (16 / VEC);          // <= 256
  static constexpr int OITEMS = C * (16 / VEC);          // 16-byte pieces of the output tile
  static_assert(2 * NK + NQ <= 31, "validity bits of one staged chunk must fit a word");
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
  uint32_t valid;  // per-load row validity (bit 2i+s: key pair i row s; 2NK+i: query i; 31: value)
};

// The LDS tiles of one staged chunk.
template <typename E, int DK, int C>
struct ChunkTiles {
  using Cfg = InterCfg<E, DK, C>;
  Tile<E> K, Q, KT, T, A, V;
  __device__ inline explicit ChunkTiles(E* base) {
    K = make_tile<E, DK>(base);
    Q = make_tile<E, DK>(base + Cfg::KS);
    KT = make_tile<E, C>(base + Cfg::KS + Cfg::QS);
    T = make_tile<E, C>(base + Cfg::KS + Cfg::QS + Cfg::KTS);
    A = make_tile<E, C>(base + Cfg::KS + Cfg::QS + Cfg::KTS + Cfg::TS);
    V = make_tile<E, 16>(base + Cfg::KS + Cfg::QS + Cfg::KTS + Cfg::TS + Cfg::AS);
  }
};

template <typename E, int DK, int C>
__global__ __launch_bounds__(512) void inter_chunk_kernel(FwdParams p) {
  using Cfg = InterCfg<E, DK, C>;
  constexpr int VEC = Cfg::VEC, NBUF = Cfg::NBUF, OLD = Cfg::OLD;
  constexpr int NBC = C / 16;          // position blocks per chunk
  constexpr int NTS = DK / 16;         // state row tiles
  constexpr int SLOTS = (NTS + 3) / 4; // state tiles per compute wave
  constexpr int KSTEP = Mfma<E>::KSTEP;

  __shared__ __attribute__((aligned(16))) E smem[Cfg::ELEMS];
  __shared__ float egs[NBUF][C], eds[NBUF][C];  // exp(gc), exp(gc_last - gc)

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const bool loader = wave >= 4;
  const int ltid = tid - 256;            // loader thread index (loader waves only)
  const int NSL = p.DV / 16;
  const int BH = p.B * p.H;

  // workgroup -> (head, slab).  Workgroups are dispatched round-robin over the 8 XCDs;
  // place all slabs of one head on the same XCD so their shared K/Q/T/A reads hit one L2.
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
  E* work = smem + NBUF * Cfg::IN;
  const Tile<E> St = make_tile<E, DK>(work);                          // S^T  [16][DK]
  const Tile<E> Yt = make_tile<E, C>(work + Cfg::STS);                // Y^T  [16][C]
  const Tile<E> Vt = make_tile<E, C>(work + Cfg::STS + Cfg::YTS);     // V~^T [16][C]
  const Tile<E> DVt = make_tile<E, C>(work + Cfg::STS + 2 * Cfg::YTS);  // (D V~)^T
  E* Os = work + Cfg::STS + 3 * Cfg::YTS;                              // [C][OLD]

  // ---------------- loader: global -> registers for chunk n.  Every lane issues the same
  // loads on every chunk (rows past the end read row 0 of the sequence and are zeroed when
  // written to LDS), so the number of outstanding loads is the same on all paths and the
  // compiler can wait for one chunk's loads while the next chunk's stay in flight.
  // Addresses are a per-chunk uniform base plus a per-lane 32-bit offset.
  const long HDK = (long)p.H * DK, HDV = (long)p.H * p.DV;
  auto load_chunk = [&](int n, Staged<E, DK, C>& st) {
    const long P0 = (long)n * C;
    const int krows = (int)min((long)C, p.Lx - P0);                  // valid positions
    const int qrows = (int)min((long)QR, (long)p.L - (long)n * QR);   // valid tokens
    const E* kb = kg + ((long)b * p.Lx + P0) * HDK + (long)h * DK;
    const E* qb = qg + ((long)b * p.L + (long)n * QR) * HDK + (long)h * DK;
    const E* vb = vg + ((long)b * p.Lx + P0) * HDV + (long)h * p.DV + slab * 16;
    const E* Tc = Tg + ((long)head * p.NT + n) * C * C;
    const E* Ac = Ag + ((long)head * p.NT + n) * C * C;
    uint32_t valid = 0;
#pragma unroll
    for (int i = 0; i < Cfg::NK; ++i) {
      const int it = min(ltid + 256 * i, Cfg::KITEMS - 1);
      const int rp = it % (C / 2), cc = it / (C / 2);
#pragma unroll
      for (int s = 0; s < 2; ++s) {
        const bool ok = 2 * rp + s < krows;
        valid |= (uint32_t)ok << (2 * i + s);
        st.k[i][s] = *reinterpret_cast<const u32x4*>(kb + (ok ? (2 * rp + s) * (int)HDK : 0) + cc * VEC);
      }
    }
#pragma unroll
    for (int i = 0; i < Cfg::NQ; ++i) {
      const int it = min(ltid + 256 * i, Cfg::QITEMS - 1);
      const int r = it / (DK / VEC), c = (it % (DK / VEC)) * VEC;
      const bool ok = r < qrows;
      valid |= (uint32_t)ok << (2 * Cfg::NK + i);
      st.q[i] = *reinterpret_cast<const u32x4*>(qb + (ok ? r * (int)HDK : 0) + c);
    }
#pragma unroll
    for (int i = 0; i < Cfg::NT; ++i) {
      const int it = min(ltid + 256 * i, Cfg::TITEMS - 1);
      st.t[i] = *reinterpret_cast<const u32x4*>(Tc + it * VEC);
      st.a[i] = *reinterpret_cast<const u32x4*>(Ac + it * VEC);
    }
    {
      const int lv = min(ltid, Cfg::VITEMS - 1);
      const int r = lv / (16 / VEC), c = (lv % (16 / VEC)) * VEC;
      const bool ok = r < krows;
      valid |= (uint32_t)ok << 31;
      st.v = *reinterpret_cast<const u32x4*>(vb + (ok ? r * (int)HDV : 0) + c);
    }
    st.gc = p.gc[((long)head * p.NT + n) * C + min(ltid, C - 1)];
    st.valid = valid;
  };

  // ---------------- loader: registers -> LDS buffer `buf`
  auto store_chunk = [&](const Staged<E, DK, C>& st, int buf) {
    const ChunkTiles<E, DK, C> in(smem + buf * Cfg::IN);
#pragma unroll
    for (int i = 0; i < Cfg::NK; ++i) {
      const int it = ltid + 256 * i;
      if (it < Cfg::KITEMS) {
        const int rp = it % (C / 2), cc = it / (C / 2);
        const u32x4 z = {0u, 0u, 0u, 0u};
        const u32x4 k0 = (st.valid >> (2 * i)) & 1u ? st.k[i][0] : z;
        const u32x4 k1 = (st.valid >> (2 * i + 1)) & 1u ? st.k[i][1] : z;
        *reinterpret_cast<u32x4*>(in.K.at(2 * rp, cc * VEC)) = k0;
        *reinterpret_cast<u32x4*>(in.K.at(2 * rp + 1, cc * VEC)) = k1;
        if constexpr (Cfg::BF) {
          // K^T rows: the two key rows of this pair are adjacent, so each K^T element pair is
          // one packed 4-byte write.  Dword w of a row holds elements 2w (low) and 2w+1 (high).
#pragma unroll
          for (int w = 0; w < 4; ++w) {
            const uint32_t lo = k0[w], hi = k1[w];
            *reinterpret_cast<uint32_t*>(in.KT.at(cc * VEC + 2 * w, 2 * rp)) = (lo & 0xFFFFu) | (hi << 16);
            *reinterpret_cast<uint32_t*>(in.KT.at(cc * VEC + 2 * w + 1, 2 * rp)) = (lo >> 16) | (hi & 0xFFFF0000u);
          }
        }
      }
    }
#pragma unroll
    for (int i = 0; i < Cfg::NQ; ++i) {
      const int it = ltid + 256 * i;
      if (it < Cfg::QITEMS) {
        const int r = it / (DK / VEC), c = (it % (DK / VEC)) * VEC;
        const u32x4 z = {0u, 0u, 0u, 0u};
        *reinterpret_cast<u32x4*>(in.Q.at(r, c)) = (st.valid >> (2 * Cfg::NK + i)) & 1u ? st.q[i] : z;
      }
    }
#pragma unroll
    for (int i = 0; i < Cfg::NT; ++i) {
      const int it = ltid + 256 * i;
      if (it < Cfg::TITEMS) {
        const int r = (it * VEC) / C, c = (it * VEC) % C;
        *reinterpret_cast<u32x4*>(in.T.at(r, c)) = st.t[i];
        *reinterpret_cast<u32x4*>(in.A.at(r, c)) = st.a[i];
      }
    }
    if (ltid < Cfg::VITEMS) {
      const int r = ltid / (16 / VEC), c = (ltid % (16 / VEC)) * VEC;
      const u32x4 z = {0u, 0u, 0u, 0u};
      *reinterpret_cast<u32x4*>(in.V.at(r, c)) = (st.valid >> 31) & 1u ? st.v : z;
    }
    if (ltid < 64) {  // C <= 64: the first loader wave owns the gate arrays
      const float gl = __shfl(st.gc, C - 1, 64);
      if (ltid < C) {
        egs[buf][ltid] = expf(st.gc);
        eds[buf][ltid] = expf(gl - st.gc);
      }
    }
  };

  // ---------------- loader: output staging tile of chunk n -> HBM (16-byte stores)
  auto store_outputs = [&](int n) {
    if (ltid < Cfg::OITEMS) {
      const int r = ltid / (16 / VEC), c = (ltid % (16 / VEC)) * VEC;
      const long tok = (long)n * QR + r;
      if (r < QR && tok < p.L)
        *reinterpret_cast<u32x4*>(Og + (((long)b * p.L + tok) * p.H + h) * p.DV + slab * 16 + c) =
            *reinterpret_cast<const u32x4*>(Os + r * OLD + c);
    }
  };

  // last position block a token row of tile t may read
  auto jmax_of = [&](int t) { return (min(16 * t + 15, QR - 1) * nh + nh - 1) / 16; };

  // The two roles run separate loops that execute the same sequence of workgroup barriers
  // (3 per chunk, plus one for a single staging buffer), so the register allocator never
  // keeps one role's values live in the other's code.
  if (loader) {
    // ---------------- loader waves
    Staged<E, DK, C> stA, stB;   // register sets, used alternately
    if (p.NT > 0) {
      load_chunk(0, stB);
      store_chunk(stB, 0);
      load_chunk(min(1, p.NT - 1), stA);
    }
    __syncthreads();
    // one chunk: `nxt` holds chunk n+1 (loads issued one chunk earlier), `ld` receives chunk
    // n+2 -- two chunks of lead time to cover HBM latency
    auto loader_step = [&](int n, Staged<E, DK, C>& nxt, Staged<E, DK, C>& ld) {
      const int cur = (NBUF == 2) ? (n & 1) : 0;
      const bool more = n + 1 < p.NT;
      if (n > 0) store_outputs(n - 1);
      load_chunk(min(n + 2, p.NT - 1), ld);   // past the end: a harmless repeat load
      __syncthreads();  // phase 1 done
      __syncthreads();  // phase 2 done
      if (NBUF == 2 && more) store_chunk(nxt, cur ^ 1);
      if constexpr (NBUF == 1) {
        __syncthreads();
        if (more) store_chunk(nxt, 0);
      }
      __syncthreads();  // phase 3 done
    };
    for (int n = 0; n < p.NT; n += 2) {
      loader_step(n, stA, stB);
      if (n + 1 < p.NT) loader_step(n + 1, stB, stA);
    }
    if (p.NT > 0) store_outputs(p.NT - 1);
    return;
  }

  // ---------------- compute waves
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
    if (t < NTS) store4<E>(St.at(col, 16 * t + rq), S[s][0], S[s][1], S[s][2], S[s][3]);
  }
  __syncthreads();

  for (int n = 0; n < p.NT; ++n) {
    const int cur = (NBUF == 2) ? (n & 1) : 0;
    const ChunkTiles<E, DK, C> in(smem + cur * Cfg::IN);
    const float* eg = egs[cur];
    const float* ed = eds[cur];

    // ---------------- phase 1: Y = V - gamma (K S); O1 = Q S
    floatx4 o1 = {0.f, 0.f, 0.f, 0.f};
    if (wave < NBC) {
      floatx4 x = {0.f, 0.f, 0.f, 0.f};
      x = mma_tile<E>(x, in.K, 16 * wave, St, 0, DK, lane);
      const int r0 = 16 * wave + rq;
      float y[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) y[r] = to_float(*in.V.at(r0 + r, col)) - eg[r0 + r] * x[r];
      store4<E>(Yt.at(col, r0), y[0], y[1], y[2], y[3]);
    }
    if (wave < NQT) o1 = mma_tile<E>(o1, in.Q, 16 * wave, St, 0, DK, lane);
    __syncthreads();

    // ---------------- phase 2: V~ = T Y (T lower triangular: k up to the row block's end)
    if (wave < NBC) {
      floatx4 vt = {0.f, 0.f, 0.f, 0.f};
      const int K2 = min(round_up(16 * (wave + 1), KSTEP), C);
      vt = mma_tile<E>(vt, in.T, 16 * wave, Yt, 0, K2, lane);
      const int r0 = 16 * wave + rq;
      store4<E>(Vt.at(col, r0), vt[0], vt[1], vt[2], vt[3]);
      store4<E>(DVt.at(col, r0), vt[0] * ed[r0], vt[1] * ed[r0 + 1], vt[2] * ed[r0 + 2], vt[3] * ed[r0 + 3]);
    }
    __syncthreads();

    // ---------------- phase 3: state update and outputs
    const float gC = eg[C - 1];
#pragma unroll
    for (int s = 0; s < SLOTS; ++s) {
      const int t = wave + 4 * s;
      if (t < NTS) {
        floatx4 acc = S[s] * gC;
        if constexpr (Cfg::BF) {
          acc = mma_tile<E>(acc, in.KT, 16 * t, DVt, 0, C, lane);
        } else {
          // fp32: A[d][r] = K[r][d] read column-wise from the row-major key tile
#pragma unroll 4
          for (int k0 = 0; k0 < C; k0 += 4) {
            const int r = k0 + (lane >> 4);
            acc = Mfma<E>::mma(*in.K.at(r, 16 * t + col), *DVt.at(col, r), acc);
          }
        }
        S[s] = acc;
        store4<E>(St.at(col, 16 * t + rq), acc[0], acc[1], acc[2], acc[3]);
      }
    }
    if (wave < NQT) {
      floatx4 o2 = {0.f, 0.f, 0.f, 0.f};
      const int K3 = min(round_up(16 * (jmax_of(wave) + 1), KSTEP), C);
      o2 = mma_tile<E>(o2, in.A, 16 * wave, Vt, 0, K3, lane);
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int trow = 16 * wave + rq + r;
        const float gq = (trow < QR) ? eg[trow * nh + nh - 1] : 0.f;
        Os[trow * OLD + col] = to_elem<E>(p.scale * (gq * o1[r] + o2[r]));
      }
    }
    if constexpr (NBUF == 1) __syncthreads();
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
  const dim3 grid((unsigned)(p.B * p.H * (p.DV / 16))), block(512);
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
