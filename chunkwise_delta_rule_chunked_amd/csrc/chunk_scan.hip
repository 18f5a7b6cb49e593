// Inter-chunk pass: carries the state across chunks and produces the outputs.
//
// Sources: "08 linear delta rule & DPLR" page, section 2.3 (chunkwise algorithm:
// pseudo-values V~ = U - W S, O = Q S + (Q K^T * M) V~, S <- S + K^T V~), section 2.5
// (V~ contracts over all of d_k, so the key dimension cannot be split across workgroups)
// and section 3 (gated form: queries decayed to the chunk start, keys to the chunk end,
// S <- gamma_C S + (K * gamma_C / gamma)^T V~, Gamma-weighted Q K^T).  DeltaProduct notes,
// section 4.1: on the expanded sequence only each token's last sub-step produces an output.
// Parallel scan over the sequence: DeltaProduct notes, section 3 (the per-step maps are
// affine in S, so they compose associatively).
//
// Per chunk, with T from the intra-chunk kernel and gamma_r = exp(gc_r):
//   Y   = V - gamma * (K S)                    (the residual the writes must correct)
//   V~  = T Y                                  (= U - W S with U = T V, W = T (gamma K))
//   O   = scale * (gamma_p * (Q S) + A V~),    A = Q K^T weighted by Gamma, causal
//   S  <- gamma_C S + K^T (gamma_C / gamma * V~)
// Forming V~ as T (V - gamma K S) instead of materialising W = T (gamma K) saves a
// C x C x d_k contraction per chunk; both are the same product.
//
// Sequence split.  The chunk map S -> gamma_C S + K^T D T (V - gamma K S) is affine, so a
// segment of chunks maps its start state to  S_end = M S_start + S_loc  with M (d_k x d_k)
// the product of the linear parts and S_loc the segment run from S = 0.  Three launches:
//   summary  for each (head, segment but the last): S_loc, and M by running the same chain
//            on d_k extra state columns that start as the identity and see V = 0 (segment 0
//            instead runs from the true S0 and needs no M);
//   combine  per (head, 16 state columns): S_start of every segment, in order, in fp32;
//   outputs  for each (head, segment): the chain from S_start, writing O (and S_final for
//            the last segment).
// With one segment (enough heads to fill the GPU) only the outputs launch runs, from S0.
//
// A (section 3's Gamma-weighted causal Q K^T) is formed in the outputs launch itself, by the
// loading wavefronts from the staged Q and K of the next chunk while the chain works on the
// current one: it never travels through HBM.
//
// Work split inside a workgroup: each of the 4 chain wavefronts owns CT 16-column tiles of
// the state for the whole segment, so the chain needs no exchange between wavefronts.  The
// state stays in MFMA accumulators: on gfx950 the accumulator layout of a 16x16 tile (lane l
// holds rows 4(l/16)..4(l/16)+3 of column l%16) is exactly the B-operand layout of a 16-deep
// bf16 MFMA, so S, Y and V~ feed the next product from registers (two tiles form one 32-deep
// step with the k order permuted consistently in A and B).  A operands (K, Q, T, A rows and
// K^T through LDS transpose reads) come from a staged chunk in LDS.  4 more wavefronts move
// data: direct global -> LDS loads of chunk n+1 into the other half of a double-buffered
// stage while chunk n is processed.  Only they have loads in flight; one workgroup barrier
// per chunk publishes the next stage.  Barriers are issued without the compiler's
// workgroup fence, which would otherwise wait for the loaders' in-flight loads.
//
// Padded positions of the last chunk: the intra-chunk kernel leaves T's padded rows and
// columns at exactly zero, so padded key, value and query rows may hold any finite data --
// they are loaded from row 0 of the sequence -- without reaching an output (padded rows of V~
// are 0, so whatever A holds in their columns multiplies zeros, and they add nothing to the
// state).
#include <type_traits>

#include "common.h"
#include "kernels.h"

namespace delta {

// MFMA whose B operand is an accumulator tile in the D layout (see above).  `A` is the lane's
// four consecutive A elements (row lane%16, columns 4(lane/16) .. +3 of a 16-wide k block).
template <typename E>
struct DOp;

template <>
struct DOp<bf16> {
  typedef bf16x4 A;
  typedef bf16x4 B;
  __device__ static inline B cvt(floatx4 d) { return bf16x4{(bf16)d[0], (bf16)d[1], (bf16)d[2], (bf16)d[3]}; }
  __device__ static inline A row4(const bf16* p) { return *reinterpret_cast<const bf16x4*>(p); }
  // M^T block: lane (g, i) gets M[r0 + 4g + j][c0 + i], j = 0..3 (transpose read; the lane
  // addresses row r0 + 4g + i/4 at column c0 + 4(i%4))
  __device__ static inline A col4(const Tile<bf16>& m, int r0, int c0, int lane) {
    const int g = lane >> 4, i = lane & 15;
    return read_tr4(m.at(r0 + 4 * g + (i >> 2), c0 + 4 * (i & 3)));
  }
  __device__ static inline floatx4 mma1(A a, B b, floatx4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, b, c, 0, 0, 0);
  }
  // two 16-deep k blocks as one 32-deep instruction: k slot 8g+j <- block 0 row 4g+j,
  // k slot 8g+4+j <- block 1 row 4g+j, in both operands
  __device__ static inline floatx4 mma2(A a0, A a1, B b0, B b1, floatx4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_shufflevector(a0, a1, 0, 1, 2, 3, 4, 5, 6, 7),
                                                   __builtin_shufflevector(b0, b1, 0, 1, 2, 3, 4, 5, 6, 7), c, 0, 0, 0);
  }
  // A fragment of a 32-deep step read as one 16-byte piece (8 consecutive elements)
  __device__ static inline bf16x8 row8(const bf16* p) { return *reinterpret_cast<const bf16x8*>(p); }
  __device__ static inline floatx4 mma8(bf16x8 a, B b0, B b1, floatx4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, __builtin_shufflevector(b0, b1, 0, 1, 2, 3, 4, 5, 6, 7), c, 0, 0, 0);
  }
  // mma2 is one instruction: a chain must not mix shapes (a dependent pair of different shapes
  // needs wait states the compiler does not insert on gfx950)
  static constexpr bool PAIRS = true;
};

template <>
struct DOp<float> {
  typedef floatx4 A;
  typedef floatx4 B;
  __device__ static inline B cvt(floatx4 d) { return d; }
  __device__ static inline A row4(const float* p) { return *reinterpret_cast<const floatx4*>(p); }
  __device__ static inline A col4(const Tile<float>& m, int r0, int c0, int lane) {
    const int g = lane >> 4, i = lane & 15;
    return floatx4{*m.at(r0 + 4 * g, c0 + i), *m.at(r0 + 4 * g + 1, c0 + i), *m.at(r0 + 4 * g + 2, c0 + i),
                   *m.at(r0 + 4 * g + 3, c0 + i)};
  }
  // v_mfma_f32_16x16x4_f32 takes k = lane/16: step j uses k index 4(lane/16) + j of the block
  __device__ static inline floatx4 mma1(A a, B b, floatx4 c) {
#pragma unroll
    for (int j = 0; j < 4; ++j) c = __builtin_amdgcn_mfma_f32_16x16x4f32(a[j], b[j], c, 0, 0, 0);
    return c;
  }
  __device__ static inline floatx4 mma2(A a0, A a1, B b0, B b1, floatx4 c) { return mma1(a1, b1, mma1(a0, b0, c)); }
  static constexpr bool PAIRS = false;
};

// Rendezvous of the loading wavefronts only (the chain wavefronts are mid-chunk): each arrives
// once per call, `target` = (calls so far) x (loading wavefronts).  Every loading wavefront runs
// the same number of calls, so the wait always ends.  The release orders this wave's completed
// LDS writes (its direct-to-LDS loads were waited for) before the count.
__device__ inline void loader_rendezvous(unsigned* ctr, unsigned target, int lane) {
  if (lane == 0) __hip_atomic_fetch_add(ctr, 1u, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_WORKGROUP);
  while (__hip_atomic_load(ctr, __ATOMIC_ACQUIRE, __HIP_MEMORY_SCOPE_WORKGROUP) < target) __builtin_amdgcn_s_sleep(1);
}

constexpr int SEG_LOADERS = 4;  // loading wavefronts per workgroup
constexpr int LDS_BUDGET = 160 * 1024;

// What a launch of seg_kernel does with each segment:
//   SEG_SUM     the segment summary (S_loc and the transition columns of M)
//   SEG_OUT     the chain from the segment's start state, writing O (and S_final)
//   SEG_STATES  the chain from the segment's start state, writing each chunk's start state
//               (bf16 when the inputs are bf16) instead of O
// and REV runs the adjoint chain of the backward pass instead (see the reverse chain below).
enum SegMode { SEG_SUM = 0, SEG_OUT = 1, SEG_STATES = 2 };

template <typename E, int DK, int C, int CT, int NCW, int MODE, bool REV>
struct SegCfg {
  static constexpr bool SUM = MODE == SEG_SUM;
  static constexpr bool QA = MODE == SEG_OUT || REV;  // Q staged and A formed per chunk
  static constexpr int ES = sizeof(E);
  static constexpr int TPG = NCW * CT;      // state column tiles per workgroup
  static constexpr int THREADS = (NCW + SEG_LOADERS) * WAVE;
  static constexpr int VWMAX = 16 * TPG;    // value columns staged per chunk
  static constexpr int KS = C * DK, QS = QA ? C * DK : 0, TS = C * C, AS = QA ? C * C : 0, VS = C * VWMAX;
  static constexpr int GS = 4 * C * 4 / ES;  // gc, exp(gc), exp(gc_last - gc), token output gates
  static constexpr int IN = KS + QS + TS + AS + VS + GS;   // one staged chunk (elements)
  static constexpr int SYNC = QA ? 16 / ES : 0;              // loader rendezvous counter
  static constexpr int NSTAGE = (2 * IN + SYNC) * ES <= LDS_BUDGET ? 2 : 1;
  static constexpr int ELEMS = NSTAGE * IN + SYNC;
  static_assert(ELEMS * ES <= LDS_BUDGET, "LDS budget");
};

template <typename E, int DK, int C, int CT, int NCW, int MODE, bool REV>
__global__ __launch_bounds__((NCW + SEG_LOADERS) * WAVE) void seg_kernel(FwdParams p) {
  using Cfg = SegCfg<E, DK, C, CT, NCW, MODE, REV>;
  constexpr bool SUM = Cfg::SUM, QA = Cfg::QA, OUT = MODE == SEG_OUT, STATES = MODE == SEG_STATES;
  static_assert(!REV || (sizeof(E) == 2 && MODE != SEG_OUT), "the reverse chain: bf16, summary or states");
  // dO rows past the sequence must read as zeros (they meet A^T columns of padded tokens): the
  // register-prefetched stages load through buffer ranges that give that, the one-stage copies
  // repeat row 0 instead
  static_assert(!REV || Cfg::NSTAGE == 2, "the reverse chain takes the double-buffered stage");
  using D = DOp<E>;
  constexpr int NB = C / 16;     // position blocks per chunk
  constexpr int NTS = DK / 16;   // state row tiles
  constexpr int TPG = Cfg::TPG;

  __shared__ __attribute__((aligned(16))) E smem[Cfg::ELEMS];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int m = lane & 15, g4 = lane >> 4;
  const int BH = p.B * p.H;
  const int NCT = p.DV / 16;
  // transition columns: the forward summary's; the reverse chain takes its transition maps from
  // the forward summary (transposed), so its summary runs the value columns only
  const int MCT = (SUM && !REV) ? DK / 16 : 0;
  const int G = (NCT + MCT + TPG - 1) / TPG;            // column groups
  const int NSEG = SUM ? p.P - 1 : p.P;                 // segments this launch handles

  // workgroup -> (segment, head, column group); the groups of one (segment, head) share
  // its K and T reads, so they go to one XCD (workgroups are dealt round-robin over 8)
  int unit, grp;
  {
    const int i = blockIdx.x;
    if ((NSEG * BH) % 8 == 0) {
      const int x = i % 8, j = i / 8;
      unit = x + 8 * (j / G);
      grp = j % G;
    } else {
      unit = i / G;
      grp = i % G;
    }
  }
  // the reverse chain numbers the segments from the end of the sequence (its segment 0 starts
  // from the gradient of S_final) and walks each segment's chunks backwards
  const int seg = unit / BH, head = unit % BH;
  const int b = head / p.H, h = head % p.H;
  const int fseg = REV ? p.P - 1 - seg : seg;              // the segment's place in the sequence
  const int n0 = fseg * p.NS, n1 = min(p.NT, n0 + p.NS);  // chunks of this segment
  const int cnt = max(0, n1 - n0);
  auto chunk_at = [&](int i) { return REV ? n1 - 1 - i : n0 + i; };
  const int nh = p.nh;
  const int QR = C / nh;                                 // tokens per chunk
  // value columns staged for this group
  const int vt0 = grp * TPG;
  const int vcnt = max(0, min(NCT - vt0, TPG));
  const int VW = 16 * vcnt;
  // segment 0 of the summary needs only the value columns
  if (SUM && seg == 0 && vcnt == 0) return;
  unsigned* rdv = reinterpret_cast<unsigned*>(smem + Cfg::NSTAGE * Cfg::IN);
  if constexpr (QA) {
    // The reverse chain contracts the staged Q and dO over all C rows, where only a chunk's
    // QR token rows are ever loaded: with several sub-steps per token the rest must hold finite
    // values (they meet zeros), so the stages start as zeros.
    if (REV && nh > 1)
      for (int i = tid; i < Cfg::NSTAGE * Cfg::IN * Cfg::ES / 16; i += Cfg::THREADS)
        reinterpret_cast<u32x4*>(smem)[i] = u32x4{0u, 0u, 0u, 0u};
    if (tid == 0) *rdv = 0u;
    barrier_lds();
  }

  if (wave >= NCW) {
    // ---------------- loading wavefronts
    const int dw = wave - NCW;
    const E* qg = reinterpret_cast<const E*>(p.q);
    const E* kg = reinterpret_cast<const E*>(p.k);
    const E* vg = reinterpret_cast<const E*>(p.v);
    const E* Tg = reinterpret_cast<const E*>(p.T);
    const int HDK = p.H * DK, HDV = p.H * p.DV;
    // copy plans of the whole-chunk case; a chunk cut short by the end of the sequence takes the
    // general copy
    CopyPlan<E, DK, C, SEG_LOADERS> pk, pq;
    CopyPlan<E, C, C, SEG_LOADERS> pt;
    CopyPlan<E, Cfg::VWMAX, C, SEG_LOADERS> pv;
    CopyPlan<float, 4, C / 4, SEG_LOADERS> pg;
    pk.init(HDK, C, dw, lane);
    pq.init(HDK, QR, dw, lane);
    pt.init(C, C, dw, lane);
    // values by position; the reverse chain's dO (in p.v) by token
    pv.init(HDV, VW > 0 ? (REV ? QR : C) : 0, dw, lane, VW * (int)sizeof(E) / 16);
    pg.init(4, C / 4, dw, lane);
    // Issues the copies of chunk n into `stage`: gate prefix, keys and queries first, then T and
    // the values.  Returns how many of this wave's copies were issued after the first three
    // (the outputs launch forms A from those three while the rest is in flight), or 0 when the
    // caller must wait for everything (a chunk cut short by the end of the sequence).
    auto issue = [&](int n, int stage) -> int {
      E* st = smem + stage * Cfg::IN;
      const long P0 = (long)n * C;
      const int krows = (int)min((long)C, p.Lx - P0);                  // valid positions
      const long tok0 = (long)n * QR;
      const int qrows = (int)min((long)QR, (long)p.L - tok0);           // valid tokens
      const E* kc = kg + ((long)b * p.Lx + P0) * HDK + (long)h * DK;
      const E* qc = qg + ((long)b * p.L + tok0) * HDK + (long)h * DK;
      const E* vc = vg + (REV ? ((long)b * p.L + tok0) : ((long)b * p.Lx + P0)) * HDV + (long)h * p.DV + 16 * vt0;
      E* sv = st + Cfg::KS + Cfg::QS + Cfg::TS + Cfg::AS;
      pg.issue(reinterpret_cast<float*>(sv + Cfg::VS), p.gc + ((long)head * p.NT + n) * C, dw);
      if (krows == C && (!QA || qrows == QR)) {
        pk.issue(st, kc, dw);
        if (QA) pq.issue(st + Cfg::KS, qc, dw);
        pt.issue(st + Cfg::KS + Cfg::QS, Tg + ((long)head * p.NT + n) * C * C, dw);
        if (VW > 0) pv.issue(sv, vc, dw);
        return pt.n + (VW > 0 ? pv.n : 0);
      }
      copy_rows_to_lds<E, DK>(st, kc, HDK, C, krows, dw, SEG_LOADERS, lane);
      if (QA) copy_rows_to_lds<E, DK>(st + Cfg::KS, qc, HDK, QR, qrows, dw, SEG_LOADERS, lane);
      pt.issue(st + Cfg::KS + Cfg::QS, Tg + ((long)head * p.NT + n) * C * C, dw);
      // the group's value columns, at the fixed row pitch VWMAX (columns past them repeat its first)
      if (VW > 0)
        copy_rows_to_lds<E, Cfg::VWMAX>(sv, vc, HDV, REV ? QR : C, REV ? qrows : krows, dw, SEG_LOADERS, lane,
                                         VW * (int)sizeof(E) / 16);
      return 0;
    };
    // exp(gc), exp(gc_last - gc) and, per token row, scale * exp(gc) at the token's last
    // sub-step (0 past the chunk's tokens) of a staged chunk, once for all chain wavefronts
    auto exps = [&](int stage) {
      if (dw == 0 && lane < C) {
        float* gcs = reinterpret_cast<float*>(smem + stage * Cfg::IN + Cfg::KS + Cfg::QS + Cfg::TS + Cfg::AS + Cfg::VS);
        const float x = gcs[lane], xl = gcs[C - 1];
        gcs[C + lane] = expf(x);
        gcs[2 * C + lane] = expf(xl - x);
        gcs[3 * C + lane] = lane < QR ? p.scale * expf(gcs[min(lane, QR - 1) * nh + nh - 1]) : 0.f;
      }
    };
    // Outputs launch: A[t][j] = scale q_t . k_j exp(gc_p - gc_j) for positions j <= p, the
    // token's last sub-step p = t n_h + n_h - 1, else 0 (rows past the chunk's tokens: 0), from
    // the staged Q and K once every loading wavefront's copies have landed.  Block (t, j) of
    // K Q^T on MFMA holds A^T: lane (g, m) gets A[16 t + m][16 j + 4 g .. + 3], one row run.
    // Every block is formed, those past the causal reach (or past the tokens: Q rows there are
    // stale, and the select drops whatever they give) as zeros, so each wave's blocks are
    // independent straight-line work.
    // The reverse chain takes A^T instead (rows: positions, columns: tokens), formed from the
    // product Q K^T: lane (g, m) gets A[16 t + 4 g .. + 3][16 j + m], a row run of A^T.
    unsigned arrivals = 0;
    auto build_a = [&](int stage) {
      if constexpr (QA) {
        arrivals += SEG_LOADERS;
        loader_rendezvous(rdv, arrivals, lane);
        E* st = smem + stage * Cfg::IN;
        const Tile<E> Kt = make_packed_tile<E, DK>(st), Qt = make_packed_tile<E, DK>(st + Cfg::KS);
        const Tile<E> At = make_packed_tile<E, C>(st + Cfg::KS + Cfg::QS + Cfg::TS);
        const float* gcs = reinterpret_cast<const float*>(st + Cfg::KS + Cfg::QS + Cfg::TS + Cfg::AS + Cfg::VS);
        constexpr int NBLK = NB * NB, PER = (NBLK + SEG_LOADERS - 1) / SEG_LOADERS;
        floatx4 d[PER];
#pragma unroll
        for (int u = 0; u < PER; ++u) {
          const int blk = dw + SEG_LOADERS * u;
          d[u] = floatx4{0.f, 0.f, 0.f, 0.f};
          if (NBLK % SEG_LOADERS == 0 || blk < NBLK)
            d[u] = REV ? mma_tile<E>(d[u], Qt, 16 * (blk / NB), Kt, 16 * (blk % NB), DK, lane)
                       : mma_tile<E>(d[u], Kt, 16 * (blk % NB), Qt, 16 * (blk / NB), DK, lane);
        }
#pragma unroll
        for (int u = 0; u < PER; ++u) {
          const int blk = dw + SEG_LOADERS * u;
          if (NBLK % SEG_LOADERS != 0 && blk >= NBLK) continue;
          const int t = blk / NB, j = blk % NB;
          if constexpr (REV) {
            const int pc = 16 * j + m;  // the lane's position; tokens 16 t + 4 g4 + r
            const float gj = gcs[pc];
            float a[4];
#pragma unroll
            for (int r = 0; r < 4; ++r) {
              const int trow = 16 * t + 4 * g4 + r, ptok = min(trow, QR - 1) * nh + nh - 1;
              const float x = p.scale * d[u][r] * gate_exp(gcs[ptok] - gj);
              a[r] = (trow < QR && pc <= ptok) ? x : 0.f;
            }
            store4<E>(At.at(pc, 16 * t + 4 * g4), a[0], a[1], a[2], a[3]);
          } else {
            const int trow = 16 * t + m, ptok = min(trow, QR - 1) * nh + nh - 1;
            const float gp = gcs[ptok];
            float a[4];
#pragma unroll
            for (int r = 0; r < 4; ++r) {
              const int pc = 16 * j + 4 * g4 + r;
              const float x = p.scale * d[u][r] * gate_exp(gp - gcs[pc]);
              a[r] = (trow < QR && pc <= ptok) ? x : 0.f;
            }
            store4<E>(At.at(trow, 16 * j + 4 * g4), a[0], a[1], a[2], a[3]);
          }
        }
      }
    };
    // stage a chunk: copies, gate tables and (outputs launch) A, which needs only the first
    // copies; everything has landed when the function returns
    auto stage_chunk = [&](int n, int stage) {
      const int late = issue(n, stage);
      if constexpr (!QA) {
        wait_vmem();
        exps(stage);
      } else {
        wait_vmem_upto(late);
        exps(stage);
        build_a(stage);
        wait_vmem();
      }
    };
    if constexpr (Cfg::NSTAGE == 2) {
      // Double-buffered stage, with the next chunk prefetched into registers: the copies of
      // chunk n+2 are loaded while chunk n is processed and written to LDS at the start of
      // chunk n+1, so neither the gate tables nor A ever wait for HBM.  Loads go through
      // buffer resources over the chunk's valid rows (rows past the sequence read 0).
      u32x4 rk[decltype(pk)::NS], rq[QA ? decltype(pq)::NS : 1], rt[decltype(pt)::NS], rv[decltype(pv)::NS],
          rg[decltype(pg)::NS];
      auto load = [&](int n) {
        const long P0 = (long)n * C;
        const int krows = (int)min((long)C, p.Lx - P0);
        const long tok0 = (long)n * QR;
        const int qrows = (int)min((long)QR, (long)p.L - tok0);
        const __amdgpu_buffer_rsrc_t kr = buffer_rsrc(const_cast<E*>(kg) + ((long)b * p.Lx + P0) * HDK + (long)h * DK,
                                                      krows * HDK * (int)sizeof(E));
        const __amdgpu_buffer_rsrc_t vr =
            REV ? buffer_rsrc(const_cast<E*>(vg) + ((long)b * p.L + tok0) * HDV + (long)h * p.DV + 16 * vt0,
                              qrows * HDV * (int)sizeof(E))
                : buffer_rsrc(const_cast<E*>(vg) + ((long)b * p.Lx + P0) * HDV + (long)h * p.DV + 16 * vt0,
                              krows * HDV * (int)sizeof(E));
        const __amdgpu_buffer_rsrc_t tr =
            buffer_rsrc(const_cast<E*>(Tg) + ((long)head * p.NT + n) * C * C, C * C * (int)sizeof(E));
        const __amdgpu_buffer_rsrc_t gr = buffer_rsrc(p.gc + ((long)head * p.NT + n) * C, C * 4);
#pragma unroll
        for (int s = 0; s < decltype(pg)::NS; ++s)
          if (s < pg.n && pg.off[s] != ~0u) rg[s] = buffer_load16(gr, (int)pg.off[s]);
#pragma unroll
        for (int s = 0; s < decltype(pk)::NS; ++s)
          if (s < pk.n && pk.off[s] != ~0u) rk[s] = buffer_load16(kr, (int)pk.off[s]);
        if constexpr (QA) {
          const __amdgpu_buffer_rsrc_t qr =
              buffer_rsrc(const_cast<E*>(qg) + ((long)b * p.L + tok0) * HDK + (long)h * DK, qrows * HDK * (int)sizeof(E));
#pragma unroll
          for (int s = 0; s < decltype(pq)::NS; ++s)
            if (s < pq.n && pq.off[s] != ~0u) rq[s] = buffer_load16(qr, (int)pq.off[s]);
        }
#pragma unroll
        for (int s = 0; s < decltype(pt)::NS; ++s)
          if (s < pt.n && pt.off[s] != ~0u) rt[s] = buffer_load16(tr, (int)pt.off[s]);
#pragma unroll
        for (int s = 0; s < decltype(pv)::NS; ++s)
          if (s < pv.n && pv.off[s] != ~0u) rv[s] = buffer_load16(vr, (int)pv.off[s]);
      };
      // the registers into stage `stage`: each piece where its direct-to-LDS copy would land
      auto store = [&](int stage) {
        E* st = smem + stage * Cfg::IN;
        E* sv = st + Cfg::KS + Cfg::QS + Cfg::TS + Cfg::AS;
        auto put = [&](E* tile, int s, const u32x4& x) {
          *reinterpret_cast<u32x4*>(tile + ((dw + SEG_LOADERS * s) * WAVE + lane) * (16 / (int)sizeof(E))) = x;
        };
#pragma unroll
        for (int s = 0; s < decltype(pg)::NS; ++s)
          if (s < pg.n && pg.off[s] != ~0u)
            *reinterpret_cast<u32x4*>(reinterpret_cast<float*>(sv + Cfg::VS) + ((dw + SEG_LOADERS * s) * WAVE + lane) * 4) = rg[s];
#pragma unroll
        for (int s = 0; s < decltype(pk)::NS; ++s)
          if (s < pk.n && pk.off[s] != ~0u) put(st, s, rk[s]);
        if constexpr (QA) {
#pragma unroll
          for (int s = 0; s < decltype(pq)::NS; ++s)
            if (s < pq.n && pq.off[s] != ~0u) put(st + Cfg::KS, s, rq[s]);
        }
#pragma unroll
        for (int s = 0; s < decltype(pt)::NS; ++s)
          if (s < pt.n && pt.off[s] != ~0u) put(st + Cfg::KS + Cfg::QS, s, rt[s]);
#pragma unroll
        for (int s = 0; s < decltype(pv)::NS; ++s)
          if (s < pv.n && pv.off[s] != ~0u) put(sv, s, rv[s]);
      };
      // (i counts the segment's chunks in processing order)
      if (cnt > 0) {
        load(chunk_at(0));
        store(0);
        exps(0);
        build_a(0);
        if (cnt > 1) load(chunk_at(1));
      }
      barrier_lds();  // first chunk staged
      for (int i = 0; i < cnt; ++i) {
        if (i + 1 < cnt) {
          const int stage = (i + 1) & 1;
          store(stage);  // chunk i+1, loaded during chunk i-1
          if (i + 2 < cnt) load(chunk_at(i + 2));
          exps(stage);
          build_a(stage);
        }
        barrier_lds();  // chunk i done, chunk i+1 staged (the loads in flight are not waited for)
      }
    } else {
      for (int i = 0; i < cnt; ++i) {
        stage_chunk(chunk_at(i), 0);
        barrier_all();  // chunk n staged
        barrier_all();  // chunk n done
      }
    }
    return;
  }

  // ---------------- chain wavefronts: tiles vt0 + CT*wave + c, c < CT
  int tile[CT];
  bool live[CT], isv[CT];
#pragma unroll
  for (int c = 0; c < CT; ++c) {
    tile[c] = vt0 + CT * wave + c;
    isv[c] = tile[c] < NCT;
    // segment 0 of the summary starts from the true S0 and needs no transition columns
    live[c] = tile[c] < NCT + ((SUM && seg == 0) ? 0 : MCT);
  }

  // State rows.  With pairs of 32-deep steps (DP), the two row tiles 2u, 2u+1 of a pair interleave
  // their d_k indices so that lane group g's k slots 8g .. 8g+7 of the pair are d_k indices
  // 32u + 8g .. 32u + 8g + 7: the A fragment of K S and Q S is then one contiguous 16-byte read.
  // Accumulator row 4g + j of tile t holds d_k index dkrow(t, 4g + j).
  constexpr bool DP = D::PAIRS && NTS % 2 == 0;
  auto dkrow = [](int t, int r) {
    return DP ? 32 * (t >> 1) + 8 * (r >> 2) + 4 * (t & 1) + (r & 3) : 16 * t + r;
  };
  // state init: column m of tile c
  floatx4 S[CT][NTS];
#pragma unroll
  for (int c = 0; c < CT; ++c)
#pragma unroll
    for (int t = 0; t < NTS; ++t) {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int row = dkrow(t, 4 * g4 + j);
        float x = 0.f;
        if (live[c]) {
          if (isv[c]) {
            const long col = 16 * tile[c] + m;
            if (!SUM && p.P > 1) {
              // with a split every segment, the first too, starts from the start state the
              // summary and combine launches wrote: this launch then reads no caller tensor that
              // it also writes (S_final may be S0 itself, written by the last segment)
              x = p.Sst[(((long)head * p.P + seg) * DK + row) * p.DV + col];
            } else if (seg == 0) {
              if (p.S0) x = p.S0[((long)head * DK + row) * p.DV + col];
              if (SUM) p.Sst[((long)head * p.P * DK + row) * p.DV + col] = x;  // segment 0's start
            }
          } else {
            x = (row == 16 * (tile[c] - NCT) + m) ? 1.f : 0.f;  // identity columns of M
          }
        }
        S[c][t][j] = x;
      }
    }

  // Per-lane LDS element offsets of the fragments this lane reads.  A block of 16 rows further
  // down a tile adds a constant: for r = 16 bb + x the key depends on x alone (every mask < 16).
  constexpr unsigned CH = 16 / sizeof(E);
  constexpr int MK = PackedLayout<E, DK>::MASK, MC = PackedLayout<E, C>::MASK;
  // (column indices are never negative: unsigned chunk arithmetic is shifts and masks)
  auto swz = [](int r, int e, int ld, int mask) {
    const unsigned u = e;
    return r * ld + (int)(((u / CH) ^ (unsigned)swz_key(r, mask)) * CH + u % CH);
  };
  constexpr int MV = PackedLayout<E, Cfg::VWMAX>::MASK;
  if constexpr (Cfg::NSTAGE == 2) barrier_lds();

  E* Og = reinterpret_cast<E*>(p.O);

  for (int i = 0; i < cnt; ++i) {
    const int n = chunk_at(i);
    if constexpr (Cfg::NSTAGE == 1) barrier_lds();
    const E* Kp = smem + ((Cfg::NSTAGE == 2) ? (i & 1) : 0) * Cfg::IN;
    const E* Qp = Kp + Cfg::KS;
    const E* Tp = Qp + Cfg::QS;
    const E* Ap = Tp + Cfg::TS;
    const E* Vp = Ap + Cfg::AS;
    const float* gcp = reinterpret_cast<const float*>(Vp + Cfg::VS);
    const float* egp = gcp + C;        // exp(gc)
    const float* edp = gcp + 2 * C;    // exp(gc_last - gc)
    const float* eqp = gcp + 3 * C;    // scale * exp(gc) of each token row's last sub-step
    // Per-lane LDS element offsets of this chunk's fragment reads, recomputed every chunk from
    // a lane index the optimiser cannot see through (hoisted, they would pin ~20 registers).
    int lnL = lane;
    asm volatile("" : "+v"(lnL));
    const int mL = lnL & 15, gL = lnL >> 4;
    int offK[NTS], offKT[NTS], offT[NB], offV[CT], offTT[NB];
#pragma unroll
    for (int t = 0; t < NTS; ++t) {
      if constexpr (DP) {
        offK[t] = swz(mL, 32 * (t >> 1) + 8 * gL, DK, MK);   // K, Q rows: 16-byte pieces (t even)
        // K^T transpose reads: the lane addresses d_k columns dkrow(t, 4i .. 4i + 3), i = lane % 4
        offKT[t] = swz(4 * gL + (mL >> 2), 32 * (t >> 1) + 4 * (t & 1) + 8 * (mL & 3), DK, MK);
      } else {
        offK[t] = swz(mL, 16 * t + 4 * gL, DK, MK);                          // K, Q rows
        offKT[t] = swz(4 * gL + (mL >> 2), 16 * t + 4 * (mL & 3), DK, MK);   // K^T transpose reads
      }
    }
#pragma unroll
    for (int kb = 0; kb < NB; ++kb) {
      offT[kb] = swz(mL, 16 * kb + 4 * gL, C, MC);  // T, A rows
      // T^T transpose reads (reverse chain): column block kb of T as rows, at row block 0
      offTT[kb] = swz(4 * gL + (mL >> 2), 16 * kb + 4 * (mL & 3), C, MC);
    }
#pragma unroll
    for (int c = 0; c < CT; ++c)   // V transpose reads (D layout of the tile's 16 columns)
      offV[c] = swz(4 * gL + (mL >> 2), 16 * (isv[c] ? tile[c] - vt0 : 0) + 4 * (mL & 3), Cfg::VWMAX, MV);

    // chunk-start state as a B operand
    typename D::B Sb[CT][NTS];
#pragma unroll
    for (int c = 0; c < CT; ++c)
#pragma unroll
      for (int t = 0; t < NTS; ++t) Sb[c][t] = D::cvt(S[c][t]);

    // ---- the chunk's start state as the chain holds it (rounded to the element type), into
    // Sn [B*H, NT, d_v, d_k]: lane (g, m) holds 4 consecutive d_k rows of column 16 tile + m.  The
    // reverse chain's gradients also leave their rounding residual in Snl: the gradient of the
    // final state enters the last chunk unattenuated and can dwarf the rest of its products.
    if constexpr (STATES) {
      const long cofs = ((long)head * p.NT + n) * p.DV * DK;
#pragma unroll
      for (int c = 0; c < CT; ++c)
        if (isv[c])
#pragma unroll
          for (int t = 0; t < NTS; ++t) {
            const long e = cofs + (long)(16 * tile[c] + m) * DK + dkrow(t, 4 * g4);
            *reinterpret_cast<typename D::B*>(reinterpret_cast<E*>(p.Sn) + e) = Sb[c][t];
            if constexpr (REV) {
              const bf16x4 hi = Sb[c][t];
              *reinterpret_cast<bf16x4*>(reinterpret_cast<bf16*>(p.Snl) + e) =
                  DOp<bf16>::cvt(S[c][t] - floatx4{(float)hi[0], (float)hi[1], (float)hi[2], (float)hi[3]});
            }
          }
    }

    // ---- X = K S, contracting over d_k
    constexpr int TSTEP = (D::PAIRS && NTS % 2 == 0) ? 2 : 1;
    floatx4 X[CT][NB];
#pragma unroll
    for (int c = 0; c < CT; ++c)
#pragma unroll
      for (int bb = 0; bb < NB; ++bb) X[c][bb] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int t = 0; t < NTS; t += TSTEP)
#pragma unroll
      for (int bb = 0; bb < NB; ++bb) {
        if constexpr (DP) {
          const bf16x8 a = DOp<bf16>::row8(reinterpret_cast<const bf16*>(Kp) + 16 * bb * DK + offK[t]);
#pragma unroll
          for (int c = 0; c < CT; ++c) X[c][bb] = DOp<bf16>::mma8(a, Sb[c][t], Sb[c][t + 1], X[c][bb]);
        } else {
          const typename D::A a0 = D::row4(Kp + 16 * bb * DK + offK[t]);
#pragma unroll
          for (int c = 0; c < CT; ++c) X[c][bb] = D::mma1(a0, Sb[c][t], X[c][bb]);
        }
      }

    // ---- Y = V - gamma X (transition columns see V = 0); the reverse chain:
    // dV~ = w X + A^T dO (dO tiles read once, D layout, zero on transition columns)
    typename D::B Yb[CT][NB];
    [[maybe_unused]] typename D::B Ob[CT][NB];
    if constexpr (REV) {
#pragma unroll
      for (int kb = 0; kb < NB; ++kb)
#pragma unroll
        for (int c = 0; c < CT; ++c) {
          const bf16x4 r = read_tr4(reinterpret_cast<const bf16*>(Vp) + 16 * kb * Cfg::VWMAX + offV[c]);
          u32x2 u = __builtin_bit_cast(u32x2, r);
          u[0] = isv[c] ? u[0] : 0u;
          u[1] = isv[c] ? u[1] : 0u;
          Ob[c][kb] = __builtin_bit_cast(bf16x4, u);
        }
#pragma unroll
      for (int bb = 0; bb < NB; ++bb) {
        floatx4 acc[CT];
#pragma unroll
        for (int c = 0; c < CT; ++c) acc[c] = floatx4{0.f, 0.f, 0.f, 0.f};
        // A^T is zero past each position's causal reach; every token block is taken, so the
        // chunk body stays straight-line
#pragma unroll
        for (int kb = 0; kb < NB; kb += 2) {
          const typename D::A a0 = D::row4(Ap + 16 * bb * C + offT[kb]);
          const typename D::A a1 = D::row4(Ap + 16 * bb * C + offT[kb + 1]);
#pragma unroll
          for (int c = 0; c < CT; ++c) acc[c] = D::mma2(a0, a1, Ob[c][kb], Ob[c][kb + 1], acc[c]);
        }
        const floatx4 ed4 = *reinterpret_cast<const floatx4*>(edp + 16 * bb + 4 * g4);
#pragma unroll
        for (int c = 0; c < CT; ++c) Yb[c][bb] = D::cvt(acc[c] + ed4 * X[c][bb]);
      }
    }
#pragma unroll
    for (int bb = 0; bb < NB && !REV; ++bb) {
      const floatx4 eg4 = *reinterpret_cast<const floatx4*>(egp + 16 * bb + 4 * g4);
#pragma unroll
      for (int c = 0; c < CT; ++c) {
        // read unconditionally (offV of a transition tile addresses the stage's first value
        // columns, which may never have been loaded) and select, so the chunk body stays one
        // straight-line block
        floatx4 v4;
        if constexpr (sizeof(E) == 2) {
          const bf16x4 r = read_tr4(reinterpret_cast<const bf16*>(Vp) + 16 * bb * Cfg::VWMAX + offV[c]);
          u32x2 u = __builtin_bit_cast(u32x2, r);
          u[0] = isv[c] ? u[0] : 0u;
          u[1] = isv[c] ? u[1] : 0u;
          const bf16x4 rs = __builtin_bit_cast(bf16x4, u);
          v4 = floatx4{(float)rs[0], (float)rs[1], (float)rs[2], (float)rs[3]};
        } else {
          const Tile<E> V = make_packed_tile<E, Cfg::VWMAX>(const_cast<E*>(Vp));
          const int vc = isv[c] ? 16 * (tile[c] - vt0) : 0;
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const float x = to_float(*V.at(16 * bb + 4 * g4 + j, vc + m));
            v4[j] = isv[c] ? x : 0.f;
          }
        }
        Yb[c][bb] = D::cvt(v4 - eg4 * X[c][bb]);
      }
    }

    // ---- V~ = T Y (T lower triangular; a zero block above the diagonal may pair in); the
    // reverse chain: dY = T^T dV~ (T^T upper triangular), kept as -gamma dY for the update
    typename D::B Vb[CT][NB], DVb[CT][NB];
    if constexpr (REV) {
#pragma unroll
      for (int bb = 0; bb < NB; ++bb) {
        floatx4 vt[CT];
#pragma unroll
        for (int c = 0; c < CT; ++c) vt[c] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kb = bb & ~1; kb < NB; kb += 2) {
          const bf16x4 a0 = read_tr4(reinterpret_cast<const bf16*>(Tp) + 16 * kb * C + offTT[bb]);
          const bf16x4 a1 = read_tr4(reinterpret_cast<const bf16*>(Tp) + 16 * (kb + 1) * C + offTT[bb]);
#pragma unroll
          for (int c = 0; c < CT; ++c) vt[c] = D::mma2(a0, a1, Yb[c][kb], Yb[c][kb + 1], vt[c]);
        }
        const floatx4 eg4 = *reinterpret_cast<const floatx4*>(egp + 16 * bb + 4 * g4);
#pragma unroll
        for (int c = 0; c < CT; ++c) DVb[c][bb] = D::cvt(-eg4 * vt[c]);
      }
    }
#pragma unroll
    for (int bb = 0; bb < NB && !REV; ++bb) {
      floatx4 vt[CT];
#pragma unroll
      for (int c = 0; c < CT; ++c) vt[c] = floatx4{0.f, 0.f, 0.f, 0.f};
      if (D::PAIRS && ((bb + 2) & ~1) <= NB) {
#pragma unroll
        for (int kb = 0; kb <= bb; kb += 2) {
          const typename D::A a0 = D::row4(Tp + 16 * bb * C + offT[kb]);
          const typename D::A a1 = D::row4(Tp + 16 * bb * C + offT[kb + 1]);
#pragma unroll
          for (int c = 0; c < CT; ++c) vt[c] = D::mma2(a0, a1, Yb[c][kb], Yb[c][kb + 1], vt[c]);
        }
      } else {
#pragma unroll
        for (int kb = 0; kb <= bb; ++kb) {
          const typename D::A a0 = D::row4(Tp + 16 * bb * C + offT[kb]);
#pragma unroll
          for (int c = 0; c < CT; ++c) vt[c] = D::mma1(a0, Yb[c][kb], vt[c]);
        }
      }
      const floatx4 ed4 = *reinterpret_cast<const floatx4*>(edp + 16 * bb + 4 * g4);
#pragma unroll
      for (int c = 0; c < CT; ++c) {
        Vb[c][bb] = D::cvt(vt[c]);
        DVb[c][bb] = D::cvt(vt[c] * ed4);
      }
    }

    // ---- outputs: O = scale (gamma_p Q S + A V~), S still the chunk-start state, formed
    // transposed: with the operands of each product swapped the MFMA yields the tile of O^T
    // (O^T = S^T Q^T + V~^T A^T; the state and V~ registers serve as A operands and the Q and A
    // row fragments as B operands unchanged), so lane (g, m) holds columns 4g .. 4g + 3 of token
    // row m and stores them with one 8-byte (bf16) or 16-byte (fp32) write.  A is zero past each
    // token's causal reach, so the product runs over all position blocks.  Every row block is
    // computed (with several sub-steps per token the blocks past the chunk's tokens read stale
    // but in-bounds LDS) and the stores are masked by the buffer range check: no branch splits
    // the chunk body.
    if constexpr (OUT) {
      constexpr int KSTEPA = (D::PAIRS && NB % 2 == 0) ? 2 : 1;
      // Output addresses depend only on the lane and the chunk; hiding the lane index keeps the
      // optimiser from hoisting one register per row block and tile out of the chunk loop.
      int lo = lane;
      asm volatile("" : "+v"(lo));
      const int mo = lo & 15, go = lo >> 4;
      // this chunk's first token row of O (uniform) and the number of its rows inside the sequence
      const int HDV = p.H * p.DV;
      E* Ochunk = Og + (((long)b * p.L + (long)n * QR) * p.H + h) * p.DV;
      const int orows = min(QR, (int)((long)p.L - (long)n * QR));
      const __amdgpu_buffer_rsrc_t orsrc = buffer_rsrc(Ochunk, orows * HDV * (int)sizeof(E));
      // the lane's first element column of each tile in O; a tile past the value columns stores
      // out of range
      int ocol[CT];
#pragma unroll
      for (int c = 0; c < CT; ++c) ocol[c] = isv[c] ? 16 * tile[c] + 4 * go : orows * HDV;
#pragma unroll
      for (int tq = 0; tq < NB; ++tq) {
        floatx4 o1[CT], o2[CT];
#pragma unroll
        for (int c = 0; c < CT; ++c) o1[c] = o2[c] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int t = 0; t < NTS; t += TSTEP) {
          if constexpr (DP) {
            const bf16x8 a = DOp<bf16>::row8(reinterpret_cast<const bf16*>(Qp) + 16 * tq * DK + offK[t]);
#pragma unroll
            for (int c = 0; c < CT; ++c)
              o1[c] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                  __builtin_shufflevector(Sb[c][t], Sb[c][t + 1], 0, 1, 2, 3, 4, 5, 6, 7), a, o1[c], 0, 0, 0);
          } else {
            const typename D::A a0 = D::row4(Qp + 16 * tq * DK + offK[t]);
#pragma unroll
            for (int c = 0; c < CT; ++c) o1[c] = D::mma1(Sb[c][t], a0, o1[c]);
          }
        }
#pragma unroll
        for (int kb = 0; kb < NB; kb += KSTEPA) {
          const typename D::A a0 = D::row4(Ap + 16 * tq * C + offT[kb]);
          if constexpr (KSTEPA == 2) {
            const typename D::A a1 = D::row4(Ap + 16 * tq * C + offT[kb + 1]);
#pragma unroll
            for (int c = 0; c < CT; ++c) o2[c] = D::mma2(Vb[c][kb], Vb[c][kb + 1], a0, a1, o2[c]);
          } else {
#pragma unroll
            for (int c = 0; c < CT; ++c) o2[c] = D::mma1(Vb[c][kb], a0, o2[c]);
          }
        }
        // scale * gamma of the lane's token (its last sub-step; rows past the chunk's tokens: 0);
        // the stored A_qk already carries the scale
        const float gq = eqp[16 * tq + mo];
        const int orow = (16 * tq + mo) * HDV;
#pragma unroll
        for (int c = 0; c < CT; ++c) {
          const floatx4 o = gq * o1[c] + o2[c];
          if constexpr (sizeof(E) == 2) buffer_store8(orsrc, (orow + ocol[c]) * 2, DOp<bf16>::cvt(o));
          else buffer_store16(orsrc, (orow + ocol[c]) * 4, o);
        }
      }
    }

    // ---- S <- gamma_C S + K^T (gamma_C / gamma V~); the reverse chain:
    // G <- gamma_C G + K^T (-gamma dY) + Q^T (gamma_q dO), gamma_q = scale exp(gc) at each token's
    // last sub-step (0 past the chunk's tokens)
    {
      const float gC = egp[C - 1];
      constexpr int BSTEP = (D::PAIRS && NB % 2 == 0) ? 2 : 1;
      [[maybe_unused]] typename D::B QOb[CT][NB];
      if constexpr (REV) {
#pragma unroll
        for (int kb = 0; kb < NB; ++kb) {
          const floatx4 eq4 = *reinterpret_cast<const floatx4*>(eqp + 16 * kb + 4 * g4);
#pragma unroll
          for (int c = 0; c < CT; ++c) {
            const bf16x4 o = Ob[c][kb];
            QOb[c][kb] = D::cvt(eq4 * floatx4{(float)o[0], (float)o[1], (float)o[2], (float)o[3]});
          }
        }
      }
#pragma unroll
      for (int t = 0; t < NTS; ++t) {
#pragma unroll
        for (int c = 0; c < CT; ++c) S[c][t] *= gC;
#pragma unroll
        for (int bb = 0; bb < NB; bb += BSTEP) {
          typename D::A a0, a1;
          if constexpr (sizeof(E) == 2) {
            a0 = read_tr4(reinterpret_cast<const bf16*>(Kp) + 16 * bb * DK + offKT[t]);
            if constexpr (BSTEP == 2) a1 = read_tr4(reinterpret_cast<const bf16*>(Kp) + 16 * (bb + 1) * DK + offKT[t]);
          } else {
            const Tile<E> K = make_packed_tile<E, DK>(const_cast<E*>(Kp));
            a0 = D::col4(K, 16 * bb, 16 * t, lane);
            if constexpr (BSTEP == 2) a1 = D::col4(K, 16 * bb + 16, 16 * t, lane);
          }
          if constexpr (BSTEP == 2) {
#pragma unroll
            for (int c = 0; c < CT; ++c) S[c][t] = D::mma2(a0, a1, DVb[c][bb], DVb[c][bb + 1], S[c][t]);
          } else {
#pragma unroll
            for (int c = 0; c < CT; ++c) S[c][t] = D::mma1(a0, DVb[c][bb], S[c][t]);
          }
        }
        if constexpr (REV) {
#pragma unroll
          for (int kb = 0; kb < NB; kb += 2) {
            const bf16x4 a0 = read_tr4(reinterpret_cast<const bf16*>(Qp) + 16 * kb * DK + offKT[t]);
            const bf16x4 a1 = read_tr4(reinterpret_cast<const bf16*>(Qp) + 16 * (kb + 1) * DK + offKT[t]);
#pragma unroll
            for (int c = 0; c < CT; ++c) S[c][t] = D::mma2(a0, a1, QOb[c][kb], QOb[c][kb + 1], S[c][t]);
          }
        }
      }
    }
    barrier_lds();  // chunk done (and, with one stage, the stage may be reloaded)
  }

  // ---------------- segment results (a summary: S_loc, and M as E, in the combine's order)
#pragma unroll
  for (int c = 0; c < CT; ++c) {
    if (!live[c]) continue;
#pragma unroll
    for (int t = 0; t < NTS; ++t)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int row = dkrow(t, 4 * g4 + j);
        if constexpr (SUM) {
          float* SMs = p.SM + ((long)head * p.P + seg) * DK * (p.DV + DK);
          if (isv[c]) SMs[sloc_index(row, 16 * tile[c] + m, DK)] = S[c][t][j];
          else reinterpret_cast<E*>(SMs + (long)p.DV * DK)[mfrag_index<mfrag_width<E, DK>()>(row, 16 * (tile[c] - NCT) + m, DK)] = to_elem<E>(S[c][t][j]);
        } else if (seg == p.P - 1 && p.S_final) {
          p.S_final[((long)head * DK + row) * p.DV + 16 * tile[c] + m] = S[c][t][j];
        }
      }
  }
}

// Start states of the segments, in order: S_start(1) = S_end(0) and
// S_start(q+1) = M(q) S_start(q) + S_loc(q).  One workgroup per (head, CTW tiles of 16 state
// columns), one wavefront per 16 state rows; fp32 accumulation.  The chain is short and each
// step is a few MFMAs: the time goes into fetching the summaries, M(q) once per workgroup (so
// several column tiles share each A fragment) and S_loc(q) for the workgroup's columns.  The
// loads of up to DEPTH segments are issued together into DEPTH register sets; the current start
// state is exchanged between the wavefronts through two LDS buffers, one barrier per step.
// BF: bf16 products (M is stored in bf16; the state is rounded to bf16 as the chunk chain
// rounds it every chunk) on the 32-deep MFMA, k in natural order: the lane's A fragment is 16
// contiguous bytes of its row of M.  Otherwise fp32 products on the 4-deep MFMA with the
// contraction index permuted (consistently in both operands): lane group g takes
// k = 16 i + 4 g + e, so one load of the four lane groups of a row covers 16 contiguous elements.
template <typename E, int DK, bool BF, int CTW>
struct CombineCfg {
  static constexpr int NA = BF ? DK / 32 : DK / 16;  // A pieces per lane and segment
  static constexpr int RUNREGS = NA * (BF ? 4 : (int)sizeof(E)) + 4 * CTW;
  static constexpr int DEPTH = 192 / RUNREGS < 8 ? 192 / RUNREGS : 8;
};

template <typename E, int DK, bool BF, int CTW>
__global__ __launch_bounds__(DK / 16 * WAVE) void combine_kernel(FwdParams p) {
  using Cfg = CombineCfg<E, DK, BF, CTW>;
  constexpr int NA = Cfg::NA, DEPTH = Cfg::DEPTH;
  static_assert(!BF || (sizeof(E) == 2 && DK % 32 == 0), "bf16 products take bf16 M, 32 indices a step");
  typedef typename std::conditional<BF, bf16, float>::type SE;
  // A piece as loaded: 8 bf16 (BF), 4 E otherwise
  typedef typename std::conditional<BF, bf16x8, typename std::conditional<sizeof(E) == 2, bf16x4, floatx4>::type>::type Piece;
  // the current start state, transposed: column 16 c + m at row 16 c + m, padded by 16 bytes;
  // two buffers
  constexpr int LDT = DK + 16 / (int)sizeof(SE);
  __shared__ __attribute__((aligned(16))) SE SlT[2][16 * CTW * LDT];
  const int NG = p.DV / (16 * CTW);  // column groups per head
  // workgroups are dealt round-robin over the 8 XCDs: keep the column groups of one head on one
  // XCD so that its transitions are fetched into one L2 once
  int head, cg;
  if ((p.B * p.H) % 8 == 0) {
    const int x = blockIdx.x % 8, j = blockIdx.x / 8;
    head = x + 8 * (j / NG);
    cg = j % NG;
  } else {
    head = blockIdx.x / NG;
    cg = blockIdx.x % NG;
  }
  const int lane = threadIdx.x & 63, t = threadIdx.x >> 6, m = lane & 15, g4 = lane >> 4;
  const int col0 = 16 * CTW * cg + m;        // the lane's column of tile 0 (tile c: + 16 c)
  const long SLOT = (long)DK * (p.DV + DK);  // floats per segment summary
  const float* SMh = p.SM + (long)head * p.P * SLOT;
  float* Sst = p.Sst + (long)head * p.P * DK * p.DV;
  // Loads go through a buffer resource per segment summary, so a lane keeps two offsets: its
  // S_loc values (rows 16 t + 4 g4 .. + 3 of its column of tile 0) and its first A piece (row
  // 16 t + m of M); both layouts put a wavefront's 64 pieces of one load side by side.
  constexpr int PW = mfrag_width<E, DK>();
  static_assert(PW == (BF ? 8 : 4), "M piece width");
  const int offS = sloc_index(16 * t + 4 * g4, col0, DK) * 4;
  const int offM = p.DV * DK * 4 + mfrag_index<PW>(16 * t + m, PW * g4, DK) * (int)sizeof(E);
  constexpr int STEPM = 64 * PW * (int)sizeof(E);  // bytes between a lane's A pieces
  constexpr int STEPS = DK / 16 * 64 * 16;         // bytes between a lane's S_loc column tiles
  auto rsrc = [&](int q) { return buffer_rsrc(const_cast<float*>(SMh) + q * SLOT, (int)SLOT * 4); };
  struct Run {
    Piece a[NA];
    floatx4 sl[CTW];
  };
  auto load = [&](int q, Run& r) {
    const __amdgpu_buffer_rsrc_t rs = rsrc(q);
#pragma unroll
    for (int i = 0; i < NA; ++i) {
      if constexpr (sizeof(Piece) == 16) r.a[i] = __builtin_bit_cast(Piece, buffer_load16(rs, offM + STEPM * i));
      else r.a[i] = __builtin_bit_cast(Piece, buffer_load8(rs, offM + STEPM * i));
    }
#pragma unroll
    for (int c = 0; c < CTW; ++c) r.sl[c] = __builtin_bit_cast(floatx4, buffer_load16(rs, offS + STEPS * c));
  };
  // the new start state of q1, tile c: into LDS buffer q1 & 1 and to the start-state output
  auto put = [&](int q1, int c, floatx4 x) {
    SE* d = SlT[q1 & 1] + (16 * c + m) * LDT + 16 * t + 4 * g4;
    if constexpr (BF) *reinterpret_cast<bf16x4*>(d) = bf16x4{(bf16)x[0], (bf16)x[1], (bf16)x[2], (bf16)x[3]};
    else *reinterpret_cast<floatx4*>(d) = x;
#pragma unroll
    for (int j = 0; j < 4; ++j) Sst[((long)q1 * DK + 16 * t + 4 * g4 + j) * p.DV + col0 + 16 * c] = x[j];
  };
  // waves exchange the state only through LDS: a barrier that waits for LDS alone, so the loads
  // in flight are not drained
  auto lds_barrier = [] {
    __builtin_amdgcn_s_waitcnt(0xC07F);
    asm volatile("s_barrier" ::: "memory");
  };
  // S_start(q+1) from the run of segment q and S_start(q) in buffer q & 1
  auto step = [&](int q, const Run& r) {
    floatx4 acc0[CTW], acc1[CTW];
#pragma unroll
    for (int c = 0; c < CTW; ++c) {
      acc0[c] = r.sl[c];
      acc1[c] = floatx4{0.f, 0.f, 0.f, 0.f};
    }
#pragma unroll
    for (int i = 0; i < NA; ++i) {
#pragma unroll
      for (int c = 0; c < CTW; ++c) {
        const SE* y = SlT[q & 1] + (16 * c + m) * LDT;
        floatx4& acc = (i & 1) ? acc1[c] : acc0[c];
        if constexpr (BF) {
          const bf16x8 b = *reinterpret_cast<const bf16x8*>(y + 32 * i + 8 * g4);
          acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(r.a[i], b, acc, 0, 0, 0);
        } else {
          const floatx4 b = *reinterpret_cast<const floatx4*>(y + 16 * i + 4 * g4);
          floatx4 a;
          if constexpr (sizeof(E) == 2) a = floatx4{(float)r.a[i][0], (float)r.a[i][1], (float)r.a[i][2], (float)r.a[i][3]};
          else a = r.a[i];
#pragma unroll
          for (int e = 0; e < 4; ++e) acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a[e], b[e], acc, 0, 0, 0);
        }
      }
    }
#pragma unroll
    for (int c = 0; c < CTW; ++c) put(q + 1, c, acc0[c] + acc1[c]);
    lds_barrier();
  };
  // S_start(1) = S_end(0)
  {
    const __amdgpu_buffer_rsrc_t rs = rsrc(0);
#pragma unroll
    for (int c = 0; c < CTW; ++c) put(1, c, __builtin_bit_cast(floatx4, buffer_load16(rs, offS + STEPS * c)));
  }
  lds_barrier();
  // rounds of DEPTH segments: all of a round's loads are issued together, then its steps run
  const int last = p.P - 2;  // last segment with a transition
  for (int q0 = 1; q0 <= last; q0 += DEPTH) {
    Run r[DEPTH];
#pragma unroll
    for (int d = 0; d < DEPTH; ++d)
      if (q0 + d <= last) load(q0 + d, r[d]);
#pragma unroll
    for (int d = 0; d < DEPTH; ++d)
      if (q0 + d <= last) step(q0 + d, r[d]);
  }
}

// ------------------------------------------------------------------ launch
template <typename E, int DK, int C, int CT, int NCW, int MODE, bool REV = false>
static hipError_t launch_seg(const FwdParams& p, hipStream_t st) {
  using Cfg = SegCfg<E, DK, C, CT, NCW, MODE, REV>;
  constexpr int TPG = Cfg::TPG;
  const int NCT = p.DV / 16, MCT = (Cfg::SUM && !REV) ? DK / 16 : 0;
  const int G = (NCT + MCT + TPG - 1) / TPG;
  const int nseg = Cfg::SUM ? p.P - 1 : p.P;
  const long blocks = (long)nseg * p.B * p.H * G;
  if (blocks == 0) return hipSuccess;
  hipLaunchKernelGGL((seg_kernel<E, DK, C, CT, NCW, MODE, REV>), dim3((unsigned)blocks), dim3(Cfg::THREADS), 0, st, p);
  return hipGetLastError();
}

// Outputs: 4 chain wavefronts (plus the 4 loading ones), one 16-column tile each when d_v <= 64,
// else two.  Summary: 2 state tiles per chain wavefront; with bf16 inputs 8 chain wavefronts, so
// that one workgroup covers 16 tiles (the d_v value and d_k transition columns of a segment
// together when d_v + d_k <= 256: K and T are then staged once per segment, and a segment's
// workgroups fit the GPU in one round); fp32 state fragments need twice the registers, so fp32
// takes 4.
constexpr int OUT_NCW = 4, SUM_CT = 2;
template <typename E>
constexpr int sum_ncw() { return sizeof(E) == 2 ? 8 : 4; }

template <typename E, int DK, int C>
static hipError_t scan_phase(const FwdParams& p, int phase, hipStream_t st) {
  switch (phase) {
    case SCAN_SUMMARY:
      return p.P > 1 ? launch_seg<E, DK, C, SUM_CT, sum_ncw<E>(), SEG_SUM>(p, st) : hipSuccess;
    case SCAN_COMBINE:
      if (p.P <= 1 || p.B * p.H == 0) return hipSuccess;
    {
      // one column tile per workgroup: the workgroup's loads are what takes the time, and with
      // 2 or 4 tiles (M fetched once for more columns) the launch measured 9.8 / 13.5 us against
      // 8.2 us on the 8K-token workload
      constexpr bool BF = sizeof(E) == 2 && DK >= 32;
      hipLaunchKernelGGL((combine_kernel<E, DK, BF, 1>), dim3((unsigned)(p.B * p.H * (p.DV / 16))), dim3(DK / 16 * WAVE), 0, st, p);
      return hipGetLastError();
    }
    case SCAN_OUTPUTS:
      return p.DV / 16 <= OUT_NCW ? launch_seg<E, DK, C, 1, OUT_NCW, SEG_OUT>(p, st)
                                  : launch_seg<E, DK, C, 2, 4, SEG_OUT>(p, st);
    default:
      return hipErrorInvalidValue;
  }
}

template <typename E, int DK>
static hipError_t phase_by_c(const FwdParams& p, int phase, hipStream_t st) {
  switch (p.C) {
    case 16: return scan_phase<E, DK, 16>(p, phase, st);
    case 32: return scan_phase<E, DK, 32>(p, phase, st);
    case 48: return scan_phase<E, DK, 48>(p, phase, st);
    case 64: return scan_phase<E, DK, 64>(p, phase, st);
    default: return hipErrorInvalidValue;
  }
}

template <typename E>
static hipError_t phase_by_dk(const FwdParams& p, int phase, hipStream_t st) {
  switch (p.DK) {
    case 16: return phase_by_c<E, 16>(p, phase, st);
    case 32: return phase_by_c<E, 32>(p, phase, st);
    case 64: return phase_by_c<E, 64>(p, phase, st);
    case 128: return phase_by_c<E, 128>(p, phase, st);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_scan_phase(const FwdParams& p, bool bf16_in, int phase, hipStream_t st) {
  if (phase == SCAN_SUMMARY && scan_summary_fast_applies(p, bf16_in)) return launch_scan_summary_fast(p, st);
  return bf16_in ? phase_by_dk<bf16>(p, phase, st) : phase_by_dk<float>(p, phase, st);
}

// The backward pass's two scans over chunk states, for bf16 inputs with d_k = d_v = 128 and
// chunk 64 (bwd_scans_apply): the forward chain writing each chunk's start state, and the
// adjoint chain (summary, combine, chain) writing each chunk's end-state gradient.  Both use
// 4 chain wavefronts of 2 column tiles; the reverse summary covers the value and transition
// columns in two workgroups per segment.
bool bwd_scans_apply(const FwdParams& p, bool bf16_in) {
  return bf16_in && p.DK == 128 && p.DV == 128 && p.C == 64;
}

hipError_t launch_scan_states(const FwdParams& p, hipStream_t st) {
  if (p.DK != 128 || p.DV != 128 || p.C != 64) return hipErrorInvalidValue;
  return launch_seg<bf16, 128, 64, 2, 4, SEG_STATES>(p, st);
}

// KDA in chunks (bf16, d_k = d_v = 128, chunk 64): the summary and the chain forming the outputs by
// the summary kernel's KDA forms (scan_summary.hip), the start states by the combine launch.
hipError_t launch_kda_scan(const FwdParams& p, int phase, hipStream_t st) {
  if (p.DK != 128 || p.DV != 128 || p.C != 64) return hipErrorInvalidValue;
  switch (phase) {
    case SCAN_SUMMARY:
      return launch_scan_summary_fast_kda(p, st);
    case SCAN_COMBINE:
      return scan_phase<bf16, 128, 64>(p, SCAN_COMBINE, st);
    case SCAN_OUTPUTS:
      return launch_scan_outputs_kda(p, st);
    default:
      return hipErrorInvalidValue;
  }
}

hipError_t launch_rev_scan(const FwdParams& p, int phase, hipStream_t st) {
  if (p.DK != 128 || p.DV != 128 || p.C != 64) return hipErrorInvalidValue;
  switch (phase) {
    case SCAN_SUMMARY:
      return p.P > 1 ? launch_seg<bf16, 128, 64, 2, 4, SEG_SUM, true>(p, st) : hipSuccess;
    case SCAN_COMBINE:
      return scan_phase<bf16, 128, 64>(p, SCAN_COMBINE, st);
    case SCAN_OUTPUTS:
      return launch_seg<bf16, 128, 64, 2, 4, SEG_STATES, true>(p, st);
    default:
      return hipErrorInvalidValue;
  }
}

}  // namespace delta
