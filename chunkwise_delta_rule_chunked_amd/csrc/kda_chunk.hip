// KDA forward in chunks: the delta rule with a decay per key channel,
//     S_t = (I - beta_t k_t k_t^T) Diag(alpha_t) S_{t-1} + beta_t k_t v_t^T,   o_t = scale S_t^T q_t
// ("08 linear delta rule & DPLR" page, section 1.4 table, KDA row, and section 5), evaluated
// chunkwise for bf16 inputs with d_k = d_v = 128, chunk 64, one step per token.
//
// The pages give KDA's recurrence but not a chunk algorithm; this one follows from it as the
// scalar-gated form follows from its recurrence (the same page, sections 2.2-2.3 and 3).  With
// Gc_r = sum_{j <= r} log alpha_j per channel inside the chunk (restarting every chunk) and the
// chunk's start state S:
//     A_rj  = beta_r sum_c k_rc k_jc e^{Gc_rc - Gc_jc}          (j < r; the Gram matrix decayed
//                                                                  per channel)
//     T     = (I + A)^-1 diag(beta)                             (the UT transform, ut_solve.h)
//     V~    = T (V - K+ S),            K+ = K e^{Gc}
//     O     = Q+ S + Aqk V~,           Q+ = scale Q e^{Gc},  Aqk_rj = scale q_r . (k_j e^{Gc_r - Gc_j}), j <= r
//     S'    = e^{Gc_C} S + Kh^T V~,    Kh = K e^{Gc_C - Gc}     (e^{Gc_C} scales row c of S)
// Every exponent above is a decay from a later position back to an earlier one (<= 0).  The block
// products below split e^{Gc_r - Gc_j} at a reference row between the two; below the block
// diagonal both halves are decays, on it one half grows, and a bound on its span keeps it finite
// (block_row, diag_span_ok).
//
// Four launches (delta_abi.cpp runs them):
//   kda_intra_kernel   per chunk: Gc, A and Aqk, T, and the decayed tiles K+, Kh, Q+ and the
//                      chunk decay e^{Gc_C} into the workspace;
//   the inter-chunk scan in the summary kernel's KDA forms (scan_summary.hip): segment
//                      summaries, the combine launch's start states, then the chain from each
//                      segment's start state forming O and S_final.
#include "common.h"
#include "kernels.h"
#include "ut_solve.h"

namespace delta {
namespace kdac {

constexpr int DK = 128, C = 64;
constexpr int GP = DK + 4;  // float row pitch of the Gc table
constexpr int KP = DK + 8;  // bf16 row pitch of the key tile
constexpr int NTH = 256;

// Loads with the non-temporal cache policy, for inputs this kernel reads for the last time (k,
// the log decays, and q's second read, for the block products): nothing else reads them again,
// so they need not displace the decayed tiles that the scans read next from the caches (the call
// measured ~10 us faster on the 32-head 8K-token shape).  0 outside the buffer range.
__device__ inline u32x4 load16_last(__amdgpu_buffer_rsrc_t r, int off) {
  return __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 2);
}
__device__ inline float load4_last(__amdgpu_buffer_rsrc_t r, int off) {
  return __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(r, off, 0, 2));
}

// 16-lane row sum (every lane of the row gets it): quad xor 1, xor 2, half-mirror, mirror
template <int CTRL>
__device__ inline float dpp(float x) {
  return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x), CTRL, 0xF, 0xF, false));
}
__device__ inline float row_sum16(float x) {
  x += dpp<0xB1>(x);
  x += dpp<0x4E>(x);
  x += dpp<0x141>(x);
  x += dpp<0x140>(x);
  return x;
}
__device__ inline void unpack8(u32x4 r, float* x) {
  const bf16x8 v = __builtin_bit_cast(bf16x8, r);
#pragma unroll
  for (int e = 0; e < 8; ++e) x[e] = (float)v[e];
}
__device__ inline u32x4 pack8(const float* x) {
  bf16x8 v;
#pragma unroll
  for (int e = 0; e < 8; ++e) v[e] = (bf16)x[e];
  return __builtin_bit_cast(u32x4, v);
}

// LDS of the intra kernel.  The Gc table is dead once the decayed tiles and the MFMA products are
// done; A's slots and the Aqk staging tile then take its place.
struct IntraLds {
  static constexpr int GC_BYTES = C * GP * 4;
  static constexpr int SLOT_BYTES = UtSlots<C>::BYTES;
  static constexpr int AQ_LD = C + 8;  // bf16 row pitch of the Aqk tile
  static constexpr int AQ_BYTES = C * AQ_LD * 2;
  static_assert(SLOT_BYTES + AQ_BYTES <= GC_BYTES, "A's slots and Aqk must fit in the Gc table");
  union {
    float Gc[C][GP];
    struct {
      unsigned char slots[SLOT_BYTES];
      bf16 Aq[C][AQ_LD];
    } a;
  } u;
  bf16 Kl[C][KP];
  float bs[C];
};

// Largest per-channel decay span (Gc at the row before a 16-row block minus Gc at its last row,
// i.e. minus the sum of the block's log decays) for which the block's diagonal entries are taken
// on the MFMA: its B factors reach e^{span}, its A factors e^{-span}, both far inside float32's
// normal range.
constexpr float DIAG_SPAN = 64.f;

// x = hi + lo in bf16 (hi the round-to-nearest of x, lo that of the remainder): a product of two
// such pairs, hi hi + hi lo + lo hi on the bf16 MFMA, is the float32 product to about 2^-16.
__device__ inline void split8(const float* x, bf16x8& hi, bf16x8& lo) {
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    hi[e] = (bf16)x[e];
    lo[e] = (bf16)(x[e] - (float)hi[e]);
  }
}
__device__ inline floatx4 mma3(bf16x8 ah, bf16x8 al, bf16x8 bh, bf16x8 bl, floatx4 c) {
  c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ah, bh, c, 0, 0, 0);
  c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ah, bl, c, 0, 0, 0);
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(al, bh, c, 0, 0, 0);
}

// Entries of row block I of A and Aqk against column blocks J0 .. J0 + NJ - 1 (J <= I), each a
// 16 x 16 product over d_k on the bf16 MFMA with split operands (split8), into accumulators
// OFF .. OFF + NJ - 1.  The reference is the row just before the block, rho = 16 I - 1 (Gc_rho = 0
// for I = 0): the A operand is k_r e^{Gc_r - Gc_rho} (scale q_r e^{...} for Aqk), the B operand
// k_j e^{Gc_rho - Gc_j}.  Below the diagonal block (j <= rho) both factors are decays (<= 1; a
// product that underflows is below either factor); on the diagonal block the B factor is a
// growth bounded by e^{span}, which diag_span_ok checks.  Lane (g, m) of a 16x16x32 step takes
// channels 32 u + 8 g .. + 7 of row m.
template <int I, int J0, int NJ, int OFF, int NA>
__device__ __forceinline__ void block_row(const IntraLds& s, __amdgpu_buffer_rsrc_t qrs, long HD, float scale,
                                          floatx4 (&gram)[NA], floatx4 (&aqk)[NA], int lane) {
  const int g4 = lane >> 4, m = lane & 15, ra = 16 * I + m;
  constexpr int rho = 16 * I - 1;
  u32x4 qa[4];
#pragma unroll
  for (int u = 0; u < 4; ++u) qa[u] = load16_last(qrs, (int)((ra * HD + 32 * u + 8 * g4) * 2));  // 0 past the sequence
#pragma unroll
  for (int t = 0; t < NJ; ++t) gram[OFF + t] = aqk[OFF + t] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const int c = 32 * u + 8 * g4;
    float ga[8], gr[8], av[8], aq[8];
    *reinterpret_cast<floatx4*>(ga) = *reinterpret_cast<const floatx4*>(&s.u.Gc[ra][c]);
    *reinterpret_cast<floatx4*>(ga + 4) = *reinterpret_cast<const floatx4*>(&s.u.Gc[ra][c + 4]);
    if (rho >= 0) {
      *reinterpret_cast<floatx4*>(gr) = *reinterpret_cast<const floatx4*>(&s.u.Gc[rho][c]);
      *reinterpret_cast<floatx4*>(gr + 4) = *reinterpret_cast<const floatx4*>(&s.u.Gc[rho][c + 4]);
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e) gr[e] = 0.f;
    }
    const bf16x8 ka = *reinterpret_cast<const bf16x8*>(&s.Kl[ra][c]);
    const bf16x8 q8 = __builtin_bit_cast(bf16x8, qa[u]);
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float ea = gate_exp(ga[e] - gr[e]);
      av[e] = (float)ka[e] * ea;
      aq[e] = scale * (float)q8[e] * ea;
    }
    bf16x8 ah, al, qh, ql;
    split8(av, ah, al);
    split8(aq, qh, ql);
#pragma unroll
    for (int t = 0; t < NJ; ++t) {
      const int rb = 16 * (J0 + t) + m;
      float gb[8], bv[8];
      *reinterpret_cast<floatx4*>(gb) = *reinterpret_cast<const floatx4*>(&s.u.Gc[rb][c]);
      *reinterpret_cast<floatx4*>(gb + 4) = *reinterpret_cast<const floatx4*>(&s.u.Gc[rb][c + 4]);
      const bf16x8 kb = *reinterpret_cast<const bf16x8*>(&s.Kl[rb][c]);
#pragma unroll
      for (int e = 0; e < 8; ++e) bv[e] = (float)kb[e] * gate_exp(gr[e] - gb[e]);
      bf16x8 bh, bl;
      split8(bv, bh, bl);
      gram[OFF + t] = mma3(ah, al, bh, bl, gram[OFF + t]);
      aqk[OFF + t] = mma3(qh, ql, bh, bl, aqk[OFF + t]);
    }
  }
}

// Whether every channel's decay span over diagonal block I is within DIAG_SPAN (NaN is not), for
// the whole wave.
template <int I>
__device__ __forceinline__ bool diag_span_ok(const IntraLds& s, int lane) {
  constexpr int rho = 16 * I - 1, e = 16 * I + 15;
  const float s0 = (rho >= 0 ? s.u.Gc[rho][lane] : 0.f) - s.u.Gc[e][lane];
  const float s1 = (rho >= 0 ? s.u.Gc[rho][lane + 64] : 0.f) - s.u.Gc[e][lane + 64];
  return __all(s0 <= DIAG_SPAN && s1 <= DIAG_SPAN);
}

// The accumulators of block_row into A's slots (times beta of the row; on the diagonal block the
// entries j < r) and into the Aqk tile (j <= r; zeros above the diagonal, also when diag_exact
// takes the diagonal block).  Lane (g, m) holds rows
// 4 g .. 4 g + 3 of column m of each block.
template <int I, int J0, int NJ, int OFF, int NA>
__device__ __forceinline__ void store_row(IntraLds& s, const floatx4 (&gram)[NA], const floatx4 (&aqk)[NA], bool diag_ok,
                                          int lane) {
  constexpr int LDB = UtSlots<C>::LDB, BLK = UtSlots<C>::BLK;
  const int g4 = lane >> 4, m = lane & 15;
  float* As = reinterpret_cast<float*>(s.u.a.slots);
#pragma unroll
  for (int t = 0; t < NJ; ++t) {
    const int J = J0 + t;
    const bool mf = J < I || diag_ok;  // else diag_exact writes the entries j <= r
    float* blk = As + lower_block(I, J) * BLK;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int rl = 4 * g4 + j, r = 16 * I + rl;
      if (mf && (J < I || m < rl)) blk[rl * LDB + m] = s.bs[r] * gram[OFF + t][j];
      if (J < I || m <= rl) {
        if (mf) s.u.a.Aq[r][16 * J + m] = (bf16)aqk[OFF + t][j];
      } else {
        s.u.a.Aq[r][16 * J + m] = (bf16)0.f;
      }
    }
  }
}

// Diagonal block I of A and Aqk entry by entry with the exact per-channel factor e^{Gc_r - Gc_j}
// (j <= r), for blocks whose span is beyond DIAG_SPAN (a reset, very strong decay, NaN), by one
// wave from global memory (the Gc table is gone by then): 16-lane group g takes the block's rows
// g, 7 - g, 8 + g and 15 - g (34 entries), lane l of the group channels 8 l .. 8 l + 7.  For a row
// r the factor runs down from j = r as a product of the per-token decays (factor_{j-1} =
// factor_j e^{log alpha_j}), each entry a DPP row sum.  Rows past the sequence have k = q = 0 and
// decay by nothing.
__device__ __noinline__ void diag_exact(IntraLds& s, const bf16* qb, const bf16* kb, const float* ab, long HD,
                                        int valid, float scale, int I, int lane) {
  constexpr int LDB = UtSlots<C>::LDB, BLK = UtSlots<C>::BLK;
  const int grp = lane >> 4, gl = lane & 15, c = 8 * gl;
  float* blk = reinterpret_cast<float*>(s.u.a.slots) + lower_block(I, I) * BLK;
  const int rl4[4] = {grp, 7 - grp, 8 + grp, 15 - grp};
  for (int u = 0; u < 4; ++u) {
    const int rl = rl4[u], r = 16 * I + rl;
    float kr[8], qr[8], f[8];
    unpack8(r < valid ? *reinterpret_cast<const u32x4*>(kb + r * HD + c) : u32x4{0, 0, 0, 0}, kr);
    unpack8(r < valid ? *reinterpret_cast<const u32x4*>(qb + r * HD + c) : u32x4{0, 0, 0, 0}, qr);
#pragma unroll
    for (int e = 0; e < 8; ++e) f[e] = 1.f;
    for (int jl = rl; jl >= 0; --jl) {
      const int j = 16 * I + jl;
      float kj[8];
      unpack8(j < valid ? *reinterpret_cast<const u32x4*>(kb + j * HD + c) : u32x4{0, 0, 0, 0}, kj);
      float sg = 0.f, sq = 0.f;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float kd = kj[e] * f[e];
        sg += kr[e] * kd;
        sq += qr[e] * kd;
      }
      if (j < valid) {  // the factor for j - 1 takes in token j's decay
        const floatx4 a0 = *reinterpret_cast<const floatx4*>(ab + j * HD + c);
        const floatx4 a1 = *reinterpret_cast<const floatx4*>(ab + j * HD + c + 4);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          f[e] *= gate_exp(a0[e] < LOG_GATE_FLOOR ? LOG_GATE_FLOOR : a0[e]);
          f[4 + e] *= gate_exp(a1[e] < LOG_GATE_FLOOR ? LOG_GATE_FLOOR : a1[e]);
        }
      }
      sg = row_sum16(sg);
      sq = row_sum16(sq);
      if (gl == 0) {
        if (jl < rl) blk[rl * LDB + jl] = s.bs[r] * sg;
        s.u.a.Aq[r][j] = (bf16)(scale * sq);
      }
    }
  }
}

// One workgroup of 4 wavefronts per (sequence, head, chunk).
//   1. keys to LDS (rows past the sequence: 0), beta, Gc per channel (two half-chunk scans)
//   2. the decayed tiles K+, Kh, Q+ and e^{Gc_C} stored
//   3. the 10 blocks of A and Aqk on or below the block diagonal on the MFMA (block_row; wave 0:
//      row block 3 against column blocks 0, 1 and row block 0; wave 1: row block 3 against 2, 3;
//      wave 2: row block 2; wave 3: row block 1), held in registers
//   4. with the Gc table dead, the products into A's slots and the Aqk tile; a diagonal block
//      whose span is too large entry by entry (diag_exact)
//   5. T by ut_solve_store; Aqk stored in the outputs chain's fragment order
__global__ __launch_bounds__(NTH) __attribute__((amdgpu_waves_per_eu(3))) void kda_intra_kernel(KdaChunkParams p) {
  __shared__ IntraLds s;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int n = (int)(blockIdx.x % p.NT), bh = (int)(blockIdx.x / p.NT), b = bh / p.H, h = bh % p.H;
  const long P0 = (long)n * C, chunk = (long)bh * p.NT + n;
  const int valid = (int)min((long)C, (long)p.L - P0);
  const long HD = (long)p.H * DK;
  const long row0 = ((long)b * p.L + P0) * p.H + h;  // this chunk's first row of [B, L, H, .]
  const bf16* kb = static_cast<const bf16*>(p.k) + row0 * DK;
  const bf16* qb = static_cast<const bf16*>(p.q) + row0 * DK;
  const float* ab = p.a_log + row0 * DK;
  constexpr int PIECES = C * DK / 8 / NTH;  // 16-byte pieces of a 64 x 128 bf16 tile per thread
  // rows past the sequence read 0 through the buffer range check (no select waits for a load)
  const int span_rows = (int)((valid - 1) * HD + DK);
  const auto krs = buffer_rsrc(const_cast<bf16*>(kb), span_rows * 2);
  const auto qrs = buffer_rsrc(const_cast<bf16*>(qb), span_rows * 2);
  const auto ars = buffer_rsrc(const_cast<float*>(ab), span_rows * 4);

  // ---- 1. keys, beta, Gc (every thread's loads issued before its first use)
  {
    u32x4 kv[PIECES];
#pragma unroll
    for (int u = 0; u < PIECES; ++u) {
      const int idx = tid + NTH * u, r = idx >> 4, c = (idx & 15) * 8;
      kv[u] = load16_last(krs, (int)((r * HD + c) * 2));
    }
    // thread t scans channel t % 128 over rows 32 (t / 128) .. + 31; positions past the sequence
    // decay by nothing; each log decay is raised to the floor (a -inf reset then decays to
    // exactly 0 while prefix differences stay finite); NaN passes through
    const int c = tid & (DK - 1), r0 = 32 * (tid >> 7);
    float x[32];
#pragma unroll
    for (int i = 0; i < 32; ++i) {
      const float a = load4_last(ars, (int)(((r0 + i) * HD + c) * 4));
      x[i] = a < LOG_GATE_FLOOR ? LOG_GATE_FLOOR : a;
    }
    if (tid < C) s.bs[tid] = tid < valid ? p.beta[row0 + (long)tid * p.H] : 0.f;
#pragma unroll
    for (int u = 0; u < PIECES; ++u) {
      const int idx = tid + NTH * u, r = idx >> 4, cc = (idx & 15) * 8;
      *reinterpret_cast<u32x4*>(&s.Kl[r][cc]) = kv[u];
    }
    float run = 0.f;
#pragma unroll
    for (int i = 0; i < 32; ++i) {
      run += x[i];
      x[i] = run;
      if (r0 == 0) s.u.Gc[i][c] = run;
    }
    __syncthreads();
    if (r0 != 0) {  // the second half adds the first half's total
      const float base = s.u.Gc[31][c];
#pragma unroll
      for (int i = 0; i < 32; ++i) s.u.Gc[32 + i][c] = x[i] + base;
    }
  }
  __syncthreads();

  // ---- 2. K+, Kh, Q+, e^{Gc_C}
  {
    u32x4 qv[PIECES];
#pragma unroll
    for (int u = 0; u < PIECES; ++u) {
      const int idx = tid + NTH * u, r = idx >> 4, c = (idx & 15) * 8;
      qv[u] = buffer_load16(qrs, (int)((r * HD + c) * 2));
    }
#pragma unroll
    for (int u = 0; u < PIECES; ++u) {
      const int idx = tid + NTH * u, r = idx >> 4, c = (idx & 15) * 8;
      if (r >= valid) continue;
      float kx[8], qx[8], kp[8], kh[8], qp[8];
      unpack8(*reinterpret_cast<const u32x4*>(&s.Kl[r][c]), kx);
      unpack8(qv[u], qx);
#pragma unroll
      for (int e4 = 0; e4 < 8; e4 += 4) {
        const floatx4 gr = *reinterpret_cast<const floatx4*>(&s.u.Gc[r][c + e4]);
        const floatx4 gl = *reinterpret_cast<const floatx4*>(&s.u.Gc[C - 1][c + e4]);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float d = gate_exp(gr[e]);
          kp[e4 + e] = kx[e4 + e] * d;
          kh[e4 + e] = kx[e4 + e] * gate_exp(gl[e] - gr[e]);
          qp[e4 + e] = p.scale * qx[e4 + e] * d;
        }
      }
      const long off = r * HD + c;
      *reinterpret_cast<u32x4*>(static_cast<bf16*>(p.kp) + row0 * DK + off) = pack8(kp);
      *reinterpret_cast<u32x4*>(static_cast<bf16*>(p.kh) + row0 * DK + off) = pack8(kh);
      *reinterpret_cast<u32x4*>(static_cast<bf16*>(p.qp) + row0 * DK + off) = pack8(qp);
    }
    if (tid < DK) p.dC[chunk * DK + tid] = gate_exp(s.u.Gc[C - 1][tid]);
  }

  // ---- 3. A and Aqk on the MFMA, in registers (up to 3 blocks per wave)
  floatx4 gram[3], aqk[3];
  bool diag_ok;
  if (wave == 0) {
    block_row<3, 0, 2, 0>(s, qrs, HD, p.scale, gram, aqk, lane);
    block_row<0, 0, 1, 2>(s, qrs, HD, p.scale, gram, aqk, lane);
    diag_ok = diag_span_ok<0>(s, lane);
  } else if (wave == 1) {
    block_row<3, 2, 2, 0>(s, qrs, HD, p.scale, gram, aqk, lane);
    diag_ok = diag_span_ok<3>(s, lane);
  } else if (wave == 2) {
    block_row<2, 0, 3, 0>(s, qrs, HD, p.scale, gram, aqk, lane);
    diag_ok = diag_span_ok<2>(s, lane);
  } else {
    block_row<1, 0, 2, 0>(s, qrs, HD, p.scale, gram, aqk, lane);
    diag_ok = diag_span_ok<1>(s, lane);
  }
  __syncthreads();  // the Gc table is dead

  // ---- 4. A's slots and the Aqk tile (blocks above the diagonal are never read)
  if (wave == 0) {
    store_row<3, 0, 2, 0>(s, gram, aqk, true, lane);
    store_row<0, 0, 1, 2>(s, gram, aqk, diag_ok, lane);
  } else if (wave == 1) {
    store_row<3, 2, 2, 0>(s, gram, aqk, diag_ok, lane);
  } else if (wave == 2) {
    store_row<2, 0, 3, 0>(s, gram, aqk, diag_ok, lane);
  } else {
    store_row<1, 0, 2, 0>(s, gram, aqk, diag_ok, lane);
  }
  if (!diag_ok) {
    const int I = wave == 0 ? 0 : wave == 1 ? 3 : wave == 2 ? 2 : 1;
    diag_exact(s, qb, kb, ab, HD, valid, p.scale, I, lane);
  }
  __syncthreads();

  // ---- 5. T, Aqk
  ut_solve_store<C>(reinterpret_cast<float*>(s.u.a.slots), s.bs, static_cast<bf16*>(p.T) + chunk * C * C,
                    static_cast<float*>(nullptr), tid);
  // Aqk in the outputs chain's fragment order (KDA_AQK_FRAGS x 64 lanes x 16 bytes per chunk)
  u32x4* aq = reinterpret_cast<u32x4*>(static_cast<char*>(p.Aqk) + chunk * KDA_AQK_CHUNK_BYTES);
  for (int idx = tid; idx < KDA_AQK_FRAGS * 64; idx += NTH) {
    const int f = idx >> 6, g = (idx >> 4) & 3, m = idx & 15;
    const int bb = kda_aqk_block(f), kp = kda_aqk_pair(f), r = 16 * bb + m, c = 32 * kp + 4 * g;
    const u32x2 lo = *reinterpret_cast<const u32x2*>(&s.u.a.Aq[r][c]);
    const u32x2 hi = 2 * kp + 1 <= bb ? *reinterpret_cast<const u32x2*>(&s.u.a.Aq[r][c + 16]) : u32x2{0, 0};
    aq[idx] = u32x4{lo[0], lo[1], hi[0], hi[1]};
  }
}

}  // namespace kdac


hipError_t launch_kda_intra(const KdaChunkParams& p, hipStream_t st) {
  const long blocks = (long)p.B * p.H * p.NT;
  if (blocks == 0) return hipSuccess;
  hipLaunchKernelGGL(kdac::kda_intra_kernel, dim3((unsigned)blocks), dim3(kdac::NTH), 0, st, p);
  return hipGetLastError();
}

}  // namespace delta
