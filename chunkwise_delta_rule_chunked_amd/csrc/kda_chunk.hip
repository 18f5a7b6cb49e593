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
// Every exponent above is a decay from a later position back to an earlier one (<= 0), so no
// factor overflows.
//
// Four steps (delta_abi.cpp runs them):
//   kda_intra_kernel   per chunk: Gc, A and Aqk, T, and the decayed tiles K+, Kh, Q+ and the
//                      chunk decay e^{Gc_C} into the workspace;
//   the inter-chunk scan (chunk_scan.hip, KDA mode): summaries, combine, then the chain that
//                      stores each chunk's start state;
//   kda_out_kernel     per chunk, all in parallel: O from the start state.
#include "common.h"
#include "kernels.h"
#include "ut_solve.h"

namespace delta {
namespace kdac {

constexpr int DK = 128, DV = 128, C = 64, NB = C / 16;
constexpr int GP = DK + 4;  // float row pitch of the Gc table
constexpr int KP = DK + 8;  // bf16 row pitch of the key tile
constexpr int NTH = 256;

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

// Diagonal block I of A and Aqk entry by entry, with the exact per-channel factor e^{Gc_r - Gc_j}
// (j <= r, never above 1), by one wave: 16-lane group g takes the block's rows g, 7 - g, 8 + g and
// 15 - g (34 entries), lane l of the group channels 8 l .. 8 l + 7, each entry a DPP row sum.
__device__ __noinline__ void diag_exact(const float (*Gc)[GP], const bf16 (*Kl)[KP], float* As, bf16 (*Aq)[C + 8],
                                        const float* bs, const bf16* qb, long HD, int valid, float scale, int I,
                                        int lane) {
  constexpr int LDB = UtSlots<C>::LDB, BLK = UtSlots<C>::BLK;
  const int grp = lane >> 4, gl = lane & 15, c = 8 * gl;
  float* blk = As + lower_block(I, I) * BLK;
  const int rl4[4] = {grp, 7 - grp, 8 + grp, 15 - grp};
  for (int u = 0; u < 4; ++u) {
    const int rl = rl4[u], r = 16 * I + rl;
    float kr[8], qr[8], gr[8];
    unpack8(*reinterpret_cast<const u32x4*>(&Kl[r][c]), kr);
    unpack8(r < valid ? *reinterpret_cast<const u32x4*>(qb + r * HD + c) : u32x4{0, 0, 0, 0}, qr);
    *reinterpret_cast<floatx4*>(gr) = *reinterpret_cast<const floatx4*>(&Gc[r][c]);
    *reinterpret_cast<floatx4*>(gr + 4) = *reinterpret_cast<const floatx4*>(&Gc[r][c + 4]);
    for (int jl = 0; jl <= rl; ++jl) {
      const int j = 16 * I + jl;
      float kj[8], gj[8];
      unpack8(*reinterpret_cast<const u32x4*>(&Kl[j][c]), kj);
      *reinterpret_cast<floatx4*>(gj) = *reinterpret_cast<const floatx4*>(&Gc[j][c]);
      *reinterpret_cast<floatx4*>(gj + 4) = *reinterpret_cast<const floatx4*>(&Gc[j][c + 4]);
      float sg = 0.f, sq = 0.f;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float kd = kj[e] * gate_exp(gr[e] - gj[e]);
        sg += kr[e] * kd;
        sq += qr[e] * kd;
      }
      sg = row_sum16(sg);
      sq = row_sum16(sq);
      if (gl == 0) {
        if (jl < rl) blk[rl * LDB + jl] = bs[r] * sg;
        Aq[r][j] = (bf16)(scale * sq);
      }
    }
  }
}

// Largest per-channel decay span (Gc at the row before a 16-row block minus Gc at its last row) for
// which the block's diagonal entries are taken on the MFMA: its B factors reach e^{span}, its A
// factors e^{-span}, both far inside float32's normal range.
constexpr float DIAG_SPAN = 64.f;

// The entries of row block I of A and Aqk against column blocks J0 .. J0 + NJ - 1 (J <= I), each a
// 16 x 16 product over d_k on the fp32 MFMA.  The reference is the row just before the block,
// rho = 16 I - 1 (Gc_rho = 0 for I = 0): the A operand is k_r e^{Gc_r - Gc_rho} (scale q_r e^{...}
// for Aqk), the B operand k_j e^{Gc_rho - Gc_j}.  Below the diagonal block (j <= rho) both factors
// are decays (<= 1; a product that underflows is below either factor); on the diagonal block the
// B factor is a growth bounded by e^{span}, so that block takes this route only when every
// channel's span is within DIAG_SPAN (NaN is not), else diag_exact below.  The contraction over
// d_k is permuted alike in both operands: lane group g takes channels 32 g .. 32 g + 31, one per
// 4-deep step.  Results go to the A slots (times beta of the row; the diagonal block's entries
// j < r) and to the Aqk tile (j <= r; above the diagonal it keeps its zeros).
template <int NJ>
__device__ __forceinline__ void block_row(const float (*Gc)[GP], const bf16 (*Kl)[KP], float* As, bf16 (*Aq)[C + 8],
                                          const float* bs, const bf16* qb, long HD, int valid, float scale, int I,
                                          int J0, int lane) {
  constexpr int LDB = UtSlots<C>::LDB, BLK = UtSlots<C>::BLK;
  const int g4 = lane >> 4, m = lane & 15, ra = 16 * I + m, rho = 16 * I - 1, c0 = 32 * g4;
  const bool has_diag = J0 + NJ - 1 == I;
  bool diag_ok = true;
  if (has_diag) {
    const int e = 16 * I + 15;
    const float s0 = (rho >= 0 ? Gc[rho][lane] : 0.f) - Gc[e][lane];
    const float s1 = (rho >= 0 ? Gc[rho][lane + 64] : 0.f) - Gc[e][lane + 64];
    diag_ok = __all(s0 <= DIAG_SPAN && s1 <= DIAG_SPAN);
  }
  float qa[32];
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const u32x4 x = ra < valid ? *reinterpret_cast<const u32x4*>(qb + ra * HD + c0 + 8 * u) : u32x4{0, 0, 0, 0};
    unpack8(x, qa + 8 * u);
  }
  floatx4 gram[NJ], aqk[NJ];
#pragma unroll
  for (int t = 0; t < NJ; ++t) gram[t] = aqk[t] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll 2
  for (int s4 = 0; s4 < 32; s4 += 4) {
    const int c = c0 + s4;
    const floatx4 ga = *reinterpret_cast<const floatx4*>(&Gc[ra][c]);
    const floatx4 gr = rho >= 0 ? *reinterpret_cast<const floatx4*>(&Gc[rho][c]) : floatx4{0.f, 0.f, 0.f, 0.f};
    const bf16x4 ka = *reinterpret_cast<const bf16x4*>(&Kl[ra][c]);
    floatx4 gb[NJ];
    bf16x4 kb[NJ];
#pragma unroll
    for (int t = 0; t < NJ; ++t) {
      gb[t] = *reinterpret_cast<const floatx4*>(&Gc[16 * (J0 + t) + m][c]);
      kb[t] = *reinterpret_cast<const bf16x4*>(&Kl[16 * (J0 + t) + m][c]);
    }
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const float ea = gate_exp(ga[s] - gr[s]), av = (float)ka[s] * ea, aq = scale * qa[s4 + s] * ea;
#pragma unroll
      for (int t = 0; t < NJ; ++t) {
        const float bv = (float)kb[t][s] * gate_exp(gr[s] - gb[t][s]);
        gram[t] = __builtin_amdgcn_mfma_f32_16x16x4f32(av, bv, gram[t], 0, 0, 0);
        aqk[t] = __builtin_amdgcn_mfma_f32_16x16x4f32(aq, bv, aqk[t], 0, 0, 0);
      }
    }
  }
  // lane (g, m) holds rows 4 g .. 4 g + 3 of column m of each block
#pragma unroll
  for (int t = 0; t < NJ; ++t) {
    const int J = J0 + t;
    if (J == I && !diag_ok) continue;
    float* blk = As + lower_block(I, J) * BLK;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int rl = 4 * g4 + j, r = 16 * I + rl;
      if (J < I || m < rl) blk[rl * LDB + m] = bs[r] * gram[t][j];
      if (J < I || m <= rl) Aq[r][16 * J + m] = (bf16)aqk[t][j];
    }
  }
  if (has_diag && !diag_ok) diag_exact(Gc, Kl, As, Aq, bs, qb, HD, valid, scale, I, lane);
}

// One workgroup of 4 wavefronts per (sequence, head, chunk).
//   1. keys to LDS (rows past the sequence: 0), beta, Gc per channel (two half-chunk scans)
//   2. the 10 blocks of A and Aqk on or below the block diagonal by row block (block_row), the
//      diagonal blocks whose decay span is too large for it entry by entry (diag_exact)
//   3. T by ut_solve_store; Aqk, K+, Kh, Q+ and e^{Gc_C} stored
__global__ __launch_bounds__(NTH) void kda_intra_kernel(KdaChunkParams p) {
  __shared__ __attribute__((aligned(16))) float Gc[C][GP];
  __shared__ __attribute__((aligned(16))) bf16 Kl[C][KP];
  __shared__ __attribute__((aligned(16))) bf16 Aq[C][C + 8];  // Aqk staged for 16-byte stores
  __shared__ __attribute__((aligned(16))) unsigned char slots[UtSlots<C>::BYTES];
  __shared__ __attribute__((aligned(16))) float bs[C];
  float* As = reinterpret_cast<float*>(slots);

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int n = (int)(blockIdx.x % p.NT), bh = (int)(blockIdx.x / p.NT), b = bh / p.H, h = bh % p.H;
  const long P0 = (long)n * C, chunk = (long)bh * p.NT + n;
  const int valid = (int)min((long)C, (long)p.L - P0);
  const long HD = (long)p.H * DK;
  const long row0 = ((long)b * p.L + P0) * p.H + h;  // this chunk's first row of [B, L, H, .]
  const bf16* kb = static_cast<const bf16*>(p.k) + row0 * DK;
  const bf16* qb = static_cast<const bf16*>(p.q) + row0 * DK;
  const float* ab = p.a_log + row0 * DK;

  // ---- 1. keys, beta, Gc (every thread's loads issued before its first use)
  {
    u32x4 kv[C * DK / 8 / NTH];
#pragma unroll
    for (int u = 0; u < C * DK / 8 / NTH; ++u) {
      const int idx = tid + NTH * u, r = idx >> 4, c = (idx & 15) * 8;
      kv[u] = r < valid ? *reinterpret_cast<const u32x4*>(kb + r * HD + c) : u32x4{0, 0, 0, 0};
    }
    // thread t scans channel t % 128 over rows 32 (t / 128) .. + 31; positions past the sequence
    // decay by nothing; each log decay is raised to the floor (a -inf reset then decays to
    // exactly 0 while prefix differences stay finite); NaN passes through
    const int c = tid & (DK - 1), r0 = 32 * (tid >> 7);
    float x[32];
#pragma unroll
    for (int i = 0; i < 32; ++i) {
      const int r = r0 + i;
      const float a = r < valid ? ab[r * HD + c] : 0.f;
      x[i] = a < LOG_GATE_FLOOR ? LOG_GATE_FLOOR : a;
    }
    if (tid < C) bs[tid] = tid < valid ? p.beta[row0 + (long)tid * p.H] : 0.f;
#pragma unroll
    for (int u = 0; u < C * DK / 8 / NTH; ++u) {
      const int idx = tid + NTH * u, r = idx >> 4, cc = (idx & 15) * 8;
      *reinterpret_cast<u32x4*>(&Kl[r][cc]) = kv[u];
      *reinterpret_cast<u32x4*>(&Aq[r][cc & 63]) = u32x4{0, 0, 0, 0};  // Aqk starts as zeros
    }
    float run = 0.f;
#pragma unroll
    for (int i = 0; i < 32; ++i) {
      run += x[i];
      x[i] = run;
      if (r0 == 0) Gc[i][c] = run;
    }
    __syncthreads();
    if (r0 != 0) {  // the second half adds the first half's total
      const float base = Gc[31][c];
#pragma unroll
      for (int i = 0; i < 32; ++i) Gc[32 + i][c] = x[i] + base;
    }
  }
  __syncthreads();

  // ---- 2. A and Aqk by 16-row blocks (block_row); wave w: w = 0 row block 3
  // against column blocks 0, 1 and row block 0; w = 1 row block 3 against 2, 3; w = 2 row block 2;
  // w = 3 row block 1 (3, 2, 3 and 2 blocks)
  if (wave == 0) {
    block_row<2>(Gc, Kl, As, Aq, bs, qb, HD, valid, p.scale, 3, 0, lane);
    block_row<1>(Gc, Kl, As, Aq, bs, qb, HD, valid, p.scale, 0, 0, lane);
  } else if (wave == 1) {
    block_row<2>(Gc, Kl, As, Aq, bs, qb, HD, valid, p.scale, 3, 2, lane);
  } else if (wave == 2) {
    block_row<3>(Gc, Kl, As, Aq, bs, qb, HD, valid, p.scale, 2, 0, lane);
  } else {
    block_row<2>(Gc, Kl, As, Aq, bs, qb, HD, valid, p.scale, 1, 0, lane);
  }
  __syncthreads();

  // ---- 3. T, Aqk, K+, Kh, Q+, e^{Gc_C}
  ut_solve_store<C>(As, bs, static_cast<bf16*>(p.T) + chunk * C * C, static_cast<float*>(nullptr), tid);
  bf16* aq = static_cast<bf16*>(p.Aqk) + chunk * C * C;
  for (int idx = tid; idx < C * C / 8; idx += NTH) {
    const int r = idx >> 3, c = (idx & 7) * 8;
    *reinterpret_cast<u32x4*>(aq + r * C + c) = *reinterpret_cast<const u32x4*>(&Aq[r][c]);
  }
  u32x4 qv[C * DK / 8 / NTH];
#pragma unroll
  for (int u = 0; u < C * DK / 8 / NTH; ++u) {
    const int idx = tid + NTH * u, r = idx >> 4, c = (idx & 15) * 8;
    qv[u] = r < valid ? *reinterpret_cast<const u32x4*>(qb + r * HD + c) : u32x4{0, 0, 0, 0};
  }
#pragma unroll
  for (int u = 0; u < C * DK / 8 / NTH; ++u) {
    const int idx = tid + NTH * u, r = idx >> 4, c = (idx & 15) * 8;
    if (r >= valid) continue;
    float kx[8], qx[8], kp[8], kh[8], qp[8];
    unpack8(*reinterpret_cast<const u32x4*>(&Kl[r][c]), kx);
    unpack8(qv[u], qx);
#pragma unroll
    for (int e4 = 0; e4 < 8; e4 += 4) {
      const floatx4 gr = *reinterpret_cast<const floatx4*>(&Gc[r][c + e4]);
      const floatx4 gl = *reinterpret_cast<const floatx4*>(&Gc[C - 1][c + e4]);
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
  if (tid < DK) p.dC[chunk * DK + tid] = gate_exp(Gc[C - 1][tid]);
}

// ------------------------------------------------------------------------------------------
// Outputs, one workgroup of 8 wavefronts per chunk, from the chunk's start state S (bf16,
// transposed [d_v][d_k], as the scan stored it): per quarter of 32 value columns
//     Y = V - K+ S;  V~ = T Y;  O = Q+ S + Aqk V~,
// wavefront w owning the 16 x 16 tile (rows 16 (w / 2), columns 16 (w % 2)) of each.  O is formed
// transposed (the operands of both products swapped), so a lane holds 4 consecutive columns of
// one row and stores them with one 8-byte write.  Fragment layouts (16x16x32 bf16): lane (g, i)
// holds A[i][8g .. 8g+7], B[8g .. 8g+7][i], D[4g .. 4g+3][i].
constexpr int QC = 32, NW = 8, NTO = NW * WAVE;
using L128 = TileLayout<bf16, 128>;
using L64 = TileLayout<bf16, 64>;
using L32 = TileLayout<bf16, QC>;

__device__ inline bf16x8 frag_rows(const Tile<bf16>& t, int r0, int k0, int lane) {
  return *reinterpret_cast<const bf16x8*>(t.at(r0 + (lane & 15), k0 + 8 * (lane >> 4)));
}
__device__ inline bf16x8 frag_cols(const Tile<bf16>& t, int k0, int c0, int lane) {
  const int g = lane >> 4, i = lane & 15;
  const int r = k0 + 8 * g + (i >> 2), e = c0 + 4 * (i & 3);
  const bf16x4 lo = read_tr4(t.at(r, e)), hi = read_tr4(t.at(r + 4, e));
  return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
}
__device__ inline floatx4 mma(bf16x8 a, bf16x8 b, floatx4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

struct __attribute__((aligned(16))) OutLds {
  bf16 Q[C * L128::LD], K[C * L128::LD];  // Q+, K+
  bf16 T[C * L64::LD], A[C * L64::LD];    // T, Aqk
  bf16 S[QC * L128::LD];                  // this quarter of S^T
  bf16 V[C * L32::LD], Y[C * L32::LD], Vt[C * L32::LD];
};

__global__ __launch_bounds__(NTO) void kda_out_kernel(KdaChunkParams p) {
  __shared__ OutLds s;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, g4 = lane >> 4, m = lane & 15;
  const int n = (int)(blockIdx.x % p.NT), bh = (int)(blockIdx.x / p.NT), b = bh / p.H, h = bh % p.H;
  const long P0 = (long)n * C, chunk = (long)bh * p.NT + n;
  const int valid = (int)min((long)C, (long)p.L - P0);
  const long HD = (long)p.H * DK;
  const long row0 = ((long)b * p.L + P0) * p.H + h;
  const Tile<bf16> Qt{s.Q, L128::LD, L128::MASK}, Kt{s.K, L128::LD, L128::MASK}, St{s.S, L128::LD, L128::MASK};
  const Tile<bf16> Tt{s.T, L64::LD, L64::MASK}, At{s.A, L64::LD, L64::MASK};
  const Tile<bf16> Vq{s.V, L32::LD, L32::MASK}, Yq{s.Y, L32::LD, L32::MASK}, Vtq{s.Vt, L32::LD, L32::MASK};
  const bf16* qp = static_cast<const bf16*>(p.qp) + row0 * DK;
  const bf16* kp = static_cast<const bf16*>(p.kp) + row0 * DK;
  const bf16* vb = static_cast<const bf16*>(p.v) + row0 * DV;
  const bf16* Sn = static_cast<const bf16*>(p.Sn) + chunk * DV * DK;

  // Q+, K+ (rows past the sequence: 0), T, Aqk
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    const int idx = tid + NTO * u, r = idx >> 4, c = (idx & 15) * 8;
    const bool ok = r < valid;
    *reinterpret_cast<u32x4*>(Qt.at(r, c)) = ok ? *reinterpret_cast<const u32x4*>(qp + r * HD + c) : u32x4{0, 0, 0, 0};
    *reinterpret_cast<u32x4*>(Kt.at(r, c)) = ok ? *reinterpret_cast<const u32x4*>(kp + r * HD + c) : u32x4{0, 0, 0, 0};
  }
  {
    const int r = tid >> 3, c = (tid & 7) * 8;
    *reinterpret_cast<u32x4*>(Tt.at(r, c)) =
        *reinterpret_cast<const u32x4*>(static_cast<const bf16*>(p.T) + chunk * C * C + r * C + c);
    *reinterpret_cast<u32x4*>(At.at(r, c)) =
        *reinterpret_cast<const u32x4*>(static_cast<const bf16*>(p.Aqk) + chunk * C * C + r * C + c);
  }
  const int rb = wave >> 1, ct = wave & 1;
  bf16* Ob = static_cast<bf16*>(p.O) + row0 * DV;
#pragma unroll 1
  for (int q = 0; q < DV / QC; ++q) {
    const int c0 = QC * q;
    // this quarter of S^T (32 d_v rows x 128 d_k) and of V (64 rows x 32 columns)
    {
      const int r = tid >> 4, c = (tid & 15) * 8;
      *reinterpret_cast<u32x4*>(St.at(r, c)) = *reinterpret_cast<const u32x4*>(Sn + (c0 + r) * DK + c);
      if (tid < C * QC / 8) {
        const int rv = tid >> 2, cv = (tid & 3) * 8;
        *reinterpret_cast<u32x4*>(Vq.at(rv, cv)) =
            rv < valid ? *reinterpret_cast<const u32x4*>(vb + rv * p.H * DV + c0 + cv) : u32x4{0, 0, 0, 0};
      }
    }
    __syncthreads();
    // Y = V - K+ S (contract d_k)
    {
      floatx4 ks = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int k0 = 0; k0 < DK; k0 += 32) ks = mma(frag_rows(Kt, 16 * rb, k0, lane), frag_rows(St, 16 * ct, k0, lane), ks);
      const bf16x4 v4 = read_tr4(Vq.at(16 * rb + 4 * g4 + (m >> 2), 16 * ct + 4 * (m & 3)));
#pragma unroll
      for (int j = 0; j < 4; ++j) *Yq.at(16 * rb + 4 * g4 + j, 16 * ct + m) = (bf16)((float)v4[j] - ks[j]);
    }
    __syncthreads();
    // V~ = T Y (T zero above the diagonal)
    {
      floatx4 vt = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int k0 = 0; k0 < C; k0 += 32)
        if (k0 <= 16 * rb) vt = mma(frag_rows(Tt, 16 * rb, k0, lane), frag_cols(Yq, k0, 16 * ct, lane), vt);
#pragma unroll
      for (int j = 0; j < 4; ++j) *Vtq.at(16 * rb + 4 * g4 + j, 16 * ct + m) = (bf16)vt[j];
    }
    __syncthreads();
    // O^T tile (value columns 16 ct .., rows 16 rb ..) = S^T Q+^T + V~^T Aqk^T (Aqk zero above the diagonal)
    {
      floatx4 o = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int k0 = 0; k0 < DK; k0 += 32) o = mma(frag_rows(St, 16 * ct, k0, lane), frag_rows(Qt, 16 * rb, k0, lane), o);
#pragma unroll
      for (int k0 = 0; k0 < C; k0 += 32)
        if (k0 <= 16 * rb) o = mma(frag_cols(Vtq, k0, 16 * ct, lane), frag_rows(At, 16 * rb, k0, lane), o);
      const int row = 16 * rb + m;
      if (row < valid)
        *reinterpret_cast<bf16x4*>(Ob + (long)row * p.H * DV + c0 + 16 * ct + 4 * g4) =
            bf16x4{(bf16)o[0], (bf16)o[1], (bf16)o[2], (bf16)o[3]};
    }
    __syncthreads();  // the quarter's tiles are rewritten next
  }
}

}  // namespace kdac


hipError_t launch_kda_intra(const KdaChunkParams& p, hipStream_t st) {
  const long blocks = (long)p.B * p.H * p.NT;
  if (blocks == 0) return hipSuccess;
  hipLaunchKernelGGL(kdac::kda_intra_kernel, dim3((unsigned)blocks), dim3(kdac::NTH), 0, st, p);
  return hipGetLastError();
}

hipError_t launch_kda_out(const KdaChunkParams& p, hipStream_t st) {
  const long blocks = (long)p.B * p.H * p.NT;
  if (blocks == 0) return hipSuccess;
  hipLaunchKernelGGL(kdac::kda_out_kernel, dim3((unsigned)blocks), dim3(kdac::NTO), 0, st, p);
  return hipGetLastError();
}

}  // namespace delta
