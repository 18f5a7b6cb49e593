// Per-chunk gradients of the backward pass on MFMA, for bf16 inputs with d_k = d_v = 128 and
// chunk 64 (other shapes use bwd_chunk_kernel in backward.hip, whose header states the
// gradients; this kernel evaluates the same formulas).  Per chunk, with N = (I + A)^-1,
// T = N diag(beta), gamma = exp(gc), w = exp(gc_C - gc), Gam_ij = exp(gc_i - gc_j) (j <= i), the
// chunk's start state S and the gradient G' of its end state:
//   KS = K S, KG = K G';  Y = V - gamma KS;  V~ = T Y
//   dV~ = w KG + P^T dO  (P = Q K^T * Gam, on and below the diagonal);  dY = T^T dV~
//   dT = dV~ Y^T, dOV = dO V~^T                        (sums over the value dimension)
//   dQ = gamma (dO S^T) + E1 K,  dK = w (V~ G'^T) - gamma (dY S^T) + E1^T Q + (dGm + dGm^T) K
// with E1 = Gam * dOV and dGm from the chunk-local C x C algebra (dA = -strictLower(N^T dT T^T),
// dGm = diag(beta) (Gam * dA)), and the gate-prefix and beta gradients from the same algebra.
// Two row sums over the value dimension that the algebra needs follow from the accumulated
// products: sum_c QS_ic dO_ic = Q_i . (dO S^T)_i, sum_c KS_ic dY_ic = K_i . (dY S^T)_i and
// sum_c KG_ic V~_ic = K_i . (V~ G'^T)_i.
//
// One workgroup of 8 wavefronts per chunk.  K, Q, V, dO (bf16), N (float32), T and P (bf16)
// are staged in LDS; the value dimension is taken in quarters of 32 columns, the next quarter's
// S and G' loaded into registers while the current one is computed.  Per quarter wavefront w owns
// the 16 x 16 tile (rows 16 (w / 2), columns 16 (w % 2)) of KS, KG, Y, V~, dV~ and dY, and
// accumulates 16 output tiles of the products that sum over the value dimension (two of dT and
// dOV, and the tiles of column block w of d_k for dO S^T, V~ G'^T, dY S^T) across the quarters.
// Products on the 16x16x32 bf16 MFMA with float32 accumulation; the C x C algebra in float32
// on the vector ALUs.
#include "common.h"
#include "kernels.h"

namespace delta {
namespace bwdm {

constexpr int C = 64, DK = 128, DV = 128, QC = 32, NW = 8, NTH = NW * WAVE;
constexpr int PC = C + 4;  // float row pitch of the C x C float32 matrices

// A 16x16x32 fragment from a tile stored with the contraction index along its rows ([n][k] for
// a B operand, [m][k] for an A operand): lane (g, i) takes row r0 + i, elements k0 + 8 g .. + 7.
__device__ inline bf16x8 frag_rows(const Tile<bf16>& t, int r0, int k0, int lane) {
  return *reinterpret_cast<const bf16x8*>(t.at(r0 + (lane & 15), k0 + 8 * (lane >> 4)));
}
// A 16x16x32 fragment from a tile stored with the contraction index down its columns ([k][n]
// for a B operand; for an A operand the tile is the transpose, [k][m]): lane (g, i) takes
// column c0 + i, elements k0 + 8 g .. + 7, by two transpose reads.
__device__ inline bf16x8 frag_cols(const Tile<bf16>& t, int k0, int c0, int lane) {
  const int g = lane >> 4, i = lane & 15;
  const int r = k0 + 8 * g + (i >> 2), e = c0 + 4 * (i & 3);
  const bf16x4 lo = read_tr4(t.at(r, e)), hi = read_tr4(t.at(r + 4, e));
  return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
}
__device__ inline floatx4 mma(bf16x8 a, bf16x8 b, floatx4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
// The accumulator tile (rows r0 + 4 g .. + 3 of column c0 + i) into a bf16 tile.
__device__ inline void put_tile(const Tile<bf16>& t, int r0, int c0, floatx4 x, int lane) {
  const int g = lane >> 4, i = lane & 15;
#pragma unroll
  for (int j = 0; j < 4; ++j) *t.at(r0 + 4 * g + j, c0 + i) = (bf16)x[j];
}
template <int CTRL>
__device__ inline float dpp(float x) {
  return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x), CTRL, 0xF, 0xF, false));
}
// sum over the 16 lanes of a DPP row (quad xor 1, xor 2, half-mirror, mirror)
__device__ inline float row_sum16(float x) {
  x += dpp<0xB1>(x);
  x += dpp<0x4E>(x);
  x += dpp<0x141>(x);
  x += dpp<0x140>(x);
  return x;
}

using L128 = TileLayout<bf16, 128>;
using L64 = TileLayout<bf16, 64>;
using L32 = TileLayout<bf16, QC>;

struct __attribute__((aligned(16))) Lds {
  bf16 K[C * L128::LD], Q[C * L128::LD], V[C * L128::LD], dO[C * L128::LD];  // V, dO: then E1, Gs
  bf16 T[C * L64::LD], P[C * L64::LD];
  float N[C][PC];
  union {
    struct {
      bf16 S[QC * L128::LD], G[QC * L128::LD], Gl[QC * L128::LD];  // this quarter of S^T, G'^T (hi, lo)
      bf16 Y[C * L32::LD], Vt[C * L32::LD], dVt[C * L32::LD], dY[C * L32::LD];
    } q;
    struct {
      float R0[C][PC], R1[C][PC], R2[C][PC];
    } m;
  } u;
  float gc[C], gam[C], w[C], beta[C], dgc[C], dw[C];
  // per-wave partial row sums (Q . dO S^T, K . dY S^T, K . V~ G'^T), then the algebra's partial
  // sums per tile and of dbeta's diagonal term per wave
  float part[4][NW][C];
  float sgs[NW];
};
static_assert(sizeof(Lds) <= 160 * 1024, "LDS budget");

__global__ __launch_bounds__(NTH) void bwd_chunk_mfma_kernel(BwdParams p) {
  __shared__ Lds s;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int g4 = lane >> 4, m = lane & 15;
  const int n = (int)(blockIdx.x % p.NT), bh = (int)(blockIdx.x / p.NT), b = bh / p.H, h = bh % p.H;
  // the chunk starts at a token boundary (C is a multiple of n_h): row r is sub-step r % n_h of
  // the chunk's token r / n_h, token index tok0 + r / n_h
  const int nh = p.nh;
  const long tok0 = (long)n * (C / nh);
  const long P0 = (long)n * C, chunk = (long)bh * p.NT + n;
  const int valid = (int)min((long)C, (long)p.Lx - P0);
  const long HD = (long)p.H * DK;  // d_k == d_v: one row stride for all four tensors

  const Tile<bf16> Kt{s.K, L128::LD, L128::MASK}, Qt{s.Q, L128::LD, L128::MASK}, Vt{s.V, L128::LD, L128::MASK},
      Ot{s.dO, L128::LD, L128::MASK};
  const Tile<bf16> Tt{s.T, L64::LD, L64::MASK}, Pt{s.P, L64::LD, L64::MASK};
  const Tile<bf16> Sq{s.u.q.S, L128::LD, L128::MASK}, Gq{s.u.q.G, L128::LD, L128::MASK},
      Glq{s.u.q.Gl, L128::LD, L128::MASK};
  const Tile<bf16> Yq{s.u.q.Y, L32::LD, L32::MASK}, Vq{s.u.q.Vt, L32::LD, L32::MASK},
      dVq{s.u.q.dVt, L32::LD, L32::MASK}, dYq{s.u.q.dY, L32::LD, L32::MASK};
  // E1 and Gs = dGm + dGm^T after the value loop, in the V and dO areas
  const Tile<bf16> E1t{s.V, L64::LD, L64::MASK}, Gst{s.dO, L64::LD, L64::MASK};

  // ---- stage K, Q (scaled, rows without a readout zero), V, dO, N and the per-position scalars
  {
    const bf16* kb = static_cast<const bf16*>(p.k) + ((long)b * p.Lx + P0) * HD + (long)h * DK;
    const bf16* vb = static_cast<const bf16*>(p.v) + ((long)b * p.Lx + P0) * HD + (long)h * DV;
    const bf16* qb = static_cast<const bf16*>(p.q) + (long)b * p.L * HD + (long)h * DK;
    const bf16* ob = static_cast<const bf16*>(p.dO) + (long)b * p.L * HD + (long)h * DV;
    u32x4 rk[2], rv[2], rq[2], ro[2];
    floatx4 rn[2];
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int idx = tid + NTH * u, r = idx >> 4, c = (idx & 15) * 8;
      const int rt = r / nh;
      const bool ok = r < valid, last = ok && r - rt * nh == nh - 1;
      const long tok = tok0 + rt;
      rk[u] = ok ? *reinterpret_cast<const u32x4*>(kb + r * HD + c) : u32x4{0, 0, 0, 0};
      rv[u] = ok ? *reinterpret_cast<const u32x4*>(vb + r * HD + c) : u32x4{0, 0, 0, 0};
      rq[u] = last ? *reinterpret_cast<const u32x4*>(qb + tok * HD + c) : u32x4{0, 0, 0, 0};
      ro[u] = last ? *reinterpret_cast<const u32x4*>(ob + tok * HD + c) : u32x4{0, 0, 0, 0};
      const int rr = idx >> 4, cc = (idx & 15) * 4;  // N: 64 rows of 16 float4
      rn[u] = *reinterpret_cast<const floatx4*>(p.N + chunk * C * C + rr * C + cc);
    }
    if (tid < C) {
      const float g = p.gc[chunk * C + tid], gC = p.gc[chunk * C + C - 1];
      s.gc[tid] = g;
      s.gam[tid] = expf(g);
      s.w[tid] = expf(gC - g);
      s.beta[tid] = tid < valid ? p.beta[(b * (long)p.Lx + P0 + tid) * p.H + h] : 0.f;
    }
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int idx = tid + NTH * u, r = idx >> 4, c = (idx & 15) * 8;
      *reinterpret_cast<u32x4*>(Kt.at(r, c)) = rk[u];
      *reinterpret_cast<u32x4*>(Vt.at(r, c)) = rv[u];
      *reinterpret_cast<u32x4*>(Ot.at(r, c)) = ro[u];
      // q scaled by the readout scale
      bf16x8 qv = __builtin_bit_cast(bf16x8, rq[u]);
#pragma unroll
      for (int e = 0; e < 8; ++e) qv[e] = (bf16)((float)qv[e] * p.scale);
      *reinterpret_cast<bf16x8*>(Qt.at(r, c)) = qv;
      const int rr = idx >> 4, cc = (idx & 15) * 4;
      *reinterpret_cast<floatx4*>(&s.N[rr][cc]) = rn[u];
    }
  }
  __syncthreads();
  // T = N diag(beta) in bf16, and P = (Q K^T) * Gam on and below the diagonal (bf16), on MFMA:
  // wave w forms P blocks (w / 4 + 2 t, w % 4), t = 0, 1
  for (int idx = tid; idx < C * C; idx += NTH) {
    const int r = idx >> 6, c = idx & 63;
    *Tt.at(r, c) = (bf16)(c <= r ? s.N[r][c] * s.beta[c] : 0.f);
  }
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    const int bi = wave / 4 + 2 * t, bj = wave % 4;
    floatx4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int k0 = 0; k0 < DK; k0 += 32) acc = mma(frag_rows(Qt, 16 * bi, k0, lane), frag_rows(Kt, 16 * bj, k0, lane), acc);
    const int c = 16 * bj + m;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int r = 16 * bi + 4 * g4 + j;
      acc[j] = c <= r ? acc[j] * gate_exp(s.gc[r] - s.gc[c]) : 0.f;
    }
    put_tile(Pt, 16 * bi, 16 * bj, acc, lane);
  }

  // ---- the value dimension in quarters
  // this wave's tile of the quarter: rows 16 rb, columns 16 ct of the quarter
  const int rb = wave >> 1, ct = wave & 1;
  // accumulators over the quarters: dT and dOV tiles (rows 16 (w / 4 + 2 t), columns 16 (w % 4)),
  // and column block w of d_k for dQraw = dO S^T, A1 = V~ G'^T, A2 = dY S^T (all 4 row blocks)
  floatx4 aT[2], aO[2], aQ[4], a1[4], a2[4];
#pragma unroll
  for (int t = 0; t < 2; ++t) aT[t] = aO[t] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int r = 0; r < 4; ++r) aQ[r] = a1[r] = a2[r] = floatx4{0.f, 0.f, 0.f, 0.f};
  float sgs = 0.f;
  // S^T and G'^T quarters (bf16, as the scans stored them, G' with its low part): 32 d_v rows x
  // 128 d_k each, one 16-byte piece per thread each
  u32x4 ps, pg, pgl;
  const bf16* Sn = static_cast<const bf16*>(p.Snt) + chunk * DV * DK;
  const bf16* Gn = static_cast<const bf16*>(p.Gnt) + chunk * DV * DK;
  const bf16* Gnl = static_cast<const bf16*>(p.Gntl) + chunk * DV * DK;
  const int fr = tid >> 4, fc = (tid & 15) * 8;
  auto fetch = [&](int q) {
    ps = *reinterpret_cast<const u32x4*>(Sn + (QC * q + fr) * DK + fc);
    pg = *reinterpret_cast<const u32x4*>(Gn + (QC * q + fr) * DK + fc);
    pgl = *reinterpret_cast<const u32x4*>(Gnl + (QC * q + fr) * DK + fc);
  };
  fetch(0);
#pragma unroll 1
  for (int q = 0; q < DV / QC; ++q) {
    // lane-derived offsets are formed again in every quarter from a lane index the optimiser
    // cannot see through (kept live across the loop, they spill)
    int lq = lane;
    asm volatile("" : "+v"(lq));
    const int mq = lq & 15, gq = lq >> 4, frq = (lq + WAVE * wave) >> 4, fcq = (lq & 15) * 8;
    __syncthreads();  // the previous quarter's tiles are no longer read
    *reinterpret_cast<u32x4*>(Sq.at(frq, fcq)) = ps;
    *reinterpret_cast<u32x4*>(Gq.at(frq, fcq)) = pg;
    *reinterpret_cast<u32x4*>(Glq.at(frq, fcq)) = pgl;
    {
      const bf16x8 sv = __builtin_bit_cast(bf16x8, ps), gv = __builtin_bit_cast(bf16x8, pg),
                   gl = __builtin_bit_cast(bf16x8, pgl);
#pragma unroll
      for (int e = 0; e < 8; ++e) sgs += (float)sv[e] * ((float)gv[e] + (float)gl[e]);
    }
    if (q + 1 < DV / QC) fetch(q + 1);  // in flight during this quarter
    __syncthreads();
    const int c0 = QC * q;
    // KS and KG (contract d_k), then Y = V - gamma KS
    floatx4 ks = {0.f, 0.f, 0.f, 0.f}, kg = ks;
#pragma unroll
    for (int k0 = 0; k0 < DK; k0 += 32) {
      const bf16x8 ka = frag_rows(Kt, 16 * rb, k0, lq);
      ks = mma(ka, frag_rows(Sq, 16 * ct, k0, lq), ks);
      kg = mma(ka, frag_rows(Gq, 16 * ct, k0, lq), kg);
      kg = mma(ka, frag_rows(Glq, 16 * ct, k0, lq), kg);
    }
    floatx4 y;
    {
      const bf16x4 v4 = read_tr4(Vt.at(16 * rb + 4 * gq + (mq >> 2), c0 + 16 * ct + 4 * (mq & 3)));
#pragma unroll
      for (int j = 0; j < 4; ++j) y[j] = (float)v4[j] - s.gam[16 * rb + 4 * gq + j] * ks[j];
    }
    put_tile(Yq, 16 * rb, 16 * ct, y, lq);
    __syncthreads();
    // V~ = T Y (T zero above the diagonal), dV~ = w KG + P^T dO (P^T zero below it).  T enters V~
    // as a bf16 pair (high part and rounding residual, from N and beta): the log-gate gradient
    // sums large terms that cancel between the V~ products and the N-based algebra, and a T
    // rounded to 8 bits in one of them only leaves a residue of the size of those terms.
    floatx4 vt = {0.f, 0.f, 0.f, 0.f}, dvt = vt;
#pragma unroll
    for (int k0 = 0; k0 < C; k0 += 32) {
      if (k0 <= 16 * rb) {
        const int r = 16 * rb + mq, kk = k0 + 8 * gq;
        const floatx4 n0 = *reinterpret_cast<const floatx4*>(&s.N[r][kk]);
        const floatx4 n1 = *reinterpret_cast<const floatx4*>(&s.N[r][kk + 4]);
        const floatx4 b0 = *reinterpret_cast<const floatx4*>(&s.beta[kk]);
        const floatx4 b1 = *reinterpret_cast<const floatx4*>(&s.beta[kk + 4]);
        bf16x8 th, tl;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float x = kk + e <= r ? (e < 4 ? n0[e] * b0[e] : n1[e - 4] * b1[e - 4]) : 0.f;
          th[e] = (bf16)x;
          tl[e] = (bf16)(x - (float)th[e]);
        }
        const bf16x8 yb = frag_cols(Yq, k0, 16 * ct, lq);
        vt = mma(tl, yb, mma(th, yb, vt));
      }
      if (k0 + 32 > 16 * rb)
        dvt = mma(frag_cols(Pt, k0, 16 * rb, lq), frag_cols(Ot, k0, c0 + 16 * ct, lq), dvt);
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) dvt[j] += s.w[16 * rb + 4 * gq + j] * kg[j];
    put_tile(Vq, 16 * rb, 16 * ct, vt, lq);
    put_tile(dVq, 16 * rb, 16 * ct, dvt, lq);
    __syncthreads();
    // dY = T^T dV~ (T^T zero below the diagonal)
    {
      floatx4 dy = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int k0 = 0; k0 < C; k0 += 32)
        if (k0 + 32 > 16 * rb) dy = mma(frag_cols(Tt, k0, 16 * rb, lq), frag_cols(dVq, k0, 16 * ct, lq), dy);
      put_tile(dYq, 16 * rb, 16 * ct, dy, lq);
      // dY is dv
      float* dvp = p.dv + ((long)b * p.Lx + P0) * p.H * DV + (long)h * DV + c0 + 16 * ct + mq;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int row = 16 * rb + 4 * gq + j;
        if (row < valid) dvp[(long)row * p.H * DV] = dy[j];
      }
    }
    __syncthreads();
    // the products that sum over this quarter's 32 columns (one 32-deep step each)
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      const int bi = wave / 4 + 2 * t, bj = wave % 4;
      aT[t] = mma(frag_rows(dVq, 16 * bi, 0, lq), frag_rows(Yq, 16 * bj, 0, lq), aT[t]);
      aO[t] = mma(frag_rows(Ot, 16 * bi, c0, lq), frag_rows(Vq, 16 * bj, 0, lq), aO[t]);
    }
    {
      const bf16x8 sb = frag_cols(Sq, 0, 16 * wave, lq), gb = frag_cols(Gq, 0, 16 * wave, lq),
                   gbl = frag_cols(Glq, 0, 16 * wave, lq);
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        aQ[r] = mma(frag_rows(Ot, 16 * r, c0, lq), sb, aQ[r]);
        const bf16x8 vr = frag_rows(Vq, 16 * r, 0, lq);
        a1[r] = mma(vr, gbl, mma(vr, gb, a1[r]));
        a2[r] = mma(frag_rows(dYq, 16 * r, 0, lq), sb, a2[r]);
      }
    }
  }

  // ---- row sums over the value dimension from the accumulated products (this wave: d_k block w)
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    float pq[4], pa2[4], pa1[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int row = 16 * r + 4 * g4 + j, d = 16 * wave + m;
      const float qv = (float)*Qt.at(row, d), kv = (float)*Kt.at(row, d);
      pq[j] = row_sum16(qv * aQ[r][j]);
      pa2[j] = row_sum16(kv * a2[r][j]);
      pa1[j] = row_sum16(kv * a1[r][j]);
    }
    if (m == 0) {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int row = 16 * r + 4 * g4 + j;
        s.part[0][wave][row] = pq[j];
        s.part[1][wave][row] = pa2[j];
        s.part[2][wave][row] = pa1[j];
      }
    }
  }
  {
    float x = sgs;
    for (int o = 32; o > 0; o >>= 1) x += __shfl_xor(x, o, WAVE);
    if (lane == 0) s.sgs[wave] = x;
  }
  __syncthreads();  // the quarter tiles are dead: R0..R2 overwrite them
  // dT -> R0, dOV -> R1; K K^T (strictly lower) -> R2; per-position row sums
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    const int bi = wave / 4 + 2 * t, bj = wave % 4;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      s.u.m.R0[16 * bi + 4 * g4 + j][16 * bj + m] = aT[t][j];
      s.u.m.R1[16 * bi + 4 * g4 + j][16 * bj + m] = aO[t][j];
    }
  }
  for (int t = wave; t < 10; t += NW) {  // the 10 lower 16 x 16 blocks of K K^T
    int bi = 0;
    while ((bi + 1) * (bi + 2) / 2 <= t) ++bi;
    const int bj = t - bi * (bi + 1) / 2;
    floatx4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int k0 = 0; k0 < DK; k0 += 32) acc = mma(frag_rows(Kt, 16 * bi, k0, lane), frag_rows(Kt, 16 * bj, k0, lane), acc);
#pragma unroll
    for (int j = 0; j < 4; ++j) s.u.m.R2[16 * bi + 4 * g4 + j][16 * bj + m] = acc[j];
  }
  if (tid < C) {
    float q = 0.f, k2 = 0.f, k1 = 0.f;
#pragma unroll
    for (int w = 0; w < NW; ++w) {
      q += s.part[0][w][tid];
      k2 += s.part[1][w][tid];
      k1 += s.part[2][w][tid];
    }
    s.dgc[tid] = s.gam[tid] * (q - k2);  // gamma_i (sum_c QS dO - sum_c KS dY)
    s.dw[tid] = k1;                      // sum_c KG V~
  }
  __syncthreads();

  // ---- chunk-local C x C algebra (float32).  The two C x C x C products, X = dT diag(beta) N^T
  // (= dT T^T) and dA = -strictLower(N^T X), run on the fp32 MFMA (16x16x4: lane (g, m) supplies
  // A[m][g] and B[g][m] of each 4-deep step and holds D[4 g .. 4 g + 3][m]).  The per-entry
  // terms then work on each wave's lower dA tiles in that layout; their row and column sums are
  // reduced across lanes, left per tile in LDS and summed in a fixed order.
  auto& N = s.N;
  auto& R0 = s.u.m.R0;
  auto& R1 = s.u.m.R1;
  auto& R2 = s.u.m.R2;
  auto mma4 = [](float a, float b, floatx4 acc) { return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, acc, 0, 0, 0); };
  // dbeta's diagonal term diag(N^T dT), rows 8 w .. 8 w + 7 by wave w
  {
    const int i = lane;
    float acc = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int r = 8 * wave + e;
      acc += r >= i ? N[r][i] * R0[r][i] : 0.f;
    }
    s.part[3][wave][i] = acc;
  }
  // X tiles (w / 2, w % 2) and (w / 2, 3 - w % 2), equal depth per wave (N[j][k] = 0 for k > j)
  floatx4 xt[2];
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    const int bi = wave >> 1, bj = t == 0 ? (wave & 1) : 3 - (wave & 1);
    floatx4 acc = {0.f, 0.f, 0.f, 0.f};
    for (int k0 = 0; k0 < 16 * (bj + 1); k0 += 4) {
      const int k = k0 + g4;
      acc = mma4(R0[16 * bi + m][k], s.beta[k] * N[16 * bj + m][k], acc);
    }
    xt[t] = acc;
  }
  __syncthreads();  // dT is no longer read
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    const int bi = wave >> 1, bj = t == 0 ? (wave & 1) : 3 - (wave & 1);
#pragma unroll
    for (int j = 0; j < 4; ++j) R0[16 * bi + 4 * g4 + j][16 * bj + m] = xt[t][j];
  }
  __syncthreads();
  // The 10 lower tiles of dA, tile l = (bi, bj) with l = bi (bi + 1) / 2 + bj, dealt to the waves
  // so that their depths (64 - 16 bi) even out: waves 0-6 take tile w, waves 3-5 also 12 - w.
  int tbi[2], tbj[2];
  floatx4 da[2];
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    const int l = t == 0 ? (wave < 7 ? wave : -1) : (wave >= 3 && wave <= 5 ? 12 - wave : -1);
    const int bi = l >= 6 ? 3 : l >= 3 ? 2 : l >= 1 ? 1 : 0;
    tbi[t] = l < 0 ? -1 : bi;
    tbj[t] = l - bi * (bi + 1) / 2;
    floatx4 acc = {0.f, 0.f, 0.f, 0.f};
    if (l >= 0)
      for (int k0 = 16 * bi; k0 < C; k0 += 4) {  // N[k][i] = 0 for k < i
        const int k = k0 + g4;
        acc = mma4(N[k][16 * bi + m], R0[k][16 * tbj[t] + m], acc);
      }
    da[t] = acc;
  }
  __syncthreads();  // X is no longer read
  // per entry j <= i: the gate-prefix term tg, dbeta's row term ta, dGm and E1 = Gam * dOV
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    if (tbi[t] < 0) continue;
    const int bi = tbi[t], bj = tbj[t], j = 16 * bj + m;
    float rb[4], rt[4], cs = 0.f;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int i = 16 * bi + 4 * g4 + e;
      float ta = 0.f, tg = 0.f, dGm = 0.f, e1 = 0.f;
      if (j <= i) {
        const float gm = gate_exp(s.gc[i] - s.gc[j]);
        const float dA = j < i ? -da[t][e] : 0.f, dov = R1[i][j];
        ta = dA * gm * (j < i ? R2[i][j] : 0.f);
        tg = s.beta[i] * ta + (float)*Pt.at(i, j) * dov;
        dGm = s.beta[i] * gm * dA;
        e1 = gm * dov;
      }
      R0[i][j] = dGm;  // each entry is this lane's alone
      R1[i][j] = e1;
      rb[e] = row_sum16(ta);
      rt[e] = row_sum16(tg);
      cs += tg;
    }
    // column sums of tg over the tile's rows: the lane's 4, then its column's 4 lane groups
    cs += __shfl_xor(cs, 16, WAVE);
    cs += __shfl_xor(cs, 32, WAVE);
    if (m == 0)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        s.part[0][bj][16 * bi + 4 * g4 + e] = rb[e];
        s.part[1][bj][16 * bi + 4 * g4 + e] = rt[e];
      }
    if (g4 == 0) s.part[2][bi][j] = cs;
  }
  __syncthreads();
  if (tid < C) {
    const int i = tid, bi = i >> 4;
    float dbd = 0.f, rs = 0.f, col = 0.f;
#pragma unroll
    for (int w = 0; w < NW; ++w) dbd += s.part[3][w][i];
    for (int bj = 0; bj <= bi; ++bj) {
      dbd += s.part[0][bj][i];
      rs += s.part[1][bj][i];
    }
    for (int bk = bi; bk < C / 16; ++bk) col += s.part[2][bk][i];
    s.dgc[i] += rs - col - s.w[i] * s.dw[i];
    if (i < valid) p.dbeta[(b * (long)p.Lx + P0 + i) * p.H + h] = dbd;
  }
  // E1 and Gs = dGm + dGm^T in bf16 for the last products (only the lower entries were written)
  for (int idx = tid; idx < C * C; idx += NTH) {
    const int i = idx >> 6, j = idx & 63;
    *E1t.at(i, j) = (bf16)(j <= i ? R1[i][j] : 0.f);
    *Gst.at(i, j) = (bf16)((j < i ? R0[i][j] : 0.f) + (i < j ? R0[j][i] : 0.f));
  }
  __syncthreads();
  if (wave == 0 && p.dg_log) {
    // lane i: sum over positions >= i of dgc, plus (every position) the chunk-end total
    // sum_i w_i dw_i + gamma_C sum S G'; one position per lane (C == WAVE)
    static_assert(C == WAVE, "one position per lane");
    float tot = s.w[lane] * s.dw[lane] + (lane < NW ? expf(s.gc[C - 1]) * s.sgs[lane] : 0.f);
    for (int o = 32; o > 0; o >>= 1) tot += __shfl_xor(tot, o, WAVE);
    float run = s.dgc[lane];
    for (int o = 1; o < WAVE; o <<= 1) {
      const float x = __shfl_down(run, o, WAVE);
      if (lane + o < WAVE) run += x;
    }
    const int iq = lane / nh;
    if (lane < valid && lane - iq * nh == 0) p.dg_log[(b * (long)p.L + tok0 + iq) * p.H + h] = tot + run;
  }

  // ---- dQ = gamma dQraw + E1 K, dK = w A1 - gamma A2 + E1^T Q + Gs K  (d_k block w)
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    floatx4 dq, dk;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int row = 16 * r + 4 * g4 + j;
      dq[j] = s.gam[row] * aQ[r][j];
      dk[j] = s.w[row] * a1[r][j] - s.gam[row] * a2[r][j];
    }
#pragma unroll
    for (int k0 = 0; k0 < C; k0 += 32) {
      const bf16x8 kb = frag_cols(Kt, k0, 16 * wave, lane);
      dq = mma(frag_rows(E1t, 16 * r, k0, lane), kb, dq);
      dk = mma(frag_cols(E1t, k0, 16 * r, lane), frag_cols(Qt, k0, 16 * wave, lane), dk);
      dk = mma(frag_rows(Gst, 16 * r, k0, lane), kb, dk);
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int row = 16 * r + 4 * g4 + j, d = 16 * wave + m, rq = row / nh;
      if (row >= valid) continue;
      p.dk[((b * (long)p.Lx + P0 + row) * p.H + h) * DK + d] = dk[j];
      if (row - rq * nh == nh - 1) p.dq[((b * (long)p.L + tok0 + rq) * p.H + h) * DK + d] = p.scale * dq[j];
    }
  }
}

}  // namespace bwdm

bool bwd_chunk_mfma_applies(const BwdParams& p, bool bf16_in) {
  return bf16_in && p.DK == bwdm::DK && p.DV == bwdm::DV && p.C == bwdm::C;
}

hipError_t launch_bwd_chunk_mfma(const BwdParams& p, hipStream_t st) {
  hipLaunchKernelGGL(bwdm::bwd_chunk_mfma_kernel, dim3((unsigned)((long)p.NT * p.B * p.H)), dim3(bwdm::NTH), 0, st, p);
  return hipGetLastError();
}

}  // namespace delta
