// Backward pass of the chunkwise delta rule: gradients of <O, dO> + <S_final, dS_final> with
// respect to q, k, v, beta, the log gates and S0.
//
// The pages give the forward only ("08 linear delta rule & DPLR", sections 2.2-2.3 and 3:
// per chunk Y = V - gam K S, V~ = T Y, O = (gam Q) S + (Q K^T * Gam) V~,
// S' = gam_C S + K^T (w V~), w = gam_C / gam, T = (I + A)^-1 diag(beta),
// A = strictLower(diag(beta) (Gam * K K^T))).  The gradients below are that forward
// differentiated by hand, chunk by chunk; with N = (I + A)^-1 and G' the state gradient
// after a chunk:
//   dV~ = w (K G') + (Q K^T * Gam)^T dO            dY = T^T dV~ = dV
//   G   = gam_C G' - K^T (gam dY) + (gam Q)^T dO   (state gradient before the chunk)
//   dT  = dV~ Y^T,  dA = -strictLower(N^T dT T^T),  dGm = diag(beta) (Gam * dA)
//   dQ  = gam (dO S^T) + (Gam * dO V~^T) K
//   dK  = -gam (dY S^T) + w (V~ G'^T) + (Gam * dO V~^T)^T Q + (dGm + dGm^T) K
//   dbeta = diag(N^T dT) + rowsum(dA * Gam * K K^T)
// and every factor that depends on the in-chunk log-gate prefix gc adds to dgc, whose reverse
// cumulative sum within the chunk is the log-gate gradient (taken at each token's first
// sub-step).  Q and dO rows exist only at a token's last sub-step (DeltaProduct notes,
// section 4.1); the readout scale is folded into Q.
//
// Four launches follow the intra-chunk launch (which leaves T in float32 and gc in the
// workspace):
//   bwd_qk_kernel        one workgroup per (head, chunk): P = Q K^T * Gam (lower) into the
//                        workspace
//   bwd_states_kernel    one workgroup per (head, 16 state columns), chunks in order: stores
//                        each chunk's start state S_n
//   bwd_dstates_kernel   same split, chunks in reverse: stores each chunk's end-state gradient
//                        G'_n, writes dV and dS0
//   bwd_chunk_kernel     one workgroup per (head, chunk): everything that sums over the value
//                        dimension (streamed in 16-column tiles of S_n and G'_n), then the
//                        chunk-local C x C algebra, writes dq, dk, dbeta, dlog g
// All arithmetic is float32 on the vector ALUs.
#include <hip/hip_runtime.h>

#include "common.h"
#include "kernels.h"

namespace delta {
namespace {

constexpr int CM = 64;   // largest chunk
constexpr int NTH = 256; // threads per workgroup
constexpr int NTC = 512; // threads per workgroup of the per-chunk gradient kernel

// Eight bf16 or four floats of a 16-byte vector, as floats.
template <typename E>
__device__ inline void unpack16(u32x4 r, float* x);
template <>
__device__ inline void unpack16<bf16>(u32x4 r, float* x) {
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    x[2 * e] = __uint_as_float(r[e] << 16);
    x[2 * e + 1] = __uint_as_float(r[e] & 0xffff0000u);
  }
}
template <>
__device__ inline void unpack16<float>(u32x4 r, float* x) {
#pragma unroll
  for (int e = 0; e < 4; ++e) x[e] = __uint_as_float(r[e]);
}

// A tile of up to MAXR rows x WIDTH elements of E, moved in 16-byte vectors: issue() fetches
// every vector of the calling thread into registers (all loads in flight together), commit()
// later unpacks them into a float LDS tile.  rowptr(i) gives row i's first element, or nullptr
// for a row of zeros.
template <typename E, int WIDTH, int MAXR, int NTHR = NTH>
struct RowTile {
  static constexpr int VE = 16 / (int)sizeof(E), VPR = WIDTH / VE;
  static constexpr int NV = (MAXR * VPR + NTHR - 1) / NTHR;
  u32x4 r[NV];
  template <typename F>
  __device__ inline void issue(F rowptr, int tid) {
#pragma unroll
    for (int u = 0; u < NV; ++u) {
      const int idx = tid + NTHR * u, i = idx / VPR, j = (idx % VPR) * VE;
      const E* q = i < MAXR ? rowptr(i) : nullptr;
      r[u] = q ? *reinterpret_cast<const u32x4*>(q + j) : u32x4{0, 0, 0, 0};
    }
  }
  template <int PITCH, bool TRANSPOSE = false>
  __device__ inline void commit(float (*dst)[PITCH], int rows, int tid, float mul = 1.f) const {
#pragma unroll
    for (int u = 0; u < NV; ++u) {
      const int idx = tid + NTHR * u, i = idx / VPR, j = (idx % VPR) * VE;
      if (i < rows) {
        float x[VE];
        unpack16<E>(r[u], x);
#pragma unroll
        for (int e = 0; e < VE; ++e) {
          if (TRANSPOSE)
            dst[j + e][i] = mul * x[e];
          else
            dst[i][j + e] = mul * x[e];
        }
      }
    }
  }
};

// A C x C float matrix stored contiguously (C <= CM), moved the same way.
template <int NTHR = NTH>
struct SquareTile {
  static constexpr int NV = CM * CM / 4 / NTHR;
  u32x4 r[NV];
  __device__ inline void issue(const float* src, int C, int tid) {
#pragma unroll
    for (int u = 0; u < NV; ++u) {
      const int idx = tid + NTHR * u;
      r[u] = idx < C * C / 4 ? *reinterpret_cast<const u32x4*>(src + 4 * idx) : u32x4{0, 0, 0, 0};
    }
  }
  template <int PITCH, bool TRANSPOSE = false>
  __device__ inline void commit(float (*dst)[PITCH], int C, int tid) const {
#pragma unroll
    for (int u = 0; u < NV; ++u) {
      const int idx = tid + NTHR * u;
      if (idx < C * C / 4) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int x = 4 * idx + e;
          if (TRANSPOSE)
            dst[x % C][x / C] = __uint_as_float(r[u][e]);
          else
            dst[x / C][x % C] = __uint_as_float(r[u][e]);
        }
      }
    }
  }
};

typedef float f4 __attribute__((ext_vector_type(4)));
__device__ inline f4 ld4(const float* p) { return *reinterpret_cast<const f4*>(p); }
__device__ inline float dot4(f4 a, f4 b) { return a.x * b.x + a.y * b.y + a.z * b.z + a.w * b.w; }

// Chunk rows i of a 16-column tile are owned by threads with (tid >> 4) == i % 16, column tid & 15.

// The two scans run 512 threads per (head, 16 state columns): thread (r0, c) = (tid >> 4,
// tid & 15) owns state rows r0 + 32 u and chunk rows r0 + 32 u of column c.  K (and Q, T, P)
// sit in LDS both as loaded and transposed, so that every product reads 16-byte vectors along
// its summed index.
constexpr int NTS = 512, RSS = NTS / 16;

template <typename E, int DK>
__global__ __launch_bounds__(NTS) void bwd_states_kernel(BwdParams p) {
  constexpr int RD = (DK + RSS - 1) / RSS, NU = CM / RSS;
  __shared__ __attribute__((aligned(16))) float Kl[CM][DK + 4];
  __shared__ __attribute__((aligned(16))) float Kt[DK][CM + 4];
  __shared__ __attribute__((aligned(16))) float Tl[CM][CM + 4];
  __shared__ float Sl[DK][17];
  __shared__ float Yl[CM][17];  // V, then Y in place
  __shared__ float Wv[CM][17];  // w * V~
  __shared__ float gcl[CM], gam[CM], wl[CM];
  const int tid = threadIdx.x, c = tid & 15, r0 = tid >> 4;
  const int ntile = p.DV / 16, c0 = (int)(blockIdx.x % ntile) * 16, bh = (int)(blockIdx.x / ntile);
  const int b = bh / p.H, h = bh % p.H;
  const int C = p.C, DV = p.DV, NT = p.NT;
  const long HDK = (long)p.H * DK, HDV = (long)p.H * DV;
  const E* kb = static_cast<const E*>(p.k) + (long)b * p.Lx * HDK + (long)h * DK;
  const E* vb = static_cast<const E*>(p.v) + (long)b * p.Lx * HDV + (long)h * DV + c0;
  float S[RD];
#pragma unroll
  for (int u = 0; u < RD; ++u) {
    const int d = r0 + RSS * u;
    S[u] = p.S0 && d < DK ? p.S0[((long)bh * DK + d) * DV + c0 + c] : 0.f;
  }

  RowTile<E, DK, CM, NTS> kt;
  RowTile<E, 16, CM, NTS> vt;
  SquareTile<NTS> tt;
  float gv = 0.f;
  auto issue = [&](int n) {
    const long P0 = (long)n * C;
    const int valid = (int)min((long)C, (long)p.Lx - P0);
    kt.issue([&](int i) -> const E* { return i < valid ? kb + (P0 + i) * HDK : nullptr; }, tid);
    vt.issue([&](int i) -> const E* { return i < valid ? vb + (P0 + i) * HDV : nullptr; }, tid);
    tt.issue(p.T + ((long)bh * NT + n) * C * C, C, tid);
    gv = tid < C ? p.gc[((long)bh * NT + n) * C + tid] : 0.f;
  };
  if (NT > 0) issue(0);
  for (int n = 0; n < NT; ++n) {
    const long chunk = (long)bh * NT + n;
    kt.commit(Kl, C, tid);
    kt.template commit<CM + 4, true>(Kt, C, tid);
    vt.commit(Yl, C, tid);
    tt.template commit<CM + 4>(Tl, C, tid);
    if (tid < C) gcl[tid] = gv;
#pragma unroll
    for (int u = 0; u < RD; ++u) {
      const int d = r0 + RSS * u;
      if (d < DK) {
        p.Sn[(chunk * DK + d) * DV + c0 + c] = S[u];
        Sl[d][c] = S[u];
      }
    }
    __syncthreads();
    const float gC = gcl[C - 1];
    if (tid < C) {
      gam[tid] = expf(gcl[tid]);
      wl[tid] = expf(gC - gcl[tid]);
    }
    if (n + 1 < NT) issue(n + 1);  // the next chunk's loads fly while this one computes
    __syncthreads();
    // Y = V - gam K S
    {
      float acc[NU] = {};
      for (int d = 0; d < DK; d += 4) {
        f4 sv;
#pragma unroll
        for (int e = 0; e < 4; ++e) sv[e] = Sl[d + e][c];
#pragma unroll
        for (int u = 0; u < NU; ++u)
          if (r0 + RSS * u < C) acc[u] += dot4(ld4(&Kl[r0 + RSS * u][d]), sv);
      }
#pragma unroll
      for (int u = 0; u < NU; ++u)
        if (r0 + RSS * u < C) Yl[r0 + RSS * u][c] -= gam[r0 + RSS * u] * acc[u];
    }
    __syncthreads();
    // w * V~ with V~ = T Y (T zero above the diagonal: j up to the thread's last row)
    {
      float acc[NU] = {};
      const int jend = r0 < C ? (r0 + RSS * ((C - 1 - r0) / RSS) + 4) & ~3 : 0;
      for (int j = 0; j < jend; j += 4) {
        f4 y;
#pragma unroll
        for (int e = 0; e < 4; ++e) y[e] = Yl[j + e][c];
#pragma unroll
        for (int u = 0; u < NU; ++u)
          if (r0 + RSS * u < C) acc[u] += dot4(ld4(&Tl[r0 + RSS * u][j]), y);
      }
#pragma unroll
      for (int u = 0; u < NU; ++u)
        if (r0 + RSS * u < C) Wv[r0 + RSS * u][c] = wl[r0 + RSS * u] * acc[u];
    }
    __syncthreads();
    // S <- gam_C S + K^T (w V~)
    {
      const float eC = expf(gC);
      float acc[RD] = {};
      for (int i = 0; i < C; i += 4) {
        f4 x;
#pragma unroll
        for (int e = 0; e < 4; ++e) x[e] = Wv[i + e][c];
#pragma unroll
        for (int u = 0; u < RD; ++u)
          if (r0 + RSS * u < DK) acc[u] += dot4(ld4(&Kt[r0 + RSS * u][i]), x);
      }
#pragma unroll
      for (int u = 0; u < RD; ++u) S[u] = eC * S[u] + acc[u];
    }
    __syncthreads();
  }
}

// P = Q K^T * Gam on and below the diagonal, per chunk (Q scaled, zero rows where a token has
// no readout), for the reverse scan and the per-chunk gradients.
template <typename E, int DK>
__global__ __launch_bounds__(NTH) void bwd_qk_kernel(BwdParams p) {
  __shared__ float Kl[CM][DK + 1];
  __shared__ float Ql[CM][DK + 1];
  __shared__ float gcl[CM];
  const int tid = threadIdx.x;
  const int n = (int)(blockIdx.x % p.NT), bh = (int)(blockIdx.x / p.NT), b = bh / p.H, h = bh % p.H;
  const int C = p.C, nh = p.nh;
  const long HDK = (long)p.H * DK, P0 = (long)n * C, chunk = (long)bh * p.NT + n;
  const int valid = (int)min((long)C, (long)p.Lx - P0);
  const E* kb = static_cast<const E*>(p.k) + (long)b * p.Lx * HDK + (long)h * DK;
  const E* qb = static_cast<const E*>(p.q) + (long)b * p.L * HDK + (long)h * DK;
  RowTile<E, DK, CM> kt, qt;
  kt.issue([&](int i) -> const E* { return i < valid ? kb + (P0 + i) * HDK : nullptr; }, tid);
  qt.issue([&](int i) -> const E* {
    return i < valid && (P0 + i) % nh == nh - 1 ? qb + (P0 + i) / nh * HDK : nullptr;
  }, tid);
  if (tid < C) gcl[tid] = p.gc[chunk * C + tid];
  kt.commit(Kl, C, tid);
  qt.commit(Ql, C, tid, p.scale);
  __syncthreads();
  float* out = p.Pm + chunk * C * C;
  for (int idx = tid; idx < C * C; idx += NTH) {
    const int i = idx / C, j = idx % C;
    float acc = 0.f;
    if (j <= i) {
#pragma unroll 8
      for (int d = 0; d < DK; ++d) acc += Ql[i][d] * Kl[j][d];
      acc *= expf(gcl[i] - gcl[j]);
    }
    out[idx] = acc;
  }
}

template <typename E, int DK>
__global__ __launch_bounds__(NTS) void bwd_dstates_kernel(BwdParams p) {
  constexpr int RD = (DK + RSS - 1) / RSS, NU = CM / RSS;
  __shared__ __attribute__((aligned(16))) float Kl[CM][DK + 4];
  __shared__ __attribute__((aligned(16))) float Kt[DK][CM + 4];
  __shared__ __attribute__((aligned(16))) float Qt[DK][CM + 4];
  __shared__ __attribute__((aligned(16))) float Tt[CM][CM + 4];  // T^T
  __shared__ __attribute__((aligned(16))) float Pt[CM][CM + 4];  // P^T
  __shared__ float Gl[DK][17];
  __shared__ float dOl[CM][17];
  __shared__ float dVt[CM][17];
  __shared__ float dYl[CM][17];
  __shared__ __attribute__((aligned(16))) float gam[CM];
  __shared__ float gcl[CM], wl[CM];
  const int tid = threadIdx.x, c = tid & 15, r0 = tid >> 4;
  const int ntile = p.DV / 16, c0 = (int)(blockIdx.x % ntile) * 16, bh = (int)(blockIdx.x / ntile);
  const int b = bh / p.H, h = bh % p.H;
  const int C = p.C, DV = p.DV, nh = p.nh, NT = p.NT;
  const long HDK = (long)p.H * DK, HDV = (long)p.H * DV;
  const E* kb = static_cast<const E*>(p.k) + (long)b * p.Lx * HDK + (long)h * DK;
  const E* qb = static_cast<const E*>(p.q) + (long)b * p.L * HDK + (long)h * DK;
  const E* ob = static_cast<const E*>(p.dO) + (long)b * p.L * HDV + (long)h * DV + c0;
  float G[RD];
#pragma unroll
  for (int u = 0; u < RD; ++u) {
    const int d = r0 + RSS * u;
    G[u] = p.dS_final && d < DK ? p.dS_final[((long)bh * DK + d) * DV + c0 + c] : 0.f;
  }

  RowTile<E, DK, CM, NTS> kt, qt;
  RowTile<E, 16, CM, NTS> ot;
  SquareTile<NTS> tt, pt;
  float gv = 0.f;
  auto issue = [&](int n) {
    const long P0 = (long)n * C, chunk = (long)bh * NT + n;
    const int valid = (int)min((long)C, (long)p.Lx - P0);
    auto last = [&](int i) { return i < valid && (P0 + i) % nh == nh - 1; };
    kt.issue([&](int i) -> const E* { return i < valid ? kb + (P0 + i) * HDK : nullptr; }, tid);
    qt.issue([&](int i) -> const E* { return last(i) ? qb + (P0 + i) / nh * HDK : nullptr; }, tid);
    ot.issue([&](int i) -> const E* { return last(i) ? ob + (P0 + i) / nh * HDV : nullptr; }, tid);
    tt.issue(p.T + chunk * C * C, C, tid);
    pt.issue(p.Pm + chunk * C * C, C, tid);
    gv = tid < C ? p.gc[chunk * C + tid] : 0.f;
  };
  if (NT > 0) issue(NT - 1);
  for (int n = NT - 1; n >= 0; --n) {
    const long P0 = (long)n * C;
    const int valid = (int)min((long)C, (long)p.Lx - P0);
    const long chunk = (long)bh * NT + n;
    kt.commit(Kl, C, tid);
    kt.template commit<CM + 4, true>(Kt, C, tid);
    qt.template commit<CM + 4, true>(Qt, C, tid, p.scale);
    ot.commit(dOl, C, tid);
    tt.template commit<CM + 4, true>(Tt, C, tid);
    pt.template commit<CM + 4, true>(Pt, C, tid);
    if (tid < C) gcl[tid] = gv;
#pragma unroll
    for (int u = 0; u < RD; ++u) {
      const int d = r0 + RSS * u;
      if (d < DK) {
        p.Gn[(chunk * DK + d) * DV + c0 + c] = G[u];
        Gl[d][c] = G[u];
      }
    }
    __syncthreads();
    const float gC = gcl[C - 1];
    if (tid < C) {
      gam[tid] = expf(gcl[tid]);
      wl[tid] = expf(gC - gcl[tid]);
    }
    if (n > 0) issue(n - 1);
    __syncthreads();
    // dV~ = w (K G') + P^T dO  (P^T zero below the diagonal: j from the thread's first row)
    {
      float kg[NU] = {}, acc[NU] = {};
      for (int d = 0; d < DK; d += 4) {
        f4 gv4;
#pragma unroll
        for (int e = 0; e < 4; ++e) gv4[e] = Gl[d + e][c];
#pragma unroll
        for (int u = 0; u < NU; ++u)
          if (r0 + RSS * u < C) kg[u] += dot4(ld4(&Kl[r0 + RSS * u][d]), gv4);
      }
      for (int j = r0 & ~3; j < C; j += 4) {
        f4 o;
#pragma unroll
        for (int e = 0; e < 4; ++e) o[e] = dOl[j + e][c];
#pragma unroll
        for (int u = 0; u < NU; ++u)
          if (r0 + RSS * u < C) acc[u] += dot4(ld4(&Pt[r0 + RSS * u][j]), o);
      }
#pragma unroll
      for (int u = 0; u < NU; ++u)
        if (r0 + RSS * u < C) dVt[r0 + RSS * u][c] = wl[r0 + RSS * u] * kg[u] + acc[u];
    }
    __syncthreads();
    // dY = T^T dV~, which is dV  (T^T zero below the diagonal)
    {
      float acc[NU] = {};
      for (int j = r0 & ~3; j < C; j += 4) {
        f4 x;
#pragma unroll
        for (int e = 0; e < 4; ++e) x[e] = dVt[j + e][c];
#pragma unroll
        for (int u = 0; u < NU; ++u)
          if (r0 + RSS * u < C) acc[u] += dot4(ld4(&Tt[r0 + RSS * u][j]), x);
      }
#pragma unroll
      for (int u = 0; u < NU; ++u) {
        const int i = r0 + RSS * u;
        if (i < C) {
          dYl[i][c] = acc[u];
          if (i < valid) p.dv[((b * (long)p.Lx + P0 + i) * p.H + h) * DV + c0 + c] = acc[u];
        }
      }
    }
    __syncthreads();
    // G <- gam_C G' - K^T (gam dY) + (gam Q)^T dO
    {
      const float eC = expf(gC);
      float acc[RD] = {};
      for (int i = 0; i < C; i += 4) {
        const f4 g4 = ld4(&gam[i]);
        f4 o, y;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          o[e] = g4[e] * dOl[i + e][c];
          y[e] = g4[e] * dYl[i + e][c];
        }
#pragma unroll
        for (int u = 0; u < RD; ++u)
          if (r0 + RSS * u < DK)
            acc[u] += dot4(ld4(&Qt[r0 + RSS * u][i]), o) - dot4(ld4(&Kt[r0 + RSS * u][i]), y);
      }
#pragma unroll
      for (int u = 0; u < RD; ++u) G[u] = eC * G[u] + acc[u];
    }
    __syncthreads();
  }
  if (p.dS0) {
#pragma unroll
    for (int u = 0; u < RD; ++u) {
      const int d = r0 + RSS * u;
      if (d < DK) p.dS0[((long)bh * DK + d) * DV + c0 + c] = G[u];
    }
  }
}

// Sum over the 16 lanes of a row group (lanes that share tid >> 4 within the wave).
__device__ inline float sum16(float x) {
  x += __shfl_xor(x, 8, 16);
  x += __shfl_xor(x, 4, 16);
  x += __shfl_xor(x, 2, 16);
  x += __shfl_xor(x, 1, 16);
  return x;
}

// Rows padded to a multiple of 4 floats so that 16-byte LDS reads stay aligned.
template <int DK>
struct __attribute__((aligned(16))) ChunkLds {
  float K[CM][DK + 4];
  float Q[CM][DK + 4];
  float N[CM][CM + 4];   // (I + A)^-1
  float Pt[CM][CM + 4];  // P^T, P = Q K^T * Gam on and below the diagonal
  union {
    struct {  // one 16-column tile of the value dimension
      float St[DK][20], Gt[DK][20];
      float Y[CM][20], dO[CM][20], Vt[CM][20], dVt[CM][20], dY[CM][20];
    } t;
    struct {  // chunk-local C x C algebra
      float R0[CM][CM + 4], R1[CM][CM + 4], R2[CM][CM + 4];
    } m;
  } u;
  float gc[CM], gam[CM], w[CM], beta[CM], dbd[CM], dgc[CM], dw[CM], rsum[CM];
  float sgs[NTC / WAVE];
};

template <typename E, int DK>
__global__ __launch_bounds__(NTC) void bwd_chunk_kernel(BwdParams p) {
  __shared__ ChunkLds<DK> s;
  // 512 threads: chunk rows r0 + 32 u (u < 2) of column c, two waves per SIMD
  constexpr int RS = NTC / 16, NU = CM / RS;
  const int tid = threadIdx.x, c = tid & 15, r0 = tid >> 4;
  const int n = (int)(blockIdx.x % p.NT), bh = (int)(blockIdx.x / p.NT), b = bh / p.H, h = bh % p.H;
  const int C = p.C, DV = p.DV, nh = p.nh, CU = C / 16;
  constexpr int SD = DK / 16;
  const long P0 = (long)n * C;
  const int valid = (int)min((long)C, (long)p.Lx - P0);
  const long chunk = (long)bh * p.NT + n;

  const long HDK = (long)p.H * DK, HDV = (long)p.H * DV;
  const E* kb = static_cast<const E*>(p.k) + (long)b * p.Lx * HDK + (long)h * DK;
  const E* qb = static_cast<const E*>(p.q) + (long)b * p.L * HDK + (long)h * DK;
  const E* vb = static_cast<const E*>(p.v) + (long)b * p.Lx * HDV + (long)h * DV;
  const E* ob = static_cast<const E*>(p.dO) + (long)b * p.L * HDV + (long)h * DV;
  auto last = [&](int i) { return i < valid && (P0 + i) % nh == nh - 1; };
  {
    RowTile<E, DK, CM, NTC> kt, qt;
    SquareTile<NTC> pt;
    kt.issue([&](int i) -> const E* { return i < valid ? kb + (P0 + i) * HDK : nullptr; }, tid);
    qt.issue([&](int i) -> const E* { return last(i) ? qb + (P0 + i) / nh * HDK : nullptr; }, tid);
    pt.issue(p.Pm + chunk * C * C, C, tid);
    kt.commit(s.K, C, tid);
    qt.commit(s.Q, C, tid, p.scale);
    pt.template commit<CM + 4, true>(s.Pt, C, tid);
  }
  const float gC = p.gc[chunk * C + C - 1];
  if (tid < C) {
    const float g = p.gc[chunk * C + tid];
    s.gc[tid] = g;
    s.gam[tid] = expf(g);
    s.w[tid] = expf(gC - g);
    s.beta[tid] = tid < valid ? p.beta[(b * (long)p.Lx + P0 + tid) * p.H + h] : 0.f;
  }
  __syncthreads();
  // A = strictLower(diag(beta) (Gam * K K^T)) into R0
  for (int idx = tid; idx < C * C; idx += NTC) {
    const int i = idx / C, j = idx % C;
    float kk = 0.f;
    if (j < i) {
#pragma unroll 8
      for (int d = 0; d < DK; d += 4) kk += dot4(ld4(&s.K[i][d]), ld4(&s.K[j][d]));
      kk *= s.beta[i] * expf(s.gc[i] - s.gc[j]);
    }
    s.u.m.R0[i][j] = kk;
  }
  __syncthreads();
  // N = (I + A)^-1 by forward substitution, one row per step
  for (int i = 0; i < C; ++i) {
    if (tid < C) {
      const int m = tid;
      float acc = m == i ? 1.f : 0.f;
      for (int j = m; j < i; ++j) acc -= s.u.m.R0[i][j] * s.N[j][m];
      s.N[i][m] = m <= i ? acc : 0.f;
    }
    __syncthreads();
  }

  // ---- value-dimension tiles; each tile's loads are issued one tile ahead
  float dT[NU][4] = {}, dOV[NU][4] = {}, dQa[NU][SD] = {}, dKa[NU][SD] = {};
  float dgcr[NU] = {}, dwr[NU] = {}, sgs = 0.f;
  RowTile<float, 16, DK, NTC> st, gt;
  RowTile<E, 16, CM, NTC> vt, ot;
  auto issue = [&](int c0) {
    const float* sb = p.Sn + chunk * DK * DV + c0;
    const float* gb = p.Gn + chunk * DK * DV + c0;
    st.issue([&](int d) -> const float* { return sb + (long)d * DV; }, tid);
    gt.issue([&](int d) -> const float* { return gb + (long)d * DV; }, tid);
    vt.issue([&](int i) -> const E* { return i < valid ? vb + (P0 + i) * HDV + c0 : nullptr; }, tid);
    ot.issue([&](int i) -> const E* { return last(i) ? ob + (P0 + i) / nh * HDV + c0 : nullptr; }, tid);
  };
  issue(0);
  for (int c0 = 0; c0 < DV; c0 += 16) {
    st.commit(s.u.t.St, DK, tid);
    gt.commit(s.u.t.Gt, DK, tid);
    vt.commit(s.u.t.Y, C, tid);
    ot.commit(s.u.t.dO, C, tid);
    __syncthreads();
    if (c0 + 16 < DV) issue(c0 + 16);
    for (int d = r0; d < DK; d += RS) sgs += s.u.t.St[d][c] * s.u.t.Gt[d][c];
    // K S, Q S and K G' on the thread's rows (four key dimensions per step)
    float ks[NU] = {}, qs[NU] = {}, kg[NU] = {};
#pragma unroll 2
    for (int d = 0; d < DK; d += 4) {
      f4 sv, gv;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        sv[e] = s.u.t.St[d + e][c];
        gv[e] = s.u.t.Gt[d + e][c];
      }
#pragma unroll
      for (int u = 0; u < NU; ++u)
        if (r0 + RS * u < C) {
          const f4 kv = ld4(&s.K[r0 + RS * u][d]);
          ks[u] += dot4(kv, sv);
          qs[u] += dot4(ld4(&s.Q[r0 + RS * u][d]), sv);
          kg[u] += dot4(kv, gv);
        }
    }
#pragma unroll
    for (int u = 0; u < NU; ++u)
      if (r0 + RS * u < C) s.u.t.Y[r0 + RS * u][c] -= s.gam[r0 + RS * u] * ks[u];
    __syncthreads();
    // V~ = N diag(beta) Y; N is zero above the diagonal
    float vt[NU] = {};
    {
      // up to the thread's last row, rounded up to 4
      const int jend = r0 < C ? (r0 + RS * ((C - 1 - r0) / RS) + 4) & ~3 : 0;
      for (int j = 0; j < jend; j += 4) {
        const f4 bj = ld4(&s.beta[j]);
        f4 y;
#pragma unroll
        for (int e = 0; e < 4; ++e) y[e] = s.u.t.Y[j + e][c] * bj[e];
#pragma unroll
        for (int u = 0; u < NU; ++u)
          if (r0 + RS * u < C) vt[u] += dot4(ld4(&s.N[r0 + RS * u][j]), y);
      }
    }
#pragma unroll
    for (int u = 0; u < NU; ++u)
      if (r0 + RS * u < C) s.u.t.Vt[r0 + RS * u][c] = vt[u];
    __syncthreads();
    // dV~ = w (K G') + P^T dO; P^T is zero below the diagonal
    {
      float dvt[NU];
#pragma unroll
      for (int u = 0; u < NU; ++u) dvt[u] = r0 + RS * u < C ? s.w[r0 + RS * u] * kg[u] : 0.f;
      for (int j = r0 & ~3; j < C; j += 4) {
        f4 o;
#pragma unroll
        for (int e = 0; e < 4; ++e) o[e] = s.u.t.dO[j + e][c];
#pragma unroll
        for (int u = 0; u < NU; ++u)
          if (r0 + RS * u < C) dvt[u] += dot4(ld4(&s.Pt[r0 + RS * u][j]), o);
      }
#pragma unroll
      for (int u = 0; u < NU; ++u)
        if (r0 + RS * u < C) s.u.t.dVt[r0 + RS * u][c] = dvt[u];
    }
    __syncthreads();
    // dY = diag(beta) N^T dV~
    {
      float dy[NU] = {};
      for (int j = r0; j < C; ++j) {
        const float x = s.u.t.dVt[j][c];
#pragma unroll
        for (int u = 0; u < NU; ++u)
          if (r0 + RS * u < C) dy[u] += s.N[j][r0 + RS * u] * x;
      }
#pragma unroll
      for (int u = 0; u < NU; ++u) {
        const int i = r0 + RS * u;
        if (r0 + RS * u < C) {
          const float acc = dy[u] * s.beta[i];
          s.u.t.dY[i][c] = acc;
          dgcr[u] += sum16(s.gam[i] * (qs[u] * s.u.t.dO[i][c] - ks[u] * acc));
          dwr[u] += sum16(kg[u] * vt[u]);
        }
      }
    }
    __syncthreads();
    // dT += dV~ Y^T, dOV += dO V~^T; dQa += gam dO S^T, dKa += -gam dY S^T + w V~ G'^T
#pragma unroll
    for (int e = 0; e < 16; e += 4) {
      f4 a[NU], o[NU], dy4[NU], vt4[NU];
#pragma unroll
      for (int u = 0; u < NU; ++u)
        if (r0 + RS * u < C) {
          const int i = r0 + RS * u;
          a[u] = ld4(&s.u.t.dVt[i][e]);
          o[u] = ld4(&s.u.t.dO[i][e]);
          dy4[u] = ld4(&s.u.t.dY[i][e]);
          vt4[u] = ld4(&s.u.t.Vt[i][e]);
        }
#pragma unroll
      for (int v = 0; v < 4; ++v)
        if (v < CU) {
          const int j = c + 16 * v;
          const f4 yv = ld4(&s.u.t.Y[j][e]), vv = ld4(&s.u.t.Vt[j][e]);
#pragma unroll
          for (int u = 0; u < NU; ++u)
            if (r0 + RS * u < C) {
              dT[u][v] += dot4(a[u], yv);
              dOV[u][v] += dot4(o[u], vv);
            }
        }
#pragma unroll
      for (int v = 0; v < SD; ++v) {
        const int d = c + 16 * v;
        const f4 sv = ld4(&s.u.t.St[d][e]), gv = ld4(&s.u.t.Gt[d][e]);
#pragma unroll
        for (int u = 0; u < NU; ++u)
          if (r0 + RS * u < C) {
            const int i = r0 + RS * u;
            dQa[u][v] += s.gam[i] * dot4(o[u], sv);
            dKa[u][v] += s.w[i] * dot4(vt4[u], gv) - s.gam[i] * dot4(dy4[u], sv);
          }
      }
    }
    __syncthreads();
  }

  // ---- chunk-local algebra
  // sum of S_n * G'_n over the whole state: per-wave partial sums, then one total
  {
    float x = sgs;
    for (int o = 32; o > 0; o >>= 1) x += __shfl_xor(x, o, WAVE);
    if ((tid & (WAVE - 1)) == 0) s.sgs[tid / WAVE] = x;
  }
  if (c == 0) {
#pragma unroll
    for (int u = 0; u < NU; ++u)
      if (r0 + RS * u < C) {
        s.dgc[r0 + RS * u] = dgcr[u];
        s.dw[r0 + RS * u] = dwr[u];
      }
  }
#pragma unroll
  for (int u = 0; u < NU; ++u)
#pragma unroll
    for (int v = 0; v < 4; ++v)
      if (r0 + RS * u < C && v < CU) {
        s.u.m.R0[r0 + RS * u][c + 16 * v] = dT[u][v];
        s.u.m.R1[r0 + RS * u][c + 16 * v] = dOV[u][v];
      }
  __syncthreads();
  // diag(N^T dT), and X = dT diag(beta) N^T (= dT T^T) into registers
  if (tid < C) {
    float acc = 0.f;
    for (int i = tid; i < C; ++i) acc += s.N[i][tid] * s.u.m.R0[i][tid];
    s.dbd[tid] = acc;
  }
  float X[NU][4];
#pragma unroll
  for (int u = 0; u < NU; ++u)
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      X[u][v] = 0.f;
      if (r0 + RS * u < C && v < CU) {
        const int i = r0 + RS * u, j = c + 16 * v;
        // N is zero above the diagonal: k runs to j rounded up to 4
        for (int k = 0; k <= j; k += 4)
          X[u][v] += dot4(ld4(&s.u.m.R0[i][k]) * ld4(&s.beta[k]), ld4(&s.N[j][k]));
      }
    }
  __syncthreads();
#pragma unroll
  for (int u = 0; u < NU; ++u)
#pragma unroll
    for (int v = 0; v < 4; ++v)
      if (r0 + RS * u < C && v < CU) s.u.m.R0[r0 + RS * u][c + 16 * v] = X[u][v];
  __syncthreads();
  // dA = -strictLower(N^T X); K K^T recomputed into R2
  float dA[NU][4];
#pragma unroll
  for (int u = 0; u < NU; ++u)
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      dA[u][v] = 0.f;
      const int i = r0 + RS * u, j = c + 16 * v;
      if (r0 + RS * u < C && v < CU) {
        if (j < i) {
          float acc = 0.f;
          for (int k = i; k < C; ++k) acc += s.N[k][i] * s.u.m.R0[k][j];
          dA[u][v] = -acc;
        }
        float kk = 0.f;
        if (j < i) {
#pragma unroll 8
          for (int d = 0; d < DK; d += 4) kk += dot4(ld4(&s.K[i][d]), ld4(&s.K[j][d]));
        }
        s.u.m.R2[i][j] = kk;
      }
    }
  __syncthreads();
  // per entry: the gate-prefix term t, dbeta's row term, dGm and E1 = Gam * dOV (lower)
  float t[NU][4], dGm[NU][4], E1[NU][4], rb[NU] = {}, rt[NU] = {};
#pragma unroll
  for (int u = 0; u < NU; ++u)
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      t[u][v] = dGm[u][v] = E1[u][v] = 0.f;
      const int i = r0 + RS * u, j = c + 16 * v;
      if (r0 + RS * u < C && v < CU && j <= i) {
        const float gm = expf(s.gc[i] - s.gc[j]);
        const float kk = s.u.m.R2[i][j], dov = s.u.m.R1[i][j];
        const float ta = dA[u][v] * gm * kk;  // zero on the diagonal
        rb[u] += ta;
        t[u][v] = s.beta[i] * ta + s.Pt[j][i] * dov;
        dGm[u][v] = s.beta[i] * gm * dA[u][v];
        E1[u][v] = gm * dov;
        rt[u] += t[u][v];
      }
    }
  __syncthreads();
#pragma unroll
  for (int u = 0; u < NU; ++u) {
    rb[u] = sum16(rb[u]);
    rt[u] = sum16(rt[u]);
#pragma unroll
    for (int v = 0; v < 4; ++v)
      if (r0 + RS * u < C && v < CU) {
        const int i = r0 + RS * u, j = c + 16 * v;
        s.u.m.R0[i][j] = dGm[u][v];
        s.u.m.R1[i][j] = E1[u][v];
        s.u.m.R2[i][j] = t[u][v];
      }
    if (c == 0 && r0 + RS * u < C) {
      const int i = r0 + RS * u;
      s.dbd[i] += rb[u];
      s.rsum[i] = rt[u];
    }
  }
  __syncthreads();
  if (tid < C) {
    const int i = tid;
    float col = 0.f;
    for (int r = i; r < C; ++r) col += s.u.m.R2[r][i];
    s.dgc[i] += s.rsum[i] - col - s.w[i] * s.dw[i];
    if (i < valid) p.dbeta[(b * (long)p.Lx + P0 + i) * p.H + h] = s.dbd[i];
  }
  __syncthreads();
  if (tid == 0 && p.dg_log) {
    float tot = 0.f;
    for (int i = 0; i < C; ++i) tot += s.w[i] * s.dw[i];
    for (int o = 0; o < NTC / WAVE; ++o) tot += expf(gC) * s.sgs[o];
    // reverse cumulative sum over the chunk; the last position also collects the total above
    float run = tot;
    for (int i = C - 1; i >= 0; --i) {
      run += s.dgc[i];
      const long pos = P0 + i;
      if (i < valid && pos % nh == 0) p.dg_log[(b * (long)p.L + pos / nh) * p.H + h] = run;
    }
  }
  // dQ = dQa + E1 K,  dK = dKa + E1^T Q + (dGm + dGm^T) K  (E1 lower, dGm strictly lower)
  for (int j = 0; j < C; ++j) {
    float kj[SD], qj[SD];
#pragma unroll
    for (int v = 0; v < SD; ++v) {
      kj[v] = s.K[j][c + 16 * v];
      qj[v] = s.Q[j][c + 16 * v];
    }
#pragma unroll
    for (int u = 0; u < NU; ++u)
      if (r0 + RS * u < C) {
        const int i = r0 + RS * u;
        const float e1 = s.u.m.R1[i][j], e1t = s.u.m.R1[j][i], gs = s.u.m.R0[i][j] + s.u.m.R0[j][i];
#pragma unroll
        for (int v = 0; v < SD; ++v) {
          dQa[u][v] += e1 * kj[v];
          dKa[u][v] += e1t * qj[v] + gs * kj[v];
        }
      }
  }
#pragma unroll
  for (int u = 0; u < NU; ++u) {
    const int i = r0 + RS * u;
    if (i >= C || i >= valid) continue;
    const long pos = P0 + i;
    const bool is_last = pos % nh == nh - 1;
#pragma unroll
    for (int v = 0; v < SD; ++v) {
      const int d = c + 16 * v;
      p.dk[((b * (long)p.Lx + pos) * p.H + h) * DK + d] = dKa[u][v];
      if (is_last) p.dq[((b * (long)p.L + pos / nh) * p.H + h) * DK + d] = p.scale * dQa[u][v];
    }
  }
}

template <typename E>
hipError_t launch_by_dk(const BwdParams& p, int which, hipStream_t st) {
  const dim3 block(NTH);
  // one-dimensional grids: (head, column tile) and (head, chunk), tile or chunk fastest
  const dim3 gs((unsigned)((long)p.DV / 16 * p.B * p.H)), gc((unsigned)((long)p.NT * p.B * p.H));
#define DELTA_BWD_CASE(D)                                                                        \
  case D:                                                                                        \
    if (which == 0) hipLaunchKernelGGL((bwd_states_kernel<E, D>), gs, dim3(NTS), 0, st, p);     \
    else if (which == 1) hipLaunchKernelGGL((bwd_dstates_kernel<E, D>), gs, dim3(NTS), 0, st, p); \
    else if (which == 2) hipLaunchKernelGGL((bwd_chunk_kernel<E, D>), gc, dim3(NTC), 0, st, p); \
    else hipLaunchKernelGGL((bwd_qk_kernel<E, D>), gc, block, 0, st, p);                         \
    break;
  switch (p.DK) {
    DELTA_BWD_CASE(16)
    DELTA_BWD_CASE(32)
    DELTA_BWD_CASE(64)
    DELTA_BWD_CASE(128)
    default: return hipErrorInvalidValue;
  }
#undef DELTA_BWD_CASE
  return hipGetLastError();
}

}  // namespace

hipError_t launch_bwd_phase(const BwdParams& p, bool bf16_in, int phase, hipStream_t st) {
  return bf16_in ? launch_by_dk<bf16>(p, phase, st) : launch_by_dk<float>(p, phase, st);
}

}  // namespace delta
