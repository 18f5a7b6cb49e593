// KDA forward over a sequence, token by token: the delta rule with a decay per key channel,
//     S_t = (I - beta_t k_t k_t^T) Diag(alpha_t) S_{t-1} + beta_t k_t v_t^T,   o_t = scale S_t^T q_t
// ("08 linear delta rule & DPLR" page, section 1.4 table, KDA row, and section 5, where the same
// update is written as a DPLR step with the diagonal applied first).
//
// Organisation.  One workgroup of 4 wavefronts per (sequence, head, 16 value columns); lane
// (c, g) = (lane / 16, lane % 16) of wavefront w holds column 4 w + c of the slab, rows
// g RPL .. g RPL + RPL - 1 of the state (RPL = d_k / 16), in registers for the whole sequence.
// Per token, with alpha = exp(a_log), the two sums over d_k share one pass over the pre-token
// state:
//     a  = sum_r s_r alpha_r k_r          (S_{t-1}^T Diag(alpha) k: the value the write corrects)
//     oq = sum_r s_r alpha_r q_r
//     e  = v - a,   o = scale (oq + beta (k . q) e),   s_r <- alpha_r s_r + beta k_r e
// (o = S_t^T q expands to Diag(alpha)-decayed state read by q plus the rank-1 write's share).
// The 16 row groups of a column sit in one row of 16 lanes, so the sums finish with four DPP
// steps, no LDS and no barrier.  Tokens come in blocks of 16: every thread loads one token's
// 1/16 of k, q and a_log (and one value element), the block's per-token vectors alpha k,
// alpha q, beta k, alpha and the scalar beta (k . q) are formed once and staged in LDS (block n+1
// is loaded into registers while block n is processed and written to LDS after it), and each
// block's outputs leave through LDS as 16-column rows.
//
// Bound: the recurrence is a chain of L dependent steps per state slab; each step is ~4 RPL
// fused multiply-adds per lane plus the two row sums, so the kernel is latency- and issue-bound,
// not bandwidth-bound (the chunkwise form, which turns the steps into matrix products, is the
// fast path for the scalar gate).
#include "common.h"
#include "kernels.h"

namespace delta {

namespace kda {

constexpr int TB = 16;  // tokens per staged block (16 threads per token, 256 threads)

// x taken from another lane of the same 16-lane row (DPP control CTRL)
template <int CTRL>
__device__ inline float dpp(float x) {
  return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x), CTRL, 0xF, 0xF, false));
}

// Sum over the 16 lanes of a DPP row: quad permutations xor 1 (0xB1) and xor 2 (0x4E) leave every
// lane with its quad's sum, the half-mirror (lane i <-> 7 - i, 0x141) pairs the quads of each
// 8, the mirror (i <-> 15 - i, 0x140) the halves; every lane of the row receives the total.
__device__ inline float row_sum16(float x) {
  x += dpp<0xB1>(x);
  x += dpp<0x4E>(x);
  x += dpp<0x141>(x);
  x += dpp<0x140>(x);
  return x;
}

// RPL consecutive floats of LDS: 16-byte reads when RPL is a multiple of 4 (the rows of a lane
// then start 16-byte aligned), single reads otherwise.
template <int RPL>
__device__ inline void read_rows(float (&x)[RPL], const float* src) {
  if constexpr (RPL % 4 == 0) {
#pragma unroll
    for (int j = 0; j < RPL; j += 4) {
      const floatx4 v = *reinterpret_cast<const floatx4*>(src + j);
      x[j] = v[0], x[j + 1] = v[1], x[j + 2] = v[2], x[j + 3] = v[3];
    }
  } else {
#pragma unroll
    for (int j = 0; j < RPL; ++j) x[j] = src[j];
  }
}

// N consecutive elements of E (N * sizeof(E) bytes, aligned to that size up to 16) as floats, in
// pieces of up to 16 bytes.
template <typename E, int N>
__device__ inline void load_vec(float (&x)[N], const E* src) {
  constexpr int BYTES = N * (int)sizeof(E);
  constexpr int PIECE = BYTES >= 16 ? 16 : BYTES;
  constexpr int PER = PIECE / (int)sizeof(E);
#pragma unroll
  for (int i = 0; i < N / PER; ++i) {
    E tmp[PER];
    if constexpr (PIECE == 16) *reinterpret_cast<u32x4*>(tmp) = reinterpret_cast<const u32x4*>(src)[i];
    else if constexpr (PIECE == 8) *reinterpret_cast<u32x2*>(tmp) = reinterpret_cast<const u32x2*>(src)[i];
    else if constexpr (PIECE == 4) *reinterpret_cast<uint32_t*>(tmp) = reinterpret_cast<const uint32_t*>(src)[i];
    else tmp[0] = src[i];
#pragma unroll
    for (int j = 0; j < PER; ++j) x[i * PER + j] = to_float(tmp[j]);
  }
}

template <int DK>
struct Stage {
  float kt[TB][DK];   // alpha * k
  float qt[TB][DK];   // alpha * q
  float bk[TB][DK];   // beta * k
  float al[TB][DK];   // alpha
  float vv[TB][16];   // the slab's value columns
  float bkq[TB];      // beta (k . q)
  float o[TB][16];    // outputs of the block
};

// One token's operands for a lane: its RPL rows of alpha k, alpha q, beta k and alpha, its value
// element and beta (k . q).
template <int RPL>
struct Ops {
  float kt[RPL], qt[RPL], bk[RPL], al[RPL], v, bkq;
};

template <int DK, int RPL>
__device__ inline void fetch(Ops<RPL>& o, const Stage<DK>& s, int t, int g, int cc) {
  read_rows<RPL>(o.kt, &s.kt[t][g * RPL]);
  read_rows<RPL>(o.qt, &s.qt[t][g * RPL]);
  read_rows<RPL>(o.bk, &s.bk[t][g * RPL]);
  read_rows<RPL>(o.al, &s.al[t][g * RPL]);
  o.v = s.vv[t][cc];
  o.bkq = s.bkq[t];
}

}  // namespace kda

template <typename E, int DK>
__global__ __launch_bounds__(256) void kda_fwd_kernel(KdaParams p) {
  using kda::TB;
  constexpr int RPL = DK / 16;   // state rows per lane
  constexpr int EPT = DK / 16;   // elements of a token's vectors per staging thread
  __shared__ __attribute__((aligned(16))) kda::Stage<DK> s;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int nsl = p.DV / 16;
  const int head = blockIdx.x / nsl, slab = blockIdx.x % nsl;
  const int b = head / p.H, h = head % p.H;
  // compute role: column cc of the slab, rows g*RPL ..
  const int c = lane >> 4, g = lane & 15;
  const int cc = 4 * wave + c;
  const int col = 16 * slab + cc;
  // staging role: token tt of the block, elements se*EPT .. of its vectors; value column se
  const int tt = tid >> 4, se = tid & 15;

  const E* qg = reinterpret_cast<const E*>(p.q);
  const E* kg = reinterpret_cast<const E*>(p.k);
  const E* vg = reinterpret_cast<const E*>(p.v);

  // registers of one staged token slice
  float rk[EPT], rq[EPT], ra[EPT], rv, rb;
  auto load = [&](int blk) {
    const long t = (long)blk * TB + tt;
    const bool ok = t < p.L;
    const long tok = ((long)b * p.L + (ok ? t : 0)) * p.H + h;
    kda::load_vec<E, EPT>(rk, kg + tok * DK + se * EPT);
    kda::load_vec<E, EPT>(rq, qg + tok * DK + se * EPT);
    kda::load_vec<float, EPT>(ra, p.a_log + tok * DK + se * EPT);
    rv = to_float(vg[tok * p.DV + 16 * slab + se]);
    rb = p.beta[tok];
    if (!ok) {  // past the sequence: a write of strength 0 (the block's tail is not read)
#pragma unroll
      for (int i = 0; i < EPT; ++i) rk[i] = rq[i] = ra[i] = 0.f;
      rv = rb = 0.f;
    }
  };
  auto store = [&]() {
    float kq = 0.f;
#pragma unroll
    for (int i = 0; i < EPT; ++i) {
      const float a = gate_exp(ra[i]);
      s.kt[tt][se * EPT + i] = a * rk[i];
      s.qt[tt][se * EPT + i] = a * rq[i];
      s.bk[tt][se * EPT + i] = rb * rk[i];
      s.al[tt][se * EPT + i] = a;
      kq += rk[i] * rq[i];
    }
    kq = kda::row_sum16(kq);  // the 16 staging threads of a token are one DPP row
    if (se == 0) s.bkq[tt] = rb * kq;
    s.vv[tt][se] = rv;
  };

  float S[RPL];
#pragma unroll
  for (int j = 0; j < RPL; ++j) S[j] = p.S0 ? p.S0[((long)head * DK + g * RPL + j) * p.DV + col] : 0.f;

  const int nblk = (p.L + TB - 1) / TB;
  if (nblk > 0) {
    load(0);
    store();
    if (nblk > 1) load(1);
  }
  __syncthreads();
  for (int n = 0; n < nblk; ++n) {
    const int ntok = min(TB, p.L - n * TB);
    // The block's 16 tokens as straight-line code: nothing inside writes LDS, so every operand
    // read can be issued ahead of the dependent chain.  Tokens past the sequence were staged as
    // no-ops (alpha = 1, k = q = v = beta = 0).  Every lane of a row ends a token with the row's
    // output; lane g keeps token g's.
    float myo = 0.f;
    kda::Ops<RPL> ops[2];
    kda::fetch<DK, RPL>(ops[0], s, 0, g, cc);
#pragma unroll
    for (int t = 0; t < TB; ++t) {
      const kda::Ops<RPL>& x = ops[t & 1];
      // token t+1's operands are read before token t's chain, which then never waits on LDS
      if (t + 1 < TB) kda::fetch<DK, RPL>(ops[(t + 1) & 1], s, t + 1, g, cc);
      __builtin_amdgcn_sched_barrier(0);
      float a0 = 0.f, a1 = 0.f, o0 = 0.f, o1 = 0.f;
#pragma unroll
      for (int j = 0; j < RPL; j += 2) {
        a0 += S[j] * x.kt[j];
        o0 += S[j] * x.qt[j];
        if (j + 1 < RPL) {
          a1 += S[j + 1] * x.kt[j + 1];
          o1 += S[j + 1] * x.qt[j + 1];
        }
      }
      const float a = kda::row_sum16(a0 + a1);
      const float oq = kda::row_sum16(o0 + o1);
      const float e = x.v - a;
      const float o = p.scale * (oq + x.bkq * e);
      myo = (g == t) ? o : myo;
#pragma unroll
      for (int j = 0; j < RPL; ++j) S[j] = x.al[j] * S[j] + x.bk[j] * e;
    }
    s.o[g][cc] = myo;
    __syncthreads();  // block n processed: its outputs are in LDS and its inputs are dead
    if (tt < ntok) {  // outputs of block n: 16 tokens x 16 columns, one element per thread
      E* Og = reinterpret_cast<E*>(p.O) + (((long)b * p.L + (long)n * TB + tt) * p.H + h) * p.DV + 16 * slab + se;
      *Og = to_elem<E>(s.o[tt][se]);
    }
    if (n + 1 < nblk) {
      store();  // block n+1, loaded during block n
      if (n + 2 < nblk) load(n + 2);
    }
    __syncthreads();
  }
#pragma unroll
  for (int j = 0; j < RPL; ++j)
    if (p.S_final) p.S_final[((long)head * DK + g * RPL + j) * p.DV + col] = S[j];
}

template <typename E>
static hipError_t kda_by_dk(const KdaParams& p, hipStream_t st) {
  const dim3 grid((unsigned)(p.B * p.H * (p.DV / 16))), block(256);
  switch (p.DK) {
    case 16: hipLaunchKernelGGL((kda_fwd_kernel<E, 16>), grid, block, 0, st, p); break;
    case 32: hipLaunchKernelGGL((kda_fwd_kernel<E, 32>), grid, block, 0, st, p); break;
    case 64: hipLaunchKernelGGL((kda_fwd_kernel<E, 64>), grid, block, 0, st, p); break;
    case 128: hipLaunchKernelGGL((kda_fwd_kernel<E, 128>), grid, block, 0, st, p); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_kda_fwd(const KdaParams& p, bool bf16_in, hipStream_t st) {
  return bf16_in ? kda_by_dk<bf16>(p, st) : kda_by_dk<float>(p, st);
}

}  // namespace delta
