// Segment summaries of the inter-chunk pass, for bf16 inputs with d_k = d_v = 128 and chunk 64:
// per (segment, head) the segment run from S = 0 on the d_v value columns (segment 0: from S0)
// and the segment's transition map on d_k columns that start as the identity and see V = 0.
//
// Sources: "08 linear delta rule & DPLR" page, section 2.3 (chunkwise algorithm: pseudo-values
// V~ = U - W S, S <- S + K^T V~), section 2.5 (V~ contracts over all of d_k, so the key dimension
// stays inside one workgroup) and section 3 (gated form: keys decayed to the chunk end).
// DeltaProduct notes, section 3 (the chunk maps are affine in S, so a segment composes them).
//
// Per chunk, with T from the intra-chunk kernel and gamma_r = exp(gc_r):
//   Y = V - gamma * (K S);   V~ = T Y;   S <- gamma_C S + K^T (gamma_C / gamma * V~).
//
// Organisation.  One workgroup of 8 wavefronts per (segment, head), two per SIMD; each
// wavefront owns 2 of the 16 state tiles of 16 columns (wavefronts 0-3: value columns, 4-7:
// transition columns) and also loads an eighth of every chunk: chunk n+1's tiles arrive in
// registers during chunk n, are written to the free half of a double-buffered LDS stage at the
// start of chunk n+1, and chunk n+2's loads are issued into the registers just freed.  The
// state stays in registers as MFMA accumulators (on gfx950 a 16x16 accumulator tile is already
// the B operand of the 16x16x32 bf16 MFMA; two tiles form one 32-deep step).  A operands (K
// rows, K^T through transpose reads, T rows) come from LDS.  One workgroup barrier per chunk.
//
// This file is built with MFMA accumulators in VGPRs and a scheduling hint that interleaves the
// operand reads with the products (see the build script): with the default allocation the
// compiler keeps the state in AGPRs, copies it through VGPRs for every vector operation, and
// waits for each LDS operand read before issuing the next.
//
// SM_OUT (KDA): the same chain on the value columns alone, from each segment's start state
// (written by the combine launch; S0 when the sequence is not split), one 16-column tile per
// wavefront, forming each chunk's outputs and, for the last segment, S_final:
//     O = Q+ S + Aqk V~   (Q+ = scale Q e^{Gc} staged as a fifth tile, Aqk from the intra kernel),
// transposed (O^T = S^T Q+^T + V~^T Aqk^T): the state's B-operand registers are the A operand of
// the first product and V~'s of the second, so a lane's accumulator holds four consecutive value
// columns of one token, stored with one 8-byte write.  Aqk's fragments are loaded per lane from
// global memory into registers (two stages with Aqk staged would not fit the LDS), during the
// chunk before; the intra kernel stores them in that order (KDA_AQK_*, kernels.h), so each load
// is 1 KB contiguous per wavefront.
//
// KDA (kda_chunk.hip; a decay per key channel): K is K e^{Gc}, Y = V - K S with no row gate, V~
// enters the update unweighted, the update's keys are K e^{Gc_C - Gc} (a fourth staged tile), and
// row r of the state decays by its channel's e^{Gc_C} (staged in place of the gate tables).
//
// Fragment layouts (16x16x32 bf16): lane (g, m) (g = lane / 16, m = lane % 16) holds
// A[m][8g .. 8g+7], B[8g .. 8g+7][m] and D[4g .. 4g+3][m].  State row tiles 2u, 2u+1 interleave
// their d_k indices so that the K S A-fragment is one 16-byte LDS read.
#include <type_traits>

#include "common.h"
#include "kernels.h"

namespace delta {
namespace summary {

constexpr int DK = 128, C = 64, DV = 128;
constexpr int NB = C / 16, NTS = DK / 16, NCT = DV / 16;
constexpr int NW = 8;                          // wavefronts
constexpr int CT = 2 * NCT / NW;               // 16-column state tiles per wavefront
constexpr int NKP = C * DK / 8 / (NW * WAVE);  // 16-byte pieces of K and V per lane and chunk
constexpr int NTP = C * C / 8 / (NW * WAVE);   // of T

// one stage (bf16 elements): K [C][DK], T [C][C], V [C][DV], then fp32 gc, exp(gc) and
// exp(gc_last - gc) tables of C
// (KDA: the tables hold e^{Gc_C} per channel, and K e^{Gc_C - Gc} [C][DK] follows them)
constexpr int K_OFF = 0, T_OFF = K_OFF + C * DK, V_OFF = T_OFF + C * C, G_OFF = V_OFF + C * DV;
constexpr int K2_OFF = G_OFF + 3 * C * 2;
constexpr int Q_OFF = K2_OFF + C * DK;  // KDA outputs: Q+ [C][DK]
enum SumMode { SM_SUMMARY = 0, SM_OUT = 2 };
template <bool KDA, int MODE>
constexpr int stage_elems() { return K2_OFF + (KDA ? C * DK : 0) + (MODE == SM_OUT ? C * DK : 0); }
static_assert(2 * stage_elems<true, SM_OUT>() * 2 <= 160 * 1024, "LDS budget");
static_assert(3 * C * 2 >= DK * 2, "the tables hold d_k floats");

// This lane's share of one chunk's input.
template <bool KDA, int MODE>
struct Regs {
  u32x4 k[NKP];
  u32x4 t[NTP];
  u32x4 v[NKP];
  u32x4 kh[KDA ? NKP : 1];
  u32x4 q[MODE == SM_OUT ? NKP : 1];
  std::conditional_t<KDA, u32x2, unsigned> gc;  // gc of token `lane` (KDA: e^{Gc_C} of channels 2 lane, + 1)
};

__device__ inline bf16x8 lds8(const bf16* p) { return *reinterpret_cast<const bf16x8*>(p); }
__device__ inline bf16x4 lds4(const bf16* p) { return *reinterpret_cast<const bf16x4*>(p); }
__device__ inline bf16x4 cvt4(floatx4 d) { return bf16x4{(bf16)d[0], (bf16)d[1], (bf16)d[2], (bf16)d[3]}; }
__device__ inline bf16x8 cat8(bf16x4 a, bf16x4 b) { return __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7); }
__device__ inline floatx4 mma(bf16x8 a, bf16x8 b, floatx4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// The LDS writes of the prefetched pieces, with the stage offset as the instruction's immediate
// (the compiler waits for each piece's load before its write).
__device__ inline unsigned lds_addr(const void* p) {
  return (unsigned)reinterpret_cast<unsigned long>((const __attribute__((address_space(3))) void*)p);
}
template <int OFF>
__device__ inline void write16(unsigned addr, const u32x4& x) {
  asm volatile("ds_write_b128 %0, %1 offset:%2" ::"v"(addr), "v"(x), "n"(OFF) : "memory");
}
__device__ inline void lds_barrier() {
  __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): this wave's LDS traffic has landed
  asm volatile("s_barrier" ::: "memory");
}

// swizzled element offset of (row r, column e) in a tile whose rows hold `ld` elements
// (16-byte chunks XOR-permuted by swz_key(r, mask))
__device__ inline int swz(int r, int e, int ld, int mask) {
  const unsigned u = e;
  return r * ld + (int)(((u >> 3) ^ (unsigned)swz_key(r, mask)) * 8 + (u & 7));
}

template <bool KDA, int MODE = SM_SUMMARY>
__global__ __launch_bounds__(NW * WAVE) __attribute__((amdgpu_waves_per_eu(2, 2))) void summary_kernel(FwdParams p) {
  constexpr bool OUT = MODE == SM_OUT, CHAIN = MODE != SM_SUMMARY;
  static_assert(!OUT || KDA, "the outputs form is KDA's");
  constexpr int STAGE = stage_elems<KDA, MODE>();
  constexpr int CT = CHAIN ? 1 : summary::CT;  // state tiles per wavefront
  using R_t = Regs<KDA, MODE>;
  __shared__ __attribute__((aligned(16))) bf16 smem[2 * STAGE];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int m = lane & 15, g4 = lane >> 4;
  const int BH = p.B * p.H;
  // workgroup -> (segment, head); segment P-1 needs no summary
  const int seg = blockIdx.x / BH, head = blockIdx.x % BH;
  const int b = head / p.H, h = head % p.H;
  const int n0 = seg * p.NS, n1 = min(p.NT, n0 + p.NS);
  const int cnt = n1 - n0;
  const int HDK = p.H * DK, HDV = p.H * DV;

  const bf16* kg = reinterpret_cast<const bf16*>(p.k) + (long)h * DK;
  const bf16* vg = reinterpret_cast<const bf16*>(p.v) + (long)h * DV;
  const bf16* Tg = reinterpret_cast<const bf16*>(p.T) + (long)head * p.NT * C * C;
  const float* gcg = KDA ? p.dC + (long)head * p.NT * DK : p.gc + (long)head * p.NT * C;
  const bf16* khg = KDA ? reinterpret_cast<const bf16*>(p.kh) + (long)h * DK : nullptr;
  const bf16* qg = reinterpret_cast<const bf16*>(p.q) + (long)h * DK;  // outputs: Q+

  // this lane's pieces of a chunk: piece 64 (NKP wave + i) + lane of the K (V) tile is row q / 16,
  // chunk q % 16; of the T tile, piece 64 (NTP wave + i) + lane
  int offG_k[NKP], offG_v[NKP], offL_k[NKP], offL_t[NTP];
#pragma unroll
  for (int i = 0; i < NKP; ++i) {
    const int q = (NKP * wave + i) * WAVE + lane, r = q >> 4, c = q & 15;
    offG_k[i] = (r * HDK + c * 8) * 2;
    offG_v[i] = (r * HDV + c * 8) * 2;
    offL_k[i] = (r * DK + ((c ^ swz_key(r, 15)) << 3)) * 2;
  }
#pragma unroll
  for (int i = 0; i < NTP; ++i) {
    const int q = (NTP * wave + i) * WAVE + lane, r = q >> 3, c = q & 7;
    offL_t[i] = (T_OFF + r * C + ((c ^ swz_key(r, 7)) << 3)) * 2;
  }

  // loads of chunk n (clamped to the segment's last chunk: past the end they repeat it) into
  // registers; rows past the sequence read 0
  auto load = [&](int n, R_t& R) __attribute__((always_inline)) {
    n = min(n, n1 - 1);
    const long P0 = (long)n * C;
    const unsigned krows = (unsigned)min((long)C, p.Lx - P0);
    const __amdgpu_buffer_rsrc_t kd = buffer_rsrc(const_cast<bf16*>(kg) + ((long)b * p.Lx + P0) * HDK, krows * HDK * 2);
    const __amdgpu_buffer_rsrc_t vd = buffer_rsrc(const_cast<bf16*>(vg) + ((long)b * p.Lx + P0) * HDV, krows * HDV * 2);
    const __amdgpu_buffer_rsrc_t td = buffer_rsrc(const_cast<bf16*>(Tg) + (long)n * C * C, C * C * 2);
#pragma unroll
    for (int i = 0; i < NKP; ++i) R.k[i] = buffer_load16(kd, offG_k[i]);
#pragma unroll
    for (int i = 0; i < NTP; ++i) R.t[i] = buffer_load16(td, ((NTP * wave + i) * WAVE + lane) * 16);
#pragma unroll
    for (int i = 0; i < NKP; ++i) R.v[i] = buffer_load16(vd, offG_v[i]);
    if constexpr (KDA) {
      const __amdgpu_buffer_rsrc_t hd =
          buffer_rsrc(const_cast<bf16*>(khg) + ((long)b * p.Lx + P0) * HDK, krows * HDK * 2);
#pragma unroll
      for (int i = 0; i < NKP; ++i) R.kh[i] = buffer_load16(hd, offG_k[i]);
      R.gc = buffer_load8(buffer_rsrc(const_cast<float*>(gcg) + (long)n * DK, DK * 4), lane * 8);
      if constexpr (OUT) {
        const __amdgpu_buffer_rsrc_t qd =
            buffer_rsrc(const_cast<bf16*>(qg) + ((long)b * p.Lx + P0) * HDK, krows * HDK * 2);
#pragma unroll
        for (int i = 0; i < NKP; ++i) R.q[i] = buffer_load16(qd, offG_k[i]);
      }
    } else {
      R.gc = __builtin_bit_cast(unsigned, buffer_load4(buffer_rsrc(const_cast<float*>(gcg) + (long)n * C, C * 4), lane * 4));
    }
  };

  // registers -> LDS stage; wavefront 0 also writes the gate tables
  auto write_stage = [&](bf16* st, const R_t& R) __attribute__((always_inline)) {
    const unsigned base = lds_addr(st);
#pragma unroll
    for (int i = 0; i < NKP; ++i) {
      write16<0>(base + offL_k[i], R.k[i]);
      write16<V_OFF * 2>(base + offL_k[i], R.v[i]);
    }
#pragma unroll
    for (int i = 0; i < NTP; ++i) write16<0>(base + offL_t[i], R.t[i]);
    if constexpr (KDA) {
#pragma unroll
      for (int i = 0; i < NKP; ++i) write16<K2_OFF * 2>(base + offL_k[i], R.kh[i]);
      if constexpr (OUT) {
#pragma unroll
        for (int i = 0; i < NKP; ++i) write16<Q_OFF * 2>(base + offL_k[i], R.q[i]);
      }
      if (wave == 0) *reinterpret_cast<u32x2*>(reinterpret_cast<float*>(st + G_OFF) + 2 * lane) = R.gc;
    } else if (wave == 0) {
      float* G = reinterpret_cast<float*>(st + G_OFF);
      const float x = __builtin_bit_cast(float, R.gc), xl = __shfl(x, C - 1, WAVE);
      G[lane] = x;
      G[C + lane] = gate_exp(x);
      G[2 * C + lane] = gate_exp(xl - x);
    }
  };

  // per-lane fragment offsets (elements)
  int offK[4];  // K row m, d_k 32 u + 8 g .. + 7 (row blocks further down add 16 DK)
#pragma unroll
  for (int u = 0; u < 4; ++u) offK[u] = swz(m, 32 * u + 8 * g4, DK, 15);
  int offKT[NTS];  // K^T transpose reads: the lane addresses d_k columns dkrow(t, 4i ..)
#pragma unroll
  for (int t = 0; t < NTS; ++t) offKT[t] = swz(4 * g4 + (m >> 2), 32 * (t >> 1) + 4 * (t & 1) + 8 * (m & 3), DK, 15);
  int offT[NB];
#pragma unroll
  for (int kb = 0; kb < NB; ++kb) offT[kb] = swz(m, 16 * kb + 4 * g4, C, 7);

  // state: tiles CT*wave + c (0..7 value, 8..15 transition); accumulator row 4g + j of tile t
  // holds d_k index dkrow(t, 4g + j)
  const int tile0 = CT * wave;
  const bool isv = CHAIN || tile0 < NCT;  // wave-uniform
  auto dkrow = [](int t, int r) { return 32 * (t >> 1) + 8 * (r >> 2) + 4 * (t & 1) + (r & 3); };
  floatx4 S[CT][NTS];
#pragma unroll
  for (int c = 0; c < CT; ++c)
#pragma unroll
    for (int t = 0; t < NTS; ++t)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int row = dkrow(t, 4 * g4 + j), col = 16 * (tile0 + c) + m;
        float x;
        if (CHAIN && p.P > 1) x = p.Sst[(((long)head * p.P + seg) * DK + row) * DV + col];
        else if (isv) x = (seg == 0 && p.S0) ? p.S0[((long)head * DK + row) * DV + col] : 0.f;
        else x = (row == col - DV) ? 1.f : 0.f;  // identity columns of the transition map
        S[c][t][j] = x;
      }
  // the compiler waits for these loads at their first use: use them here, before any prefetch
  // is in flight, so that wait does not also drain the prefetches
#pragma unroll
  for (int c = 0; c < CT; ++c)
#pragma unroll
    for (int t = 0; t < NTS; ++t) asm volatile("" ::"v"(S[c][t]));

  // V transposed reads (D layout of each of this wave's tiles); transition waves read value
  // tiles and discard them
  int offV[CT];
#pragma unroll
  for (int c = 0; c < CT; ++c) offV[c] = swz(4 * g4 + (m >> 2), 16 * (isv ? tile0 + c : c) + 4 * (m & 3), DV, 15);

  // outputs: this lane's fragments of chunk n's Aqk as the B operand of O^T += V~^T Aqk^T, for the
  // token blocks bb and 32-token pairs kp <= bb / 2 at or left of the diagonal: Aqk row 16 bb + m,
  // tokens 32 kp + 4 g .. + 3 and 32 kp + 16 + 4 g .. + 3 (the order of V~'s registers), stored
  // so by the intra kernel
  constexpr int NAQ = OUT ? KDA_AQK_FRAGS : 1;
  u32x4 aqf[NAQ];
  auto load_aq = [&](int n) __attribute__((always_inline)) {
    if constexpr (OUT) {
      n = min(n, n1 - 1);
      const __amdgpu_buffer_rsrc_t ar = buffer_rsrc(
          static_cast<char*>(const_cast<void*>(p.Aqk)) + ((long)head * p.NT + n) * KDA_AQK_CHUNK_BYTES, KDA_AQK_CHUNK_BYTES);
#pragma unroll
      for (int f = 0; f < NAQ; ++f) aqf[f] = buffer_load16(ar, (f * WAVE + lane) * 16);
    }
  };

  // one chunk on stage st; Rw (chunk n+1) goes to the other stage, then takes chunk n+2
  // (ISV: this wavefront's tiles are value columns; transition columns see V = 0 and read no V)
  auto body = [&](int i, R_t& Rw, auto isv_tag) __attribute__((always_inline)) {
    constexpr bool ISV = decltype(isv_tag)::value;
    bf16* st = smem + (i & 1) * STAGE;
    bf16* sn = smem + ((i & 1) ^ 1) * STAGE;
    write_stage(sn, Rw);  // chunk n+1 (the compiler waits for its loads)
    load(n0 + i + 2, Rw);
    __builtin_amdgcn_iglp_opt(1);

    const bf16* K = st + K_OFF;
    const bf16* T = st + T_OFF;
    const bf16* V = st + V_OFF;
    const float* G = reinterpret_cast<const float*>(st + G_OFF);
    const bf16* K2 = st + K2_OFF;

    // X = K S, contracting over d_k in 4 steps of 32
    floatx4 X[CT][NB];
#pragma unroll
    for (int c = 0; c < CT; ++c)
#pragma unroll
      for (int bb = 0; bb < NB; ++bb) X[c][bb] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      bf16x8 Bs[CT];
#pragma unroll
      for (int c = 0; c < CT; ++c) Bs[c] = cat8(cvt4(S[c][2 * u]), cvt4(S[c][2 * u + 1]));
#pragma unroll
      for (int bb = 0; bb < NB; ++bb) {
        const bf16x8 a = lds8(K + 16 * bb * DK + offK[u]);
#pragma unroll
        for (int c = 0; c < CT; ++c) X[c][bb] = mma(a, Bs[c], X[c][bb]);
      }
    }

    // Y = V - gamma X (KDA: V - X; transition columns see V = 0)
    bf16x4 Yb[CT][NB];
#pragma unroll
    for (int bb = 0; bb < NB; ++bb) {
      const floatx4 eg = KDA ? floatx4{1.f, 1.f, 1.f, 1.f} : *reinterpret_cast<const floatx4*>(G + C + 16 * bb + 4 * g4);
#pragma unroll
      for (int c = 0; c < CT; ++c) {
        if constexpr (ISV) {
          const bf16x4 r = read_tr4(V + 16 * bb * DV + offV[c]);
          const floatx4 v4 = floatx4{(float)r[0], (float)r[1], (float)r[2], (float)r[3]};
          Yb[c][bb] = cvt4(v4 - eg * X[c][bb]);
        } else {
          Yb[c][bb] = cvt4(-(eg * X[c][bb]));
        }
      }
    }
    // V~ = T Y (T lower triangular: block pairs at or left of the diagonal), weighted by
    // gamma_C / gamma for the state update (KDA: unweighted)
    bf16x8 DVb[CT][NB / 2];
    bf16x4 dlo[CT];
#pragma unroll
    for (int bb = 0; bb < NB; ++bb) {
      floatx4 vt[CT];
#pragma unroll
      for (int c = 0; c < CT; ++c) vt[c] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kb = 0; kb <= bb; kb += 2) {
        const bf16x8 a = cat8(lds4(T + 16 * bb * C + offT[kb]), lds4(T + 16 * bb * C + offT[kb + 1]));
#pragma unroll
        for (int c = 0; c < CT; ++c) vt[c] = mma(a, cat8(Yb[c][kb], Yb[c][kb + 1]), vt[c]);
      }
      const floatx4 ed = KDA ? floatx4{1.f, 1.f, 1.f, 1.f} : *reinterpret_cast<const floatx4*>(G + 2 * C + 16 * bb + 4 * g4);
#pragma unroll
      for (int c = 0; c < CT; ++c) {
        if (bb & 1) DVb[c][bb >> 1] = cat8(dlo[c], cvt4(vt[c] * ed));
        else dlo[c] = cvt4(vt[c] * ed);
      }
    }

    // outputs, O^T = S^T Q+^T + V~^T Aqk^T per block of 16 tokens (S still the chunk's start state)
    if constexpr (OUT) {
      const bf16* Q = st + Q_OFF;
      const long P0 = (long)(n0 + i) * C;
      const int valid = (int)min((long)C, (long)p.L - P0);
      bf16* Og = reinterpret_cast<bf16*>(p.O) + (((long)b * p.L + P0) * p.H + h) * DV + 16 * tile0 + 4 * g4;
      int f = 0;
#pragma unroll
      for (int bb = 0; bb < NB; ++bb) {
        floatx4 o = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int u = 0; u < 4; ++u)
          o = mma(cat8(cvt4(S[0][2 * u]), cvt4(S[0][2 * u + 1])), lds8(Q + 16 * bb * DK + offK[u]), o);
#pragma unroll
        for (int kp = 0; kp <= bb / 2; ++kp, ++f)
          o = mma(DVb[0][kp], __builtin_bit_cast(bf16x8, aqf[f]), o);
        const int row = 16 * bb + m;
        if (row < valid) *reinterpret_cast<bf16x4*>(Og + (long)row * p.H * DV) = cvt4(o);
      }
      load_aq(n0 + i + 1);  // the next chunk's, into the registers just read
    }

    // S <- gamma_C S + K^T (gamma_C / gamma V~)  (KDA: e^{Gc_C} S + (K e^{Gc_C - Gc})^T V~, row r
    // of S decayed by its channel's factor; a lane's four rows are consecutive channels)
    const float gC = KDA ? 1.f : G[C + C - 1];
    const bf16* Ku = KDA ? K2 : K;
#pragma unroll
    for (int t = 0; t < NTS; ++t) {
      const floatx4 d4 = KDA ? *reinterpret_cast<const floatx4*>(G + dkrow(t, 4 * g4)) : floatx4{gC, gC, gC, gC};
#pragma unroll
      for (int c = 0; c < CT; ++c) S[c][t] *= d4;
#pragma unroll
      for (int kp = 0; kp < NB / 2; ++kp) {
        const bf16x8 a = cat8(read_tr4(Ku + 32 * kp * DK + offKT[t]), read_tr4(Ku + (32 * kp + 16) * DK + offKT[t]));
#pragma unroll
        for (int c = 0; c < CT; ++c) S[c][t] = mma(a, DVb[c][kp], S[c][t]);
      }
    }
    lds_barrier();  // chunk n done (stage st free); chunk n+1 staged
  };

  // prologue: chunk n0 staged, chunk n0+1 in flight
  R_t R;
  load_aq(n0);
  load(n0, R);
  write_stage(smem, R);
  load(n0 + 1, R);
  lds_barrier();
  if (isv) {
    for (int i = 0; i < cnt; ++i) body(i, R, std::true_type{});
  } else {
    for (int i = 0; i < cnt; ++i) body(i, R, std::false_type{});
  }
  if constexpr (CHAIN) {
    if (seg == p.P - 1 && p.S_final)
#pragma unroll
      for (int t = 0; t < NTS; ++t)
#pragma unroll
        for (int j = 0; j < 4; ++j) p.S_final[((long)head * DK + dkrow(t, 4 * g4 + j)) * DV + 16 * tile0 + m] = S[0][t][j];
    return;
  }

  // the summary (S_loc: a lane's four consecutive rows are one 16-byte store; M in bf16, which
  // its consumer rounds it to for its products); segment 0 starts from S0 and needs no
  // transition map
  float* SMs = p.SM + ((long)head * p.P + seg) * DK * (DV + DK);
  // segment 0's start state, which the outputs launch reads instead of S0 (copied here, after the
  // chunk loop, so that the loop's schedule is not disturbed by these stores)
  if (seg == 0 && isv) {
    for (int i = lane + WAVE * (wave & 3); i < DK * DV / 4; i += 4 * WAVE) {
      const long off = (long)head * DK * DV + 4L * i;
      const floatx4 x = p.S0 ? *reinterpret_cast<const floatx4*>(p.S0 + off) : floatx4{0.f, 0.f, 0.f, 0.f};
      *reinterpret_cast<floatx4*>(p.Sst + (long)head * p.P * DK * DV + 4L * i) = x;
    }
  }
#pragma unroll
  for (int c = 0; c < CT; ++c)
#pragma unroll
    for (int t = 0; t < NTS; ++t) {
      const int row = dkrow(t, 4 * g4), col = 16 * (tile0 + c) + m;
      if (isv) {
        *reinterpret_cast<floatx4*>(SMs + sloc_index(row, col, DK)) = S[c][t];
      } else if (seg > 0) {
        bf16* Ms = reinterpret_cast<bf16*>(SMs + DV * DK);
#pragma unroll
        for (int j = 0; j < 4; ++j) Ms[mfrag_index<mfrag_width<bf16, DK>()>(row + j, col - DV, DK)] = (bf16)S[c][t][j];
        if (p.SMr) {  // M^T: the lane's four rows are four consecutive k of one row of M^T
          bf16* Mt = reinterpret_cast<bf16*>(p.SMr + ((long)head * p.P + p.P - 1 - seg) * DK * (DV + DK) + DV * DK);
          *reinterpret_cast<bf16x4*>(Mt + mfrag_index<mfrag_width<bf16, DK>()>(col - DV, row, DK)) =
              bf16x4{(bf16)S[c][t][0], (bf16)S[c][t][1], (bf16)S[c][t][2], (bf16)S[c][t][3]};
        }
      }
    }
}

}  // namespace summary

bool scan_summary_fast_applies(const FwdParams& p, bool bf16_in) {
  return bf16_in && p.DK == summary::DK && p.DV == summary::DV && p.C == summary::C && p.NT >= 1;
}

hipError_t launch_scan_summary_fast(const FwdParams& p, hipStream_t st) {
  if (p.P <= 1) return hipSuccess;
  hipLaunchKernelGGL((summary::summary_kernel<false, summary::SM_SUMMARY>), dim3((unsigned)((p.P - 1) * p.B * p.H)), dim3(summary::NW * WAVE), 0, st, p);
  return hipGetLastError();
}

hipError_t launch_scan_outputs_kda(const FwdParams& p, hipStream_t st) {
  if (p.DK != summary::DK || p.DV != summary::DV || p.C != summary::C) return hipErrorInvalidValue;
  hipLaunchKernelGGL((summary::summary_kernel<true, summary::SM_OUT>), dim3((unsigned)(p.P * p.B * p.H)),
                     dim3(summary::NW * WAVE), 0, st, p);
  return hipGetLastError();
}

hipError_t launch_scan_summary_fast_kda(const FwdParams& p, hipStream_t st) {
  if (p.P <= 1) return hipSuccess;
  if (p.DK != summary::DK || p.DV != summary::DV || p.C != summary::C) return hipErrorInvalidValue;
  hipLaunchKernelGGL((summary::summary_kernel<true, summary::SM_SUMMARY>), dim3((unsigned)((p.P - 1) * p.B * p.H)), dim3(summary::NW * WAVE), 0, st, p);
  return hipGetLastError();
}

}  // namespace delta
