// Device helpers shared by the delta-rule kernels (gfx950 / CDNA4 only).
//
// MFMA fragments follow the gfx950 lane layouts of the 16x16 output tiles:
//   v_mfma_f32_16x16x32_bf16: lane l holds A[l%16][8*(l/16) + 0..7],
//                             B[8*(l/16) + 0..7][l%16], D[4*(l/16) + 0..3][l%16]
//   v_mfma_f32_16x16x4_f32:   lane l holds A[l%16][l/16], B[l/16][l%16], D as above.
// Operands are kept in LDS "K-contiguous": an A operand as [m][k] rows, a B operand
// transposed as [n][k] rows, so each lane's fragment is one contiguous LDS read (Tile below).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace delta {

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float floatx4 __attribute__((ext_vector_type(4)));

constexpr int WAVE = 64;

// Element traits: how one MFMA k-step reads its operands from a K-contiguous row.
template <typename E>
struct Mfma;

template <>
struct Mfma<bf16> {
  static constexpr int KSTEP = 32;  // k covered by one instruction
  static constexpr int KTAIL = 16;  // a 16-deep instruction finishes K % 32 == 16
  typedef bf16x8 frag;
  __device__ static inline floatx4 mma(frag a, frag b, floatx4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
  }
  // v_mfma_f32_16x16x16_bf16: lane l holds A[l%16][4*(l/16) + 0..3], B[4*(l/16) + 0..3][l%16];
  // a and b point at this lane's four elements
  __device__ static inline floatx4 mma_tail(const bf16* a, const bf16* b, floatx4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(*reinterpret_cast<const bf16x4*>(a),
                                                      *reinterpret_cast<const bf16x4*>(b), c, 0, 0, 0);
  }
};

template <>
struct Mfma<float> {
  static constexpr int KSTEP = 4;
  static constexpr int KTAIL = 4;
  typedef float frag;
  __device__ static inline floatx4 mma(frag a, frag b, floatx4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
  }
  __device__ static inline floatx4 mma_tail(const float* a, const float* b, floatx4 c) { return mma(*a, *b, c); }
};

// Layout of a segment summary (S_loc, M) in the order the start-state combine reads it: every
// wavefront load there is 64 lanes x one contiguous 16-byte piece (or 8 bytes), so a load covers
// whole cache lines.  Lane (g, m) of the wavefront for rows 16 t .. 16 t + 15 takes:
//   S_loc, column tile ct: rows 16 t + 4 g .. + 3 of column 16 ct + m (fp32), at
//     sloc_index(r, c) = ((c / 16 * (DK / 16) + r / 16) * 64 + (r % 16) / 4 * 16 + c % 16) * 4 + r % 4;
//   M, contraction block i: its A fragment, row 16 t + m, k = i KB + g PW .. + PW - 1, at
//     mfrag_index(r, k) = ((r / 16 * (DK / KB) + k / KB) * 64 + (k % KB) / PW * 16 + r % 16) * PW + k % PW
//   with PW = 8 elements (bf16 products on the 32-deep MFMA, KB = 32) or 4 (KB = 16).
__host__ __device__ constexpr int sloc_index(int r, int c, int DK) {
  return ((c / 16 * (DK / 16) + r / 16) * 64 + (r % 16) / 4 * 16 + c % 16) * 4 + r % 4;
}
template <int PW>
__host__ __device__ constexpr int mfrag_index(int r, int k, int DK) {
  return ((r / 16 * (DK / (4 * PW)) + k / (4 * PW)) * 64 + (k % (4 * PW)) / PW * 16 + r % 16) * PW + k % PW;
}
// piece width of M for element type E and key width DK (bf16 products need DK >= 32)
template <typename E, int DK>
__host__ __device__ constexpr int mfrag_width() {
  return sizeof(E) == 2 && DK >= 32 ? 8 : 4;
}

// XOR key of row r for a swizzle mask: the 16-byte chunks of row r are permuted by chunk ^ key.
// With 16 chunks per row (256-byte rows, mask 15) the key is the linear map over GF(2) that
// takes row bits 0, 1, 2, 3 to 0x2, 0x6, 0xd, 0xe.  It was chosen by timing all 20160 invertible
// 4-bit linear keys on gfx950 for the three reads of such tiles in the chain kernels: 16-byte
// fragment reads of 16 rows at one logical chunk (238 B/cycle/CU, conflict-free), and transpose
// reads of column runs of the key tile (122, the ds_read_b64_tr_b16 rate) and of the value tile
// (189); swapping the two 2-bit fields of the row, the previous key, gave 124 / 121 / 121.  With 8
// chunks per row (128-byte rows, mask 7) two consecutive rows share one 256-byte bank sweep, so
// the key is (r / 2) % 8: 16 rows read at one chunk fall on 16 distinct bank groups.
__host__ __device__ constexpr int swz_key(int r, int mask) {
  return mask == 15 ? (((r & 1) ? 0x2 : 0) ^ ((r & 2) ? 0x6 : 0) ^ ((r & 4) ? 0xd : 0) ^ ((r & 8) ? 0xe : 0))
       : mask == 7 ? ((r >> 1) & 7)
                   : (r & mask);
}

// A matrix tile in LDS.  Element (r, e) lives at p + r * ld + swizzled column, where the
// 16-byte chunks of a row are permuted by XOR with swz_key(r, mask).  With bf16 operands each lane
// of an MFMA fragment read takes one 16-byte chunk of one of 16 rows; on gfx950 such a read
// is free of bank conflicts when the rows are 128 or 256 bytes long and chunks are swizzled
// (mask = chunks per row - 1), or when the row stride is an odd multiple of 32 bytes
// (measured with rocprofv3 SQ_LDS_BANK_CONFLICT).  TileLayout picks one of the two.
template <typename E>
struct Tile {
  E* p;
  int ld;    // row stride in elements
  int mask;  // chunk swizzle mask (0 = none)
  __device__ inline E* at(int r, int e) const {
    constexpr unsigned CH = 16 / sizeof(E);  // elements per 16-byte chunk
    const unsigned u = e;                      // column indices are never negative: shifts, not divides
    return p + r * ld + (int)((((u / CH) ^ (unsigned)swz_key(r, mask))) * CH + u % CH);
  }
};

// Smallest odd multiple of 32 that is >= b.
constexpr int odd_multiple_of_32(int b) {
  return ((b + 31) / 32) % 2 ? (b + 31) / 32 * 32 : (b + 31) / 32 * 32 + 32;
}

// Layout of a tile whose rows hold L elements of E.
template <typename E, int L>
struct TileLayout {
  static constexpr int BYTES = L * (int)sizeof(E);
  static constexpr bool SWZ = sizeof(E) == 2 && (BYTES == 128 || BYTES == 256);
  static constexpr int MASK = SWZ ? BYTES / 16 - 1 : 0;
  // otherwise pad: bf16 rows to an odd multiple of 32 bytes, fp32 rows by 16 bytes
  static constexpr int LD = SWZ ? L : (sizeof(E) == 2 ? odd_multiple_of_32(BYTES) / 2 : L + 4);
};

template <typename E, int L>
__device__ inline Tile<E> make_tile(E* p) {
  return Tile<E>{p, TileLayout<E, L>::LD, TileLayout<E, L>::MASK};
}

// Unpadded layout for tiles filled by direct-to-LDS loads (each such load writes 64 consecutive
// 16-byte chunks, so rows must be contiguous).  Chunks are XOR-swizzled with the row number
// within the largest power-of-two group of chunks that divides the row (at most 16), which keeps
// every swizzled chunk inside its row.
constexpr int pow2_part(int x) { return (x & -x) > 16 ? 16 : (x & -x); }
template <typename E, int L>
struct PackedLayout {
  static constexpr int CPR = L * (int)sizeof(E) / 16;  // 16-byte chunks per row
  static constexpr int LD = L;
  static constexpr int MASK = pow2_part(CPR) - 1;
};

template <typename E, int L>
__device__ inline Tile<E> make_packed_tile(E* p) {
  return Tile<E>{p, PackedLayout<E, L>::LD, PackedLayout<E, L>::MASK};
}

typedef __attribute__((address_space(3))) void* lds_ptr;

// Direct global -> LDS copy of 16 bytes per lane (global_load_lds_dwordx4).  The LDS address is
// wave-uniform: lane l writes lds_base + 16 l.  Completion is tracked by vmcnt.
__device__ inline void copy16_to_lds(const void* g, void* lds_base) {
  __builtin_amdgcn_global_load_lds(g, (lds_ptr)lds_base, 16, 0, 0);
}

// Wait until every vector memory operation of this wave has completed (vmcnt = 0).
__device__ inline void wait_vmem() { __builtin_amdgcn_s_waitcnt(0x0F70); }
// Waits until at most k (wave-uniform, clamped to [0, 15]) of this wave's vector memory loads are
// outstanding: loads complete in issue order, so all but the k most recent have landed.
template <int K = 15>
__device__ inline void wait_vmem_upto(int k) {
  if constexpr (K == 0) {
    __builtin_amdgcn_s_waitcnt(0x0F70);
  } else {
    if (k >= K) __builtin_amdgcn_s_waitcnt(0x0F70 | K);
    else wait_vmem_upto<K - 1>(k);
  }
}

// Copies rows [0, nrows) of a row-major global matrix (rows of L elements, row stride gstride
// elements) into a PackedLayout tile with direct-to-LDS loads issued by wave w of nw waves.
// Rows at or past `valid` read row 0 instead (finite data that the caller's products cancel).
// Chunks of a row at or past `cvalid` (16-byte chunks) read the row's first chunk instead.
template <typename E, int L>
__device__ inline void copy_rows_to_lds(E* tile, const E* g, int gstride, int nrows, int valid, int w, int nw,
                                        int lane, int cvalid = PackedLayout<E, L>::CPR) {
  constexpr int CPR = PackedLayout<E, L>::CPR, MASK = PackedLayout<E, L>::MASK, VEC = 16 / sizeof(E);
  const int total = nrows * CPR;
  for (int i = w; i * WAVE < total; i += nw) {
    const int q = i * WAVE + lane;
    const int r = q / CPR, pc = q % CPR;
    const int src = r < valid ? r : 0;
    const int lc = pc ^ swz_key(r, MASK);
    if (q < total) copy16_to_lds(g + src * gstride + (lc < cvalid ? lc : 0) * VEC, tile + i * WAVE * VEC);
  }
}

// The direct-to-LDS copies of one tile that one of `nw` waves issues, with the per-lane source
// byte offsets worked out once: copy instruction i = w + nw s (s < NS) moves LDS chunks
// [64 i, 64 i + 64) of the tile; rows are assumed valid (a partial tile takes copy_rows_to_lds).
// Issuing then costs no vector ALU work: a uniform base plus a 32-bit lane offset per copy.
template <typename E, int L, int ROWS, int NW>
struct CopyPlan {
  static constexpr int CPR = PackedLayout<E, L>::CPR, MASK = PackedLayout<E, L>::MASK, VEC = 16 / sizeof(E);
  static constexpr int NS = ((ROWS * CPR + WAVE - 1) / WAVE + NW - 1) / NW;
  unsigned off[NS];
  int n;  // copies this wave issues
  __device__ inline void init(int gstride, int nrows, int w, int lane, int cvalid = CPR) {
    const int total = nrows * CPR;
    n = 0;
#pragma unroll
    for (int s = 0; s < NS; ++s) {
      const int q = (w + NW * s) * WAVE + lane;
      const int r = q / CPR, lc = (q % CPR) ^ swz_key(r, MASK);
      off[s] = q < total ? (unsigned)((r * gstride + (lc < cvalid ? lc : 0) * VEC) * (int)sizeof(E)) : ~0u;
      if ((w + NW * s) * WAVE < total) n = s + 1;
    }
  }
  __device__ inline void issue(E* tile, const E* g, int w) const {
#pragma unroll
    for (int s = 0; s < NS; ++s)
      if (s < n && off[s] != ~0u)
        copy16_to_lds(reinterpret_cast<const char*>(g) + off[s], tile + (w + NW * s) * WAVE * VEC);
  }
};

// ds_read_b64_tr_b16 (gfx950): within each group of 16 lanes, lane i receives element i % 4 of
// the 4-element (8-byte) pieces addressed by lanes i / 4, 4 + i / 4, 8 + i / 4, 12 + i / 4 of its
// group, in that order.  (Lane semantics measured on the device.)
__device__ inline bf16x4 read_tr4(const bf16* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4bf16((__attribute__((address_space(3))) bf16x4*)(p));
}

// C(16x16) += M^T(16 x K) * B(K x 16) for bf16, where M is a row-major [K][.] tile (here the
// key tile, K = positions) and the A operand is M^T[d0 .. d0+16)[0 .. K): transpose reads give
// each lane its column run of M directly.  B^T rows b_r0.. of tile b are K-contiguous.
// One instruction shape per chain, as in mma_tile.
template <int K>
__device__ inline floatx4 mma_tn(floatx4 acc, const Tile<bf16>& m, int d0, const Tile<bf16>& b, int b_r0, int lane) {
  const int g = lane >> 4, i = lane & 15;
  const int e = d0 + 4 * (i & 3);  // column of the 8-byte piece this lane addresses
  if constexpr (K % 32 == 0) {
#pragma unroll
    for (int k0 = 0; k0 < K; k0 += 32) {
      const int r = k0 + 8 * g + (i >> 2);
      const bf16x4 lo = read_tr4(m.at(r, e)), hi = read_tr4(m.at(r + 4, e));
      const bf16x8 a = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
      acc = Mfma<bf16>::mma(a, *reinterpret_cast<const bf16x8*>(b.at(b_r0 + i, k0 + 8 * g)), acc);
    }
  } else {
#pragma unroll
    for (int k0 = 0; k0 < K; k0 += 16) {
      const bf16x4 a = read_tr4(m.at(k0 + 4 * g + (i >> 2), e));
      acc = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, *reinterpret_cast<const bf16x4*>(b.at(b_r0 + i, k0 + 4 * g)),
                                                      acc, 0, 0, 0);
    }
  }
  return acc;
}

// C(16x16) += A(16 x K) * B(K x 16): A rows a_r0.. of tile a (K along the row), B^T rows
// b_r0.. of tile b (the B operand stored transposed, K along the row).  K must be a multiple
// of 16 (of 4 for float).  One accumulation chain uses one instruction shape: a contraction
// whose K is not a multiple of the long step runs entirely on the 16-deep instruction.  On
// gfx950 an MFMA that reads the previous MFMA's result as its accumulator input needs wait
// states when the two differ in shape (16x16x32 vs 16x16x16 bf16, either order), and the
// compiler issues such a pair back to back: measured, about half the entries come out wrong.
// Same-shape pairs, separate accumulators, or 16 wait states between give exact sums.
template <typename E>
__device__ inline floatx4 mma_tile(floatx4 acc, const Tile<E>& a, int a_r0, const Tile<E>& b, int b_r0, int K,
                                   int lane) {
  const int ra = a_r0 + (lane & 15), rb = b_r0 + (lane & 15);
  if (K % Mfma<E>::KSTEP == 0) {
    const int ko = (Mfma<E>::KSTEP / 4) * (lane >> 4);  // 8 (bf16) or 1 (fp32) per lane group
    for (int k0 = 0; k0 < K; k0 += Mfma<E>::KSTEP)
      acc = Mfma<E>::mma(*reinterpret_cast<const typename Mfma<E>::frag*>(a.at(ra, k0 + ko)),
                         *reinterpret_cast<const typename Mfma<E>::frag*>(b.at(rb, k0 + ko)), acc);
  } else {
    const int ko = (Mfma<E>::KTAIL / 4) * (lane >> 4);
    for (int k0 = 0; k0 < K; k0 += Mfma<E>::KTAIL) acc = Mfma<E>::mma_tail(a.at(ra, k0 + ko), b.at(rb, k0 + ko), acc);
  }
  return acc;
}

template <typename E>
__device__ inline E to_elem(float x);
template <>
__device__ inline float to_elem<float>(float x) { return x; }
template <>
__device__ inline bf16 to_elem<bf16>(float x) { return (bf16)x; }  // round to nearest even

template <typename E>
__device__ inline float to_float(E x) { return (float)x; }

// Store 4 consecutive elements (one lane's D column run, transposed) to LDS.
template <typename E>
__device__ inline void store4(E* dst, float a, float b, float c, float d);
template <>
__device__ inline void store4<float>(float* dst, float a, float b, float c, float d) {
  *reinterpret_cast<floatx4*>(dst) = floatx4{a, b, c, d};
}
template <>
__device__ inline void store4<bf16>(bf16* dst, float a, float b, float c, float d) {
  *reinterpret_cast<bf16x4*>(dst) = bf16x4{(bf16)a, (bf16)b, (bf16)c, (bf16)d};
}

// 16-byte vector type for global<->LDS copies.
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// Raw buffer resource over [base, base + bytes) (stride 0; descriptor word 3 = 32-bit data
// format, the raw-buffer setting of gfx9-family parts).  A buffer access whose byte offset lies
// outside the range is dropped by the hardware's range check, so rows past the end of a
// sequence can be masked with no branch and no per-lane exec mask.
__device__ inline __amdgpu_buffer_rsrc_t buffer_rsrc(void* base, int bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(base, 0, bytes, 0x00020000);
}
__device__ inline void buffer_store8(__amdgpu_buffer_rsrc_t r, int off, bf16x4 x) {
  __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(u32x2, x), r, off, 0, 0);
}
__device__ inline u32x4 buffer_load16(__amdgpu_buffer_rsrc_t r, int off) {  // 0 outside the range
  return __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0);
}
__device__ inline u32x2 buffer_load8(__amdgpu_buffer_rsrc_t r, int off) {   // 0 outside the range
  return __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, 0);
}
__device__ inline float buffer_load4(__amdgpu_buffer_rsrc_t r, int off) {   // 0 outside the range
  return __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(r, off, 0, 0));
}
__device__ inline void buffer_store16(__amdgpu_buffer_rsrc_t r, int off, floatx4 x) {
  __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, x), r, off, 0, 0);
}
__device__ inline void buffer_store4(__amdgpu_buffer_rsrc_t r, int off, float x) {
  __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, x), r, off, 0, 0);  // data operand is a u32
}

// Barrier without the compiler's workgroup fence: waits for this wave's own LDS operations
// (and, for barrier_all, its vector memory operations) and then synchronises.  Global loads
// still in flight stay in flight (the compiler waits for them where their registers are used).
__device__ inline void barrier_lds() {
  __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
  asm volatile("s_barrier" ::: "memory");
}
__device__ inline void barrier_all() {
  __builtin_amdgcn_s_waitcnt(0x0070);  // vmcnt(0) lgkmcnt(0)
  asm volatile("s_barrier" ::: "memory");
}

__device__ inline float gate_exp(float x) { return __builtin_amdgcn_exp2f(x * 1.4426950408889634f); }

// Lower bound applied to each token's log gate on the chunkwise path.  exp(-150) ~ 7e-66 is far
// below the smallest float32 subnormal (1.4e-45), so any decay spanning a clamped position is
// exactly 0; a true log gate below the floor differs from it by a factor under 1e-65.
constexpr float LOG_GATE_FLOOR = -150.f;

// Inclusive prefix sum across the 64 lanes of a wave.
__device__ inline float wave_inclusive_scan(float x, int lane) {
#pragma unroll
  for (int off = 1; off < WAVE; off <<= 1) {
    float y = __shfl_up(x, off, WAVE);
    if (lane >= off) x += y;
  }
  return x;
}

__device__ inline float wave_sum(float x) {
#pragma unroll
  for (int off = WAVE / 2; off > 0; off >>= 1) x += __shfl_xor(x, off, WAVE);
  return x;
}

}  // namespace delta
