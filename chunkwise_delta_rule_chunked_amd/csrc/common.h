// Device helpers shared by the delta-rule kernels (gfx950 / CDNA4 only).
//
// MFMA fragments follow the gfx950 lane layouts of the 16x16 output tiles:
//   v_mfma_f32_16x16x32_bf16: lane l holds A[l%16][8*(l/16) + 0..7],
//                             B[8*(l/16) + 0..7][l%16], D[4*(l/16) + 0..3][l%16]
//   v_mfma_f32_16x16x4_f32:   lane l holds A[l%16][l/16], B[l/16][l%16], D as above.
// Operands are kept in LDS "K-contiguous": an A operand as [m][k] rows, a B operand
// transposed as [n][k] rows, so each lane's fragment is one contiguous LDS read.
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
  // fragment of row `row` (pointer to its first element), k-step starting at k0
  __device__ static inline frag load(const bf16* row, int k0, int lane) {
    return *reinterpret_cast<const bf16x8*>(row + k0 + 8 * (lane >> 4));
  }
  __device__ static inline floatx4 mma(frag a, frag b, floatx4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
  }
  // v_mfma_f32_16x16x16_bf16: lane l holds A[l%16][4*(l/16) + 0..3], B[4*(l/16) + 0..3][l%16]
  __device__ static inline floatx4 mma_tail(const bf16* a, const bf16* b, int k0, int lane, floatx4 c) {
    bf16x4 fa = *reinterpret_cast<const bf16x4*>(a + k0 + 4 * (lane >> 4));
    bf16x4 fb = *reinterpret_cast<const bf16x4*>(b + k0 + 4 * (lane >> 4));
    return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(fa, fb, c, 0, 0, 0);
  }
};

template <>
struct Mfma<float> {
  static constexpr int KSTEP = 4;
  static constexpr int KTAIL = 4;
  typedef float frag;
  __device__ static inline frag load(const float* row, int k0, int lane) {
    return row[k0 + (lane >> 4)];
  }
  __device__ static inline floatx4 mma(frag a, frag b, floatx4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
  }
  __device__ static inline floatx4 mma_tail(const float* a, const float* b, int k0, int lane, floatx4 c) {
    return mma(load(a, k0, lane), load(b, k0, lane), c);
  }
};

// C(16x16) += A(16 x K) * B(K x 16): A rows at a_row0 (stride lda elements),
// B^T rows at b_row0 (stride ldb).  K must be a multiple of 16 (of 4 for float).
// One accumulation chain uses one instruction shape: a contraction whose K is not a
// multiple of the long step runs entirely on the 16-deep instruction (a dependent
// 16x16x32 -> 16x16x16 pair on one accumulator gave intermittently wrong sums on gfx950).
template <typename E>
__device__ inline floatx4 mma_tile(floatx4 acc, const E* a_row0, int lda, const E* b_row0, int ldb,
                                   int K, int lane) {
  const E* a = a_row0 + (lane & 15) * lda;
  const E* b = b_row0 + (lane & 15) * ldb;
  if (K % Mfma<E>::KSTEP == 0) {
    for (int k0 = 0; k0 < K; k0 += Mfma<E>::KSTEP)
      acc = Mfma<E>::mma(Mfma<E>::load(a, k0, lane), Mfma<E>::load(b, k0, lane), acc);
  } else {
    for (int k0 = 0; k0 < K; k0 += Mfma<E>::KTAIL) acc = Mfma<E>::mma_tail(a, b, k0, lane, acc);
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
