// la_device.h -- device-side building blocks shared by the chunk kernels.
//
// Target: gfx950 (CDNA4), wave64.  Matrix products use the 16x16 MFMA
// instructions with fp32 accumulation:
//   bf16 inputs: v_mfma_f32_16x16x32_bf16 (8 bf16 per lane per operand)
//   fp32 inputs: v_mfma_f32_16x16x4_f32   (1 fp32 per lane per operand)
// Operand layout (both): lane l feeds row / column (l % 16) of the 16-wide
// A / B tile and the lane group g = l / 16 feeds a fixed set of E slots of
// the contraction dimension; the accumulator tile gives lane l column
// (l % 16) and rows 4 g .. 4 g + 3.  Since A and B use the same slot
// assignment, any bijection from (g, e) to the contraction index computes the
// same product -- the kernels use that to feed accumulator tiles straight back
// as operands without a trip through LDS.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace la {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));

constexpr int CH = 64;     // tokens per chunk
constexpr int NTHR = 256;  // threads per workgroup: 4 waves of 64

// ---------------------------------------------------------------- element traits
template <typename T>
struct Elt;

template <>
struct Elt<__bf16> {
  static constexpr int E = 8;  // operand elements per lane
  typedef bf16x8 op_t;
  __device__ static inline f32x4 mfma(op_t a, op_t b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
  }
  __device__ static inline float to_f(__bf16 x) { return (float)x; }
  __device__ static inline __bf16 from_f(float x) { return (__bf16)x; }
};

template <>
struct Elt<float> {
  static constexpr int E = 1;
  typedef float op_t;
  __device__ static inline f32x4 mfma(op_t a, op_t b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
  }
  __device__ static inline float to_f(float x) { return x; }
  __device__ static inline float from_f(float x) { return x; }
};

// ---------------------------------------------------------------- LDS tiles
// A ROWS x COLS tile of T in LDS, each row cut into 16-byte granules whose
// order is XOR-swizzled per row so that the operand reads of 8 consecutive
// rows and the transposed writes of one column hit distinct banks.
//   SW = 1: granule ^= row & 7
//   SW = 2: granule ^= (row ^ (row >> 3)) & 7
template <typename T, int ROWS, int COLS, int SW>
struct Tile {
  static constexpr int ROWB = COLS * (int)sizeof(T);
  static constexpr int GPR = ROWB / 16;
  static constexpr int TPG = 16 / (int)sizeof(T);
  static constexpr int BYTES = ROWS * ROWB;
  static_assert(GPR >= 8, "swizzle needs at least 8 granules per row");
  __device__ static inline int swz(int row) {
    return (SW == 1 ? (row & 7) : ((row ^ (row >> 3)) & 7));
  }
  // byte offset of element (row, col)
  __device__ static inline int off(int row, int col) {
    return row * ROWB + (((col / TPG) ^ swz(row)) << 4) + (col % TPG) * (int)sizeof(T);
  }
};

// ---------------------------------------------------------------- small helpers
__device__ inline float pow_lam(float lg2, float n) {
  // lambda^n = 2^(n log2 lambda); only non-negative n are formed.
  return exp2f(n * lg2);
}

template <typename T>
__device__ inline void lds_store16(char* lds, int off, u32x4 v) {
  *reinterpret_cast<u32x4*>(lds + off) = v;
}

// operand fetch of E contiguous elements (16 bytes for bf16, 4 for fp32)
template <typename T>
__device__ inline typename Elt<T>::op_t lds_op(const char* lds, int off) {
  return *reinterpret_cast<const typename Elt<T>::op_t*>(lds + off);
}

}  // namespace la
