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
// order is XOR-swizzled per row so that the reads of 16 consecutive rows, and
// the transposed reads of rows {8g + e : g, e < 4}, hit distinct banks.
//   SW = 1: granule ^= row & 7
//   SW = 2: granule ^= (row ^ (row >> 3)) & 7
//   SW = 3: granule ^= (row & 15) ^ (((row >> 4) & 1) << 2)   (16+ granules per row)
template <typename T, int ROWS, int COLS, int SW>
struct Tile {
  static constexpr int ROWB = COLS * (int)sizeof(T);
  static constexpr int GPR = ROWB / 16;
  static constexpr int TPG = 16 / (int)sizeof(T);
  static constexpr int BYTES = ROWS * ROWB;
  static_assert(GPR >= 8, "swizzle needs at least 8 granules per row");
  static_assert(SW != 3 || GPR >= 16, "SW=3 needs 16 granules per row");
  __device__ static inline int swz(int row) {
    if (SW == 1) return row & 7;
    if (SW == 2) return (row ^ (row >> 3)) & 7;
    return (row & 15) ^ (((row >> 4) & 1) << 2);
  }
  // byte offset of element (row, col)
  __device__ static inline int off(int row, int col) {
    return row * ROWB + (((col / TPG) ^ swz(row)) << 4) + (col % TPG) * (int)sizeof(T);
  }
};

// ---------------------------------------------------------------- synchronisation
// Workgroup barrier WITHOUT a memory fence, preceded by a wait until at most
// N of this wave's vector-memory operations are outstanding and all its LDS
// operations are done.  Vector loads (including loads that write LDS
// directly) complete in issue order, so N = "loads issued after the ones we
// need" is enough.  The asm statement is also a compiler-level memory barrier.
template <int N>
__device__ inline void wait_vm_barrier() {
  asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" ::"n"(N) : "memory");
}
__device__ inline void lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// 16 bytes per lane from global memory straight into LDS: lane l's bytes
// land at lds_block + 16 l (lds_block must be wave-uniform; M0 holds it).
// Issued as inline asm so that the compiler does not treat later
// transposing LDS reads as aliasing an in-flight load and wait for every
// outstanding load before them: completion is waited for explicitly
// (wait_vm_barrier) before a chunk is read.
__device__ inline void dma16(const void* gsrc, char* lds_block) {
  const unsigned lds = __builtin_amdgcn_readfirstlane(
      (unsigned)(size_t)(__attribute__((address_space(3))) char*)lds_block);
  asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(gsrc), "s"(lds)
               : "memory", "m0");
}

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

// ---------------------------------------------------------------- transposed operand
// MFMA operand that contracts over tokens, read from a token-major tile:
// lane (g = lane / 16, n = lane % 16) receives column col0 + n of the E
// consecutive tokens j0 + E g .. j0 + E g + E - 1 (the lane's contraction
// slots).  bf16: two ds_read_b64_tr_b16.  Within each 16-lane group that
// instruction hands output lane d the element (d % 4) of source lane
// 4 e + d / 4, e = 0..3; so source lane s points at token j0 + 8 g + s / 4
// (+ 4 for the second read) and columns col0 + 4 (s % 4) .. + 3.
// fp32: one scalar read of token j0 + g, column col0 + n.
template <typename T, class TL>
__device__ inline typename Elt<T>::op_t tr_op(const char* tile, int j0, int col0, int lane) {
  const int g = lane >> 4, s = lane & 15;
  if constexpr (sizeof(T) == 2) {
    typedef short v4i16 __attribute__((ext_vector_type(4)));
    typedef __attribute__((address_space(3))) v4i16 lds_v4;
    const int row = j0 + 8 * g + (s >> 2);
    const int col = col0 + 4 * (s & 3);
    const v4i16 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4*)(tile + TL::off(row, col)));
    const v4i16 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4*)(tile + TL::off(row + 4, col)));
    typedef short v8i16 __attribute__((ext_vector_type(8)));
    const v8i16 both = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
    return __builtin_bit_cast(bf16x8, both);
  } else {
    return *reinterpret_cast<const float*>(tile + TL::off(j0 + g, col0 + s));
  }
}

}  // namespace la
