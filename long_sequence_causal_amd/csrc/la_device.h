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
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
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
// A ROWS x COLS tile of T in LDS, token-major, each row padded by 16 bytes.
// With a row stride of an odd number of 16-byte granules, 16 consecutive rows
// start on 16 different bank groups, so the reads this code makes -- 16 B
// (or two 8 B pieces) from each of 16 consecutive rows, and transposing
// reads over 16 consecutive rows -- take the minimum number of LDS cycles.
// Addresses stay affine in (row, col): unrolled accesses share one base
// register and differ by immediates.
template <typename T, int ROWS, int COLS>
struct PadTile {
  static constexpr int ROWB = COLS * (int)sizeof(T);
  static constexpr int RS = ROWB + 16;  // row stride in bytes
  static constexpr int G = RS / 16;     // 16-byte granules per row (odd)
  static constexpr int BYTES = ROWS * RS;
  static_assert(ROWB % 32 == 0 && (G & 1) == 1, "row stride must be an odd number of granules");
  __device__ static inline int off(int row, int col) { return row * RS + col * (int)sizeof(T); }
};

// The 10 nonzero 16x16 blocks (key block jb <= query block ib) of the 64x64
// intra-chunk score matrix P, stored compactly, block (jb, ib) at slot
// ib (ib + 1) / 2 + jb.  Inside a block the 16 keys are split into 4 slabs of
// 4 (the keys one MFMA lane group holds, see perm16), each slab stored
// [query row][4 keys]: a 16-lane group touching one slab covers 16
// consecutive 8-byte (bf16) pieces, so 8-byte accesses by lanes 0..31 or
// 32..63 hit all 64 banks once.
template <typename T>
struct PBlocks {
  static constexpr int SLAB = 16 * 4 * (int)sizeof(T);
  static constexpr int BLK = 4 * SLAB;
  static constexpr int BYTES = 10 * BLK;
  __device__ static inline int at(int ib, int jb, int slab, int row) {
    return (ib * (ib + 1) / 2 + jb) * BLK + slab * SLAB + row * 4 * (int)sizeof(T);
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

// LDS address (byte offset in the workgroup's LDS) of a pointer into a
// __shared__ array.
__device__ inline unsigned lds_address(const void* p) {
  return (unsigned)(size_t)(const __attribute__((address_space(3))) char*)p;
}

// 16 bytes per lane from global memory straight into LDS: lane l reads
// sbase + voff (sbase wave-uniform, voff a 32-bit byte offset) and its bytes
// land at LDS address lds + 16 l (lds wave-uniform; M0 holds it).
// Issued as inline asm so that the compiler does not treat later
// transposing LDS reads as aliasing an in-flight load and wait for every
// outstanding load before them: completion is waited for explicitly
// (wait_vm_barrier) before a chunk is read.
__device__ inline void dma16(const void* sbase, unsigned voff, unsigned lds) {
  asm volatile("s_mov_b32 m0, %2\n\tglobal_load_lds_dwordx4 %0, %1" ::"v"(voff), "s"(sbase),
               "s"(__builtin_amdgcn_readfirstlane(lds))
               : "memory", "m0");
}

// 4 bytes per lane from global memory straight into LDS: lane l's 4 B land
// at LDS address lds + 4 l (as dma16, one dword per lane).
__device__ inline void dma4(const void* sbase, unsigned voff, unsigned lds) {
  asm volatile("s_mov_b32 m0, %2\n\tglobal_load_lds_dword %0, %1" ::"v"(voff), "s"(sbase),
               "s"(__builtin_amdgcn_readfirstlane(lds))
               : "memory", "m0");
}

// ---------------------------------------------------------------- wave-wide prefix sum
// Inclusive prefix sum over the 64 lanes of a wave with DPP (VALU only, no
// LDS round trip): Hillis-Steele inside each row of 16 lanes (row_shr 1, 2,
// 4, 8; lanes whose source lies outside the row add 0), then the last lane of
// row 0 into row 1 and of row 2 into row 3 (row_bcast:15), then lane 31 into
// rows 2 and 3 (row_bcast:31).
template <int CTRL, int ROWMASK>
__device__ inline float dpp_or_zero(float x) {
  return __builtin_bit_cast(
      float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), CTRL, ROWMASK, 0xF, false));
}
__device__ inline float wave_prefix_sum(float x) {
  x += dpp_or_zero<0x111, 0xF>(x);  // row_shr:1
  x += dpp_or_zero<0x112, 0xF>(x);  // row_shr:2
  x += dpp_or_zero<0x114, 0xF>(x);  // row_shr:4
  x += dpp_or_zero<0x118, 0xF>(x);  // row_shr:8
  x += dpp_or_zero<0x142, 0xA>(x);  // row_bcast:15 -> rows 1, 3
  x += dpp_or_zero<0x143, 0xC>(x);  // row_bcast:31 -> rows 2, 3
  return x;
}
// sum of x over each row of 16 lanes, in every lane of the row (rotations
// within the row: row_ror 8, 4, 2, 1; no LDS permutes)
__device__ inline float row16_sum(float x) {
  x += dpp_or_zero<0x128, 0xF>(x);
  x += dpp_or_zero<0x124, 0xF>(x);
  x += dpp_or_zero<0x122, 0xF>(x);
  x += dpp_or_zero<0x121, 0xF>(x);
  return x;
}
__device__ inline float lane_value(float x, int lane) {  // x of a wave-uniform lane
  return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, x), lane));
}

// ---------------------------------------------------------------- small helpers
// 2^x for x <= 0 (a decay factor): the hardware exponential alone.  Results
// below 2^-126, which the denormal-safe exp2f would keep, flush to zero;
// such a factor weighs nothing next to the terms of size 1 it is summed with.
__device__ inline float exp2_np(float x) { return __builtin_amdgcn_exp2f(x); }

__device__ inline float pow_lam(float lg2, float n) {
  // lambda^n = 2^(n log2 lambda); only non-negative n are formed.  n = 0 is
  // exactly 1 for every lambda, 0 included (log2 0 = -inf would give NaN).
  return n == 0.0f ? 1.0f : exp2f(n * lg2);
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

// ---------------------------------------------------------------- token order
// LDS bank model of gfx950 (64 banks of 4 bytes), as measured with the
// hardware's bank-conflict counter: 8-byte reads, including the transposing
// ones, serve lanes 0..31 in one cycle and 32..63 in the next; 16-byte reads
// serve 16 lanes per cycle, in each half of the wave the lane quads 0, 3, 5, 6
// and then 1, 2, 4, 7 (quads of even, then odd, bit count).  The paired-offset
// forms (two 8-byte pieces per lane) run at half rate and are avoided.
//
// With rows padded to an odd number of 16-byte granules (PadTile), row r
// starts on bank 4 r mod 64 (d = 128) and the orders below make every
// transposing read, score-operand read and P access conflict-free:
//   tr_row(g, e): row of contraction slot e (0..3) of lane group g within a
//     16-token block.  Groups 0, 1 get the even rows, 2, 3 the odd ones, so an
//     8-byte transposing read over lanes 0..31 touches 8 rows 8 banks apart.
//   perm16(s) = tr_row(s / 4, s % 4): the token held by row s of a 16-row
//     score operand; rows 0..3, 12..15 map to {0..3, 8..11}, a set closed
//     under +8, and the rest to its complement.
//   score_granule<D>(ks, g): 16-byte feature granule of slot group g in step
//     ks.  d = 128: groups 0/1 and 2/3 sit 8 granules apart, which with the
//     row sets above gives each 16-lane cycle of a 16-byte read 16 distinct
//     bank quads.  d = 64 has only 8 granules per row and keeps the natural
//     order (its 16-byte score reads then meet two-way conflicts).
__device__ inline int tr_row(int g, int e) {
  return ((0x1540 >> (4 * g)) & 15) + 2 * (e & 1) + 8 * (e >> 1);
}
template <typename T>
__device__ inline int perm16(int s) {
  if constexpr (sizeof(T) == 2) return tr_row(s >> 2, s & 3);
  else return s;
}
template <int D>
__device__ inline int score_granule(int ks, int g) {
  if constexpr (D == 128) return ks + 8 * (g & 1) + 4 * (g >> 1);
  else return 4 * ks + g;
}

// ---------------------------------------------------------------- transposed operand
// MFMA operand that contracts over tokens, read from a token-major tile:
// lane (g = lane / 16, n = lane % 16) receives column col0 + n of the tokens
// of its contraction slots.  bf16: slot e = 0..3 is token j0 + tr_row(g, e)
// and slot 4 + e is token j0 + 16 + tr_row(g, e), read by two
// ds_read_b64_tr_b16.  Within each 16-lane group that instruction hands
// output lane d the element (d % 4) of source lane 4 e + d / 4, e = 0..3; so
// source lane s points at the row of slot s / 4 and columns col0 + 4 (s % 4)
// .. + 3.  Every operand paired with this one uses the same slot order.
// fp32: one scalar read of token j0 + g, column col0 + n.
template <typename T, class TL>
__device__ inline typename Elt<T>::op_t tr_op(const char* tile, int j0, int col0, int lane) {
  const int g = lane >> 4, s = lane & 15;
  if constexpr (sizeof(T) == 2) {
    typedef short v4i16 __attribute__((ext_vector_type(4)));
    typedef __attribute__((address_space(3))) v4i16 lds_v4;
    const int row = j0 + tr_row(g, s >> 2);
    const int col = col0 + 4 * (s & 3);
    const v4i16 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4*)(tile + TL::off(row, col)));
    const v4i16 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4*)(tile + TL::off(row + 16, col)));
    typedef short v8i16 __attribute__((ext_vector_type(8)));
    const v8i16 both = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
    return __builtin_bit_cast(bf16x8, both);
  } else {
    return *reinterpret_cast<const float*>(tile + TL::off(j0 + g, col0 + s));
  }
}

// token of contraction slot x of lane group g in the step starting at j0
// (the order tr_op uses)
template <typename T>
__device__ inline int slot_token(int j0, int g, int x) {
  if constexpr (sizeof(T) == 2) return j0 + (x < 4 ? tr_row(g, x) : 16 + tr_row(g, x - 4));
  else return j0 + g;
}

// Separate 8-byte LDS read that the compiler may not fuse with a neighbour
// into the half-rate paired form.
__device__ inline u32x2 lds_read8(const char* p) {
  typedef const volatile __attribute__((address_space(3))) u32x2 lds_u32x2;
  return *(lds_u32x2*)((const __attribute__((address_space(3))) char*)p);
}

}  // namespace la
