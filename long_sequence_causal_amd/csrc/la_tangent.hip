// la_tangent.hip -- gradient of the loss with respect to the fixed decay of
// each head, by forward-mode differentiation of the chunkwise recurrence.
//
// With T_t = d S_t / d lambda (the tangent state), differentiating
//   S_t = lambda S_{t-1} + k_t v_t^T,   o_t = q_t^T S_t
// gives T_t = lambda T_{t-1} + S_{t-1} with T_0 = 0 (S_0 is an input), and
// for the loss l = sum_t <dO_t, o_t> + <dS_end, S_end>
//   d l / d lambda = sum_t dO_t . (q_t^T T_t) + <dS_end, T_end>.
// The kernels carry U = lambda T, which obeys U_t = lambda (U_{t-1} + S_{t-1})
// and takes the same powers of lambda as the forward pass.  Per 64-token
// chunk (tokens i, j = 0..cl-1; S, U the states before it):
//   sum_i dO_i . (q_i^T U_i) = <U, M1> + <S, M2>
//                            + sum_{j<i} (i-j) lambda^(i-j) (q_i . k_j) (dO_i . v_j)
//   M1 = sum_i lambda^(i+1) q_i dO_i^T,   M2 = sum_i (i+1) lambda^(i+1) q_i dO_i^T
//   U <- lambda^cl (U + cl S) + sum_j (cl-1-j) lambda^(cl-1-j) k_j v_j^T
//   S <- lambda^cl S + sum_j lambda^(cl-1-j) k_j v_j^T
// and d l / d lambda = (1 / lambda) (sum_t dO_t . (q_t^T U_t) + <dS_end, U_end>).
// Every term enters the result as it is; no partial sums cancel.  Still,
// the result is a small difference of many terms (their absolute sum can be
// hundreds of times larger), and U varies slowly along the sequence, so a
// per-token rounding feeding U or M would add up coherently: in bf16 the
// decayed operands (the weighted dO of M1 and M2, the weighted V of both
// updates) go through the MFMA as hi + lo, and U, S never leave fp32.  (The
// weighted V of the U update as one rounded bf16 saves about 9 % of the
// walk's time and keeps the benchmark's heads within 2.6e-3 of their own
// size, but a single head whose gradient is small next to its terms, e.g.
// 72.7 at 2176 tokens, came out 8.5 % off; hi + lo: 1e-5.)  (The
// reverse-mode identity d l / d lambda = (1 / lambda) sum_u u (q_u . dq_u -
// k_u . dk_u) + ... does cancel: its terms exceed the result by a factor
// that grows with the sequence length, which bf16 gradients cannot carry.)
//
// Parallel plan, as the forward's: sub-segments of Lp tokens.  Over n tokens
// the pair moves as
//   U <- lambda^n (U + n S) + dU,   S <- lambda^n S + dS
// (the Jordan block of the derivative of lambda^n) with (dS, dU) the
// sub-segment's local pair from zero.  The pre-pass forms
// the local pairs (K, V only; last chunk first, each chunk's weights
// carrying the decay of the m tokens after it: lambda^(m + cl-1-j) and
// (m + cl-1-j) lambda^(m + cl-1-j), so the pair is never rescaled), the scan
// chains them from (S0, 0), the main
// pass walks every sub-segment from its start pair and sums its share, and
// the last kernel adds each head's shares in a fixed order.
//
// Inside a workgroup the layout is the forward walker's: wave w holds state
// columns [16 w, 16 w + 16) of S and of U in MFMA accumulators; Q, K, V, dO
// chunks go from HBM straight to padded token-major LDS tiles (double
// buffered where two stages fit).  Intra-chunk scores K Q^T and V dO^T are
// formed tile by tile in the same accumulator layout, so their product is
// taken in registers without a P matrix in LDS; M1 and M2 are formed tile
// by tile in the state's layout (the same transposed operands as the
// update) and dotted with U and S at once, so neither is ever stored.
#include "la_internal.h"
#include "la_walk.h"

namespace la {

namespace {

// bf16 hi + lo of a pair of fp32 values, each packed as two bf16 (element
// 0 in the low half), returned as {hi, lo}: hi = round-to-nearest-even(x),
// lo = the same rounding of the residual x - hi, which is exact in fp32.
// One conversion serves both values of a pair.
__device__ inline u32x2 split_hi_lo(float x0, float x1) {
  typedef float f32x2 __attribute__((ext_vector_type(2)));
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
  const f32x2 x = {x0, x1};
  const unsigned hi = __builtin_bit_cast(unsigned, __builtin_convertvector(x, bf16x2));
  const f32x2 h = {__builtin_bit_cast(float, hi << 16), __builtin_bit_cast(float, hi & 0xffff0000u)};
  const unsigned lo = __builtin_bit_cast(unsigned, __builtin_convertvector(x - h, bf16x2));
  return u32x2{hi, lo};
}

template <typename T, int D, bool MAIN>
struct TanLayout {
  typedef PadTile<T, CH, D> TN;
  static constexpr int NTEN = MAIN ? 4 : 2;  // Q, K, V, dO  or  K, V
  static constexpr int TB = TN::BYTES;
  static constexpr int STAGE = NTEN * TB;
  static constexpr int STAGES = 2 * STAGE <= LDS_MAX ? 2 : 1;
  static constexpr int BYTES = STAGES * STAGE;
  static constexpr int NW = D / 16;  // waves: one per 16 state columns
  static constexpr int NT = 64 * NW;
  // bf16 keeps two waves per SIMD; the pre-pass (LDS for two workgroups a
  // CU, 128 registers) four, since its arithmetic, not HBM, binds it
  static constexpr int WAVES_PER_EU = sizeof(T) == 2 ? (MAIN ? 2 : 4) : 1;
  static_assert(BYTES <= LDS_MAX, "LDS budget");
  static_assert(TB == TN::G * 1024, "a tile is G loads of 1 KiB");
};

template <typename T, int D, bool MAIN, bool LAZY>
__global__ __launch_bounds__((TanLayout<T, D, MAIN>::NT), (TanLayout<T, D, MAIN>::WAVES_PER_EU)) void
k_tangent(TanArgs a) {
  typedef TanLayout<T, D, MAIN> LY;
  typedef typename LY::TN TN;
  typedef Elt<T> X;
  typedef typename X::op_t op_t;
  constexpr int E = X::E;
  constexpr int KS = 4 * E;                // MFMA contraction step
  constexpr int NW = LY::NW;
  constexpr int EP = 16 / (int)sizeof(T);  // elements per 16-byte piece
  constexpr int NKT = D / 16;
  constexpr int NST = (10 + NW - 1) / NW;  // score tiles per wave (at most)
  constexpr int NKS = D / KS;
  constexpr int NJS = CH / KS;
  constexpr int S = LY::STAGES;
  constexpr int G = TN::G;
  constexpr int NBW = (G + NW - 1) / NW;   // 1 KiB blocks per tile of the busiest wave
  static_assert(G > NW, "every wave loads at least one block");
  __shared__ __attribute__((aligned(1024))) char smem[LY::BYTES];
  __shared__ double red[NW];
  // per-token factors of the current chunk in operand slot order (entry
  // 16 g + E js + x is slot x of lane group g in contraction step js):
  // update weights lambda^(cl-1-j) and query factors lambda^(j+1), 0 past cl
  __shared__ __attribute__((aligned(16))) float tabW[64];
  __shared__ __attribute__((aligned(16))) float tabQ[64];
  static_assert(NJS * E == 16, "16 update slots per lane");

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l16 = lane & 15;
  const int g = lane >> 4;
  const int col = 16 * w;

  // ---- work item: sub-segment p of sequence n (pre-pass: piece p of
  // Lp / pre_r tokens)
  const int np = MAIN ? a.split : a.pre_r * (a.split - 1);
  const int64_t n = (int64_t)blockIdx.x / np;
  const int p = (int)((int64_t)blockIdx.x % np);
  const int h = (int)((n / a.nseg) % a.H);
  const int64_t lp = MAIN ? a.Lp : a.Lp / a.pre_r;
  const int64_t t0 = (int64_t)p * lp;
  const int64_t t1 = (t0 + lp < a.Ls) ? t0 + lp : a.Ls;
  const int len = (int)(t1 > t0 ? t1 - t0 : 0);
  const int nch = (len + CH - 1) / CH;
  const float lg = log2f(a.lam[h]);
  // the main pass runs as two launches, eager (lambda < 1/2) and lazy
  // (lambda >= 1/2, below); each sub-segment is walked by the one that fits
  // its head, the other's workgroup ending here
  if (MAIN && (fabsf(lg) <= 1.0f) != LAZY) return;
  const int64_t DD = (int64_t)D * D;
  const int64_t seq0 = n * a.Ls * D;  // element offset of the sequence's first row

  // ---- start pair -> accumulators (S0 or a scanned pair; zero in the pre-pass)
  f32x4 accS[NKT], accT[NKT];  // S and U
  {
    const float* sp = nullptr;
    const float* tp = nullptr;
    if (MAIN) {
      if (p == 0) {
        sp = a.S0 ? a.S0 + n * DD : nullptr;
      } else {
        const int64_t o = (n * (int64_t)a.pre_r * (a.split - 1) + (a.pre_r * p - 1)) * DD;
        sp = a.WS + o;
        tp = a.WT + o;
      }
    }
#pragma unroll
    for (int tk = 0; tk < NKT; ++tk)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int idx = (16 * tk + 4 * g + r) * D + col + l16;
        accS[tk][r] = sp ? sp[idx] : 0.0f;
        accT[tk][r] = tp ? tp[idx] : 0.0f;
      }
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): retire them before the chunk loop
  }

  // ---- chunk loads: block blk (0..G-1) of a tile is granules 64 blk .. + 63;
  // lane l's granule (row, piece) = divmod(64 blk + l, G), the padding piece
  // of a row loading the row's first piece.  Wave w takes blocks w, w + NW,
  // ... and loads each for every tile of the stage (their offsets within a
  // tile agree), so it keeps one chunk-0 offset per block.  Rows past the end
  // are clamped to the last token (masked by the factors).  Offsets are
  // 32-bit bytes from the sequence's first row and wrap modulo 2^32 like the
  // offsets they stand for (the host keeps a sequence below 4 GiB).
  auto tensor = [&](int ten) -> const T* {
    const void* bp;
    if (MAIN)
      bp = ten == 0 ? a.Q : (ten == 1 ? a.K : (ten == 2 ? a.V : a.dO));
    else
      bp = ten == 0 ? a.K : a.V;
    return reinterpret_cast<const T*>(bp) + seq0;
  };
  auto piece_of = [&](int blk, int& row) -> int {  // lane's row; piece offset (elements)
    const int pos = 64 * blk + lane;
    row = pos / G;
    const int pc = pos % G;
    return ((pc == G - 1) ? 0 : pc) * EP;
  };
  const int nbw = (G - w + NW - 1) / NW;  // this wave's blocks (wave-uniform)
  unsigned voff0[NBW];
#pragma unroll
  for (int k = 0; k < NBW; ++k) {
    int row;
    const int po = piece_of((w + NW * k < G) ? w + NW * k : 0, row);
    voff0[k] = (unsigned)(((t0 + row) * D + po) * (int64_t)sizeof(T));
  }
  const unsigned smem_lds = lds_address(smem);
  // pre-pass over whole chunks: walked last chunk first (step c takes chunk
  // nch - 1 - c), the decay of the chunks after it carried by the update
  // weights instead of scaling the pair every chunk
  const bool lcf = !MAIN && len % CH == 0;
  auto issue = [&](int cs, int stage) {
    const int c = lcf ? nch - 1 - cs : cs;
    const bool full = (c + 1) * CH <= len;
#pragma unroll
    for (int k = 0; k < NBW; ++k) {
      if (k < NBW - 1 || nbw == NBW) {
        const int blk = w + NW * k;
        unsigned voff;
        if (full) {
          voff = voff0[k] + (unsigned)c * (unsigned)(CH * D * (int)sizeof(T));
        } else {
          int row;
          const int po = piece_of(blk, row);
          const int tt = (c * CH + row < len) ? c * CH + row : len - 1;
          voff = (unsigned)(((t0 + tt) * D + po) * (int64_t)sizeof(T));
        }
#pragma unroll
        for (int ten = 0; ten < LY::NTEN; ++ten)
          dma16(tensor(ten), voff,
                smem_lds + (unsigned)(stage * LY::STAGE + ten * LY::TB + blk * 1024));
      }
    }
  };

  // ---- factors of a chunk of cl tokens (0 past the tail)
  float wt[NST][4];    // (i-j) lambda^(i-j) for j < i on the wave's score tiles
  float dc = 1.0f;     // lambda^cl
  int clf = CH;        // cl
  auto set_factors = [&](int cl) {
    if (MAIN) {
#pragma unroll
      for (int st = 0; st < NST; ++st) {
        const int idx = w + NW * st;
        int jb = 0, ib = 0;
        if (idx < 10) score_tile(idx, jb, ib);
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          // accumulator (row 4 g + r, column l16) of tile (jb, ib): key j, query i
          const int i = 16 * ib + perm16<T>(l16), j = 16 * jb + perm16<T>(4 * g + r);
          wt[st][r] = (idx < 10 && j < i && i < cl) ? (float)(i - j) * pow_lam(lg, (float)(i - j)) : 0.0f;
        }
      }
    }
    if (tid < 64) {
      const int js = (tid & 15) / E, x = (tid & 15) % E;
      const int j = slot_token<T>(js * KS, tid >> 4, x);
      tabW[tid] = j < cl ? pow_lam(lg, (float)(cl - 1 - j)) : 0.0f;
      tabQ[tid] = j < cl ? pow_lam(lg, (float)(j + 1)) : 0.0f;
    }
    dc = pow_lam(lg, (float)cl);
    clf = cl;
  };
  set_factors(CH);  // tabW is complete at the loop's first barrier

  double dsum = 0.0;  // this lane's share of lambda * gradient (main pass)
  // Lazy main pass (lambda >= 1/2): the accumulators hold the pair divided
  // by lambda^ntok, ntok the tokens since they last held it as it is, so
  // that a chunk adds its update with weights divided by lambda^ntok (ntok
  // counting the chunk) instead of scaling both accumulators by lambda^cl;
  // its inter-chunk inner products <U, M1> + <S, M2> are multiplied by
  // lambda^ntok (ntok before the chunk) instead.  Periods of R chunks keep those divisors within 2^64; the
  // accumulators are scaled back at the end of each.  Below 1/2 one chunk's
  // divisor could leave fp32's range: the eager pass scales the pair every
  // chunk.
  const float alg = fabsf(lg);
  const int R = !LAZY ? (1 << 30) : (alg * (float)nch <= 1.0f ? nch : (int)(1.0f / alg));
  int ntok = 0;
  // The token of a contraction slot is a lane-group term plus a
  // compile-time one (slot_token(j0, g, x) = slot_token(j0, 0, x) + fB);
  // small integers, so the factors below are exact in fp32 either way.
  const float fB = (float)slot_token<T>(0, g, 0);
  if (S > 1 && nch > 0) issue(0, 0);
  for (int c0 = 0; c0 < nch; c0 += R) {
  const int c1 = (nch - c0 > R) ? c0 + R : nch;
  for (int c = c0; c < c1; ++c) {
    const int cl = (len - c * CH < CH) ? (len - c * CH) : CH;
    // fp32 at d = 128: the lane index, opaque to the compiler once per chunk,
    // so that the transposed-operand addresses are formed in the chunk from
    // one lane term and immediates instead of being held (and spilled)
    // across the loop
    int ln = lane;
    if constexpr (E == 1 && D == 128) asm volatile("" : "+v"(ln));
    int stg = 0;
    if constexpr (S == 1) {
      lds_barrier();  // every wave is done with the previous chunk
      issue(c, 0);
      wait_vm_barrier<0>();
    } else {
      wait_vm_barrier<0>();  // chunk c landed; every wave is done with chunk c - 1
      if (c + 1 < nch) issue(c + 1, (c + 1) & 1);
      stg = c & 1;
    }
    if (cl != CH) {  // the tail (every wave is past its previous use of tabW)
      set_factors(cl);
      lds_barrier();
    }
    const char* const stage = smem + stg * LY::STAGE;
    const char* const sQ = stage;
    const char* const sK = stage + (MAIN ? LY::TB : 0);
    const char* const sV = sK + LY::TB;
    const char* const sD = sV + LY::TB;

    if constexpr (MAIN) {
      float part = 0.0f;
      float pin = 0.0f;  // lazy: the inter term, in the accumulators' scale
      // ---- intra: sum_{j<i} (i-j) lambda^(i-j) (q_i . k_j)(dO_i . v_j), wave's tiles
#pragma unroll
      for (int st = 0; st < NST; ++st) {
        const int idx = w + NW * st;
        if (idx < 10) {
          int jb, ib;
          score_tile(idx, jb, ib);
          f32x4 aqk = {0.f, 0.f, 0.f, 0.f};
          f32x4 avd = {0.f, 0.f, 0.f, 0.f};
          const int l16x = ln & 15, gx = ln >> 4;  // (l16, g from the chunk's lane index)
          const int rk = 16 * jb + perm16<T>(l16x), rq = 16 * ib + perm16<T>(l16x);
#pragma unroll
          for (int ks = 0; ks < NKS; ++ks) {
            const int f = (E == 8) ? 8 * score_granule<D>(ks, gx) : ks * KS + gx;
            aqk = X::mfma(lds_op<T>(sK, TN::off(rk, f)), lds_op<T>(sQ, TN::off(rq, f)), aqk);
            avd = X::mfma(lds_op<T>(sV, TN::off(rk, f)), lds_op<T>(sD, TN::off(rq, f)), avd);
          }
#pragma unroll
          for (int r = 0; r < 4; ++r) part += aqk[r] * avd[r] * wt[st][r];
        }
      }

      // ---- inter: <U, M1> + <S, M2>, tile tk of M1, M2 = Q^T diag(.) dO at a time
      __builtin_amdgcn_sched_barrier(0);
      {
        const float* tq = tabQ + 16 * g;
        op_t D1[NJS], D1l[NJS], D2[NJS], D2l[NJS];
#pragma unroll
        for (int js = 0; js < NJS; ++js) {
          const op_t Dop = tr_op<T, TN>(sD, js * KS, col, ln);
          if constexpr (E == 8) {
            u32x4 h1, l1, h2, l2;
#pragma unroll
            for (int x = 0; x < 8; x += 2) {
              const float a10 = (float)Dop[x] * tq[8 * js + x];
              const float a11 = (float)Dop[x + 1] * tq[8 * js + x + 1];
              const float a20 = a10 * (fB + (float)(1 + slot_token<T>(js * KS, 0, x)));
              const float a21 = a11 * (fB + (float)(1 + slot_token<T>(js * KS, 0, x + 1)));
              const u32x2 s1 = split_hi_lo(a10, a11);
              h1[x / 2] = s1[0];
              l1[x / 2] = s1[1];
              const u32x2 s2 = split_hi_lo(a20, a21);
              h2[x / 2] = s2[0];
              l2[x / 2] = s2[1];
            }
            D1[js] = __builtin_bit_cast(bf16x8, h1);
            D1l[js] = __builtin_bit_cast(bf16x8, l1);
            D2[js] = __builtin_bit_cast(bf16x8, h2);
            D2l[js] = __builtin_bit_cast(bf16x8, l2);
          } else {
            D1[js] = Dop * tq[js];
            D2[js] = D1[js] * (float)(1 + slot_token<T>(js * KS, g, 0));
          }
        }
#pragma unroll
        for (int tk = 0; tk < NKT; ++tk) {
          f32x4 m1 = {0.f, 0.f, 0.f, 0.f};
          f32x4 m2 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int js = 0; js < NJS; ++js) {
            const op_t Aq = tr_op<T, TN>(sQ, js * KS, 16 * tk, ln);
            m1 = X::mfma(Aq, D1[js], m1);
            m2 = X::mfma(Aq, D2[js], m2);
            if constexpr (E == 8) {
              m1 = X::mfma(Aq, D1l[js], m1);
              m2 = X::mfma(Aq, D2l[js], m2);
            }
          }
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            if constexpr (LAZY)
              pin += accT[tk][r] * m1[r] + accS[tk][r] * m2[r];
            else
              part += accT[tk][r] * m1[r] + accS[tk][r] * m2[r];
          }
        }
      }
      dsum += LAZY ? (double)(part + pin * pow_lam(lg, (float)ntok)) : (double)part;
    }

    __builtin_amdgcn_sched_barrier(0);
    // ---- updates: U = lambda^cl (U + cl S) + K^T diag((cl-1-j) lambda^(cl-1-j)) V,
    //               S = lambda^cl S + K^T diag(lambda^(cl-1-j)) V
    {
      // last chunk first: the m = 64 c tokens after this chunk decay its
      // contribution (weights lambda^(m + cl-1-j), (m + cl-1-j) lambda^(m + cl-1-j));
      // otherwise the pair moves over the chunk first
      float fk = lcf ? pow_lam(lg, (float)(CH * c)) : 1.0f;
      if constexpr (LAZY) {
        ntok += clf;
        fk = exp2f(-(float)ntok * lg);  // lambda^-ntok <= 2^64
#pragma unroll
        for (int tk = 0; tk < NKT; ++tk) accT[tk] += (float)clf * accS[tk];
      } else if (!lcf) {
        const float dcu = dc * (float)clf;
#pragma unroll
        for (int tk = 0; tk < NKT; ++tk) {
          accT[tk] = dc * accT[tk] + dcu * accS[tk];
          accS[tk] *= dc;
        }
      }
      // V^T operands of this wave's columns, scaled per token (hi + lo in bf16)
      const float* tw = tabW + 16 * g;
      // m + clf - 1 - slot_token = cB - slot_token(., 0, .) (small integers, exact)
      const float cB = (float)(clf - 1) - fB + (lcf ? (float)(CH * c) : 0.0f);
      op_t B1[NJS], B1l[NJS], B2[NJS], B2l[NJS];
#pragma unroll
      for (int js = 0; js < NJS; ++js) {
        const op_t Vop = tr_op<T, TN>(sV, js * KS, col, ln);
        if constexpr (E == 8) {
          u32x4 b1, b1l, b2, b2l;
#pragma unroll
          for (int x = 0; x < 8; x += 2) {
            const float vw0 = LAZY ? ((float)Vop[x] * tw[8 * js + x]) * fk
                                   : (float)Vop[x] * (tw[8 * js + x] * fk);
            const float vw1 = LAZY ? ((float)Vop[x + 1] * tw[8 * js + x + 1]) * fk
                                   : (float)Vop[x + 1] * (tw[8 * js + x + 1] * fk);
            const float vu0 = vw0 * (cB - (float)slot_token<T>(js * KS, 0, x));
            const float vu1 = vw1 * (cB - (float)slot_token<T>(js * KS, 0, x + 1));
            const u32x2 s1 = split_hi_lo(vw0, vw1);
            b1[x / 2] = s1[0];
            b1l[x / 2] = s1[1];
            const u32x2 s2 = split_hi_lo(vu0, vu1);
            b2[x / 2] = s2[0];
            b2l[x / 2] = s2[1];
          }
          B1[js] = __builtin_bit_cast(bf16x8, b1);
          B1l[js] = __builtin_bit_cast(bf16x8, b1l);
          B2[js] = __builtin_bit_cast(bf16x8, b2);
          B2l[js] = __builtin_bit_cast(bf16x8, b2l);
        } else {
          B1[js] = Vop * (tw[js] * fk);
          B2[js] = B1[js] * (cB + fB - (float)slot_token<T>(js * KS, g, 0));
        }
      }
#pragma unroll
      for (int tk = 0; tk < NKT; ++tk) {
#pragma unroll
        for (int js = 0; js < NJS; ++js) {
          const op_t Ak = tr_op<T, TN>(sK, js * KS, 16 * tk, ln);
          accS[tk] = X::mfma(Ak, B1[js], accS[tk]);
          accT[tk] = X::mfma(Ak, B2[js], accT[tk]);
          if constexpr (E == 8) accT[tk] = X::mfma(Ak, B2l[js], accT[tk]);
          if constexpr (E == 8) accS[tk] = X::mfma(Ak, B1l[js], accS[tk]);
        }
      }
    }
  }
  if constexpr (LAZY) {  // back to the pair as it is
    const float sg = pow_lam(lg, (float)ntok);
#pragma unroll
    for (int tk = 0; tk < NKT; ++tk) {
      accS[tk] *= sg;
      accT[tk] *= sg;
    }
    ntok = 0;
  }
  }

  if constexpr (MAIN) {
    // the state term <dS_end, U_end>, on the sequence's last sub-segment
    if (p == a.split - 1 && a.dSe) {
      const float* ds = a.dSe + n * DD;
      // the lane's element offset, formed here: otherwise the compiler shares
      // the 32 addresses with the start-state loads and keeps them across the
      // chunk loop
      unsigned lo = (unsigned)(4 * g * D + col + l16);
      asm volatile("" : "+v"(lo));
      float e = 0.0f;
#pragma unroll
      for (int tk = 0; tk < NKT; ++tk)
#pragma unroll
        for (int r = 0; r < 4; ++r) e += ds[lo + (unsigned)((16 * tk + r) * D)] * accT[tk][r];
      dsum += (double)e;
    }
    // workgroup sum in a fixed order
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) dsum += __shfl_xor(dsum, m, 64);
    if (lane == 0) red[w] = dsum;
    __syncthreads();
    if (tid == 0) {
      double t = 0.0;
#pragma unroll
      for (int i = 0; i < NW; ++i) t += red[i];
      a.part[n * a.split + p] = t;
    }
  } else {
    const int64_t o = (n * np + p) * DD;
#pragma unroll
    for (int tk = 0; tk < NKT; ++tk)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int idx = (16 * tk + 4 * g + r) * D + col + l16;
        a.WS[o + idx] = accS[tk][r];
        a.WT[o + idx] = accT[tk][r];
      }
  }
}

// Chain the local pairs (S, U) of the pre-pass pieces 0..pre_r (split-1) - 1
// of every sequence from (S0, 0), in place: entry q becomes the start pair of
// piece q + 1.  One thread per (sequence, state element).
__global__ __launch_bounds__(256) void k_tangent_scan(TanArgs a, int64_t total, int D) {
  const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (idx >= total) return;
  const int64_t DD = (int64_t)D * D;
  const int64_t n = idx / DD, e = idx % DD;
  const int h = (int)((n / a.nseg) % a.H);
  const float lg = log2f(a.lam[h]);
  const float Lp = (float)(a.Lp / a.pre_r);  // a multiple of 64, at most 2^24: exact
  const float dl = exp2f(Lp * lg);
  const float dw = Lp * dl;
  float x = a.S0 ? a.S0[n * DD + e] : 0.0f;
  float y = 0.0f;
  const int nq = a.pre_r * (a.split - 1);
  for (int p = 0; p < nq; ++p) {
    const int64_t o = (n * nq + p) * DD + e;
    y = dl * y + dw * x + a.WT[o];
    x = dl * x + a.WS[o];
    a.WS[o] = x;
    a.WT[o] = y;
  }
}

// dlam[h] = (1 / lambda_h) * the sum of the shares of head h's sequences
// n = (b H + h) nseg + s, in a fixed order (thread-strided sums, then a tree).
__global__ __launch_bounds__(256) void k_tangent_sum(const double* part, const float* lam,
                                                     float* dlam, int64_t nseq, int H, int nseg,
                                                     int split) {
  __shared__ double red[256];
  const int h = blockIdx.x;
  const int64_t per = nseq / H * split;  // B nseg sequences of head h, split shares each
  double acc = 0.0;
  for (int64_t m = threadIdx.x; m < per; m += 256) {
    const int64_t q = m / split, pp = m % split;
    const int64_t n = (q / nseg * H + h) * nseg + q % nseg;
    acc += part[n * split + pp];
  }
  red[threadIdx.x] = acc;
  __syncthreads();
  for (int st = 128; st > 0; st >>= 1) {
    if ((int)threadIdx.x < st) red[threadIdx.x] += red[threadIdx.x + st];
    __syncthreads();
  }
  if (threadIdx.x == 0) dlam[h] = (float)(red[0] / (double)lam[h]);
}

template <typename T, int D>
hipError_t tangent_t(const TanArgs& a, int64_t nseq, float* dlam, hipStream_t s) {
  hipError_t e;
  if (nseq > 0 && a.split > 1) {
    hipLaunchKernelGGL((k_tangent<T, D, false, false>), dim3((unsigned)(nseq * a.pre_r * (a.split - 1))),
                       dim3(TanLayout<T, D, false>::NT), 0, s, a);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    const int64_t total = nseq * (int64_t)D * D;
    hipLaunchKernelGGL(k_tangent_scan, dim3((unsigned)((total + 255) / 256)), dim3(256), 0, s, a,
                       total, D);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  if (nseq > 0) {
    hipLaunchKernelGGL((k_tangent<T, D, true, false>), dim3((unsigned)(nseq * a.split)),
                       dim3(TanLayout<T, D, true>::NT), 0, s, a);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    hipLaunchKernelGGL((k_tangent<T, D, true, true>), dim3((unsigned)(nseq * a.split)),
                       dim3(TanLayout<T, D, true>::NT), 0, s, a);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  hipLaunchKernelGGL(k_tangent_sum, dim3((unsigned)a.H), dim3(256), 0, s, a.part, a.lam, dlam,
                     nseq, a.H, a.nseg, a.split);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_tangent(const TanArgs& a, int dtype, int D, int64_t nseq, float* dlam,
                          hipStream_t s) {
  if (a.H <= 0) return hipSuccess;
  if (dtype == 0) {
    if (D == 64) return tangent_t<__bf16, 64>(a, nseq, dlam, s);
    if (D == 128) return tangent_t<__bf16, 128>(a, nseq, dlam, s);
  } else {
    if (D == 64) return tangent_t<float, 64>(a, nseq, dlam, s);
    if (D == 128) return tangent_t<float, 128>(a, nseq, dlam, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace la
