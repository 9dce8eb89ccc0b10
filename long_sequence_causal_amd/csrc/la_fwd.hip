// la_fwd.hip -- chunkwise forward kernel of decayed causal linear attention.
//
// One workgroup (4 waves) walks the 64-token chunks of one sub-segment of
// one sequence in order, carrying the fp32 state S (D x D) in MFMA
// accumulators.  Per chunk c with tokens i, j = 0..cl-1 (cl = 64 except for a
// ragged tail), decay lambda and S the state before the chunk:
//
//   P[i][j]   = lambda^(i-j) (q_i . k_j)  for j <= i, else 0     (intra scores)
//   o_i       = lambda^(i+1) q_i^T S  +  sum_j P[i][j] v_j          (output)
//   S        <- lambda^cl S + sum_j lambda^(cl-1-j) k_j v_j^T       (state)
//
// which is the token recurrence S_t = lambda S_{t-1} + k_t v_t^T,
// o_t = q_t^T S_t regrouped: exact attention inside a chunk and the state
// between chunks (the Lightning Attention-2 split named in the LASP-2 page's
// related-paper list), with the state evaluated right-product-first (LASP-2
// abstract).  Only non-negative powers of lambda are formed, so nothing
// overflows however long the sequence.
//
// Work split inside the workgroup (wave w of 4):
//   * intra scores: the 10 non-zero 16x16 tiles of P^T = K Q^T are dealt
//     round-robin to the waves and written to LDS as P[i][j];
//   * wave w owns state columns v in [w D/4, (w+1) D/4): its slice of S stays
//     in registers, serves directly (rounded to bf16) as the A operand of
//     O^T = S^T Q^T, and is updated by S += Kt' V with Kt' = (diag(lambda^(cl-1-j)) K)^T;
//   * outputs are produced as O^T tiles so each lane ends up with 4
//     consecutive v of one token: one 8-byte (bf16) store per tile.
// LDS holds the chunk's Q and K (token-major, for the scores and the inter
// term), K and V transposed (d-major, for the products that contract over
// tokens) and P.  The next chunk's Q, K, V are loaded into registers while
// the current chunk computes.
#include "la_device.h"
#include "la_internal.h"

namespace la {

// The 10 lower-triangular (key block jb <= query block ib) tiles of the
// 64x64 score matrix, dealt round-robin to the 4 waves (3, 3, 2, 2 tiles).
__device__ inline void score_tile(int idx, int& jb, int& ib) {
  if (idx < 4) { jb = idx; ib = idx; }
  else if (idx < 7) { jb = idx - 4; ib = idx - 3; }
  else if (idx < 9) { jb = idx - 7; ib = idx - 5; }
  else { jb = 0; ib = 3; }
}

template <typename T, int D, bool WITH_O>
struct FwdLayout {
  typedef Tile<T, CH, D, 1> TQ;   // Q, K token-major [token][d]
  typedef Tile<T, D, CH, 2> TT;   // K', V transposed [d][token]
  typedef Tile<T, CH, CH, 1> TP;  // P [i][j]
  static constexpr int OFF_Q = 0;
  static constexpr int OFF_K = WITH_O ? TQ::BYTES : 0;
  static constexpr int OFF_KT = WITH_O ? 2 * TQ::BYTES : 0;
  static constexpr int OFF_VT = OFF_KT + TT::BYTES;
  static constexpr int OFF_P = OFF_VT + TT::BYTES;
  static constexpr int BYTES = OFF_P + (WITH_O ? TP::BYTES : 0);
};

template <typename T, int D, bool WITH_O>
__global__ __launch_bounds__(NTHR) void k_chunk_fwd(FwdArgs a) {
  typedef Elt<T> X;
  typedef typename X::op_t op_t;
  typedef FwdLayout<T, D, WITH_O> LY;
  typedef typename LY::TQ TQ;
  typedef typename LY::TT TT;
  typedef typename LY::TP TP;
  constexpr int E = X::E;           // operand elements per lane
  constexpr int KS = 4 * E;         // MFMA contraction step
  constexpr int EP = 16 / (int)sizeof(T);  // elements per 16-byte piece
  constexpr int PPR = D / EP;       // pieces per token row
  constexpr int RPP = 2 * NTHR / PPR;  // token rows per load pass
  constexpr int NPASS = CH / RPP;   // load passes per chunk
  constexpr int NVT = D / 64;       // 16-wide state-column tiles per wave
  constexpr int NKT = D / 16;       // 16-high state-row tiles
  constexpr int NKS = D / KS;       // contraction steps over d
  constexpr int NJS = CH / KS;      // contraction steps over a chunk
  static_assert(NPASS >= 1 && RPP * NPASS == CH, "load tiling");

  __shared__ __attribute__((aligned(16))) char smem[LY::BYTES];
  char* const sQ = smem + LY::OFF_Q;
  char* const sK = smem + LY::OFF_K;
  char* const sKt = smem + LY::OFF_KT;
  char* const sVt = smem + LY::OFF_VT;
  char* const sP = smem + LY::OFF_P;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = tid >> 6;
  const int l16 = lane & 15;
  const int g = lane >> 4;

  // ---- work item
  const int64_t n = (int64_t)blockIdx.x / a.p_count;
  const int p = a.p_begin + (int)((int64_t)blockIdx.x % a.p_count);
  const int h = (int)((n / a.nseg) % a.H);
  const float lg = log2f(a.lam[h]);
  const int64_t t0 = (int64_t)p * a.Lp;
  const int64_t t1 = (t0 + a.Lp < a.Ls) ? t0 + a.Lp : a.Ls;
  const int64_t len = (t1 > t0) ? t1 - t0 : 0;
  const int64_t nch = (len + CH - 1) / CH;

  const T* const Qg = reinterpret_cast<const T*>(a.Q);
  const T* const Kg = reinterpret_cast<const T*>(a.K);
  const T* const Vg = reinterpret_cast<const T*>(a.V);
  T* const Og = reinterpret_cast<T*>(a.O);
  const int64_t seq_row0 = n * a.Ls;  // first token row of sequence n
  // token row (in the flattened tensor) of position tt of sequence n
  auto row_of = [&](int64_t tt) -> int64_t {
    return seq_row0 + (a.reverse ? (a.Ls - 1 - tt) : tt);
  };

  // ---- start state -> accumulators (wave w: columns [w D/4, (w+1) D/4))
  f32x4 accS[NKT][NVT];
  {
    const float* sp = nullptr;
    if (a.start_from_state) {
      if (p == 0)
        sp = a.S0 ? a.S0 + n * D * D : nullptr;
      else
        sp = a.Sws + (n * (a.split - 1) + (p - 1)) * (int64_t)D * D;
    }
#pragma unroll
    for (int tk = 0; tk < NKT; ++tk)
#pragma unroll
      for (int vt = 0; vt < NVT; ++vt)
#pragma unroll
        for (int r = 0; r < 4; ++r)
          accS[tk][vt][r] =
              sp ? sp[(16 * tk + 4 * g + r) * D + 16 * (w * NVT + vt) + l16] : 0.0f;
  }

  // ---- chunk-independent factors
  float qf[4];        // lambda^(i+1) for the lane's query i of each 16-row block
  float pf[3][4];     // lambda^(i-j) (or 0) for the wave's score tiles
  int njs[4];         // contraction steps over keys j < 16 (it+1)
  if (WITH_O) {
#pragma unroll
    for (int it = 0; it < 4; ++it) {
      qf[it] = pow_lam(lg, (float)(16 * it + l16 + 1));
      njs[it] = (16 * (it + 1) + KS - 1) / KS;
    }
#pragma unroll
    for (int s = 0; s < 3; ++s) {
      const int idx = w + 4 * s;
      int jb = 0, ib = 0;
      if (idx < 10) score_tile(idx, jb, ib);
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int i = 16 * ib + l16, j = 16 * jb + 4 * g + r;
        pf[s][r] = (idx < 10 && j <= i) ? pow_lam(lg, (float)(i - j)) : 0.0f;
      }
    }
    // upper score tiles are never written: clear P once
    for (int o = tid * 16; o < TP::BYTES; o += NTHR * 16)
      lds_store16<T>(sP, o, u32x4{0u, 0u, 0u, 0u});
  }
  const float lamC = pow_lam(lg, (float)CH);

  // ---- global -> register staging of one chunk (16-byte pieces)
  const int pe = tid % PPR;  // piece (column group) of this thread
  const int prp = tid / PPR; // row pair inside a pass
  u32x4 rq[NPASS][2], rk[NPASS][2], rv[NPASS][2];
  auto load_chunk = [&](int64_t c) {
#pragma unroll
    for (int ps = 0; ps < NPASS; ++ps)
#pragma unroll
      for (int hh = 0; hh < 2; ++hh) {
        const int r = ps * RPP + 2 * prp + hh;
        const int64_t tt = c * CH + r;
        const bool ok = (tt < len);
        const int64_t off = ok ? (row_of(t0 + tt) * D + pe * EP) : 0;
        const u32x4 z = {0u, 0u, 0u, 0u};
        if (WITH_O) rq[ps][hh] = ok ? *reinterpret_cast<const u32x4*>(Qg + off) : z;
        rk[ps][hh] = ok ? *reinterpret_cast<const u32x4*>(Kg + off) : z;
        rv[ps][hh] = ok ? *reinterpret_cast<const u32x4*>(Vg + off) : z;
      }
  };

  // ---- registers -> LDS (token-major Q, K; transposed K' and V)
  auto store_chunk = [&](int cl) {
#pragma unroll
    for (int ps = 0; ps < NPASS; ++ps) {
      const int r0 = ps * RPP + 2 * prp;
      if (WITH_O) {
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) {
          lds_store16<T>(sQ, TQ::off(r0 + hh, pe * EP), rq[ps][hh]);
          lds_store16<T>(sK, TQ::off(r0 + hh, pe * EP), rk[ps][hh]);
        }
      }
      const float wk0 = (r0 < cl) ? pow_lam(lg, (float)(cl - 1 - r0)) : 0.0f;
      const float wk1 = (r0 + 1 < cl) ? pow_lam(lg, (float)(cl - 2 - r0)) : 0.0f;
      union U { u32x4 u; T e[EP]; };
      U k0, k1, v0, v1;
      k0.u = rk[ps][0];
      k1.u = rk[ps][1];
      v0.u = rv[ps][0];
      v1.u = rv[ps][1];
#pragma unroll
      for (int x = 0; x < EP; ++x) {
        const int row = pe * EP + x;
        T kp[2] = {X::from_f(X::to_f(k0.e[x]) * wk0), X::from_f(X::to_f(k1.e[x]) * wk1)};
        T vp[2] = {v0.e[x], v1.e[x]};
        if (sizeof(T) == 2) {
          *reinterpret_cast<unsigned int*>(sKt + TT::off(row, r0)) =
              *reinterpret_cast<unsigned int*>(kp);
          *reinterpret_cast<unsigned int*>(sVt + TT::off(row, r0)) =
              *reinterpret_cast<unsigned int*>(vp);
        } else {
          *reinterpret_cast<u32x2*>(sKt + TT::off(row, r0)) = *reinterpret_cast<u32x2*>(kp);
          *reinterpret_cast<u32x2*>(sVt + TT::off(row, r0)) = *reinterpret_cast<u32x2*>(vp);
        }
      }
    }
  };

  if (nch > 0) load_chunk(0);

  for (int64_t c = 0; c < nch; ++c) {
    const int cl = (int)((len - c * CH < CH) ? (len - c * CH) : CH);
    __syncthreads();  // the previous chunk's LDS reads are done
    store_chunk(cl);
    __syncthreads();
    if (c + 1 < nch) load_chunk(c + 1);  // in flight during this chunk's math

    if (WITH_O) {
      // ---- intra scores: P^T tiles = K Q^T, masked and decayed, to LDS as P[i][j]
#pragma unroll
      for (int s = 0; s < 3; ++s) {
        const int idx = w + 4 * s;
        if (idx < 10) {
          int jb, ib;
          score_tile(idx, jb, ib);
          f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int ks = 0; ks < NKS; ++ks) {
            const op_t A = lds_op<T>(sK, TQ::off(16 * jb + l16, ks * KS + g * E));
            const op_t B = lds_op<T>(sQ, TQ::off(16 * ib + l16, ks * KS + g * E));
            acc = X::mfma(A, B, acc);
          }
          T pv[4];
#pragma unroll
          for (int r = 0; r < 4; ++r) pv[r] = X::from_f(acc[r] * pf[s][r]);
          char* dst = sP + TP::off(16 * ib + l16, 16 * jb + 4 * g);
          if (sizeof(T) == 2)
            *reinterpret_cast<u32x2*>(dst) = *reinterpret_cast<u32x2*>(pv);
          else
            *reinterpret_cast<u32x4*>(dst) = *reinterpret_cast<u32x4*>(pv);
        }
      }
      __syncthreads();

      // ---- state before this chunk as the A operand of O^T = S^T Q^T
      op_t Sop[NVT][NKS];
#pragma unroll
      for (int vt = 0; vt < NVT; ++vt)
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks) {
          if constexpr (E == 8) {
            bf16x8 o;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
              o[r] = (__bf16)accS[2 * ks][vt][r];
              o[4 + r] = (__bf16)accS[2 * ks + 1][vt][r];
            }
            Sop[vt][ks] = o;
          } else {
            Sop[vt][ks] = accS[ks / 4][vt][ks % 4];
          }
        }

      // ---- outputs, one 16-token block at a time
#pragma unroll
      for (int it = 0; it < 4; ++it) {
        const int i = 16 * it + l16;
        f32x4 o[NVT];
#pragma unroll
        for (int vt = 0; vt < NVT; ++vt) o[vt] = f32x4{0.f, 0.f, 0.f, 0.f};
        // inter: sum_k S[k][v] q_i[k], with Q read in the permuted slot order
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks) {
          op_t B;
          if constexpr (E == 8) {
            const u32x2 lo = *reinterpret_cast<const u32x2*>(sQ + TQ::off(i, 32 * ks + 4 * g));
            const u32x2 hi = *reinterpret_cast<const u32x2*>(sQ + TQ::off(i, 32 * ks + 16 + 4 * g));
            const u32x4 both = {lo[0], lo[1], hi[0], hi[1]};
            B = __builtin_bit_cast(bf16x8, both);
          } else {
            B = *reinterpret_cast<const float*>(sQ + TQ::off(i, 16 * (ks / 4) + 4 * g + (ks % 4)));
          }
#pragma unroll
          for (int vt = 0; vt < NVT; ++vt) o[vt] = X::mfma(Sop[vt][ks], B, o[vt]);
        }
#pragma unroll
        for (int vt = 0; vt < NVT; ++vt) o[vt] *= qf[it];
        // intra: sum_j V^T[v][j] P[i][j] over key blocks j < 16 (it + 1)
#pragma unroll
        for (int js = 0; js < NJS; ++js) {
          if (js < njs[it]) {
            const op_t Bp = lds_op<T>(sP, TP::off(i, js * KS + g * E));
#pragma unroll
            for (int vt = 0; vt < NVT; ++vt) {
              const op_t Av = lds_op<T>(sVt, TT::off(16 * (w * NVT + vt) + l16, js * KS + g * E));
              o[vt] = X::mfma(Av, Bp, o[vt]);
            }
          }
        }
        // store: lane holds O[token i][v0 .. v0+3]
        if (c * CH + i < len) {
          T* orow = Og + row_of(t0 + c * CH + i) * D;
#pragma unroll
          for (int vt = 0; vt < NVT; ++vt) {
            const int v0 = 16 * (w * NVT + vt) + 4 * g;
            T ov[4];
#pragma unroll
            for (int r = 0; r < 4; ++r) ov[r] = X::from_f(o[vt][r]);
            if (sizeof(T) == 2)
              *reinterpret_cast<u32x2*>(orow + v0) = *reinterpret_cast<u32x2*>(ov);
            else
              *reinterpret_cast<u32x4*>(orow + v0) = *reinterpret_cast<u32x4*>(ov);
          }
        }
      }
    }

    // ---- state update: S = lambda^cl S + Kt' V
    {
      const float dc = (cl == CH) ? lamC : pow_lam(lg, (float)cl);
#pragma unroll
      for (int tk = 0; tk < NKT; ++tk)
#pragma unroll
        for (int vt = 0; vt < NVT; ++vt) accS[tk][vt] *= dc;
      op_t Bv[NVT][NJS];
#pragma unroll
      for (int vt = 0; vt < NVT; ++vt)
#pragma unroll
        for (int js = 0; js < NJS; ++js)
          Bv[vt][js] = lds_op<T>(sVt, TT::off(16 * (w * NVT + vt) + l16, js * KS + g * E));
#pragma unroll
      for (int tk = 0; tk < NKT; ++tk)
#pragma unroll
        for (int js = 0; js < NJS; ++js) {
          const op_t Ak = lds_op<T>(sKt, TT::off(16 * tk + l16, js * KS + g * E));
#pragma unroll
          for (int vt = 0; vt < NVT; ++vt) accS[tk][vt] = X::mfma(Ak, Bv[vt][js], accS[tk][vt]);
        }
    }
  }

  // ---- final state of this sub-segment
  if (a.Sout && p >= a.sout_p0 && p < a.sout_p0 + a.sout_np) {
    float* dst = a.Sout + (n * a.sout_np + (p - a.sout_p0)) * (int64_t)D * D;
#pragma unroll
    for (int tk = 0; tk < NKT; ++tk)
#pragma unroll
      for (int vt = 0; vt < NVT; ++vt)
#pragma unroll
        for (int r = 0; r < 4; ++r)
          dst[(16 * tk + 4 * g + r) * D + 16 * (w * NVT + vt) + l16] = accS[tk][vt][r];
  }
}

template <typename T, int D>
static hipError_t launch_fwd_t(const FwdArgs& a, bool with_o, int64_t nwg, hipStream_t s) {
  if (with_o)
    hipLaunchKernelGGL((k_chunk_fwd<T, D, true>), dim3((unsigned)nwg), dim3(NTHR), 0, s, a);
  else
    hipLaunchKernelGGL((k_chunk_fwd<T, D, false>), dim3((unsigned)nwg), dim3(NTHR), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_fwd(const FwdArgs& a, int dtype, int D, bool with_o, int64_t nwg,
                      hipStream_t s) {
  if (nwg <= 0) return hipSuccess;
  if (dtype == 0) {
    if (D == 64) return launch_fwd_t<__bf16, 64>(a, with_o, nwg, s);
    if (D == 128) return launch_fwd_t<__bf16, 128>(a, with_o, nwg, s);
  } else {
    if (D == 64) return launch_fwd_t<float, 64>(a, with_o, nwg, s);
    if (D == 128) return launch_fwd_t<float, 128>(a, with_o, nwg, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace la
