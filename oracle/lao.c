/*
 * lao.c -- CPU oracle for decayed causal linear attention (fp64).
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may include, link,
 * load or call this file or the library built from it; only the tests, the
 * smoke check and the benchmark's CPU-baseline leg do.  It shares no code,
 * header, table or helper with the HIP library.
 *
 * What it computes is the plain definition of the method, token by token,
 * in double precision:
 *
 *   state      S_t = lambda * S_{t-1} + k_t v_t^T        (d_k x d_v, row-major)
 *   output     o_t = q_t^T S_t                            (length d_v)
 *   start      S_0 = given initial state (or zero)
 *   end        S_end = S_L
 *
 * Sources on the pages:
 *  - "LASP-2: Rethinking Sequence Parallelism for Linear Attention and Its
 *    Hybrid", abstract: linear attention is evaluated right-product-first and
 *    carries an intermediate memory state whose size does not depend on the
 *    sequence length; the state above is that memory state.
 *  - "ZeCO: Zero Communication Overhead Sequence Parallelism for Linear
 *    Attention", abstract: each sequence-parallel rank needs exactly its
 *    initial operator state; S_0 here is that state, and the segment scan
 *    below is what the All-Scan collective delivers.
 *  - "Lightning Attention-2" entry of the LASP-2 page's related-paper list:
 *    conventional attention inside blocks and the linear-attention kernel
 *    trick between blocks.  The oracle deliberately does NOT use blocks: it
 *    is the token recurrence itself, which the blocked form must reproduce.
 * Readings where the pages are silent (identity feature map, no normaliser,
 * the current token included, S_0 decayed at the first token, a constant
 * decay per head) are listed in the design notes of the repository.
 *
 * Tensor conventions (all contiguous, fp64):
 *   Q, K     [B, H, L, dk]       V, O, dO  [B, H, L, dv]
 *   states   [B, H, nseg, dk, dv]           lambda [H]
 * Each (b, h) sequence is cut into nseg equal segments that are run
 * independently, segment s starting from its own S0[b, h, s].
 *
 * Parallelism: OpenMP over independent (sequence, column block) pairs or
 * (sequence, row block) pairs.  Every element of the state evolves on its
 * own under the recurrence, so splitting by columns (or rows) changes no
 * arithmetic; each reduction (over dk for o_t, over dv for dq_t / dk_t,
 * over dk for dv_t) is summed in plain index order by one thread.
 */
#include <math.h>
#include <omp.h>
#include <stddef.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define LAO_OK 0
#define LAO_EINVAL 1
#define LAO_ENOMEM 2

/* Block width for the OpenMP split over state columns / rows. */
#define LAO_BLK 16

static int lao_check(int64_t B, int64_t H, int64_t L, int64_t dk, int64_t dv,
                     int64_t nseg) {
  if (B < 0 || H < 0 || L < 0 || dk <= 0 || dv <= 0 || nseg <= 0) return 0;
  if (L % nseg != 0) return 0;
  return 1;
}

/* lambda^n for a non-negative integer n, with 0^0 = 1. */
static double lao_pow(double lam, int64_t n) {
  if (n == 0) return 1.0;
  return pow(lam, (double)n);
}

/*
 * Forward recurrence.  O may be NULL (state only), S_end may be NULL.
 * S0 may be NULL (zero initial state).
 */
int lao_fwd(int64_t B, int64_t H, int64_t L, int64_t dk, int64_t dv,
            int64_t nseg, const double* Q, const double* K, const double* V,
            const double* lam, const double* S0, double* O, double* S_end) {
  if (!lao_check(B, H, L, dk, dv, nseg)) return LAO_EINVAL;
  const int64_t Ls = L / nseg;
  const int64_t nseq = B * H * nseg;
  const int64_t ncb = (dv + LAO_BLK - 1) / LAO_BLK;
  int fail = 0;
#pragma omp parallel for collapse(2) schedule(dynamic)
  for (int64_t n = 0; n < nseq; ++n) {
    for (int64_t cb = 0; cb < ncb; ++cb) {
      const int64_t h = (n / nseg) % H;
      const double l = lam[h];
      const int64_t c0 = cb * LAO_BLK;
      const int64_t c1 = (c0 + LAO_BLK < dv) ? c0 + LAO_BLK : dv;
      const int64_t w = c1 - c0;
      double* S = (double*)malloc(sizeof(double) * (size_t)(dk * w));
      if (!S) {
        fail = 1;
        continue;
      }
      for (int64_t i = 0; i < dk; ++i)
        for (int64_t j = 0; j < w; ++j)
          S[i * w + j] = S0 ? S0[(n * dk + i) * dv + c0 + j] : 0.0;
      const double* q = Q + n * Ls * dk;
      const double* k = K + n * Ls * dk;
      const double* v = V + n * Ls * dv;
      for (int64_t t = 0; t < Ls; ++t) {
        /* S = lambda * S + k_t v_t^T */
        for (int64_t i = 0; i < dk; ++i) {
          const double ki = k[t * dk + i];
          for (int64_t j = 0; j < w; ++j)
            S[i * w + j] = l * S[i * w + j] + ki * v[t * dv + c0 + j];
        }
        /* o_t = q_t^T S  (sum over dk in index order) */
        if (O) {
          for (int64_t j = 0; j < w; ++j) {
            double acc = 0.0;
            for (int64_t i = 0; i < dk; ++i) acc += q[t * dk + i] * S[i * w + j];
            O[(n * Ls + t) * dv + c0 + j] = acc;
          }
        }
      }
      if (S_end)
        for (int64_t i = 0; i < dk; ++i)
          for (int64_t j = 0; j < w; ++j)
            S_end[(n * dk + i) * dv + c0 + j] = S[i * w + j];
      free(S);
    }
  }
  return fail ? LAO_ENOMEM : LAO_OK;
}

/*
 * Selected output rows by direct summation of the unrolled recurrence,
 *   o_t = sum_{s<=t} lambda^{t-s} (q_t . k_s) v_s + lambda^t q_t^T S0,
 * (t and s 1-indexed within the segment).  Used where running the full
 * recurrence is too slow: each row costs O(t * d).  rows[r] holds a 0-based
 * token index into the flattened [nseq, Ls] sequence axis of segment seq[r].
 * out is [nrows, dv].
 */
int lao_fwd_rows(int64_t B, int64_t H, int64_t L, int64_t dk, int64_t dv,
                 int64_t nseg, const double* Q, const double* K,
                 const double* V, const double* lam, const double* S0,
                 int64_t nrows, const int64_t* seq, const int64_t* rows,
                 double* out) {
  if (!lao_check(B, H, L, dk, dv, nseg)) return LAO_EINVAL;
  const int64_t Ls = L / nseg;
  const int64_t nseq = B * H * nseg;
  for (int64_t r = 0; r < nrows; ++r)
    if (seq[r] < 0 || seq[r] >= nseq || rows[r] < 0 || rows[r] >= Ls)
      return LAO_EINVAL;
#pragma omp parallel for schedule(dynamic)
  for (int64_t r = 0; r < nrows; ++r) {
    const int64_t n = seq[r], t = rows[r];
    const int64_t h = (n / nseg) % H;
    const double l = lam[h];
    const double* q = Q + (n * Ls + t) * dk;
    double* o = out + r * dv;
    for (int64_t j = 0; j < dv; ++j) o[j] = 0.0;
    for (int64_t s = 0; s <= t; ++s) {
      const double* k = K + (n * Ls + s) * dk;
      const double* v = V + (n * Ls + s) * dv;
      double qk = 0.0;
      for (int64_t i = 0; i < dk; ++i) qk += q[i] * k[i];
      const double wgt = lao_pow(l, t - s) * qk;
      for (int64_t j = 0; j < dv; ++j) o[j] += wgt * v[j];
    }
    if (S0) {
      /* token t (0-based) is token t+1 of the segment: lambda^{t+1} */
      const double w0 = lao_pow(l, t + 1);
      for (int64_t j = 0; j < dv; ++j) {
        double acc = 0.0;
        for (int64_t i = 0; i < dk; ++i) acc += q[i] * S0[(n * dk + i) * dv + j];
        o[j] += w0 * acc;
      }
    }
  }
  return LAO_OK;
}

/*
 * Backward of the recurrence for the loss
 *   l = sum_t <do_t, o_t> + <dS_end, S_end>.
 * With G_t = dl/dS_t (through every later use of S_t):
 *   G_t  = q_t do_t^T + U_t,   U_L = dS_end,   U_{t-1} = lambda * G_t
 *   dq_t = S_t do_t            dk_t = G_t v_t        dv_t = G_t^T k_t
 *   dS0  = U_0 = lambda * G_1
 * S0 and dS_end may be NULL (zero); dS0 may be NULL (not returned).
 * dQ, dK, dV are written in full.
 */
int lao_bwd(int64_t B, int64_t H, int64_t L, int64_t dk, int64_t dv,
            int64_t nseg, const double* Q, const double* K, const double* V,
            const double* lam, const double* S0, const double* dO,
            const double* dS_end, double* dQ, double* dK, double* dV,
            double* dS0) {
  if (!lao_check(B, H, L, dk, dv, nseg)) return LAO_EINVAL;
  const int64_t Ls = L / nseg;
  const int64_t nseq = B * H * nseg;
  const int64_t nrb = (dk + LAO_BLK - 1) / LAO_BLK;
  const int64_t ncb = (dv + LAO_BLK - 1) / LAO_BLK;
  int fail = 0;

  /* (1) dq_t = S_t do_t: forward sweep, rows of S split over threads. */
#pragma omp parallel for collapse(2) schedule(dynamic)
  for (int64_t n = 0; n < nseq; ++n) {
    for (int64_t rb = 0; rb < nrb; ++rb) {
      const int64_t h = (n / nseg) % H;
      const double l = lam[h];
      const int64_t r0 = rb * LAO_BLK;
      const int64_t r1 = (r0 + LAO_BLK < dk) ? r0 + LAO_BLK : dk;
      const int64_t w = r1 - r0;
      double* S = (double*)malloc(sizeof(double) * (size_t)(w * dv));
      if (!S) {
        fail = 1;
        continue;
      }
      for (int64_t i = 0; i < w; ++i)
        for (int64_t j = 0; j < dv; ++j)
          S[i * dv + j] = S0 ? S0[(n * dk + r0 + i) * dv + j] : 0.0;
      const double* k = K + n * Ls * dk;
      const double* v = V + n * Ls * dv;
      const double* g = dO + n * Ls * dv;
      for (int64_t t = 0; t < Ls; ++t) {
        for (int64_t i = 0; i < w; ++i) {
          const double ki = k[t * dk + r0 + i];
          double acc = 0.0;
          for (int64_t j = 0; j < dv; ++j) {
            S[i * dv + j] = l * S[i * dv + j] + ki * v[t * dv + j];
            acc += S[i * dv + j] * g[t * dv + j];
          }
          dQ[(n * Ls + t) * dk + r0 + i] = acc;
        }
      }
      free(S);
    }
  }

  /* (2) dk_t = G_t v_t and dS0: reverse sweep, rows of G split. */
#pragma omp parallel for collapse(2) schedule(dynamic)
  for (int64_t n = 0; n < nseq; ++n) {
    for (int64_t rb = 0; rb < nrb; ++rb) {
      const int64_t h = (n / nseg) % H;
      const double l = lam[h];
      const int64_t r0 = rb * LAO_BLK;
      const int64_t r1 = (r0 + LAO_BLK < dk) ? r0 + LAO_BLK : dk;
      const int64_t w = r1 - r0;
      double* U = (double*)malloc(sizeof(double) * (size_t)(w * dv));
      if (!U) {
        fail = 1;
        continue;
      }
      for (int64_t i = 0; i < w; ++i)
        for (int64_t j = 0; j < dv; ++j)
          U[i * dv + j] = dS_end ? dS_end[(n * dk + r0 + i) * dv + j] : 0.0;
      const double* q = Q + n * Ls * dk;
      const double* v = V + n * Ls * dv;
      const double* g = dO + n * Ls * dv;
      for (int64_t t = Ls - 1; t >= 0; --t) {
        for (int64_t i = 0; i < w; ++i) {
          const double qi = q[t * dk + r0 + i];
          double acc = 0.0;
          for (int64_t j = 0; j < dv; ++j) {
            const double G = qi * g[t * dv + j] + U[i * dv + j];
            acc += G * v[t * dv + j];
            U[i * dv + j] = l * G;
          }
          dK[(n * Ls + t) * dk + r0 + i] = acc;
        }
      }
      if (dS0)
        for (int64_t i = 0; i < w; ++i)
          for (int64_t j = 0; j < dv; ++j)
            dS0[(n * dk + r0 + i) * dv + j] = U[i * dv + j];
      free(U);
    }
  }

  /* (3) dv_t = G_t^T k_t: the same reverse sweep, columns of G split. */
#pragma omp parallel for collapse(2) schedule(dynamic)
  for (int64_t n = 0; n < nseq; ++n) {
    for (int64_t cb = 0; cb < ncb; ++cb) {
      const int64_t h = (n / nseg) % H;
      const double l = lam[h];
      const int64_t c0 = cb * LAO_BLK;
      const int64_t c1 = (c0 + LAO_BLK < dv) ? c0 + LAO_BLK : dv;
      const int64_t w = c1 - c0;
      double* U = (double*)malloc(sizeof(double) * (size_t)(dk * w));
      if (!U) {
        fail = 1;
        continue;
      }
      for (int64_t i = 0; i < dk; ++i)
        for (int64_t j = 0; j < w; ++j)
          U[i * w + j] = dS_end ? dS_end[(n * dk + i) * dv + c0 + j] : 0.0;
      const double* q = Q + n * Ls * dk;
      const double* k = K + n * Ls * dk;
      const double* g = dO + n * Ls * dv;
      double* acc = (double*)malloc(sizeof(double) * (size_t)w);
      if (!acc) {
        free(U);
        fail = 1;
        continue;
      }
      for (int64_t t = Ls - 1; t >= 0; --t) {
        for (int64_t j = 0; j < w; ++j) acc[j] = 0.0;
        for (int64_t i = 0; i < dk; ++i) {
          const double qi = q[t * dk + i];
          const double ki = k[t * dk + i];
          for (int64_t j = 0; j < w; ++j) {
            const double G = qi * g[t * dv + c0 + j] + U[i * w + j];
            acc[j] += G * ki;
            U[i * w + j] = l * G;
          }
        }
        for (int64_t j = 0; j < w; ++j) dV[(n * Ls + t) * dv + c0 + j] = acc[j];
      }
      free(acc);
      free(U);
    }
  }
  return fail ? LAO_ENOMEM : LAO_OK;
}

/*
 * Segment state-combine scan.  For each (b, h), with per-segment local
 * states dS[b, h, s] (each accumulated from a zero state over a segment of
 * seg_len tokens) and decay a = lambda_h^seg_len:
 *   X = S0 (or 0)
 *   for s in 0..P-1 (reverse: P-1..0):  S_start[s] = X;  X = a * X + dS[s]
 *   S_end = X
 * This is the combine that the All-Scan collective of the ZeCO abstract, or
 * the single all-gather of memory states in the LASP-2 abstract, delivers to
 * every rank.  S_start [B,H,P,dk,dv]; S_end [B,H,dk,dv] or NULL.
 */
int lao_scan(int64_t B, int64_t H, int64_t P, int64_t dk, int64_t dv,
             const double* dS, const double* lam, int64_t seg_len,
             const double* S0, double* S_start, double* S_end, int reverse) {
  if (B < 0 || H < 0 || P < 0 || dk <= 0 || dv <= 0 || seg_len < 0)
    return LAO_EINVAL;
  const int64_t E = dk * dv;
#pragma omp parallel for collapse(2) schedule(static)
  for (int64_t bh = 0; bh < B * H; ++bh) {
    for (int64_t e = 0; e < E; ++e) {
      const int64_t h = bh % H;
      const double a = lao_pow(lam[h], seg_len);
      double X = S0 ? S0[bh * E + e] : 0.0;
      for (int64_t it = 0; it < P; ++it) {
        const int64_t s = reverse ? (P - 1 - it) : it;
        S_start[(bh * P + s) * E + e] = X;
        X = a * X + dS[(bh * P + s) * E + e];
      }
      if (S_end) S_end[bh * E + e] = X;
    }
  }
  return LAO_OK;
}

/*
 * Gated forward recurrence: the decay becomes a per-token, per-head scalar
 * gate alpha_t = exp(g_t), g_t = log alpha_t <= 0,
 *
 *   S_t = alpha_t * S_{t-1} + k_t v_t^T        o_t = q_t^T S_t
 *
 * the data-dependent-gate generalisation named in the "Gated Linear Attention
 * Transformers with Hardware-Efficient Training" entry of the LASP-2 page's
 * related-paper list, in its plainest reading (one scalar gate per token and
 * head; see the design notes).  G holds g in the token layout of Q without
 * the feature axis: [B, H, L].  Everything else as lao_fwd.
 */
int lao_fwd_gated(int64_t B, int64_t H, int64_t L, int64_t dk, int64_t dv,
                  int64_t nseg, const double* Q, const double* K, const double* V,
                  const double* G, const double* S0, double* O, double* S_end) {
  if (!lao_check(B, H, L, dk, dv, nseg)) return LAO_EINVAL;
  const int64_t Ls = L / nseg;
  const int64_t nseq = B * H * nseg;
  const int64_t ncb = (dv + LAO_BLK - 1) / LAO_BLK;
  int fail = 0;
#pragma omp parallel for collapse(2) schedule(dynamic)
  for (int64_t n = 0; n < nseq; ++n) {
    for (int64_t cb = 0; cb < ncb; ++cb) {
      const int64_t c0 = cb * LAO_BLK;
      const int64_t c1 = (c0 + LAO_BLK < dv) ? c0 + LAO_BLK : dv;
      const int64_t w = c1 - c0;
      double* S = (double*)malloc(sizeof(double) * (size_t)(dk * w));
      if (!S) {
        fail = 1;
        continue;
      }
      const double* s0 = S0 ? S0 + n * dk * dv : NULL;
      for (int64_t i = 0; i < dk; ++i)
        for (int64_t j = 0; j < w; ++j) S[i * w + j] = s0 ? s0[i * dv + c0 + j] : 0.0;
      const double* q = Q + n * Ls * dk;
      const double* k = K + n * Ls * dk;
      const double* v = V + n * Ls * dv;
      const double* g = G + n * Ls;
      for (int64_t t = 0; t < Ls; ++t) {
        /* S = alpha_t * S + k_t v_t^T */
        const double a = exp(g[t]);
        for (int64_t i = 0; i < dk; ++i) {
          const double ki = k[t * dk + i];
          for (int64_t j = 0; j < w; ++j)
            S[i * w + j] = a * S[i * w + j] + ki * v[t * dv + c0 + j];
        }
        if (O) {
          for (int64_t j = 0; j < w; ++j) {
            double o = 0.0;
            for (int64_t i = 0; i < dk; ++i) o += S[i * w + j] * q[t * dk + i];
            O[(n * Ls + t) * dv + c0 + j] = o;
          }
        }
      }
      if (S_end)
        for (int64_t i = 0; i < dk; ++i)
          for (int64_t j = 0; j < w; ++j)
            S_end[(n * dk + i) * dv + c0 + j] = S[i * w + j];
      free(S);
    }
  }
  return fail ? LAO_ENOMEM : LAO_OK;
}

/*
 * Segment combine with a decay per segment: LD[b, h, s] is the log of the
 * product of the gates over segment s, so
 *   X = S0 (or 0)
 *   for s in 0..P-1 (reverse: P-1..0):  S_start[s] = X;  X = exp(LD[s]) X + dS[s]
 *   S_end = X
 * (lao_scan with a = lambda^seg_len replaced by the segment's own product).
 */
int lao_scan_gated(int64_t B, int64_t H, int64_t P, int64_t dk, int64_t dv,
                   const double* dS, const double* LD, const double* S0, double* S_start,
                   double* S_end, int reverse) {
  if (B < 0 || H < 0 || P < 0 || dk <= 0 || dv <= 0) return LAO_EINVAL;
  const int64_t E = dk * dv;
#pragma omp parallel for collapse(2) schedule(static)
  for (int64_t bh = 0; bh < B * H; ++bh) {
    for (int64_t e = 0; e < E; ++e) {
      double X = S0 ? S0[bh * E + e] : 0.0;
      for (int64_t it = 0; it < P; ++it) {
        const int64_t s = reverse ? (P - 1 - it) : it;
        S_start[(bh * P + s) * E + e] = X;
        X = exp(LD[bh * P + s]) * X + dS[(bh * P + s) * E + e];
      }
      if (S_end) S_end[bh * E + e] = X;
    }
  }
  return LAO_OK;
}

/*
 * Backward of the gated recurrence (lao_fwd_gated) for the same loss
 *   l = sum_t <do_t, o_t> + <dS_end, S_end>,
 * with G_t = dl/dS_t and the gate of token t scaling S_{t-1}:
 *   G_t  = q_t do_t^T + U_t,   U_L = dS_end,   U_{t-1} = alpha_t G_t
 *   dq_t = S_t do_t            dk_t = G_t v_t        dv_t = G_t^T k_t
 *   dS0  = U_0 = alpha_1 G_1
 *   dg_t = d l / d log(alpha_t) = alpha_t <G_t, S_{t-1}>   (Frobenius)
 * The last term needs S_{t-1} during the reverse sweep: each row block keeps
 * its state every LAO_CKPT tokens on the way forward and recomputes the
 * states of one stretch at a time on the way back (the same recurrence,
 * re-run).  Per row block the products are summed over the block's rows,
 * and the blocks' partial sums are added in block order afterwards.
 * S0, dS_end may be NULL (zero); dS0 may be NULL.  dG is [B, H, L].
 */
#define LAO_CKPT 64
int lao_bwd_gated(int64_t B, int64_t H, int64_t L, int64_t dk, int64_t dv, int64_t nseg,
                  const double* Q, const double* K, const double* V, const double* Gl,
                  const double* S0, const double* dO, const double* dS_end, double* dQ,
                  double* dK, double* dV, double* dS0, double* dG) {
  if (!lao_check(B, H, L, dk, dv, nseg)) return LAO_EINVAL;
  const int64_t Ls = L / nseg;
  const int64_t nseq = B * H * nseg;
  const int64_t nrb = (dk + LAO_BLK - 1) / LAO_BLK;
  const int64_t ncb = (dv + LAO_BLK - 1) / LAO_BLK;
  const int64_t nck = Ls / LAO_CKPT + 1;
  double* part = (double*)calloc((size_t)(nseq * nrb * (Ls > 0 ? Ls : 1)), sizeof(double));
  if (!part) return LAO_ENOMEM;
  int fail = 0;

  /* (1) dq_t = S_t do_t: forward sweep, rows of S split over threads. */
#pragma omp parallel for collapse(2) schedule(dynamic)
  for (int64_t n = 0; n < nseq; ++n) {
    for (int64_t rb = 0; rb < nrb; ++rb) {
      const int64_t r0 = rb * LAO_BLK;
      const int64_t w = ((r0 + LAO_BLK < dk) ? r0 + LAO_BLK : dk) - r0;
      double* S = (double*)malloc(sizeof(double) * (size_t)(w * dv));
      if (!S) {
        fail = 1;
        continue;
      }
      for (int64_t i = 0; i < w; ++i)
        for (int64_t j = 0; j < dv; ++j) S[i * dv + j] = S0 ? S0[(n * dk + r0 + i) * dv + j] : 0.0;
      const double* k = K + n * Ls * dk;
      const double* v = V + n * Ls * dv;
      const double* go = dO + n * Ls * dv;
      const double* gl = Gl + n * Ls;
      for (int64_t t = 0; t < Ls; ++t) {
        const double a = exp(gl[t]);
        for (int64_t i = 0; i < w; ++i) {
          const double ki = k[t * dk + r0 + i];
          double acc = 0.0;
          for (int64_t j = 0; j < dv; ++j) {
            S[i * dv + j] = a * S[i * dv + j] + ki * v[t * dv + j];
            acc += S[i * dv + j] * go[t * dv + j];
          }
          dQ[(n * Ls + t) * dk + r0 + i] = acc;
        }
      }
      free(S);
    }
  }

  /* (2) dk_t = G_t v_t, dS0 and the row block's share of <G_t, S_{t-1}>:
   * reverse sweep, rows split; S_{t-1} recomputed from checkpoints. */
#pragma omp parallel for collapse(2) schedule(dynamic)
  for (int64_t n = 0; n < nseq; ++n) {
    for (int64_t rb = 0; rb < nrb; ++rb) {
      const int64_t r0 = rb * LAO_BLK;
      const int64_t w = ((r0 + LAO_BLK < dk) ? r0 + LAO_BLK : dk) - r0;
      const size_t blk = (size_t)(w * dv);
      double* U = (double*)malloc(sizeof(double) * blk);
      double* ck = (double*)malloc(sizeof(double) * blk * (size_t)nck);
      double* run = (double*)malloc(sizeof(double) * blk * (LAO_CKPT + 1));
      if (!U || !ck || !run) {
        free(U), free(ck), free(run);
        fail = 1;
        continue;
      }
      const double* q = Q + n * Ls * dk;
      const double* k = K + n * Ls * dk;
      const double* v = V + n * Ls * dv;
      const double* go = dO + n * Ls * dv;
      const double* gl = Gl + n * Ls;
      /* forward: S_t of this row block, kept at t = 0, LAO_CKPT, 2 LAO_CKPT, ... */
      double* S = run;
      for (int64_t i = 0; i < w; ++i)
        for (int64_t j = 0; j < dv; ++j) S[i * dv + j] = S0 ? S0[(n * dk + r0 + i) * dv + j] : 0.0;
      for (int64_t t = 0; t < Ls; ++t) {
        if (t % LAO_CKPT == 0) memcpy(ck + (size_t)(t / LAO_CKPT) * blk, S, sizeof(double) * blk);
        const double a = exp(gl[t]);
        for (int64_t i = 0; i < w; ++i)
          for (int64_t j = 0; j < dv; ++j)
            S[i * dv + j] = a * S[i * dv + j] + k[t * dk + r0 + i] * v[t * dv + j];
      }
      for (int64_t i = 0; i < w; ++i)
        for (int64_t j = 0; j < dv; ++j)
          U[i * dv + j] = dS_end ? dS_end[(n * dk + r0 + i) * dv + j] : 0.0;
      /* backward, one stretch [t0, t1) at a time, last stretch first */
      for (int64_t t0 = ((Ls - 1) / LAO_CKPT) * LAO_CKPT; t0 >= 0 && Ls > 0; t0 -= LAO_CKPT) {
        const int64_t t1 = (t0 + LAO_CKPT < Ls) ? t0 + LAO_CKPT : Ls;
        /* run[m] = S_{t0 + m}, i.e. the state before token t0 + m */
        memcpy(run, ck + (size_t)(t0 / LAO_CKPT) * blk, sizeof(double) * blk);
        for (int64_t t = t0; t < t1 - 1; ++t) {
          const double a = exp(gl[t]);
          double* prev = run + (size_t)(t - t0) * blk;
          double* next = prev + blk;
          for (int64_t i = 0; i < w; ++i)
            for (int64_t j = 0; j < dv; ++j)
              next[i * dv + j] = a * prev[i * dv + j] + k[t * dk + r0 + i] * v[t * dv + j];
        }
        for (int64_t t = t1 - 1; t >= t0; --t) {
          const double a = exp(gl[t]);
          const double* Sprev = run + (size_t)(t - t0) * blk; /* S_{t-1} */
          double dot = 0.0;
          for (int64_t i = 0; i < w; ++i) {
            const double qi = q[t * dk + r0 + i];
            double acc = 0.0;
            for (int64_t j = 0; j < dv; ++j) {
              const double G = qi * go[t * dv + j] + U[i * dv + j];
              acc += G * v[t * dv + j];
              dot += G * Sprev[i * dv + j];
              U[i * dv + j] = a * G;
            }
            dK[(n * Ls + t) * dk + r0 + i] = acc;
          }
          part[(n * nrb + rb) * Ls + t] = dot;
        }
      }
      if (dS0)
        for (int64_t i = 0; i < w; ++i)
          for (int64_t j = 0; j < dv; ++j) dS0[(n * dk + r0 + i) * dv + j] = U[i * dv + j];
      free(U), free(ck), free(run);
    }
  }

  /* (3) dv_t = G_t^T k_t: the same reverse sweep, columns split. */
#pragma omp parallel for collapse(2) schedule(dynamic)
  for (int64_t n = 0; n < nseq; ++n) {
    for (int64_t cb = 0; cb < ncb; ++cb) {
      const int64_t c0 = cb * LAO_BLK;
      const int64_t w = ((c0 + LAO_BLK < dv) ? c0 + LAO_BLK : dv) - c0;
      double* U = (double*)malloc(sizeof(double) * (size_t)(dk * w));
      double* acc = (double*)malloc(sizeof(double) * (size_t)w);
      if (!U || !acc) {
        free(U), free(acc);
        fail = 1;
        continue;
      }
      for (int64_t i = 0; i < dk; ++i)
        for (int64_t j = 0; j < w; ++j)
          U[i * w + j] = dS_end ? dS_end[(n * dk + i) * dv + c0 + j] : 0.0;
      const double* q = Q + n * Ls * dk;
      const double* k = K + n * Ls * dk;
      const double* go = dO + n * Ls * dv;
      const double* gl = Gl + n * Ls;
      for (int64_t t = Ls - 1; t >= 0; --t) {
        const double a = exp(gl[t]);
        for (int64_t j = 0; j < w; ++j) acc[j] = 0.0;
        for (int64_t i = 0; i < dk; ++i) {
          const double qi = q[t * dk + i];
          const double ki = k[t * dk + i];
          for (int64_t j = 0; j < w; ++j) {
            const double G = qi * go[t * dv + c0 + j] + U[i * w + j];
            acc[j] += ki * G;
            U[i * w + j] = a * G;
          }
        }
        for (int64_t j = 0; j < w; ++j) dV[(n * Ls + t) * dv + c0 + j] = acc[j];
      }
      free(acc), free(U);
    }
  }

  /* dg_t = alpha_t * sum over row blocks (in block order) */
  if (!fail)
    for (int64_t n = 0; n < nseq; ++n)
      for (int64_t t = 0; t < Ls; ++t) {
        double sum = 0.0;
        for (int64_t rb = 0; rb < nrb; ++rb) sum += part[(n * nrb + rb) * Ls + t];
        dG[n * Ls + t] = exp(Gl[n * Ls + t]) * sum;
      }
  free(part);
  return fail ? LAO_ENOMEM : LAO_OK;
}

int lao_abi_version(void) { return 1; }

/* Number of OpenMP threads the oracle's parallel loops use. */
int lao_threads(void) {
  int n = 1;
#pragma omp parallel
  {
#pragma omp single
    n = omp_get_num_threads();
  }
  return n;
}

/* Run later calls on n OpenMP threads (n >= 1); returns the count now in
 * force.  Changes no arithmetic: every thread's share is a fixed set of
 * independent columns or rows. */
int lao_set_threads(int n) {
  if (n >= 1) omp_set_num_threads(n);
  return lao_threads();
}
