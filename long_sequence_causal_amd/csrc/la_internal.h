// la_internal.h -- host-side interface between the C ABI layer (la_api.cpp)
// and the kernel launchers (la_fwd.hip, la_scan.hip, la_gate.hip,
// la_tangent.hip, la_step.hip).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "linattn.h"

namespace la {

// Record the message la_last_error() returns on this thread (printf format)
// and return st.
la_status record_error(la_status st, const char* fmt, ...);

// Every check la_chunk_fwd makes except the workspace's: host only, no HIP
// call; LA_OK or the failing status (with la_last_error() set).
la_status check_fwd_args(const la_shape* s, const void* Q, const void* K, const void* V,
                         const float* lambda, const float* S0, const void* O, const float* S_end);

// One launch of the chunk kernel over sub-segments [p_begin, p_begin+p_count)
// of every one of nseq sequences.  Sequence n occupies token rows
// [n*Ls, (n+1)*Ls) of the flattened [nseq*Ls, D] token tensors; its head is
// (n / nseg) % H.  Sub-segment p covers tokens [p*Lp, min(Ls, (p+1)*Lp)).
struct FwdArgs {
  const void* Q;
  const void* K;
  const void* V;
  const float* lam;
  int H;
  int nseg;
  int64_t Ls;
  int64_t Lp;
  int split;
  int p_begin;
  int p_count;
  // start state: 0 = zero; 1 = S0[n] (zero if S0 is null) for p == 0 and
  // Sws[n][p-1] for p > 0
  int start_from_state;
  const float* S0;   // [nseq][D][D]
  const float* Sws;  // [nseq][sws_nper][D][D]
  // Sws holds the start states of a finer partition of each sequence into
  // sub-segments of Lp / sws_step tokens, cut the same way (ragged_first
  // alike): sws_nper = its sub-segment count - 1.  sws_step = 1 and
  // sws_nper = split - 1 is this launch's own partition.
  int64_t sws_nper;
  int sws_step;
  void* O;           // [nseq*Ls][D], null in state-only launches
  // the final state of sub-segment p is written to Sout[n][p - sout_p0] when
  // p is in [sout_p0, sout_p0 + sout_np)
  float* Sout;
  int sout_p0;
  int sout_np;
  // reverse time order (token t of a sequence is read as token Ls-1-t); used
  // by the backward's reverse sweeps
  int reverse;
  // sub-segment partition: 0 = [p Lp, min((p+1) Lp, Ls)) (a short last one);
  // 1 = the short one first, [max(0, e - Lp), e) with e = Ls - (split-1-p) Lp,
  // so that a reverse sweep cuts a sequence at the same rows m Lp as a
  // forward one
  int ragged_first;
  // gated recurrence (gated != 0): log-gates G [nseq*Ls], read only for the
  // chunks walked, and lam is never read; state-only launches write the total
  // log-gate of each sub-segment to LDout[n][p - sout_p0] beside Sout
  int gated;
  const float* G;
  float* LDout;
  // fixed decay, sub-segment 0 from S0: S0 is the state after the first
  // token's decay (S_1 = S0 + k_1 v_1^T instead of lambda S0 + k_1 v_1^T).
  // The backward's reverse sweeps start from dS_end this way, which spares
  // them a division by lambda.
  int s0_undecayed;
  // the start states are stored transposed ([col][row]; S0 and Sws
  // separately): the backward's sweeps read S0^T, dS_end^T and the dV
  // sweep's start states as the dK sweep's this way, with no transposed copy
  int s0_transposed;
  int sws_transposed;
  // state-only launches: walk each sub-segment's chunks last
  // first (the state a sub-segment ends with is the same sum, so only the
  // rounding order changes); a sub-segment with a ragged chunk walks in order
  int last_chunk_first;
  // launch_fwd_u only: each sub-segment p >= 1 also forms
  // U = sum_t w_t Q2_t Q_t^T over its tokens and writes it to
  // Uout[n][split - 1 - p] ([nseq][split-1][D][D], the numbering of a
  // reverse sweep whose sub-segments end where these start); w_t =
  // lambda^(t - t0) (t0 the first token), gated the product of the gates of
  // tokens t0+1 .. t; gated, the sub-segment's log-gate sum as that reverse
  // sweep sees it (gates shifted by one token) goes to LDrev[n][split - 1 - p]
  const void* Q2;
  float* Uout;
  float* LDrev;
  // gated, bf16, d = 128 (may be null): row dots [nseq][Ls] over the bf16
  // outputs in fp32.  launch_fwd_duo, second argument set: rk[n][row] =
  // (first set's Q row) . (second set's output row) (the gated backward's
  // k_t . dk_t); launch_fwd_u: (Q2 row) . (output row) (q_t . dq_t)
  float* rk;
  // launches with outputs (may be null): the state at every boundary row
  // y = m * dump_rows (0 < y < Ls; dump_rows a power of two, at least 64) of
  // each sequence, to
  // dump[n][m - 1] ([nseq][ceil(Ls / dump_rows) - 1][D][D]), or to
  // dump[n][ceil(Ls / dump_rows) - 1 - m] when dump_rev; written by the walk
  // whose chunk ends there (reverse sweeps: at Ls % 64 == 0 every such row
  // ends a chunk)
  float* dump;
  int dump_rows;
  int dump_rev;
};

// dst[n] = f(src[n]) for nseq D x D fp32 states: optional transpose, then a
// per-head factor (mode 0: none, 1: * lambda_h).
struct PrepArgs {
  int64_t nseq;
  int D;
  const float* src;
  float* dst;
  const float* lam;
  int H;
  int hdiv;
  int transpose;
  int mode;
};

// Segment scan over nseq sequences of P states of E floats each.
struct ScanArgs {
  int64_t nseq;
  int P;
  int64_t E;
  const float* dS;   // [nseq][P][E]
  const float* lam;  // [H]; head of sequence n is (n / hdiv) % H
  int H;
  int hdiv;
  int64_t seg_len;
  const float* S0;   // [nseq][E] or null
  float* Sout;       // [nseq][P][E], may alias dS
  float* Send;       // [nseq][E] or null
  int reverse;
  int inclusive;     // 0: Sout[s] = state before adding dS[s]; 1: after
  // the first segment decays S0 by lambda^(seg_len - 1) instead of
  // lambda^seg_len (S0 already carries the first token's decay; fixed decay)
  int s0_undecayed;
  // S0 is stored transposed (E = d * d)
  int s0_transposed;
  int d;
  // fixed decay: the first segment in scan order spans first_len tokens
  // (0: seg_len like the others), the short one of a partition cut from the
  // sequence's other end
  int64_t first_len;
  // gated != 0: segment s of sequence n decays by exp(LD[n][s]) instead of
  // lambda^seg_len (lam is then never read, LD only for s < P)
  int gated;
  const float* LD;   // [nseq][P]
};

// Decay gradient by the tangent recurrence (la_tangent.hip).  Sequence n has
// head (n / nseg) % H and Ls tokens cut into `split` sub-segments of Lp.
struct TanArgs {
  const void* Q;     // [nseq][Ls][D] (main pass only)
  const void* K;
  const void* V;
  const void* dO;    // (main pass only)
  const float* lam;  // [H]
  const float* S0;   // [nseq][D][D] or null
  const float* dSe;  // [nseq][D][D] or null
  float* WS;         // [nseq][pre_r (split-1)][D][D]: local, then start states
  float* WT;         // the same for the tangent state
  double* part;      // [nseq][split]: each sub-segment's share of the gradient
  int H;
  int nseg;
  int split;
  int64_t Ls;
  int64_t Lp;
  // the pre-pass walks pre_r pieces of Lp / pre_r tokens per sub-segment
  // (pre_r = 1 or 2, Lp / pre_r a multiple of 64); WS, WT then hold
  // pre_r (split - 1) pairs per sequence, and the start pair of sub-segment
  // p >= 1 is entry pre_r p - 1
  int pre_r;
};
// Pre-pass over sub-segments 0..split-2, the scan of (state, tangent) pairs,
// the main pass over every sub-segment and the per-head sum into dlam.
hipError_t launch_tangent(const TanArgs& a, int dtype, int D, int64_t nseq, float* dlam,
                          hipStream_t stream);

// One decode step for nseq = B * H sequences (la_step.hip); head of
// sequence n is n % H.
struct StepArgs {
  const void* q;     // [nseq][D]
  const void* k;     // [nseq][D]
  const void* v;     // [nseq][D]
  const float* lam;  // [H]
  const float* loga; // [nseq] or null: the token's log-gate per sequence, in place of lam
  const float* S;    // [nseq][D][D] or null (zero)
  float* Sout;       // [nseq][D][D], may equal S
  void* o;           // [nseq][D] or null
  int H;
};
hipError_t launch_step(const StepArgs& a, int dtype, int D, int64_t nseq, hipStream_t stream);

// Two chunk-kernel launches with outputs over nitems work items each, as one
// grid whose partner workgroups share an XCD (la_fwd.hip); a.gated == b.gated.
hipError_t launch_fwd_pair(const FwdArgs& a, const FwdArgs& b, int dtype, int D, int64_t nitems,
                           hipStream_t stream);
hipError_t launch_fwd(const FwdArgs& a, int dtype, int D, bool with_o, int64_t nwg,
                      hipStream_t stream);
// Three chunk-kernel launches with outputs over nitems work items each as one
// grid (la_fwd.hip): a's items beside the XCD-paired items of b and c;
// a.gated == b.gated == c.gated.
hipError_t launch_fwd_triple(const FwdArgs& a, const FwdArgs& b, const FwdArgs& c, int dtype,
                             int D, int64_t nitems, hipStream_t stream);
// Two chunk-kernel launches with outputs over nitems work items each whose
// recurrences have crosswise keys and values (b.K == a.V, b.V == a.K; same
// plan, decay and gates) as one workgroup per item (la_fwd.hip); bf16 only.
hipError_t launch_fwd_duo(const FwdArgs& a, const FwdArgs& b, int dtype, int D, int64_t nitems,
                          hipStream_t stream);
// The chunk kernel with outputs over nitems work items of a (fixed decay,
// a.Q2 and a.Uout set), every sub-segment also forming its U (la_fwd.hip).
hipError_t launch_fwd_u(const FwdArgs& a, int dtype, int D, int64_t nitems, hipStream_t stream);
hipError_t launch_scan(const ScanArgs& a, hipStream_t stream);
// dst[m] = src[m]^T for nmat consecutive D x D fp32 matrices (no overlap).
hipError_t launch_transpose_copy(const float* src, float* dst, int64_t nmat, int D,
                                 hipStream_t stream);
hipError_t launch_prep(const PrepArgs& a, hipStream_t stream);
// Gated backward helpers (la_gate.hip): shifted gates for the reverse
// sweeps, dS0 scaled by the first gate of each sequence, and the log-gate
// gradient from Q, dQ, K, dK (tot: [nseq][gate_grad_blocks(Ls)] floats of
// workspace; dSe and SendT may be null).
hipError_t launch_shift_gates(const float* G, float* Gs, int64_t nseq, int64_t Ls, hipStream_t s);
hipError_t launch_scale_first_gate(float* X, const float* G, int64_t nseq, int64_t Ls, int D,
                                   hipStream_t s);
int64_t gate_grad_blocks(int64_t Ls);
// Per sequence n and block b of GBLK tokens, the gate gradient at the first
// token of block b + 1: alpha_y <G_y, S_{y-1}> at y = (b+1) GBLK from the
// forward sweep's start states WfT ([nseq][nb-1] of S^T) and the reverse
// sweep's, transposed (WrT, [nseq][nb-1] of G^T, in reverse order);
// for the last block <dS_end, S_end> (dSe, SendT may be null: 0).  Written
// to tot[n][b] for launch_gate_grad_finish.  Requires 1024-token sub-segments.
hipError_t launch_gate_anchors(const float* WfT, const float* WrT, const float* G,
                               const float* dSe, const float* SendT, float* tot, int64_t nseq,
                               int64_t Ls, int D, hipStream_t s);
// dG[t] = the in-block suffix sum of r_u = q_u . dq_u - k_u . dk_u plus
// tot[n][t / GBLK].  With K and dK null, dG must already hold k_t . dk_t per
// token (the joint dV/dK walk's row dots) and is overwritten in place.
hipError_t launch_gate_grad(int dtype, int D, const void* Q, const void* dQ, const void* K,
                            const void* dK, float* dG, const float* tot, int64_t nseq, int64_t Ls,
                            hipStream_t s);
// Both row dots from the walks (rq [nseq][Ls]: q_t . dq_t from the dQ walk;
// dG: k_t . dk_t from the joint dV/dK walk): one pass that forms each block's
// anchor as launch_gate_anchors does (same arguments) and writes dG[t] = the
// in-block suffix sum of rq - dG plus the anchor, in place.
hipError_t launch_gate_grad_rows(const float* rq, float* dG, const float* WfT, const float* WrT,
                                 const float* G, const float* dSe, const float* SendT,
                                 int64_t nseq, int64_t Ls, int D, hipStream_t s);

}  // namespace la
