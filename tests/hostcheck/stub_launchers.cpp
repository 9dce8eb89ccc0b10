// stub_launchers.cpp -- host-only stand-ins for the kernel launchers of
// liblinattn.so, so that la_api.cpp (argument validation and the launch
// plan) can be built with the host compiler and its sanitizers and driven
// without a GPU.  Each stand-in launches nothing: it checks that the plan
// handed to it is self-consistent (sizes positive, sub-segments whole chunks,
// workspace pointers present when the plan needs them) and counts the call.
// Test infrastructure only; never part of the library.
#include <cstdio>
#include <cstdlib>

#include "la_internal.h"

namespace la {

int g_launches = 0;

static void expect(bool ok, const char* what) {
  if (!ok) {
    std::fprintf(stderr, "stub launcher: inconsistent plan: %s\n", what);
    std::abort();
  }
}

static void check_fwd(const FwdArgs& a, int64_t nwg) {
  expect(nwg > 0, "workgroups");
  expect(a.Ls >= 0 && a.Lp > 0 && a.Lp % 64 == 0, "sub-segment length");
  expect(a.split >= 1 && a.p_begin >= 0 && a.p_count >= 1 && a.p_begin + a.p_count <= a.split,
         "sub-segment range");
  expect(a.H >= 1 && a.nseg >= 1, "heads and segments");
  expect(a.K && a.V, "K and V");
  expect(a.gated ? a.G != nullptr : a.lam != nullptr, "decay");
  if (a.start_from_state && a.split > 1) expect(a.Sws != nullptr, "start states");
  expect(a.sws_step >= 1 && a.sws_nper >= 0, "start-state partition");
}

hipError_t launch_fwd(const FwdArgs& a, int, int D, bool with_o, int64_t nwg, hipStream_t) {
  if (nwg <= 0) return hipSuccess;
  check_fwd(a, nwg);
  expect(D == 64 || D == 128, "head dimension");
  if (with_o) expect(a.Q && a.O, "Q and O");
  ++g_launches;
  return hipSuccess;
}

hipError_t launch_fwd_pair(const FwdArgs& a, const FwdArgs& b, int, int, int64_t nitems,
                           hipStream_t) {
  if (nitems <= 0) return hipSuccess;
  check_fwd(a, nitems);
  check_fwd(b, nitems);
  expect(a.gated == b.gated, "pair of one kind");
  ++g_launches;
  return hipSuccess;
}

hipError_t launch_fwd_triple(const FwdArgs& a, const FwdArgs& b, const FwdArgs& c, int, int,
                             int64_t nitems, hipStream_t) {
  if (nitems <= 0) return hipSuccess;
  check_fwd(a, nitems);
  check_fwd(b, nitems);
  check_fwd(c, nitems);
  expect(a.gated == b.gated && a.gated == c.gated, "triple of one kind");
  expect(a.Q && a.O && b.Q && b.O && c.Q && c.O, "outputs of all three");
  ++g_launches;
  return hipSuccess;
}

hipError_t launch_fwd_u(const FwdArgs& a, int dtype, int, int64_t nitems, hipStream_t) {
  if (nitems <= 0) return hipSuccess;
  check_fwd(a, nitems);
  expect(dtype == 0, "U-forming walk is bf16");
  expect(a.Q && a.O && a.Q2 && a.Uout, "outputs and U");
  expect(!a.gated || (a.G && a.LDrev), "gated U: gates and reverse log-gates");
  expect(!a.rk || a.gated, "row dots: gated");
  ++g_launches;
  return hipSuccess;
}

hipError_t launch_fwd_duo(const FwdArgs& a, const FwdArgs& b, int dtype, int D, int64_t nitems,
                          hipStream_t) {
  if (nitems <= 0) return hipSuccess;
  expect(!a.rk && (!b.rk || (b.gated && D == 128)), "row dots: gated, d = 128, second set");
  expect(dtype == 0, "bf16");
  check_fwd(a, nitems);
  check_fwd(b, nitems);
  expect(dtype == 0, "joint dV/dK walk is bf16 only");
  expect(a.gated == b.gated && a.G == b.G, "one gate sequence");
  expect(a.K == b.V && a.V == b.K, "crosswise keys and values");
  expect(a.Ls == b.Ls && a.Lp == b.Lp && a.split == b.split && a.reverse == b.reverse &&
             a.ragged_first == b.ragged_first && a.p_begin == b.p_begin && a.p_count == b.p_count,
         "one plan");
  expect(a.Q && a.O && b.Q && b.O, "outputs of both");
  ++g_launches;
  return hipSuccess;
}

hipError_t launch_scan(const ScanArgs& a, hipStream_t) {
  expect(a.nseq >= 0 && a.P >= 0 && a.E > 0, "scan sizes");
  if (a.P > 0) expect(a.dS && a.Sout, "scan buffers");
  expect(a.gated ? (a.P == 0 || a.LD != nullptr) : a.lam != nullptr, "scan decay");
  ++g_launches;
  return hipSuccess;
}

hipError_t launch_transpose_copy(const float* src, float* dst, int64_t nmat, int D, hipStream_t) {
  if (nmat <= 0) return hipSuccess;
  expect(src && dst && src != dst && D % 32 == 0, "transpose");
  ++g_launches;
  return hipSuccess;
}

hipError_t launch_prep(const PrepArgs& a, hipStream_t) {
  expect(a.src && a.dst && a.nseq > 0 && (a.mode == 0 || a.lam), "prep");
  ++g_launches;
  return hipSuccess;
}

hipError_t launch_shift_gates(const float* G, float* Gs, int64_t, int64_t, hipStream_t) {
  expect(G && Gs, "gate shift");
  ++g_launches;
  return hipSuccess;
}

hipError_t launch_scale_first_gate(float* X, const float* G, int64_t, int64_t, int, hipStream_t) {
  expect(X && G, "first gate");
  ++g_launches;
  return hipSuccess;
}

int64_t gate_grad_blocks(int64_t Ls) { return (Ls + 1023) / 1024; }

hipError_t launch_gate_anchors(const float* WfT, const float* WrT, const float* G, const float*,
                               const float*, float* tot, int64_t, int64_t, int, hipStream_t) {
  expect(G && tot, "anchors");
  (void)WfT;
  (void)WrT;
  ++g_launches;
  return hipSuccess;
}

hipError_t launch_gate_grad(int, int, const void* Q, const void* dQ, const void* K, const void* dK,
                            float* dG, const float* tot, int64_t, int64_t, hipStream_t) {
  // K, dK null: dG holds k . dk from the joint dV/dK walk
  expect(Q && dQ && dG && tot && ((K == nullptr) == (dK == nullptr)), "gate gradient");
  ++g_launches;
  return hipSuccess;
}

hipError_t launch_gate_grad_rows(const float* rq, float* dG, const float* WfT, const float* WrT,
                                 const float* G, const float*, const float*, int64_t, int64_t,
                                 int D, hipStream_t) {
  expect(rq && dG && G && D == 128, "gate gradient from the walks' row dots");
  (void)WfT;
  (void)WrT;
  ++g_launches;
  return hipSuccess;
}

hipError_t launch_tangent(const TanArgs& a, int, int D, int64_t nseq, float* dlam, hipStream_t) {
  expect(nseq >= 0 && dlam && a.lam && (D == 64 || D == 128), "tangent");
  if (nseq > 0 && a.split > 1) expect(a.WS && a.WT && a.part, "tangent workspace");
  ++g_launches;
  return hipSuccess;
}

hipError_t launch_step(const StepArgs& a, int, int D, int64_t nseq, hipStream_t) {
  expect(nseq > 0 && a.q && a.k && a.v && (a.lam != nullptr) != (a.loga != nullptr) && a.Sout &&
             (D == 64 || D == 128),
         "step");
  ++g_launches;
  return hipSuccess;
}

}  // namespace la
