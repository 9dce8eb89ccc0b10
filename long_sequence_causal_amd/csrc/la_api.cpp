// la_api.cpp -- the C ABI of liblinattn.so (declared in include/linattn.h).
//
// Host-side only: argument validation (pure host code, before any HIP call),
// the launch plan and the sequence of kernel launches on the caller's stream.
// The library allocates no memory and keeps no device state.
//
// Launch plan.  A sequence (one segment of one (b, h)) has a carried state, so
// one workgroup walks its chunks in order.  When there are fewer sequences
// than the chip has compute units, each is cut into `split` sub-segments and
// the dependency between them is resolved the way the sequence-parallel
// schemes of the pages resolve it between ranks (ZeCO abstract: every rank
// needs precisely its initial operator state; LASP-2 abstract: one exchange of
// length-independent memory states):
//   1. local state of every sub-segment but the last, from a zero state
//      (state-only chunk kernel);
//   2. inclusive scan X <- lambda^Lp X + dS over those local states, seeded
//      with S0, giving the start state of sub-segments 1..split-1;
//   3. the full chunk kernel over all sub-segments, each from its start state.
// Step 1 re-reads K and V for (split-1)/split of the tokens: that is the price
// of the parallelism, traded against running 32 heads on 256 compute units.
#include <hip/hip_runtime.h>

#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <string>

#include "la_internal.h"
#include "linattn.h"

namespace {

constexpr int kChunk = 64;
// Workgroups the plan aims for: one per compute unit of an MI355X.
constexpr int64_t kTargetWG = 256;
// Chunks per sub-segment at or above which the chunk walks prefer two
// rounds of workgroups to one (see check_shape).
constexpr int64_t kTwoRoundChunks = 128;

thread_local std::string g_last_error;

la_status vfail(la_status st, const char* fmt, va_list ap) {
  char buf[512];
  vsnprintf(buf, sizeof(buf), fmt, ap);
  g_last_error = std::string(la_status_str(st)) + ": " + buf;
  return st;
}

la_status fail(la_status st, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  const la_status r = vfail(st, fmt, ap);
  va_end(ap);
  return r;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// A launch covers at most 2^32 - 1 work-items (blocks x threads per block).
// Every launch of a plan is sized by one of these counts, checked on the host
// before anything is launched.
constexpr double kMaxItems = 4294967295.0;
bool fits_grid(double items) { return items <= kMaxItems; }

struct Plan {
  int64_t nseq = 0;  // B * H * nseg independent sequences
  int64_t Ls = 0;    // tokens per sequence
  int split = 1;     // sub-segments per sequence
  int64_t Lp = kChunk;  // tokens per sub-segment (multiple of 64; the last is shorter)
  int D = 0;
  bool ragged_first = false;  // the short sub-segment first (gated reverse sweeps)
};

// Shape checks shared by forward and backward.  No HIP call.
// two_rounds: the automatic split may double so that the chunk walks fill
// the chip twice (measured faster for the fixed-decay forward and backward
// when each sub-segment still spans at least kTwoRoundChunks chunks, e.g.
// 16 sequences of 256K tokens: 512 walks of 8K tokens beat 256 of 16K; the
// tangent walks of la_decay_grad, bound by their arithmetic, do not gain).
la_status check_shape(const la_shape* s, Plan* plan, bool two_rounds = true) {
  if (!s) return fail(LA_ERR_INVALID_ARG, "shape is NULL");
  if (s->B < 0 || s->H < 0 || s->L < 0)
    return fail(LA_ERR_INVALID_ARG, "negative size (B=%lld H=%lld L=%lld)", (long long)s->B,
                (long long)s->H, (long long)s->L);
  if (s->dk <= 0 || s->dv <= 0) return fail(LA_ERR_INVALID_ARG, "dk and dv must be positive");
  if (s->nseg < 1) return fail(LA_ERR_INVALID_ARG, "nseg must be >= 1");
  if (s->L % s->nseg != 0)
    return fail(LA_ERR_INVALID_ARG, "L=%lld is not a multiple of nseg=%d", (long long)s->L, s->nseg);
  if (s->dtype != LA_BF16 && s->dtype != LA_FP32)
    return fail(LA_ERR_INVALID_ARG, "unknown dtype %d", s->dtype);
  if (s->split < 0) return fail(LA_ERR_INVALID_ARG, "split must be >= 0");
  if (s->reserved != 0) return fail(LA_ERR_INVALID_ARG, "reserved must be 0");
  if (s->dk != s->dv) return fail(LA_ERR_UNSUPPORTED, "dk != dv (%d, %d)", s->dk, s->dv);
  if (s->dk != 64 && s->dk != 128) return fail(LA_ERR_UNSUPPORTED, "d=%d not in {64, 128}", s->dk);
  // sizes must stay far from int64 overflow in element offsets
  const double elems = (double)s->B * (double)s->H * (double)s->L * (double)s->dk;
  const double states = (double)s->B * (double)s->H * (double)s->nseg * s->dk * s->dv;
  if (elems > 4.0e18 || states > 4.0e18) return fail(LA_ERR_INVALID_ARG, "tensor too large");
  if ((double)s->B * s->H * s->nseg > 2.0e9) return fail(LA_ERR_INVALID_ARG, "too many sequences");

  plan->nseq = s->B * s->H * (int64_t)s->nseg;
  plan->Ls = s->L / s->nseg;
  // the kernels address one sequence's tokens with 32-bit byte offsets
  const int64_t elt = s->dtype == LA_FP32 ? 4 : 2;
  if ((double)plan->Ls * s->dk * elt >= 4294967296.0)
    return fail(LA_ERR_UNSUPPORTED, "one segment spans %lld tokens; at most 2^32 bytes per segment",
                (long long)plan->Ls);
  plan->D = s->dk;
  const int64_t nchunks = (plan->Ls + kChunk - 1) / kChunk;
  int64_t want = s->split > 0 ? s->split
                              : (plan->nseq > 0 ? (kTargetWG + plan->nseq - 1) / plan->nseq : 1);
  if (s->split == 0 && two_rounds && plan->nseq * 2 * want <= 2 * kTargetWG &&
      nchunks >= 2 * want * kTwoRoundChunks)
    want *= 2;
  if (want > nchunks) want = nchunks;
  if (want < 1) want = 1;
  const int64_t cps = nchunks > 0 ? (nchunks + want - 1) / want : 1;  // chunks per sub-segment
  plan->Lp = cps * kChunk;
  plan->split = nchunks > 0 ? (int)((nchunks + cps - 1) / cps) : 1;
  // launch sizes: paired chunk walks (D/16 waves per workgroup), one thread
  // per state element (scans, transposes, prepared states) and per token
  // (gates)
  const double walks = (double)plan->nseq * plan->split;
  if (!fits_grid(2.0 * walks * 4.0 * plan->D) ||
      !fits_grid(walks * (double)plan->D * plan->D) ||
      !fits_grid((double)plan->nseq * ((double)plan->Ls + 1024.0)))
    return fail(LA_ERR_UNSUPPORTED, "%lld sequences of %lld tokens exceed one launch's grid",
                (long long)plan->nseq, (long long)plan->Ls);
  return LA_OK;
}

size_t scan_ws_bytes(const Plan& p) {
  return (size_t)p.nseq * (size_t)(p.split - 1) * (size_t)p.D * (size_t)p.D * sizeof(float);
}

// la_chunk_bwd's workspace: the sub-segment start states of the dQ sweep and
// of the dV sweep (the dK sweep reads the dV sweep's transposed)
size_t bwd_ws_bytes(const Plan& p) { return 2 * scan_ws_bytes(p); }

la_status hip_fail(hipError_t e, const char* what) {
  return fail(LA_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

// Arguments of the chunk kernel shared by every launch of one recurrence.
la::FwdArgs flow_args(const Plan& pl, int H, int nseg, const void* Q, const void* K, const void* V,
                      const float* lam, int reverse) {
  la::FwdArgs fa;
  std::memset(&fa, 0, sizeof(fa));
  fa.Q = Q;
  fa.K = K;
  fa.V = V;
  fa.lam = lam;
  fa.H = H;
  fa.nseg = nseg;
  fa.Ls = pl.Ls;
  fa.Lp = pl.Lp;
  fa.split = pl.split;
  fa.reverse = reverse;
  fa.ragged_first = pl.ragged_first;
  fa.sws_nper = pl.split - 1;
  fa.sws_step = 1;
  return fa;
}

// Start states of sub-segments 1..split-1 of one recurrence into W
// ([nseq][split-1][D][D]): state-only pre-pass over sub-segments
// 0..split-2 from zero, then an inclusive scan seeded with `start` (null =
// zero).  Nothing to do when split == 1.
la_status run_states(const Plan& pl, int dtype, int H, int nseg, const void* K, const void* V,
                     const float* lam, const float* start, float* W, int reverse, hipStream_t st,
                     bool gated = false, const float* G = nullptr, float* LDw = nullptr,
                     bool start_undecayed = false, bool start_transposed = false) {
  if (pl.nseq == 0 || pl.split <= 1) return LA_OK;
  la::FwdArgs pa = flow_args(pl, H, nseg, nullptr, K, V, lam, reverse);
  pa.gated = gated;  // gated: sub-segment log-gates to LDw for the combine
  pa.G = G;
  pa.LDout = LDw;
  pa.p_begin = 0;
  pa.p_count = pl.split - 1;
  pa.start_from_state = 0;
  pa.Sout = W;
  pa.sout_p0 = 0;
  pa.sout_np = pl.split - 1;
  // last chunk first: the chunks this pass reads last are the ones the main
  // pass reads first, so those are still in the last-level cache then
  pa.last_chunk_first = 1;
  hipError_t e = la::launch_fwd(pa, dtype, pl.D, false, pl.nseq * (pl.split - 1), st);
  if (e != hipSuccess) return hip_fail(e, "state pre-pass launch");
  la::ScanArgs sa;
  std::memset(&sa, 0, sizeof(sa));
  sa.nseq = pl.nseq;
  sa.P = pl.split - 1;
  sa.E = (int64_t)pl.D * pl.D;
  sa.dS = W;
  sa.lam = lam;
  sa.H = H;
  sa.hdiv = nseg;
  sa.seg_len = pl.Lp;
  sa.S0 = start;
  sa.Sout = W;
  sa.Send = nullptr;
  sa.reverse = 0;
  sa.inclusive = 1;
  sa.s0_undecayed = start_undecayed;
  sa.s0_transposed = start_transposed;
  sa.d = pl.D;
  sa.gated = gated;
  sa.LD = LDw;
  e = la::launch_scan(sa, st);
  if (e != hipSuccess) return hip_fail(e, "state scan launch");
  return LA_OK;
}

// The chunk kernel over every sub-segment from its start state (`start` for
// sub-segment 0, W for the others), writing O and/or Send.  With O null only
// the last sub-segment runs (state only).
la::FwdArgs main_args(const Plan& pl, int H, int nseg, const void* Q, const void* K,
                      const void* V, const float* lam, const float* start, void* O, float* Send,
                      const float* W, int reverse, bool gated, const float* G) {
  la::FwdArgs ma = flow_args(pl, H, nseg, Q, K, V, lam, reverse);
  ma.gated = gated;
  ma.G = G;
  ma.start_from_state = 1;
  ma.S0 = start;
  ma.Sws = W;
  ma.O = O;
  ma.Sout = Send;
  ma.sout_p0 = pl.split - 1;
  ma.sout_np = 1;
  if (O) {
    ma.p_begin = 0;
    ma.p_count = pl.split;
  } else {
    ma.p_begin = pl.split - 1;
    ma.p_count = 1;
  }
  return ma;
}

la_status run_main(const Plan& pl, int dtype, int H, int nseg, const void* Q, const void* K,
                   const void* V, const float* lam, const float* start, void* O, float* Send,
                   const float* W, int reverse, hipStream_t st, bool gated = false,
                   const float* G = nullptr) {
  if (pl.nseq == 0 || (!O && !Send)) return LA_OK;
  const la::FwdArgs ma = main_args(pl, H, nseg, Q, K, V, lam, start, O, Send, W, reverse, gated, G);
  hipError_t e = la::launch_fwd(ma, dtype, pl.D, O != nullptr, pl.nseq * ma.p_count, st);
  if (e != hipSuccess) return hip_fail(e, "chunk kernel launch");
  return LA_OK;
}

// One forward recurrence over nseq sequences (optionally in reverse time):
// start states when split > 1, then the main pass.  `start` [nseq][D][D]
// may be null (zero).  O may be null (state only); Send may be null.
la_status run_flow(const Plan& pl, int dtype, int H, int nseg, const void* Q, const void* K,
                   const void* V, const float* lam, const float* start, void* O, float* Send,
                   float* W, int reverse, hipStream_t st, bool gated = false,
                   const float* G = nullptr, float* LDw = nullptr) {
  if (pl.nseq == 0 || (!O && !Send)) return LA_OK;
  la_status r = run_states(pl, dtype, H, nseg, K, V, lam, start, W, reverse, st, gated, G, LDw);
  if (r != LA_OK) return r;
  return run_main(pl, dtype, H, nseg, Q, K, V, lam, start, O, Send, W, reverse, st, gated, G);
}

// The backward's three sweeps from their start states (aq: dQ; av, ak: dV
// and dK, whose keys and values are crosswise the same Q and dO).  bf16: the
// dQ sweep, then one workgroup per item walking both dV and dK over one
// stream of Q, K, V, dO tiles (4 tile loads per chunk instead of 6, one set
// of barriers and decay factors for two walks).  fp32: one launch of the
// three, the paired dV and dK workgroups on one XCD beside the dQ walks.
hipError_t launch_sweeps(const la::FwdArgs& aq, const la::FwdArgs& av, const la::FwdArgs& ak,
                         int dtype, int D, int64_t nitems, hipStream_t st) {
  if (dtype == LA_BF16) {
    hipError_t e = la::launch_fwd(aq, dtype, D, true, nitems, st);
    if (e != hipSuccess) return e;
    return la::launch_fwd_duo(av, ak, dtype, D, nitems, st);
  }
  return la::launch_fwd_triple(aq, av, ak, dtype, D, nitems, st);
}

// Workspace of la_decay_grad: the local, then start, pairs (S, U) of
// sub-segments 1..split-1 (S and U in separate blocks) and one fp64 share per
// sub-segment.
struct TangentWs {
  size_t WS = 0, WT = 0, part = 0, total = 0;
};
// pieces per sub-segment of the tangent pre-pass: two when they stay whole
// chunks (the pre-pass runs two workgroups a CU and has twice as many to
// place)
int tangent_pre_r(const Plan& p) { return (p.Lp % (2 * kChunk) == 0) ? 2 : 1; }
TangentWs tangent_ws(const Plan& p) {
  auto up = [](size_t x) { return (x + 255) / 256 * 256; };
  TangentWs w;
  const size_t st = (size_t)tangent_pre_r(p) * scan_ws_bytes(p);
  w.WS = 0;
  w.WT = up(st);
  w.part = w.WT + up(st);
  w.total = w.part + up((size_t)p.nseq * (size_t)p.split * sizeof(double));
  return w;
}

// gated forward workspace: the start states, then the sub-segment log-gates
size_t gated_ws_bytes(const Plan& p) {
  if (p.split <= 1) return 0;
  return scan_ws_bytes(p) + ((size_t)p.nseq * (size_t)(p.split - 1) * sizeof(float) + 255) / 256 * 256;
}

}  // namespace

la_status la::record_error(la_status st, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  const la_status r = vfail(st, fmt, ap);
  va_end(ap);
  return r;
}

extern "C" {

int la_version(void) { return 1; }

const char* la_status_str(la_status s) {
  switch (s) {
    case LA_OK: return "LA_OK";
    case LA_ERR_INVALID_ARG: return "LA_ERR_INVALID_ARG";
    case LA_ERR_UNSUPPORTED: return "LA_ERR_UNSUPPORTED";
    case LA_ERR_WORKSPACE: return "LA_ERR_WORKSPACE";
    case LA_ERR_HIP: return "LA_ERR_HIP";
  }
  return "LA_ERR_UNKNOWN";
}

const char* la_last_error(void) { return g_last_error.c_str(); }

size_t la_fwd_workspace_bytes(const la_shape* shape) {
  Plan pl;
  std::string keep = g_last_error;
  if (check_shape(shape, &pl) != LA_OK) {
    g_last_error = keep;
    return 0;
  }
  return scan_ws_bytes(pl);
}

size_t la_bwd_workspace_bytes(const la_shape* shape) {
  Plan pl;
  std::string keep = g_last_error;
  if (check_shape(shape, &pl) != LA_OK) {
    g_last_error = keep;
    return 0;
  }
  return bwd_ws_bytes(pl);
}

}  // extern "C"

// Every check of la_chunk_fwd but the workspace's (host only, no HIP call).
la_status la::check_fwd_args(const la_shape* s, const void* Q, const void* K, const void* V,
                             const float* lambda, const float* S0, const void* O,
                             const float* S_end) {
  Plan pl;
  la_status r = check_shape(s, &pl);
  if (r != LA_OK) return r;
  const bool has_tokens = pl.nseq > 0 && pl.Ls > 0;
  if (has_tokens && (!Q || !K || !V)) return fail(LA_ERR_INVALID_ARG, "Q, K and V are required");
  if (pl.nseq > 0 && !lambda) return fail(LA_ERR_INVALID_ARG, "lambda is required");
  if (!O && !S_end) return fail(LA_ERR_INVALID_ARG, "O and S_end are both NULL");
  const void* ptrs[] = {Q, K, V, lambda, S0, O, S_end};
  for (const void* p : ptrs)
    if (p && !aligned16(p)) return fail(LA_ERR_INVALID_ARG, "pointer %p is not 16-byte aligned", p);
  return LA_OK;
}

extern "C" {

la_status la_chunk_fwd(const la_shape* s, const void* Q, const void* K, const void* V,
                       const float* lambda, const float* S0, void* O, float* S_end, void* ws,
                       size_t ws_bytes, void* stream) {
  la_status r = la::check_fwd_args(s, Q, K, V, lambda, S0, O, S_end);
  if (r != LA_OK) return r;
  Plan pl;
  check_shape(s, &pl);
  if (ws && !aligned16(ws)) return fail(LA_ERR_INVALID_ARG, "pointer %p is not 16-byte aligned", ws);
  const size_t need = scan_ws_bytes(pl);
  if (need > 0 && (!ws || ws_bytes < need))
    return fail(LA_ERR_WORKSPACE, "workspace of %zu bytes needed, %zu given", need,
                ws ? ws_bytes : (size_t)0);
  if (pl.nseq == 0) return LA_OK;
  return run_flow(pl, s->dtype, (int)s->H, s->nseg, Q, K, V, lambda, S0, O, S_end,
                  static_cast<float*>(ws), 0, static_cast<hipStream_t>(stream));
}

size_t la_fwd_gated_workspace_bytes(const la_shape* shape) {
  Plan pl;
  std::string keep = g_last_error;
  if (check_shape(shape, &pl) != LA_OK) {
    g_last_error = keep;
    return 0;
  }
  return gated_ws_bytes(pl);
}

la_status la_chunk_fwd_gated(const la_shape* s, const void* Q, const void* K, const void* V,
                             const float* log_alpha, const float* S0, void* O, float* S_end,
                             void* ws, size_t ws_bytes, void* stream) {
  Plan pl;
  la_status r = check_shape(s, &pl);
  if (r != LA_OK) return r;
  const bool has_tokens = pl.nseq > 0 && pl.Ls > 0;
  if (has_tokens && (!Q || !K || !V || !log_alpha))
    return fail(LA_ERR_INVALID_ARG, "Q, K, V and log_alpha are required");
  if (!O && !S_end) return fail(LA_ERR_INVALID_ARG, "O and S_end are both NULL");
  const void* ptrs[] = {Q, K, V, log_alpha, S0, O, S_end, ws};
  for (const void* p : ptrs)
    if (p && !aligned16(p)) return fail(LA_ERR_INVALID_ARG, "pointer %p is not 16-byte aligned", p);
  const size_t need = gated_ws_bytes(pl);
  if (need > 0 && (!ws || ws_bytes < need))
    return fail(LA_ERR_WORKSPACE, "workspace of %zu bytes needed, %zu given", need,
                ws ? ws_bytes : (size_t)0);
  if (pl.nseq == 0) return LA_OK;
  float* W = static_cast<float*>(ws);
  float* LDw = W ? W + scan_ws_bytes(pl) / sizeof(float) : nullptr;
  return run_flow(pl, s->dtype, (int)s->H, s->nseg, Q, K, V, nullptr, S0, O, S_end, W, 0,
                  static_cast<hipStream_t>(stream), true, log_alpha, LDw);
}

// The gated backward forms the sweeps' states on sub-segments of exactly 1024
// tokens (whatever `split` asks for): the start states at their boundaries
// anchor the log-gate gradient (launch_gate_anchors, or inside
// launch_gate_grad_rows), so that its suffix sums never run over more than
// 1024 tokens.  The reverse sweeps take the short
// sub-segment first, which puts their boundaries on the same rows.
constexpr int64_t kGateBlock = 1024;
Plan gated_bwd_plan(const Plan& p) {
  Plan g = p;
  const int64_t nchunks = (p.Ls + kChunk - 1) / kChunk;
  const int64_t cps = kGateBlock / kChunk;
  g.Lp = kGateBlock;
  g.split = nchunks > 0 ? (int)((nchunks + cps - 1) / cps) : 1;
  return g;
}

// The gated sweeps themselves walk coarser sub-segments: the automatic
// plan's (p0), rounded up to whole 1024-token blocks, i.e. `step` blocks
// each, and take their start states from every step-th entry of the
// 1024-token states (short walks measured slower).  Cut the same way as the
// fine plan, so every coarse boundary is a fine one.
Plan gated_sweep_plan(const Plan& p0, const Plan& fine, int64_t* step) {
  Plan c = fine;
  const int64_t blocks = (p0.Lp + kGateBlock - 1) / kGateBlock;
  *step = blocks > 0 ? blocks : 1;
  c.Lp = *step * kGateBlock;
  const int64_t nchunks = (p0.Ls + kChunk - 1) / kChunk;
  const int64_t cps = c.Lp / kChunk;
  c.split = nchunks > 0 ? (int)((nchunks + cps - 1) / cps) : 1;
  return c;
}

// Every sub-segment p >= 1 of the coarse plan c starts on a boundary of the
// fine plan f, whose start state sits in slot [0, f.split - 2] (the slot
// rule of the chunk kernel, sws_slot).
bool sweep_slots_valid(const Plan& c, const Plan& f, int64_t step) {
  const int64_t nper = f.split - 1;
  for (int64_t p = 1; p < c.split; ++p) {
    const int64_t slot = c.ragged_first ? nper - (c.split - p) * step : p * step - 1;
    if (slot < 0 || slot >= nper) return false;
    const int64_t fp = slot + 1;  // fine sub-segment starting there
    const int64_t fstart = f.ragged_first ? f.Ls - (f.split - fp) * f.Lp : fp * f.Lp;
    const int64_t cstart = c.ragged_first ? c.Ls - (c.split - p) * c.Lp : p * c.Lp;
    if (fstart != cstart) return false;
  }
  return true;
}

// gated backward workspace (in order): the prepared start states of the dQ
// sweep (S0^T) and of the dK sweep (dS_end^T) [nseq][D][D] each, the forward
// sweep's start states W, the dV sweep's W2 and their transposes W3 for the
// dK sweep (each [nseq][split-1][D][D]; W and W3 also feed the anchors), the
// sweeps' sub-segment log-gates (reused), shifted gates [nseq][Ls], the final
// dQ-sweep state [nseq][D][D] and one anchor per 1024-token block
struct GatedBwdWs {
  size_t W, W2, W3, Wc, W2c, LD, LDr, Gs, RQ, SE, TOT, total;
};
GatedBwdWs gated_bwd_ws(const Plan& p0) {
  const Plan p = gated_bwd_plan(p0);
  int64_t step = 1;
  const Plan pc = gated_sweep_plan(p0, p, &step);
  GatedBwdWs w;
  auto up = [](size_t b) { return (b + 255) / 256 * 256; };
  const size_t DD4 = (size_t)p.D * p.D * sizeof(float);
  size_t o = 0;
  w.W = o;  o += up(scan_ws_bytes(p));   // 1024-row states (forward)
  w.W2 = o; o += up(scan_ws_bytes(p));
  w.W3 = o; o += up(scan_ws_bytes(p));   // (reverse, transposed)
  w.Wc = o;  o += up(scan_ws_bytes(pc));  // the sweeps' own start states
  w.W2c = o; o += up(scan_ws_bytes(pc));
  w.LD = o; o += up((size_t)p.nseq * (size_t)(p.split > 1 ? p.split - 1 : 0) * sizeof(float));
  w.LDr = o; o += up((size_t)pc.nseq * (size_t)(pc.split > 1 ? pc.split - 1 : 0) * sizeof(float));
  w.Gs = o; o += up((size_t)p.nseq * (size_t)p.Ls * sizeof(float));
  w.RQ = o; o += up((size_t)p.nseq * (size_t)p.Ls * sizeof(float));  // q_t . dq_t
  w.SE = o; o += up((size_t)p.nseq * DD4);
  w.TOT = o; o += up((size_t)p.nseq * (size_t)la::gate_grad_blocks(p.Ls) * sizeof(float));
  w.total = o;
  return w;
}

size_t la_bwd_gated_workspace_bytes(const la_shape* shape) {
  Plan pl;
  std::string keep = g_last_error;
  if (check_shape(shape, &pl) != LA_OK) {
    g_last_error = keep;
    return 0;
  }
  return gated_bwd_ws(pl).total;
}

// The backward of la_chunk_fwd_gated; with from_fwd, fwd_starts holds the
// start states S [nseq][split-1][D][D] a la_chunk_fwd_gated call of the same
// shape left in its workspace, which the dQ sweep reads transposed when it
// walks that call's sub-segments.
static la_status chunk_bwd_gated(const la_shape* s, const void* Q, const void* K,
                                 const void* V, const float* log_alpha, const float* S0,
                                 const void* dO, const float* dS_end, const float* fwd_starts,
                                 bool from_fwd, void* dQ, void* dK, void* dV, float* dS0,
                                 float* dlog_alpha, void* ws, size_t ws_bytes, void* stream) {
  Plan pl0;
  la_status r = check_shape(s, &pl0);
  if (r != LA_OK) return r;
  // 1024-token blocks: one workgroup of 256 each (anchors, gate gradient),
  // their start states one thread per element
  const double gblocks = (double)pl0.nseq * (double)((pl0.Ls + kGateBlock - 1) / kGateBlock + 1);
  if (!fits_grid(gblocks * 256.0) || !fits_grid(gblocks * (double)pl0.D * pl0.D) ||
      !fits_grid(gblocks * 2.0 * 4.0 * pl0.D))
    return fail(LA_ERR_UNSUPPORTED, "too many 1024-token blocks for one launch");
  const Plan pl = gated_bwd_plan(pl0);  // forward sweep's 1024-token states
  Plan plr = pl;                        // reverse sweeps'
  plr.ragged_first = true;
  int64_t step = 1;
  const Plan plc = gated_sweep_plan(pl0, pl, &step);  // the sweeps' own walks
  Plan plrc = plc;
  plrc.ragged_first = true;
  if (!sweep_slots_valid(plc, pl, step) || !sweep_slots_valid(plrc, plr, step))
    return fail(LA_ERR_UNSUPPORTED, "sweep plan does not align with the 1024-token states");
  const bool has_tokens = pl.nseq > 0 && pl.Ls > 0;
  if (has_tokens && (!Q || !K || !V || !log_alpha || !dO || !dQ || !dK || !dV))
    return fail(LA_ERR_INVALID_ARG, "Q, K, V, log_alpha, dO, dQ, dK and dV are required");
  if (from_fwd && pl0.nseq > 0 && pl0.split > 1 && !fwd_starts)
    return fail(LA_ERR_INVALID_ARG, "fwd_ws is required (this shape splits sequences)");
  const void* ptrs[] = {Q, K, V, log_alpha, S0, dO, dS_end, dQ, dK, dV, dS0, dlog_alpha, ws,
                        fwd_starts};
  for (const void* p : ptrs)
    if (p && !aligned16(p)) return fail(LA_ERR_INVALID_ARG, "pointer %p is not 16-byte aligned", p);
  const GatedBwdWs L = gated_bwd_ws(pl0);
  if (L.total > 0 && (!ws || ws_bytes < L.total))
    return fail(LA_ERR_WORKSPACE, "workspace of %zu bytes needed, %zu given", L.total,
                ws ? ws_bytes : (size_t)0);
  if (pl.nseq == 0) return LA_OK;
  hipStream_t st = static_cast<hipStream_t>(stream);
  char* base = static_cast<char*>(ws);
  float* W = reinterpret_cast<float*>(base + L.W);    // forward sweep: S^T starts
  float* W2 = reinterpret_cast<float*>(base + L.W2);  // dV sweep: G starts
  float* W3 = reinterpret_cast<float*>(base + L.W3);  // dK sweep: G^T starts
  float* Wc = reinterpret_cast<float*>(base + L.Wc);  // the same on the sweeps' plan
  float* W2c = reinterpret_cast<float*>(base + L.W2c);
  float* LDw = reinterpret_cast<float*>(base + L.LD);
  float* LDr = reinterpret_cast<float*>(base + L.LDr);
  float* RQ = reinterpret_cast<float*>(base + L.RQ);
  float* Gs = reinterpret_cast<float*>(base + L.Gs);
  float* SE = reinterpret_cast<float*>(base + L.SE);
  float* TOT = reinterpret_cast<float*>(base + L.TOT);
  const int H = (int)s->H;
  hipError_t e;

  // dq_t = S_t dO_t: the gated forward recurrence of S^T read by dO, from
  // S0^T (S0 read transposed); it ends with S_end^T, kept for the log-gate
  // gradient
  // The sweeps walk plc (sub-segments of step x 1024 tokens) from start
  // states formed on that plan, and write the 1024-row states the log-gate
  // anchors need (W and W3) themselves as they pass those rows; every such
  // row then has to end a chunk of the reverse sweeps too, which holds when
  // Ls % 64 == 0.  Otherwise (with the log-gate gradient asked for) the
  // pre-passes and scans run on the 1024-token plan, which gives those
  // states directly, and the sweeps start from every step-th of them.
  const bool fine = dlog_alpha && pl.Ls % kChunk != 0;
  const Plan& pf = fine ? pl : plc;    // plan of the forward start states
  const Plan& prf = fine ? plr : plrc;  // and of the reverse ones
  float* const Wf = fine ? W : Wc;
  float* const W2f = fine ? W2 : W2c;
  const int sstep = fine ? (int)step : 1;
  const bool dumps = dlog_alpha && !fine;
  const bool need_send = dlog_alpha && dS_end;
  // the forward's start states serve when the sweeps walk its own sub-segments
  const bool reuse = from_fwd && !fine && pf.split > 1 && pf.Lp == pl0.Lp &&
                     pf.split == pl0.split && pf.ragged_first == pl0.ragged_first;
  if (!reuse) {
    r = run_states(pf, s->dtype, H, s->nseg, V, K, nullptr, S0, Wf, 0, st, true, log_alpha, LDw,
                   false, true);
    if (r != LA_OK) return r;
  }
  la::FwdArgs aq = main_args(plc, H, s->nseg, dO, V, K, nullptr, S0, dQ,
                             need_send ? SE : nullptr, Wf, 0, true, log_alpha);
  aq.s0_transposed = 1;
  aq.sws_nper = pf.split - 1;
  aq.sws_step = sstep;
  if (reuse) {
    aq.Sws = fwd_starts;
    aq.sws_transposed = 1;
  }
  if (dumps) {
    aq.dump = W;
    aq.dump_rows = (int)kGateBlock;
    aq.dump_rev = 0;
  }

  // reverse sweeps: from token t+1 back to t with alpha_{t+1}
  if ((e = la::launch_shift_gates(log_alpha, Gs, pl.nseq, pl.Ls, st)) != hipSuccess)
    return hip_fail(e, "gate shift launch");
  // dv_t = G_t^T k_t, G accumulating q dO^T from dS_end (the first reverse
  // step multiplies by 1); its final value G_1 gives dS0 = alpha_1 G_1.
  // dk_t = G_t v_t: the same reverse recurrence for G^T, whose sub-segment
  // start states are the transposes of the dV sweep's.  One set of local
  // states and one scan serve both, and the two sweeps share their Q and dO
  // reads (launch_sweeps).
  //
  // bf16 on the sweeps' plan: the dQ walk (four tiles: dO, V, K, Q) forms the
  // reverse sweeps' local states U = sum_t (gates of t0+1 .. t) q_t dO_t^T
  // and their reverse log-gates itself, instead of a pre-pass reading Q and
  // dO again, and at d = 128 leaves q_t . dq_t per token for the log-gate
  // gradient.
  const bool fused = s->dtype == LA_BF16 && !fine;
  const bool rk_from_walk = dlog_alpha && s->dtype == LA_BF16 && pl.D == 128;
  const bool rq_from_walk = rk_from_walk && fused;
  if (fused) {
    aq.Q2 = Q;
    aq.Uout = W2f;
    aq.LDrev = LDr;
    if (rq_from_walk) aq.rk = RQ;
    if ((e = la::launch_fwd_u(aq, s->dtype, pl.D, plc.nseq * plc.split, st)) != hipSuccess)
      return hip_fail(e, "dQ sweep launch");
    if (plc.split > 1) {
      la::ScanArgs sa;
      std::memset(&sa, 0, sizeof(sa));
      sa.nseq = plc.nseq;
      sa.P = plc.split - 1;
      sa.E = (int64_t)plc.D * plc.D;
      sa.dS = W2f;
      sa.H = H;
      sa.hdiv = s->nseg;
      sa.seg_len = plc.Lp;
      sa.S0 = dS_end;
      sa.Sout = W2f;
      sa.inclusive = 1;
      sa.gated = 1;
      sa.LD = LDr;
      if ((e = la::launch_scan(sa, st)) != hipSuccess) return hip_fail(e, "state scan launch");
    }
  } else {
    r = run_states(prf, s->dtype, H, s->nseg, Q, dO, nullptr, dS_end, W2f, 1, st, true, Gs, LDw);
    if (r != LA_OK) return r;
  }
  // (the 1024-token plan's anchors read the reverse states transposed from W3)
  if (fine && prf.split > 1) {
    e = la::launch_transpose_copy(W2f, W3, prf.nseq * (prf.split - 1), prf.D, st);
    if (e != hipSuccess) return hip_fail(e, "transpose launch");
  }
  {
    // the dV and dK sweeps (with the dQ sweep unless it ran above): the start
    // states are ready, and both plans have plc.split walks per sequence
    la::FwdArgs av = main_args(plrc, H, s->nseg, K, Q, dO, nullptr, dS_end, dV, dS0, W2f, 1,
                               true, Gs);
    la::FwdArgs ak = main_args(plrc, H, s->nseg, V, dO, Q, nullptr, dS_end, dK, nullptr, W2f, 1,
                               true, Gs);
    ak.s0_transposed = ak.sws_transposed = 1;  // dS_end^T, G^T
    av.sws_nper = ak.sws_nper = prf.split - 1;
    av.sws_step = ak.sws_step = sstep;
    if (dumps) {
      ak.dump = W3;  // G^T at the 1024-token rows, numbered from the end
      ak.dump_rows = (int)kGateBlock;
      ak.dump_rev = 1;
    }
    // the joint dV/dK walk (bf16, d = 128) also leaves k_t . dk_t per token
    // in dlog_alpha for the log-gate gradient below
    if (rk_from_walk) ak.rk = dlog_alpha;
    if (fused)
      e = la::launch_fwd_duo(av, ak, s->dtype, pl.D, plc.nseq * plc.split, st);
    else
      e = launch_sweeps(aq, av, ak, s->dtype, pl.D, plc.nseq * plc.split, st);
    if (e != hipSuccess) return hip_fail(e, "sweep launch");
  }
  if (dS0 && (e = la::launch_scale_first_gate(dS0, log_alpha, pl.nseq, pl.Ls, pl.D, st)) != hipSuccess)
    return hip_fail(e, "dS0 scale launch");

  // d l / d log(alpha_t) = sum_{u >= t} (q_u . dq_u - k_u . dk_u) + <dS_end, S_end>, the sum
  // anchored at every sub-segment boundary y by its exact value alpha_y <G_y, S_{y-1}>
  if (dlog_alpha && rq_from_walk) {
    e = la::launch_gate_grad_rows(RQ, dlog_alpha, W, W3, log_alpha, dS_end,
                                  need_send ? SE : nullptr, pl.nseq, pl.Ls, pl.D, st);
    if (e != hipSuccess) return hip_fail(e, "gate gradient launch");
  } else if (dlog_alpha) {
    e = la::launch_gate_anchors(W, W3, log_alpha, dS_end, need_send ? SE : nullptr, TOT, pl.nseq,
                                pl.Ls, pl.D, st);
    if (e != hipSuccess) return hip_fail(e, "gate anchor launch");
    e = la::launch_gate_grad(s->dtype, pl.D, Q, dQ, rk_from_walk ? nullptr : K,
                             rk_from_walk ? nullptr : dK, dlog_alpha, TOT, pl.nseq, pl.Ls, st);
    if (e != hipSuccess) return hip_fail(e, "gate gradient launch");
  }
  return LA_OK;
}

la_status la_chunk_bwd_gated(const la_shape* s, const void* Q, const void* K, const void* V,
                             const float* log_alpha, const float* S0, const void* dO,
                             const float* dS_end, void* dQ, void* dK, void* dV, float* dS0,
                             float* dlog_alpha, void* ws, size_t ws_bytes, void* stream) {
  return chunk_bwd_gated(s, Q, K, V, log_alpha, S0, dO, dS_end, nullptr, false, dQ, dK, dV, dS0,
                         dlog_alpha, ws, ws_bytes, stream);
}

la_status la_chunk_bwd_gated_from_fwd(const la_shape* s, const void* Q, const void* K,
                                      const void* V, const float* log_alpha, const float* S0,
                                      const void* dO, const float* dS_end, const void* fwd_ws,
                                      void* dQ, void* dK, void* dV, float* dS0,
                                      float* dlog_alpha, void* ws, size_t ws_bytes,
                                      void* stream) {
  return chunk_bwd_gated(s, Q, K, V, log_alpha, S0, dO, dS_end, static_cast<const float*>(fwd_ws),
                         true, dQ, dK, dV, dS0, dlog_alpha, ws, ws_bytes, stream);
}

size_t la_decay_grad_workspace_bytes(const la_shape* shape) {
  Plan pl;
  std::string keep = g_last_error;
  if (check_shape(shape, &pl, false) != LA_OK) {
    g_last_error = keep;
    return 0;
  }
  return tangent_ws(pl).total;
}

la_status la_decay_grad(const la_shape* s, const void* Q, const void* K, const void* V,
                        const float* lambda, const float* S0, const void* dO,
                        const float* dS_end, float* dlambda, void* ws, size_t ws_bytes,
                        void* stream) {
  Plan pl;
  la_status r = check_shape(s, &pl, false);
  if (r != LA_OK) return r;
  const bool has_tokens = pl.nseq > 0 && pl.Ls > 0;
  if (has_tokens && (!Q || !K || !V || !dO))
    return fail(LA_ERR_INVALID_ARG, "Q, K, V and dO are required");
  if (s->H > 0 && (!lambda || !dlambda))
    return fail(LA_ERR_INVALID_ARG, "lambda and dlambda are required");
  const void* ptrs[] = {Q, K, V, lambda, S0, dO, dS_end, dlambda, ws};
  for (const void* p : ptrs)
    if (p && !aligned16(p)) return fail(LA_ERR_INVALID_ARG, "pointer %p is not 16-byte aligned", p);
  const TangentWs L = tangent_ws(pl);
  if (L.total > 0 && (!ws || ws_bytes < L.total))
    return fail(LA_ERR_WORKSPACE, "workspace of %zu bytes needed, %zu given", L.total,
                ws ? ws_bytes : (size_t)0);
  if (s->H == 0) return LA_OK;
  char* base = static_cast<char*>(ws);
  la::TanArgs ta;
  std::memset(&ta, 0, sizeof(ta));
  ta.Q = Q;
  ta.K = K;
  ta.V = V;
  ta.dO = dO;
  ta.lam = lambda;
  ta.S0 = S0;
  ta.dSe = dS_end;
  ta.WS = reinterpret_cast<float*>(base + L.WS);
  ta.WT = reinterpret_cast<float*>(base + L.WT);
  ta.part = reinterpret_cast<double*>(base + L.part);
  ta.H = (int)s->H;
  ta.nseg = s->nseg;
  ta.split = pl.split;
  ta.Ls = pl.Ls;
  ta.Lp = pl.Lp;
  ta.pre_r = tangent_pre_r(pl);
  hipError_t e = la::launch_tangent(ta, s->dtype, pl.D, pl.nseq, dlambda,
                                    static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "decay gradient launch");
  return LA_OK;
}

// One decode step, with the per-head decay lambda or (gated, lambda null) the
// token's log-gate per sequence.
static la_status step(int64_t B, int64_t H, int32_t dk, int32_t dv, int32_t dtype, const void* q,
                      const void* k, const void* v, const float* lambda, const float* log_alpha,
                      const float* S, float* S_out, void* o, void* stream) {
  if (B < 0 || H < 0) return fail(LA_ERR_INVALID_ARG, "negative size (B=%lld H=%lld)",
                                  (long long)B, (long long)H);
  if (dk <= 0 || dv <= 0) return fail(LA_ERR_INVALID_ARG, "dk and dv must be positive");
  if (dtype != LA_BF16 && dtype != LA_FP32) return fail(LA_ERR_INVALID_ARG, "unknown dtype %d", dtype);
  if (dk != dv) return fail(LA_ERR_UNSUPPORTED, "dk != dv (%d, %d)", dk, dv);
  if (dk != 64 && dk != 128) return fail(LA_ERR_UNSUPPORTED, "d=%d not in {64, 128}", dk);
  // one workgroup of 256 per 32-column slab of every state
  if (!fits_grid((double)B * (double)H * (dk / 32) * 256.0))
    return fail(LA_ERR_UNSUPPORTED, "too many sequences for one launch");
  const int64_t nseq = B * H;
  if (nseq == 0) return LA_OK;
  if (!q || !k || !v || !S_out || (!lambda && !log_alpha))
    return fail(LA_ERR_INVALID_ARG, "q, k, v, %s and S_out are required",
                log_alpha || !lambda ? "log_alpha" : "lambda");
  const void* ptrs[] = {q, k, v, lambda, log_alpha, S, S_out, o};
  for (const void* p : ptrs)
    if (p && !aligned16(p)) return fail(LA_ERR_INVALID_ARG, "pointer %p is not 16-byte aligned", p);
  const size_t sbytes = (size_t)nseq * (size_t)dk * (size_t)dv * sizeof(float);
  if (S && S != S_out) {
    const char* a0 = reinterpret_cast<const char*>(S);
    const char* b0 = reinterpret_cast<const char*>(S_out);
    if (a0 < b0 + sbytes && b0 < a0 + sbytes)
      return fail(LA_ERR_INVALID_ARG, "S and S_out overlap without being the same buffer");
  }
  la::StepArgs sa;
  std::memset(&sa, 0, sizeof(sa));
  sa.q = q;
  sa.k = k;
  sa.v = v;
  sa.lam = lambda;
  sa.loga = log_alpha;
  sa.S = S;
  sa.Sout = S_out;
  sa.o = o;
  sa.H = (int)H;
  hipError_t e = la::launch_step(sa, dtype, dk, nseq, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "decode step launch");
  return LA_OK;
}

la_status la_step(int64_t B, int64_t H, int32_t dk, int32_t dv, int32_t dtype, const void* q,
                  const void* k, const void* v, const float* lambda, const float* S,
                  float* S_out, void* o, void* stream) {
  if (!lambda && B > 0 && H > 0) return fail(LA_ERR_INVALID_ARG, "lambda is required");
  return step(B, H, dk, dv, dtype, q, k, v, lambda, nullptr, S, S_out, o, stream);
}

la_status la_step_gated(int64_t B, int64_t H, int32_t dk, int32_t dv, int32_t dtype,
                        const void* q, const void* k, const void* v, const float* log_alpha,
                        const float* S, float* S_out, void* o, void* stream) {
  if (!log_alpha && B > 0 && H > 0) return fail(LA_ERR_INVALID_ARG, "log_alpha is required");
  return step(B, H, dk, dv, dtype, q, k, v, nullptr, log_alpha, S, S_out, o, stream);
}

la_status la_state_scan_gated(int64_t B, int64_t H, int32_t P, int32_t dk, int32_t dv,
                              const float* dS, const float* log_decay, const float* S0,
                              float* S_start, float* S_end, int32_t reverse, void* stream) {
  if (B < 0 || H < 0 || P < 0) return fail(LA_ERR_INVALID_ARG, "negative size");
  if (dk <= 0 || dv <= 0) return fail(LA_ERR_INVALID_ARG, "dk and dv must be positive");
  if ((double)B * H * ((double)P + 1) * dk * dv > 4.0e18)
    return fail(LA_ERR_INVALID_ARG, "tensor too large");
  if (!fits_grid((double)B * H * dk * dv + 256.0))
    return fail(LA_ERR_UNSUPPORTED, "too many state elements for one launch");
  const int64_t nseq = B * H;
  if (nseq > 0 && P > 0 && (!dS || !S_start || !log_decay))
    return fail(LA_ERR_INVALID_ARG, "dS, log_decay and S_start are required");
  const void* ptrs[] = {dS, log_decay, S0, S_start, S_end};
  for (const void* p : ptrs)
    if (p && !aligned16(p)) return fail(LA_ERR_INVALID_ARG, "pointer %p is not 16-byte aligned", p);
  if (nseq == 0 || (P == 0 && !S_end)) return LA_OK;
  la::ScanArgs sa;
  std::memset(&sa, 0, sizeof(sa));
  sa.nseq = nseq;
  sa.P = P;
  sa.E = (int64_t)dk * dv;
  sa.dS = dS;
  sa.lam = nullptr;
  sa.H = (int)H;
  sa.hdiv = 1;
  sa.seg_len = 0;
  sa.S0 = S0;
  sa.Sout = S_start;
  sa.Send = S_end;
  sa.reverse = reverse != 0;
  sa.inclusive = 0;
  sa.gated = 1;
  sa.LD = log_decay;  // with P == 0 the kernel only writes S_end = S0 (or zero)
  hipError_t e = la::launch_scan(sa, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "state scan launch");
  return LA_OK;
}

la_status la_state_scan(int64_t B, int64_t H, int32_t P, int32_t dk, int32_t dv, const float* dS,
                        const float* lambda, int64_t seg_len, const float* S0, float* S_start,
                        float* S_end, int32_t reverse, void* stream) {
  if (B < 0 || H < 0 || P < 0 || seg_len < 0)
    return fail(LA_ERR_INVALID_ARG, "negative size or length");
  if (dk <= 0 || dv <= 0) return fail(LA_ERR_INVALID_ARG, "dk and dv must be positive");
  if ((double)B * H * ((double)P + 1) * dk * dv > 4.0e18)
    return fail(LA_ERR_INVALID_ARG, "tensor too large");
  if (!fits_grid((double)B * H * dk * dv + 256.0))
    return fail(LA_ERR_UNSUPPORTED, "too many state elements for one launch");
  const int64_t nseq = B * H;
  if (nseq > 0 && !lambda) return fail(LA_ERR_INVALID_ARG, "lambda is required");
  if (nseq > 0 && P > 0 && (!dS || !S_start))
    return fail(LA_ERR_INVALID_ARG, "dS and S_start are required");
  const void* ptrs[] = {dS, lambda, S0, S_start, S_end};
  for (const void* p : ptrs)
    if (p && !aligned16(p)) return fail(LA_ERR_INVALID_ARG, "pointer %p is not 16-byte aligned", p);
  if (nseq == 0) return LA_OK;
  la::ScanArgs sa;
  std::memset(&sa, 0, sizeof(sa));
  sa.nseq = nseq;
  sa.P = P;
  sa.E = (int64_t)dk * dv;
  sa.dS = dS;
  sa.lam = lambda;
  sa.H = (int)H;
  sa.hdiv = 1;
  sa.seg_len = seg_len;
  sa.S0 = S0;
  sa.Sout = S_start;
  sa.Send = S_end;
  sa.reverse = reverse != 0;
  sa.inclusive = 0;
  if (P == 0 && !S_end) return LA_OK;  // nothing to write
  hipError_t e = la::launch_scan(sa, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "state scan launch");
  return LA_OK;
}

// The backward of la_chunk_bwd; with fwd_starts (the sub-segment start states
// S [nseq][split-1][D][D] a la_chunk_fwd call of the same shape left in its
// workspace) the dQ sweep takes their transposes instead of recomputing them.
static la_status chunk_bwd(const la_shape* s, const void* Q, const void* K, const void* V,
                           const float* lambda, const float* S0, const void* dO,
                           const float* dS_end, const float* fwd_starts, bool from_fwd, void* dQ,
                           void* dK, void* dV, float* dS0, void* ws, size_t ws_bytes,
                           void* stream) {
  Plan pl;
  la_status r = check_shape(s, &pl);
  if (r != LA_OK) return r;
  const bool has_tokens = pl.nseq > 0 && pl.Ls > 0;
  if (has_tokens && (!Q || !K || !V || !dO || !dQ || !dK || !dV))
    return fail(LA_ERR_INVALID_ARG, "Q, K, V, dO, dQ, dK and dV are required");
  if (pl.nseq > 0 && !lambda) return fail(LA_ERR_INVALID_ARG, "lambda is required");
  if (from_fwd && pl.nseq > 0 && pl.split > 1 && !fwd_starts)
    return fail(LA_ERR_INVALID_ARG, "fwd_ws is required (this shape splits sequences)");
  const void* ptrs[] = {Q, K, V, lambda, S0, dO, dS_end, dQ, dK, dV, dS0, ws, fwd_starts};
  for (const void* p : ptrs)
    if (p && !aligned16(p)) return fail(LA_ERR_INVALID_ARG, "pointer %p is not 16-byte aligned", p);
  const size_t need = bwd_ws_bytes(pl);
  if (need > 0 && (!ws || ws_bytes < need))
    return fail(LA_ERR_WORKSPACE, "workspace of %zu bytes needed, %zu given", need,
                ws ? ws_bytes : (size_t)0);
  if (pl.nseq == 0) return LA_OK;
  hipStream_t st = static_cast<hipStream_t>(stream);
  const size_t Wn = scan_ws_bytes(pl) / sizeof(float);
  float* W = static_cast<float*>(ws);  // sub-segment start states: dQ sweep
  float* Wv = W + Wn;                  // dV sweep (read transposed by the dK sweep)
  const int H = (int)s->H;
  la::PrepArgs pa;
  std::memset(&pa, 0, sizeof(pa));
  pa.nseq = pl.nseq;
  pa.D = pl.D;
  pa.lam = lambda;
  pa.H = H;
  pa.hdiv = s->nseg;
  hipError_t e;

  // dq_t = S_t dO_t: the forward recurrence of S^T = sum v k^T read by dO,
  // started from S0^T (S0 read transposed); its sub-segment start states
  // from a pre-pass and scan over (V, K), or the ones a forward call left,
  // read transposed.
  if (!(from_fwd && pl.split > 1)) {
    r = run_states(pl, s->dtype, H, s->nseg, V, K, lambda, S0, W, 0, st, false, nullptr, nullptr,
                   false, true);
    if (r != LA_OK) return r;
  }

  // dv_t = G_t^T k_t: in reverse time G accumulates q dO^T like a state.
  // Its seed dS_end = lambda G_{L+1} already carries the decay of the first
  // reverse step, so the sweeps and the scan take it undecayed (G_L = dS_end +
  // q_L dO_L^T; no division by lambda anywhere); its final value G_1 gives
  // dS0 = lambda G_1.  dk_t = G_t v_t: the same reverse recurrence for G^T =
  // sum dO q^T over the same pairs (q_t, dO_t) with the roles swapped, seeded
  // with the transposed seed, so its sub-segment start states are the
  // transposes of the dV sweep's: one set of local states and one scan serve
  // both (the dK sweep reads them, and dS_end, transposed).
  la::FwdArgs aq0 = main_args(pl, H, s->nseg, dO, V, K, lambda, S0, dQ, nullptr, W, 0, false,
                              nullptr);
  aq0.s0_transposed = 1;
  if (from_fwd) {
    aq0.Sws = fwd_starts;
    aq0.sws_transposed = 1;
  }
  if (s->dtype == LA_BF16) {
    // The reverse sweeps cut each sequence at the forward one's rows (the
    // short sub-segment first in reverse time), and the dQ sweep, which
    // streams dO anyway, forms their local states U = sum_t lambda^(t - t0)
    // q_t dO_t^T on its way (four tiles a stage: dO, V, K, Q); then the
    // reverse scan, and the dV and dK sweeps as one workgroup per item.
    Plan plr = pl;
    plr.ragged_first = true;
    if (pl.split > 1) {
      la::FwdArgs aq = aq0;
      aq.Q2 = Q;
      aq.Uout = Wv;
      if ((e = la::launch_fwd_u(aq, s->dtype, pl.D, pl.nseq * pl.split, st)) != hipSuccess)
        return hip_fail(e, "dQ sweep launch");
      la::ScanArgs sa;
      std::memset(&sa, 0, sizeof(sa));
      sa.nseq = pl.nseq;
      sa.P = pl.split - 1;
      sa.E = (int64_t)pl.D * pl.D;
      sa.dS = Wv;
      sa.lam = lambda;
      sa.H = H;
      sa.hdiv = s->nseg;
      sa.seg_len = pl.Lp;
      sa.first_len = pl.Ls - (int64_t)(pl.split - 1) * pl.Lp;
      sa.S0 = dS_end;
      sa.Sout = Wv;
      sa.inclusive = 1;
      sa.s0_undecayed = 1;
      if ((e = la::launch_scan(sa, st)) != hipSuccess) return hip_fail(e, "state scan launch");
    } else if ((e = la::launch_fwd(aq0, s->dtype, pl.D, true, pl.nseq, st)) != hipSuccess) {
      return hip_fail(e, "dQ sweep launch");
    }
    la::FwdArgs av = main_args(plr, H, s->nseg, K, Q, dO, lambda, dS_end, dV, dS0, Wv, 1, false,
                               nullptr);
    la::FwdArgs ak = main_args(plr, H, s->nseg, V, dO, Q, lambda, dS_end, dK, nullptr, Wv, 1,
                               false, nullptr);
    av.s0_undecayed = ak.s0_undecayed = 1;
    ak.s0_transposed = ak.sws_transposed = 1;
    if ((e = la::launch_fwd_duo(av, ak, s->dtype, pl.D, pl.nseq * pl.split, st)) != hipSuccess)
      return hip_fail(e, "dV/dK sweep launch");
  } else {
    // fp32: a pre-pass over (Q, dO) and the scan give the reverse start
    // states, then the three sweeps in one launch
    r = run_states(pl, s->dtype, H, s->nseg, Q, dO, lambda, dS_end, Wv, 1, st, false, nullptr,
                   nullptr, true);
    if (r != LA_OK) return r;
    la::FwdArgs av = main_args(pl, H, s->nseg, K, Q, dO, lambda, dS_end, dV, dS0, Wv, 1, false,
                               nullptr);
    la::FwdArgs ak = main_args(pl, H, s->nseg, V, dO, Q, lambda, dS_end, dK, nullptr, Wv, 1,
                               false, nullptr);
    av.s0_undecayed = ak.s0_undecayed = 1;
    ak.s0_transposed = ak.sws_transposed = 1;
    if ((e = launch_sweeps(aq0, av, ak, s->dtype, pl.D, pl.nseq * pl.split, st)) != hipSuccess)
      return hip_fail(e, "sweep launch");
  }
  // (with no tokens the sweep's final state is its seed, dS0 = dS_end: no factor)
  if (dS0 && pl.Ls > 0) {
    pa.src = dS0;
    pa.dst = dS0;
    pa.transpose = 0;
    pa.mode = 1;
    if ((e = la::launch_prep(pa, st)) != hipSuccess) return hip_fail(e, "prep launch");
  }
  return LA_OK;
}

la_status la_chunk_bwd(const la_shape* s, const void* Q, const void* K, const void* V,
                       const float* lambda, const float* S0, const void* dO, const float* dS_end,
                       void* dQ, void* dK, void* dV, float* dS0, void* ws, size_t ws_bytes,
                       void* stream) {
  return chunk_bwd(s, Q, K, V, lambda, S0, dO, dS_end, nullptr, false, dQ, dK, dV, dS0, ws,
                   ws_bytes, stream);
}

la_status la_chunk_bwd_from_fwd(const la_shape* s, const void* Q, const void* K, const void* V,
                                const float* lambda, const float* S0, const void* dO,
                                const float* dS_end, const void* fwd_ws, void* dQ, void* dK,
                                void* dV, float* dS0, void* ws, size_t ws_bytes, void* stream) {
  return chunk_bwd(s, Q, K, V, lambda, S0, dO, dS_end, static_cast<const float*>(fwd_ws), true,
                   dQ, dK, dV, dS0, ws, ws_bytes, stream);
}

}  // extern "C"
