// la_fwd.hip -- chunkwise forward kernel of decayed causal linear attention.
//
// One workgroup (d/16 waves) per (sequence, sub-segment) walks the
// sub-segment's 64-token chunks in order from its start state (S0, a scanned
// state or zero), carrying the fp32 state in MFMA accumulators (la_walk.h),
// and writes the state it ends with when asked.  With O the chunks also give
// the outputs; without O (state-only) only K and V are read.
#include "la_internal.h"
#include "la_walk.h"

namespace la {

// Slot in a.Sws of the start state of sub-segment p >= 1: the finer
// partition's sub-segment that starts on the same row (counted from the
// sequence's start, or from its end when the short sub-segment comes first).
__device__ inline int64_t sws_slot(const FwdArgs& a, int p) {
  return a.ragged_first ? a.sws_nper - (int64_t)(a.split - p) * a.sws_step
                        : (int64_t)p * a.sws_step - 1;
}

// Work item `wg` of a launch over a0: sub-segment p_begin + wg % p_count of
// sequence wg / p_count.  NH = 2: the same item of a1 as well, walked by
// the same waves beside it (a1 has a0's plan, positions and decay, and a0's
// values and keys as its keys and values).
template <typename T, int D, bool WITH_O, bool GATED, int NH = 1, bool ACCU = false, bool RK = false,
          bool DUMP = false>
__device__ __forceinline__ void chunk_item(const FwdArgs& a0, const FwdArgs& a1, int64_t wg) {
  constexpr int NSLOT = (NH == 2 || ACCU) ? 4 : (WITH_O ? 3 : 2);
  typedef FwdLayout<T, D, NSLOT, GATED, NH> LY;
  constexpr int NKT = D / 16;
  __shared__ __attribute__((aligned(1024))) char smem[LY::BYTES];

  const int lane = threadIdx.x & 63;
  const int l16 = lane & 15;
  const int g = lane >> 4;
  const int col = 16 * __builtin_amdgcn_readfirstlane((int)threadIdx.x >> 6);

  // ---- work item: sub-segment p of sequence n
  const FwdArgs& a = a0;  // the plan (shared by a1)
  const int64_t n = wg / a.p_count;
  const int p = a.p_begin + (int)(wg % a.p_count);
  const int h = (int)((n / a.nseg) % a.H);
  int64_t t0, t1;  // positions of the sub-segment (the short one last, or first)
  if (a.ragged_first) {
    t1 = a.Ls - (int64_t)(a.split - 1 - p) * a.Lp;
    t0 = (t1 - a.Lp > 0) ? t1 - a.Lp : 0;
  } else {
    t0 = (int64_t)p * a.Lp;
    t1 = (t0 + a.Lp < a.Ls) ? t0 + a.Lp : a.Ls;
  }
  const int64_t seq_elem0 = n * a.Ls * D;
  WalkJob jb[NH];
  f32x4 accS[NH][NKT];
#pragma unroll
  for (int u = 0; u < NH; ++u) {
    const FwdArgs& x = u ? a1 : a0;
    jb[u].Q = WITH_O ? (const void*)(reinterpret_cast<const T*>(x.Q) + seq_elem0) : nullptr;
    jb[u].K = reinterpret_cast<const T*>(x.K) + seq_elem0;
    jb[u].V = reinterpret_cast<const T*>(x.V) + seq_elem0;
    jb[u].O = WITH_O ? (void*)(reinterpret_cast<T*>(x.O) + seq_elem0) : nullptr;
    jb[u].t0 = t0;
    jb[u].len = (int)((t1 > t0) ? t1 - t0 : 0);
    jb[u].Ls = a.Ls;
    jb[u].reverse = a.reverse;
    jb[u].lg = GATED ? 0.0f : log2f(a.lam[h]);
    jb[u].G = GATED ? a.G + n * a.Ls : nullptr;
    jb[u].last_chunk_first = a.last_chunk_first;
    jb[u].first_undecayed = !GATED && x.s0_undecayed && x.start_from_state && p == 0;
    jb[u].rk = (RK && u == NH - 1) ? x.rk + n * a.Ls : nullptr;
    jb[u].dump = nullptr;
    if (DUMP && WITH_O && x.dump) {
      jb[u].dump_shift = __builtin_ctz((unsigned)x.dump_rows);  // a power of two (host-checked)
      jb[u].ndump = (int)((a.Ls + x.dump_rows - 1) / x.dump_rows - 1);
      jb[u].dump_rev = x.dump_rev;
      jb[u].dump = x.dump + n * (int64_t)jb[u].ndump * D * D;
    }

    // ---- start state -> accumulators (wave w: columns [16 w, 16 w + 16))
    const float* sp = nullptr;
    bool tr = false;  // stored transposed (wave-uniform)
    if (x.start_from_state) {
      if (p == 0) {
        sp = x.S0 ? x.S0 + n * D * D : nullptr;
        tr = x.s0_transposed;
      } else {
        sp = x.Sws + (n * x.sws_nper + sws_slot(x, p)) * (int64_t)D * D;
        tr = x.sws_transposed;
      }
    }
    if (sp && tr) {
      // element (row 16 tk + 4 g + r, column col + l16) at [col + l16][row]:
      // 16 bytes of one stored row per tile
#pragma unroll
      for (int tk = 0; tk < NKT; ++tk) {
        const f32x4 t4 = *reinterpret_cast<const f32x4*>(sp + (col + l16) * D + 16 * tk + 4 * g);
#pragma unroll
        for (int r = 0; r < 4; ++r) accS[u][tk][r] = t4[r];
      }
    } else {
#pragma unroll
      for (int tk = 0; tk < NKT; ++tk)
#pragma unroll
        for (int r = 0; r < 4; ++r)
          accS[u][tk][r] = sp ? sp[(16 * tk + 4 * g + r) * D + col + l16] : 0.0f;
    }
  }
  f32x4 accU[NKT];
  if constexpr (ACCU) {
    jb[0].Q2 = reinterpret_cast<const T*>(a.Q2) + seq_elem0;
#pragma unroll
    for (int tk = 0; tk < NKT; ++tk) accU[tk] = f32x4{0.f, 0.f, 0.f, 0.f};
  }
  if constexpr (NH == 2) {
    jb[0].src4[0] = jb[0].Q;
    jb[0].src4[1] = jb[1].Q;
    jb[0].src4[2] = jb[0].K;
    jb[0].src4[3] = jb[0].V;
  }
  // Retire the start-state loads here, visibly to the compiler (vmcnt(0)
  // only): otherwise it waits for them at their first use inside the chunk
  // loop, i.e. on every chunk, which would also drain the chunk prefetches.
  __builtin_amdgcn_s_waitcnt(0x0F70);

  const float lgate = walk<T, D, WITH_O, NSLOT, GATED, NH, RK, DUMP>(smem, jb, accS, accU);
  if constexpr (ACCU) {
    if (p >= 1) {
      const int64_t slot = n * (a.split - 1) + (a.split - 1 - p);
      float* dst = a.Uout + slot * (int64_t)D * D;
#pragma unroll
      for (int tk = 0; tk < NKT; ++tk)
#pragma unroll
        for (int r = 0; r < 4; ++r) dst[(16 * tk + 4 * g + r) * D + col + l16] = accU[tk][r];
      // gated: the sub-segment's total log-gate as the reverse sweep steps
      // through it (token t takes g_{t+1}; the sequence's last token 0)
      if (GATED && threadIdx.x == 0) {
        const float* gs = a.G + n * a.Ls;
        a.LDrev[slot] = lgate - gs[t0] + (t1 < a.Ls ? gs[t1] : 0.0f);
      }
    }
  }

  // ---- final state of this sub-segment (and its total log-gate)
#pragma unroll
  for (int u = 0; u < NH; ++u) {
    const FwdArgs& x = u ? a1 : a0;
    if (x.Sout && p >= x.sout_p0 && p < x.sout_p0 + x.sout_np) {
      if (GATED && x.LDout && threadIdx.x == 0) x.LDout[n * x.sout_np + (p - x.sout_p0)] = lgate;
      float* dst = x.Sout + (n * x.sout_np + (p - x.sout_p0)) * (int64_t)D * D;
#pragma unroll
      for (int tk = 0; tk < NKT; ++tk)
#pragma unroll
        for (int r = 0; r < 4; ++r) dst[(16 * tk + 4 * g + r) * D + col + l16] = accS[u][tk][r];
    }
  }
}

template <typename T, int D, bool WITH_O, bool GATED>
__global__ __launch_bounds__((FwdLayout<T, D, WITH_O ? 3 : 2, GATED>::NT),
                             (FwdLayout<T, D, WITH_O ? 3 : 2, GATED>::WAVES_PER_EU)) void k_chunk_fwd(
    FwdArgs a) {
  chunk_item<T, D, WITH_O, GATED>(a, a, blockIdx.x);
}

// Two launches over the same number of work items in one grid, interleaved
// in blocks of 8 workgroups: blocks 16 j + r and 16 j + 8 + r (r < 8) run
// item 8 j + r of a and of b.  Workgroups are dealt to the 8 XCDs round-robin
// by index, so the two partners share an XCD and its L2, and when a and b
// walk the same rows (the backward's dV and dK sweeps, which both read Q and
// dO) one partner's loads mostly find the other's lines there.
template <typename T, int D, bool GATED>
__global__ __launch_bounds__((FwdLayout<T, D, 3, GATED>::NT),
                             (FwdLayout<T, D, 3, GATED>::WAVES_PER_EU)) void k_chunk_fwd_pair(
    FwdArgs a, FwdArgs b, int64_t nitems) {
  const int64_t blk = blockIdx.x;
  const int64_t item = 8 * (blk / 16) + (blk % 8);
  if (item >= nitems) return;
  if ((blk & 8) == 0)
    chunk_item<T, D, true, GATED>(a, a, item);
  else
    chunk_item<T, D, true, GATED>(b, b, item);
}

// Three launches with outputs over nitems work items each as one grid, in
// groups of 24 workgroups: blocks 24 j + r run item 8 j + r of a (r < 8), of
// b (8 <= r < 16) and of c (r >= 16), so b's and c's items keep the pair
// kernel's XCD sharing (blocks 8 apart) while a's walks run beside them.  The
// backward uses it for its dQ sweep (a) and the dV and dK sweeps (b, c): the
// paired sweeps are bound by the latency of their walks rather than by HBM,
// the dQ sweep by HBM, so side by side they share the chip's time better than
// one after the other.
template <typename T, int D, bool GATED>
__global__ __launch_bounds__((FwdLayout<T, D, 3, GATED>::NT),
                             (FwdLayout<T, D, 3, GATED>::WAVES_PER_EU)) void k_chunk_fwd_triple(
    FwdArgs a, FwdArgs b, FwdArgs c, int64_t nitems) {
  const int64_t blk = blockIdx.x;
  const int r = (int)(blk % 24);
  const int64_t item = 8 * (blk / 24) + (r % 8);
  if (item >= nitems) return;
  // (the gated backward asks its dQ and dK walks for their 1024-row states)
  if (r < 8)
    chunk_item<T, D, true, GATED, 1, false, false, GATED>(a, a, item);
  else if (r < 16)
    chunk_item<T, D, true, GATED, 1, false, false, GATED>(b, b, item);
  else
    chunk_item<T, D, true, GATED, 1, false, false, GATED>(c, c, item);
}

// A dump's row count must be a power of two of at least one chunk (the
// walks test boundary rows with a mask and a shift).
static bool bad_dump(const FwdArgs& a) {
  return a.dump && (a.dump_rows < 64 || (a.dump_rows & (a.dump_rows - 1)) != 0);
}

template <typename T, int D>
static hipError_t launch_triple_t(const FwdArgs& a, const FwdArgs& b, const FwdArgs& c,
                                  int64_t nitems, hipStream_t s) {
  const unsigned grid = (unsigned)(24 * ((nitems + 7) / 8));
  if (a.gated)
    hipLaunchKernelGGL((k_chunk_fwd_triple<T, D, true>), dim3(grid),
                       dim3(FwdLayout<T, D, 3, true>::NT), 0, s, a, b, c, nitems);
  else
    hipLaunchKernelGGL((k_chunk_fwd_triple<T, D, false>), dim3(grid),
                       dim3(FwdLayout<T, D, 3, false>::NT), 0, s, a, b, c, nitems);
  return hipGetLastError();
}

hipError_t launch_fwd_triple(const FwdArgs& a, const FwdArgs& b, const FwdArgs& c, int dtype,
                             int D, int64_t nitems, hipStream_t s) {
  if (nitems <= 0) return hipSuccess;
  if (a.gated != b.gated || a.gated != c.gated) return hipErrorInvalidValue;
  if (bad_dump(a) || bad_dump(b) || bad_dump(c)) return hipErrorInvalidValue;
  if (dtype == 0) {
    if (D == 64) return launch_triple_t<__bf16, 64>(a, b, c, nitems, s);
    if (D == 128) return launch_triple_t<__bf16, 128>(a, b, c, nitems, s);
  } else {
    if (D == 64) return launch_triple_t<float, 64>(a, b, c, nitems, s);
    if (D == 128) return launch_triple_t<float, 128>(a, b, c, nitems, s);
  }
  return hipErrorInvalidValue;
}

// Two launches with outputs over the same work items whose recurrences have
// crosswise keys and values (b.K = a.V, b.V = a.K: the backward's dV and dK
// sweeps, both over q dO^T) as one workgroup per item, every wave walking
// its columns of both: one stream of four tiles per chunk feeds both.
template <typename T, int D, bool GATED, bool RK>
__global__ __launch_bounds__((FwdLayout<T, D, 4, GATED, 2>::NT),
                             (FwdLayout<T, D, 4, GATED, 2>::WAVES_PER_EU)) void k_chunk_fwd_duo(
    FwdArgs a, FwdArgs b) {
  chunk_item<T, D, true, GATED, 2, false, RK, GATED>(a, b, blockIdx.x);
}

template <typename T, int D>
static hipError_t launch_duo_t(const FwdArgs& a, const FwdArgs& b, int64_t nitems, hipStream_t s) {
  if (a.gated) {
    if (!b.rk)
      hipLaunchKernelGGL((k_chunk_fwd_duo<T, D, true, false>), dim3((unsigned)nitems),
                         dim3(FwdLayout<T, D, 4, true, 2>::NT), 0, s, a, b);
    else if constexpr (D == 128)
      hipLaunchKernelGGL((k_chunk_fwd_duo<T, D, true, true>), dim3((unsigned)nitems),
                         dim3(FwdLayout<T, D, 4, true, 2>::NT), 0, s, a, b);
    else
      return hipErrorInvalidValue;  // row dots: d = 128
  } else {
    if (b.rk) return hipErrorInvalidValue;  // (only the gated backward asks for the row dots)
    hipLaunchKernelGGL((k_chunk_fwd_duo<T, D, false, false>), dim3((unsigned)nitems),
                       dim3(FwdLayout<T, D, 4, false, 2>::NT), 0, s, a, b);
  }
  return hipGetLastError();
}

hipError_t launch_fwd_duo(const FwdArgs& a, const FwdArgs& b, int dtype, int D, int64_t nitems,
                          hipStream_t s) {
  if (nitems <= 0) return hipSuccess;
  // one plan and decay, crosswise keys and values
  if (a.gated != b.gated || a.G != b.G || a.K != b.V || a.V != b.K || a.lam != b.lam ||
      a.H != b.H || a.nseg != b.nseg || a.Ls != b.Ls || a.Lp != b.Lp || a.split != b.split ||
      a.p_begin != b.p_begin || a.p_count != b.p_count || a.reverse != b.reverse ||
      a.ragged_first != b.ragged_first || a.last_chunk_first != b.last_chunk_first)
    return hipErrorInvalidValue;
  if (dtype != 0) return hipErrorInvalidValue;  // bf16 only
  if (a.rk || (b.rk && D != 128)) return hipErrorInvalidValue;  // row dots: b, d = 128
  if (bad_dump(a) || bad_dump(b)) return hipErrorInvalidValue;
  if (D == 64) return launch_duo_t<__bf16, 64>(a, b, nitems, s);
  if (D == 128) return launch_duo_t<__bf16, 128>(a, b, nitems, s);
  return hipErrorInvalidValue;
}

// The gated chunk kernel with outputs that also writes the state at the
// boundary rows a.dump asks for (the gated backward's dQ sweep).
template <typename T, int D>
__global__ __launch_bounds__((FwdLayout<T, D, 3, true>::NT),
                             (FwdLayout<T, D, 3, true>::WAVES_PER_EU)) void k_chunk_fwd_dump(FwdArgs a) {
  chunk_item<T, D, true, true, 1, false, false, true>(a, a, blockIdx.x);
}

// The chunk kernel with outputs whose walks also form each sub-segment's U
// (four tiles a stage: Q, K, V and Q2).  Gated: also the sub-segments'
// reverse log-gates (LDrev), the states at a.dump's rows, and with RK the
// row dots of the outputs with Q2 (a.rk).
template <typename T, int D, bool GATED, bool RK>
__global__ __launch_bounds__((FwdLayout<T, D, 4, GATED>::NT),
                             (FwdLayout<T, D, 4, GATED>::WAVES_PER_EU)) void k_chunk_fwd_u(FwdArgs a) {
  chunk_item<T, D, true, GATED, 1, true, RK, GATED>(a, a, blockIdx.x);
}

template <int D>
static hipError_t launch_u_t(const FwdArgs& a, int64_t nitems, hipStream_t s) {
  typedef __bf16 T;
  const dim3 grid((unsigned)nitems);
  if (!a.gated)
    hipLaunchKernelGGL((k_chunk_fwd_u<T, D, false, false>), grid,
                       dim3(FwdLayout<T, D, 4, false>::NT), 0, s, a);
  else if (!a.rk)
    hipLaunchKernelGGL((k_chunk_fwd_u<T, D, true, false>), grid,
                       dim3(FwdLayout<T, D, 4, true>::NT), 0, s, a);
  else if constexpr (D == 128)
    hipLaunchKernelGGL((k_chunk_fwd_u<T, D, true, true>), grid,
                       dim3(FwdLayout<T, D, 4, true>::NT), 0, s, a);
  else
    return hipErrorInvalidValue;  // row dots: d = 128
  return hipGetLastError();
}

hipError_t launch_fwd_u(const FwdArgs& a, int dtype, int D, int64_t nitems, hipStream_t s) {
  if (nitems <= 0) return hipSuccess;
  if (!a.Q2 || !a.Uout || !a.O || (a.gated && (!a.G || !a.LDrev)) || (a.rk && !a.gated))
    return hipErrorInvalidValue;
  if (dtype != 0 || bad_dump(a)) return hipErrorInvalidValue;  // bf16 only
  if (D == 64) return launch_u_t<64>(a, nitems, s);
  if (D == 128) return launch_u_t<128>(a, nitems, s);
  return hipErrorInvalidValue;
}

template <typename T, int D, bool GATED>
static hipError_t launch_fwd_t(const FwdArgs& a, bool with_o, int64_t nwg, hipStream_t s) {
  if (a.dump) {
    if (!GATED || !with_o || bad_dump(a)) return hipErrorInvalidValue;  // (gated dQ sweep only)
    hipLaunchKernelGGL((k_chunk_fwd_dump<T, D>), dim3((unsigned)nwg),
                       dim3(FwdLayout<T, D, 3, true>::NT), 0, s, a);
  } else if (with_o)
    hipLaunchKernelGGL((k_chunk_fwd<T, D, true, GATED>), dim3((unsigned)nwg),
                       dim3(FwdLayout<T, D, 3, GATED>::NT), 0, s, a);
  else
    hipLaunchKernelGGL((k_chunk_fwd<T, D, false, GATED>), dim3((unsigned)nwg),
                       dim3(FwdLayout<T, D, 2, GATED>::NT), 0, s, a);
  return hipGetLastError();
}

template <typename T, int D>
static hipError_t launch_fwd_g(const FwdArgs& a, bool with_o, int64_t nwg, hipStream_t s) {
  return a.gated ? launch_fwd_t<T, D, true>(a, with_o, nwg, s)
                 : launch_fwd_t<T, D, false>(a, with_o, nwg, s);
}

template <typename T, int D>
static hipError_t launch_pair_t(const FwdArgs& a, const FwdArgs& b, int64_t nitems, hipStream_t s) {
  const unsigned grid = (unsigned)(16 * ((nitems + 7) / 8));
  if (a.gated)
    hipLaunchKernelGGL((k_chunk_fwd_pair<T, D, true>), dim3(grid), dim3(FwdLayout<T, D, 3, true>::NT),
                       0, s, a, b, nitems);
  else
    hipLaunchKernelGGL((k_chunk_fwd_pair<T, D, false>), dim3(grid),
                       dim3(FwdLayout<T, D, 3, false>::NT), 0, s, a, b, nitems);
  return hipGetLastError();
}

hipError_t launch_fwd_pair(const FwdArgs& a, const FwdArgs& b, int dtype, int D, int64_t nitems,
                           hipStream_t s) {
  if (nitems <= 0) return hipSuccess;
  if (a.gated != b.gated) return hipErrorInvalidValue;
  if (dtype == 0) {
    if (D == 64) return launch_pair_t<__bf16, 64>(a, b, nitems, s);
    if (D == 128) return launch_pair_t<__bf16, 128>(a, b, nitems, s);
  } else {
    if (D == 64) return launch_pair_t<float, 64>(a, b, nitems, s);
    if (D == 128) return launch_pair_t<float, 128>(a, b, nitems, s);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_fwd(const FwdArgs& a, int dtype, int D, bool with_o, int64_t nwg,
                      hipStream_t s) {
  if (nwg <= 0) return hipSuccess;
  if (dtype == 0) {
    if (D == 64) return launch_fwd_g<__bf16, 64>(a, with_o, nwg, s);
    if (D == 128) return launch_fwd_g<__bf16, 128>(a, with_o, nwg, s);
  } else {
    if (D == 64) return launch_fwd_g<float, 64>(a, with_o, nwg, s);
    if (D == 128) return launch_fwd_g<float, 128>(a, with_o, nwg, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace la
