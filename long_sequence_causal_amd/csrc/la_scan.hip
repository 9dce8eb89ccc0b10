// la_scan.hip -- segment state-combine scan and small state transforms.
//
// The scan is the combine X <- lambda^Ls X + dS[s] across segments that the
// All-Scan of ZeCO (abstract) and the all-gather of memory states of LASP-2
// (abstract) exist to deliver; on one GPU it runs over segments held in HBM.
// Each thread owns one state element of one sequence and walks the P
// segments in order; consecutive threads own consecutive elements, so every
// step is one coalesced read (and write) across the wave.  It is purely
// HBM-bound: 4 B read + 4 B written per element and segment.
#include "la_device.h"
#include "la_internal.h"

namespace la {

template <bool GATED>
__global__ __launch_bounds__(256) void k_state_scan(ScanArgs a) {
  const int64_t gid = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (gid >= a.nseq * a.E) return;
  const int64_t n = gid / a.E;
  const int64_t e = gid - n * a.E;
  // lambda^seg_len = 2^(seg_len log2 lambda); underflow to 0 is intended
  const float lg = GATED ? 0.0f : log2f(a.lam[(int)((n / a.hdiv) % a.H)]);
  const float dec = GATED ? 0.0f : pow_lam(lg, (float)a.seg_len);
  // decay of the first segment (first_len tokens when it is the short
  // one): a seed that already carries the first token's decay takes one
  // power fewer
  const int64_t len0 = a.first_len > 0 ? a.first_len : a.seg_len;
  float dcur = GATED ? 0.0f
                     : pow_lam(lg, (float)((a.s0_undecayed && len0 > 0) ? len0 - 1 : len0));
  const int64_t e0 = a.s0_transposed ? (e % a.d) * a.d + e / a.d : e;
  float x = a.S0 ? a.S0[n * a.E + e0] : 0.0f;
  // Segments go in groups of PF whose inputs are all loaded before any of
  // the group's outputs is stored: Sout may be dS itself, so the compiler
  // cannot move a load above an earlier store, and one segment per memory
  // round trip would make a long scan latency-bound.  Each output element is
  // written only after its own input was read, so in place stays correct.
  constexpr int PF = 16;
  auto seg = [&](int it) { return a.reverse ? (a.P - 1 - it) : it; };
  for (int it = 0; it < a.P; it += PF) {
    // (the last group may be partial: the same count for every thread)
    const int cnt = (a.P - it < PF) ? a.P - it : PF;
    float d[PF], f[PF];
#pragma unroll
    for (int j = 0; j < PF; ++j) {
      d[j] = 0.0f;
      f[j] = 0.0f;
      if (j < cnt) {
        const int s = seg(it + j);
        d[j] = a.dS[(n * a.P + s) * a.E + e];
        if (GATED) f[j] = a.LD[n * a.P + s];
      }
    }
#pragma unroll
    for (int j = 0; j < PF; ++j) {
      if (j < cnt) {
        const int64_t idx = (n * a.P + seg(it + j)) * a.E + e;
        if (!a.inclusive) a.Sout[idx] = x;
        // gated: the segment's own product of gates, exp(LD)
        x = (GATED ? expf(f[j]) : dcur) * x + d[j];
        dcur = dec;
        if (a.inclusive) a.Sout[idx] = x;
      }
    }
  }
  if (a.Send) a.Send[n * a.E + e] = x;
}

__global__ __launch_bounds__(256) void k_prep_state(PrepArgs a) {
  const int64_t DD = (int64_t)a.D * a.D;
  const int64_t gid = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (gid >= a.nseq * DD) return;
  const int64_t n = gid / DD;
  const int64_t e = gid - n * DD;
  const int r = (int)(e / a.D), c = (int)(e % a.D);
  const int64_t se = a.transpose ? ((int64_t)c * a.D + r) : e;
  float x = a.src[n * DD + se];
  if (a.mode == 1) x *= a.lam[(n / a.hdiv) % a.H];
  a.dst[gid] = x;
}

// dst[m] = src[m]^T for nmat D x D matrices (D a multiple of 32), in
// 32 x 32 tiles through LDS so that every global read and write is a
// coalesced row segment: workgroup (m, bi, bj) reads tile (bi, bj) of src[m]
// and writes it transposed as tile (bj, bi) of dst[m].  src and dst must not
// overlap.
__global__ __launch_bounds__(256) void k_transpose_copy(const float* src, float* dst, int D) {
  __shared__ float t[32][33];
  const int nt = D / 32;
  const int64_t m = blockIdx.x / (nt * nt);
  const int bi = (int)(blockIdx.x % (nt * nt)) / nt, bj = (int)(blockIdx.x % nt);
  const int64_t DD = (int64_t)D * D;
  const float* sm = src + m * DD;
  float* dm = dst + m * DD;
  const int c = threadIdx.x & 31, r0 = threadIdx.x >> 5;  // 8 rows per pass
#pragma unroll
  for (int r = r0; r < 32; r += 8) t[r][c] = sm[(int64_t)(32 * bi + r) * D + 32 * bj + c];
  __syncthreads();
#pragma unroll
  for (int r = r0; r < 32; r += 8) dm[(int64_t)(32 * bj + r) * D + 32 * bi + c] = t[c][r];
}

hipError_t launch_transpose_copy(const float* src, float* dst, int64_t nmat, int D, hipStream_t s) {
  const int nt = D / 32;
  if (nmat <= 0) return hipSuccess;
  if (D % 32 != 0) return hipErrorInvalidValue;
  hipLaunchKernelGGL(k_transpose_copy, dim3((unsigned)(nmat * nt * nt)), dim3(256), 0, s, src, dst,
                     D);
  return hipGetLastError();
}

hipError_t launch_scan(const ScanArgs& a, hipStream_t s) {
  const int64_t tot = a.nseq * a.E;
  if (tot <= 0) return hipSuccess;
  if (a.gated)
    hipLaunchKernelGGL(k_state_scan<true>, dim3((unsigned)((tot + 255) / 256)), dim3(256), 0, s, a);
  else
    hipLaunchKernelGGL(k_state_scan<false>, dim3((unsigned)((tot + 255) / 256)), dim3(256), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_prep(const PrepArgs& a, hipStream_t s) {
  const int64_t tot = a.nseq * (int64_t)a.D * a.D;
  if (tot <= 0) return hipSuccess;
  hipLaunchKernelGGL(k_prep_state, dim3((unsigned)((tot + 255) / 256)), dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace la
