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

__global__ __launch_bounds__(256) void k_state_scan(ScanArgs a) {
  const int64_t gid = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (gid >= a.nseq * a.E) return;
  const int64_t n = gid / a.E;
  const int64_t e = gid - n * a.E;
  const int h = (int)((n / a.hdiv) % a.H);
  // lambda^seg_len = 2^(seg_len log2 lambda); underflow to 0 is intended
  const float dec = exp2f((float)a.seg_len * log2f(a.lam[h]));
  float x = a.S0 ? a.S0[n * a.E + e] : 0.0f;
  for (int it = 0; it < a.P; ++it) {
    const int s = a.reverse ? (a.P - 1 - it) : it;
    const int64_t idx = (n * a.P + s) * a.E + e;
    const float d = a.dS[idx];
    if (!a.inclusive) a.Sout[idx] = x;
    x = dec * x + d;
    if (a.inclusive) a.Sout[idx] = x;
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
  if (a.mode != 0) {
    const float l = a.lam[(n / a.hdiv) % a.H];
    x = (a.mode == 1) ? x * l : x / l;
  }
  a.dst[gid] = x;
}

// One thread per element (i, j) with i < j of a matrix swaps it with (j, i).
__global__ __launch_bounds__(256) void k_transpose_inplace(float* W, int64_t nmat, int D) {
  const int64_t DD = (int64_t)D * D;
  const int64_t gid = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (gid >= nmat * DD) return;
  const int64_t m = gid / DD;
  const int64_t e = gid - m * DD;
  const int i = (int)(e / D), j = (int)(e % D);
  if (i >= j) return;
  float* M = W + m * DD;
  const float x = M[(int64_t)i * D + j];
  M[(int64_t)i * D + j] = M[(int64_t)j * D + i];
  M[(int64_t)j * D + i] = x;
}

hipError_t launch_transpose(float* W, int64_t nmat, int D, hipStream_t s) {
  const int64_t tot = nmat * (int64_t)D * D;
  if (tot <= 0) return hipSuccess;
  hipLaunchKernelGGL(k_transpose_inplace, dim3((unsigned)((tot + 255) / 256)), dim3(256), 0, s, W,
                     nmat, D);
  return hipGetLastError();
}

hipError_t launch_scan(const ScanArgs& a, hipStream_t s) {
  const int64_t tot = a.nseq * a.E;
  if (tot <= 0) return hipSuccess;
  hipLaunchKernelGGL(k_state_scan, dim3((unsigned)((tot + 255) / 256)), dim3(256), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_prep(const PrepArgs& a, hipStream_t s) {
  const int64_t tot = a.nseq * (int64_t)a.D * a.D;
  if (tot <= 0) return hipSuccess;
  hipLaunchKernelGGL(k_prep_state, dim3((unsigned)((tot + 255) / 256)), dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace la
