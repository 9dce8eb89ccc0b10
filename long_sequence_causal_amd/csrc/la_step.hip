// la_step.hip -- one recurrent decode step for a batch of sequences:
//   S' = lambda_h S + k v^T,   o = q^T S'
// for every (b, h): the token recurrence itself, the constant-memory
// inference form named in the LASP-2 page's abstract; gated, the decay is
// the token's own gate alpha = exp(log alpha) of the sequence (the per-token
// gates of the Gated Linear Attention entry of that page's related-paper
// list).  The work is a
// rank-one update of the fp32 state and a matrix-vector product: a few
// flops per state element, so the step is bound by HBM, reading the state
// once and writing it once.
//
// One workgroup per (head, slab of 32 state columns): lane (row group rr,
// column quad c4) holds rows rr, rr + 32, .. of columns v0 + c4 .. + 3 (16
// bytes, so eight lanes cover a row's 128-byte slab piece).  All of a lane's
// state loads are issued before any arithmetic; o is summed over rows per
// lane, then over the 32 row groups through LDS in a fixed order.
#include "la_internal.h"
#include "la_device.h"

namespace la {

namespace {

constexpr int VB = 32;  // state columns per workgroup

template <typename T>
__device__ inline float ld(const T* p) {
  return Elt<T>::to_f(*p);
}

template <typename T, int D>
__global__ __launch_bounds__(256) void k_step(StepArgs a) {
  constexpr int NSLAB = D / VB;
  constexpr int NP = D / 32;  // rows per lane
  __shared__ float red[32][VB + 1];
  const int tid = threadIdx.x;
  const int64_t n = (int64_t)blockIdx.x / NSLAB;  // sequence (b, h)
  const int v0 = (int)(blockIdx.x % NSLAB) * VB;
  const int h = (int)(n % a.H);
  const int rr = tid >> 3;
  const int c4 = (tid & 7) * 4;
  const int64_t DD = (int64_t)D * D;
  // gated: alpha = 2^(log alpha * log2 e), as the chunk walks form their
  // gate factors
  const float lam = a.loga ? exp2f(a.loga[n] * 1.4426950408889634f) : a.lam[h];

  const float* S = a.S ? a.S + n * DD : nullptr;
  float* So = a.Sout + n * DD;
  const T* q = reinterpret_cast<const T*>(a.q) + n * D;
  const T* k = reinterpret_cast<const T*>(a.k) + n * D;
  const T* v = reinterpret_cast<const T*>(a.v) + n * D + v0 + c4;

  f32x4 s[NP];
#pragma unroll
  for (int p = 0; p < NP; ++p) {
    const int r = 32 * p + rr;
    s[p] = S ? *reinterpret_cast<const f32x4*>(S + r * D + v0 + c4) : f32x4{0.f, 0.f, 0.f, 0.f};
  }
  f32x4 vv;
#pragma unroll
  for (int j = 0; j < 4; ++j) vv[j] = ld(v + j);
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int p = 0; p < NP; ++p) {
    const int r = 32 * p + rr;
    const float kr = ld(k + r);
    const f32x4 s1 = lam * s[p] + kr * vv;
    *reinterpret_cast<f32x4*>(So + r * D + v0 + c4) = s1;
    acc += ld(q + r) * s1;
  }
  if (!a.o) return;
#pragma unroll
  for (int j = 0; j < 4; ++j) red[rr][c4 + j] = acc[j];
  __syncthreads();
  if (tid < VB) {
    float o = 0.0f;
#pragma unroll 8
    for (int i = 0; i < 32; ++i) o += red[i][tid];
    reinterpret_cast<T*>(a.o)[n * D + v0 + tid] = Elt<T>::from_f(o);
  }
}

template <typename T, int D>
hipError_t step_t(const StepArgs& a, int64_t nseq, hipStream_t s) {
  hipLaunchKernelGGL((k_step<T, D>), dim3((unsigned)(nseq * (D / VB))), dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_step(const StepArgs& a, int dtype, int D, int64_t nseq, hipStream_t s) {
  if (nseq <= 0) return hipSuccess;
  if (dtype == 0) {
    if (D == 64) return step_t<__bf16, 64>(a, nseq, s);
    if (D == 128) return step_t<__bf16, 128>(a, nseq, s);
  } else {
    if (D == 64) return step_t<float, 64>(a, nseq, s);
    if (D == 128) return step_t<float, 128>(a, nseq, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace la
