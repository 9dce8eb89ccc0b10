// la_gate.hip -- the small kernels of the gated backward.
//
// Gated recurrence S_t = alpha_t S_{t-1} + k_t v_t^T (the data-dependent
// gates of the Gated Linear Attention entry of the LASP-2 page's
// related-paper list, one scalar gate per token and head), loss
// l = sum_t <do_t, o_t> + <dS_end, S_end>:
//
//   * the reverse sweeps step from token t+1 back to t with alpha_{t+1}:
//     k_shift_gates writes g'_t = g_{t+1} (0 for a segment's last token);
//   * dS0 = alpha_1 G_1: k_scale_first_gate;
//   * d l / d log(alpha_t) = alpha_t <G_t, S_{t-1}>
//                          = sum_{u >= t} (q_u . dq_u - k_u . dk_u) + <dS_end, S_end>
//     within each segment (g_t enters only through the cumulative log-gates,
//     which scale q_u by exp(c_u), k_u by exp(-c_u) and S_end by exp(c_L)).
//     The suffix sums run only inside blocks of 1024 tokens
//     (k_gate_grad_blocks forms r_u = q_u . dq_u - k_u . dk_u and its reverse
//     cumulative sum there, k_gate_grad_rows when the walks formed both row
//     dots); the value at the first token of the next block is taken exactly
//     from the first form, with S and G the fp32 start states the two sweeps
//     already hold at that row (block_anchor: k_gate_anchors, then
//     k_gate_grad_finish adds it; k_gate_grad_rows forms and adds it itself).  Summing r over a whole long segment
//     instead would carry the rounding of dq and dk (and of the sweeps'
//     bf16 operands) over every token: about 15 % at 256K tokens.
#include "la_device.h"
#include "la_internal.h"

namespace la {

constexpr int GBLK = 1024;  // tokens per block of the gate-gradient scan

int64_t gate_grad_blocks(int64_t Ls) { return (Ls + GBLK - 1) / GBLK; }

__global__ __launch_bounds__(256) void k_shift_gates(const float* G, float* Gs, int64_t nseq,
                                                     int64_t Ls) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= nseq * Ls) return;
  const int64_t t = i % Ls;
  Gs[i] = (t + 1 < Ls) ? G[i + 1] : 0.0f;
}

// X[n] *= exp(G[n][0]) for nseq D x D states
__global__ __launch_bounds__(256) void k_scale_first_gate(float* X, const float* G, int64_t nseq,
                                                          int64_t Ls, int64_t DD) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= nseq * DD) return;
  const int64_t n = i / DD;
  X[i] *= expf(G[n * Ls]);
}

template <typename T>
__device__ inline float dot8(const T* a, const T* b) {
  float s = 0.0f;
#pragma unroll
  for (int e = 0; e < 8; ++e) s += (float)a[e] * (float)b[e];
  return s;
}

// One workgroup per (sequence, block of GBLK tokens).  Sixteen lanes share a
// token (8 features each, D / 8 lanes in use), reduce across the 16 with
// shuffles, then the block's reverse cumulative sum is taken in LDS:
// dG[t] = sum_{u >= t in block} r_u, and the block total goes to tot[n][b]
// (when tot is not null).  MODE 1: k_u . dk_u comes from dG itself (formed
// by the joint dV/dK walk), read before the block's values are written.
template <typename T, int D, int MODE>
__global__ __launch_bounds__(256) void k_gate_grad_blocks(const T* Q, const T* dQ, const T* K,
                                                          const T* dK, float* dG, float* tot,
                                                          int64_t Ls, int64_t nb) {
  static_assert(D / 8 <= 16, "16 lanes of 8 features cover a row");
  __shared__ float r[GBLK];
  const int64_t n = blockIdx.x / nb;
  const int64_t b = blockIdx.x % nb;
  const int64_t t0 = b * GBLK;
  const int len = (int)((t0 + GBLK < Ls) ? GBLK : Ls - t0);
  const int sub = threadIdx.x & 15;   // lane within the token's group
  const int tok = threadIdx.x >> 4;   // 16 tokens per pass
  for (int i = tok; i < GBLK; i += 16) {
    float s = 0.0f;
    if (i < len && sub < D / 8) {
      const int64_t row = (n * Ls + t0 + i) * D + 8 * sub;
      s = MODE == 1 ? dot8(Q + row, dQ + row) : dot8(Q + row, dQ + row) - dot8(K + row, dK + row);
    }
#pragma unroll
    for (int m = 8; m >= 1; m >>= 1) s += __shfl_xor(s, m, 16);
    if (MODE == 1 && i < len) s -= dG[n * Ls + t0 + i];
    if (sub == 0) r[i] = s;  // tokens past the end hold 0
  }
  __syncthreads();
  // reverse inclusive scan of r[0 .. GBLK) (Hillis-Steele, ping-pong free:
  // each step reads before the barrier, writes after it)
  for (int d = 1; d < GBLK; d <<= 1) {
    float add[GBLK / 256];
#pragma unroll
    for (int j = 0; j < GBLK / 256; ++j) {
      const int i = threadIdx.x + 256 * j;
      add[j] = (i + d < GBLK) ? r[i + d] : 0.0f;
    }
    __syncthreads();
#pragma unroll
    for (int j = 0; j < GBLK / 256; ++j) r[threadIdx.x + 256 * j] += add[j];
    __syncthreads();
  }
  for (int i = threadIdx.x; i < len; i += 256) dG[n * Ls + t0 + i] = r[i];
  if (threadIdx.x == 0 && tot) tot[n * nb + b] = r[0];
}

// The same when both row dots come from the walks (q_u . dq_u in rq, k_u .
// dk_u in dG), with the anchors already in tot: one workgroup of 256 lanes
// Elementwise dot of two fp32 arrays of n4 four-float vectors by one
// workgroup of 256 lanes: each lane takes vectors j, j + 256, ..., four loads
// of each operand in flight, products and the lane's partial sum in fp32;
// the lanes' partials are returned to the caller's fp64 sum.
__device__ inline float block_dot(const f32x4* x, const f32x4* y, int64_t n4, int j) {
  constexpr int U = 4;
  float e = 0.0f;
  for (int64_t i0 = j; i0 < n4; i0 += 256 * U) {
    f32x4 a[U], c[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t i = i0 + 256 * u;
      a[u] = (i < n4) ? x[i] : f32x4{0.0f, 0.0f, 0.0f, 0.0f};
      c[u] = (i < n4) ? y[i] : f32x4{0.0f, 0.0f, 0.0f, 0.0f};
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const f32x4 p = a[u] * c[u];
      e += (p[0] + p[1]) + (p[2] + p[3]);
    }
  }
  return e;
}

// The gate gradient at the first token y = (b+1) GBLK of block b + 1 of
// sequence n, alpha_y <G_y, S_{y-1}>: an elementwise dot of S^T (the forward
// sweep's start state of sub-segment b + 1) and G^T (the reverse sweep's
// start state at row y, transposed; the reverse sweep numbers its
// sub-segments from the end); for the last block <dS_end, S_end> (S_end
// given transposed; either null: 0).  Products in fp32, the 256 lanes'
// partials summed in fp64 in a fixed order (by waves, then the four waves in
// order); the result is returned to every lane.
__device__ inline float block_anchor(const float* WfT, const float* WrT, const float* G,
                                     const float* dSe, const float* SendT, int64_t n, int64_t b,
                                     int64_t Ls, int64_t nb, int D, double* wred) {
  const int j = threadIdx.x, lane = j & 63, w = j >> 6;
  const int64_t DD = (int64_t)D * D;
  float e = 0.0f;
  double scale = 1.0;
  if (b < nb - 1) {
    e = block_dot(reinterpret_cast<const f32x4*>(WfT + (n * (nb - 1) + b) * DD),
                  reinterpret_cast<const f32x4*>(WrT + (n * (nb - 1) + (nb - 2 - b)) * DD),
                  DD / 4, j);
    scale = exp((double)G[n * Ls + (b + 1) * GBLK]);
  } else if (dSe && SendT) {
    for (int64_t i = j; i < DD; i += 256) {
      const int64_t kk = i / D, vv = i % D;
      e += dSe[n * DD + i] * SendT[n * DD + vv * D + kk];
    }
  }
  double x = (double)e;
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) x += __shfl_down(x, off, 64);
  if (lane == 0) wred[w] = x;
  __syncthreads();
  const double t = ((wred[0] + wred[1]) + (wred[2] + wred[3])) * scale;
  return (float)t;
}

// One workgroup per (sequence, block of GBLK tokens): the block's anchor
// (block_anchor), then dG[t] = sum_{u >= t in block} r_u + anchor with
// r_u = rq[u] - dG[u] (q.dq from the dQ walk, k.dk already in dG from the
// joint dV/dK walk), written in place.  Lane j takes tokens 4 j .. 4 j + 3:
// each lane sums its four from the end, the lanes' totals are summed from
// the end across each wave by shuffles and across the four waves in LDS.
__global__ __launch_bounds__(256) void k_gate_grad_rows(const float* rq, float* dG,
                                                        const float* WfT, const float* WrT,
                                                        const float* G, const float* dSe,
                                                        const float* SendT, int64_t Ls,
                                                        int64_t nb, int D) {
  static_assert(GBLK == 4 * 256, "four tokens a lane");
  __shared__ float wsum[4];
  __shared__ double wred[4];
  const int64_t n = blockIdx.x / nb;
  const int64_t b = blockIdx.x % nb;
  const int64_t base = n * Ls + b * GBLK;
  const int len = (int)((b * GBLK + GBLK < Ls) ? GBLK : Ls - b * GBLK);
  const int j = threadIdx.x, lane = j & 63, w = j >> 6;
  float r[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) {  // tokens past the end add 0
    const int i = 4 * j + e;
    r[e] = (i < len) ? rq[base + i] - dG[base + i] : 0.0f;
  }
  const float anchor = block_anchor(WfT, WrT, G, dSe, SendT, n, b, Ls, nb, D, wred);
  float s[4];
  float acc = 0.0f;
#pragma unroll
  for (int e = 3; e >= 0; --e) {
    acc += r[e];
    s[e] = acc;
  }
  // inclusive suffix sum of the lanes' totals within the wave
  float x = acc;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const float y = __shfl_down(x, off, 64);
    if (lane + off < 64) x += y;
  }
  if (lane == 0) wsum[w] = x;
  __syncthreads();
  float later = x - acc;  // lanes after this one in the wave
  for (int ww = w + 1; ww < 4; ++ww) later += wsum[ww];
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const int i = 4 * j + e;
    if (i < len) dG[base + i] = (s[e] + later) + anchor;
  }
}

// One workgroup per (sequence n, block b): tot[n][b] = block_anchor.
__global__ __launch_bounds__(256) void k_gate_anchors(const float* WfT, const float* WrT,
                                                      const float* G, const float* dSe,
                                                      const float* SendT, float* tot, int64_t Ls,
                                                      int64_t nb, int D) {
  __shared__ double wred[4];
  const int64_t n = (int64_t)blockIdx.x / nb;
  const int64_t b = (int64_t)blockIdx.x % nb;
  const float t = block_anchor(WfT, WrT, G, dSe, SendT, n, b, Ls, nb, D, wred);
  if (threadIdx.x == 0) tot[n * nb + b] = t;
}

__global__ __launch_bounds__(256) void k_gate_grad_finish(float* dG, const float* tot, int64_t nseq,
                                                          int64_t Ls, int64_t nb) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= nseq * Ls) return;
  const int64_t n = i / Ls, t = i % Ls;
  dG[i] += tot[n * nb + t / GBLK];
}

hipError_t launch_shift_gates(const float* G, float* Gs, int64_t nseq, int64_t Ls, hipStream_t s) {
  const int64_t tot = nseq * Ls;
  if (tot <= 0) return hipSuccess;
  hipLaunchKernelGGL(k_shift_gates, dim3((unsigned)((tot + 255) / 256)), dim3(256), 0, s, G, Gs,
                     nseq, Ls);
  return hipGetLastError();
}

hipError_t launch_scale_first_gate(float* X, const float* G, int64_t nseq, int64_t Ls, int D,
                                   hipStream_t s) {
  const int64_t DD = (int64_t)D * D, tot = nseq * DD;
  if (tot <= 0 || Ls <= 0) return hipSuccess;
  hipLaunchKernelGGL(k_scale_first_gate, dim3((unsigned)((tot + 255) / 256)), dim3(256), 0, s, X,
                     G, nseq, Ls, DD);
  return hipGetLastError();
}

hipError_t launch_gate_anchors(const float* WfT, const float* WrT, const float* G,
                               const float* dSe, const float* SendT, float* tot, int64_t nseq,
                               int64_t Ls, int D, hipStream_t s) {
  const int64_t nb = gate_grad_blocks(Ls);
  if (nseq <= 0 || nb <= 0) return hipSuccess;
  hipLaunchKernelGGL(k_gate_anchors, dim3((unsigned)(nseq * nb)), dim3(256), 0, s, WfT, WrT, G, dSe,
                     SendT, tot, Ls, nb, D);
  return hipGetLastError();
}

hipError_t launch_gate_grad_rows(const float* rq, float* dG, const float* WfT, const float* WrT,
                                 const float* G, const float* dSe, const float* SendT,
                                 int64_t nseq, int64_t Ls, int D, hipStream_t s) {
  const int64_t nb = gate_grad_blocks(Ls);
  if (nseq <= 0 || nb <= 0) return hipSuccess;
  hipLaunchKernelGGL(k_gate_grad_rows, dim3((unsigned)(nseq * nb)), dim3(256), 0, s, rq, dG, WfT,
                     WrT, G, dSe, SendT, Ls, nb, D);
  return hipGetLastError();
}

template <typename T, int D>
static hipError_t gate_grad_t(const void* Q, const void* dQ, const void* K, const void* dK,
                              float* dG, const float* tot, int64_t nseq, int64_t Ls,
                              hipStream_t s) {
  const int64_t nb = gate_grad_blocks(Ls);
  const dim3 grid((unsigned)(nseq * nb));
  // the block totals are not needed: tot already holds the anchors
  if (K && dK)
    hipLaunchKernelGGL((k_gate_grad_blocks<T, D, 0>), grid, dim3(256), 0, s, (const T*)Q,
                       (const T*)dQ, (const T*)K, (const T*)dK, dG, nullptr, Ls, nb);
  else
    hipLaunchKernelGGL((k_gate_grad_blocks<T, D, 1>), grid, dim3(256), 0, s, (const T*)Q,
                       (const T*)dQ, nullptr, nullptr, dG, nullptr, Ls, nb);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int64_t all = nseq * Ls;
  hipLaunchKernelGGL(k_gate_grad_finish, dim3((unsigned)((all + 255) / 256)), dim3(256), 0, s, dG,
                     tot, nseq, Ls, nb);
  return hipGetLastError();
}

hipError_t launch_gate_grad(int dtype, int D, const void* Q, const void* dQ, const void* K,
                            const void* dK, float* dG, const float* tot, int64_t nseq, int64_t Ls,
                            hipStream_t s) {
  if (nseq <= 0 || Ls <= 0) return hipSuccess;
  if (dtype == 0) {
    if (D == 64) return gate_grad_t<__bf16, 64>(Q, dQ, K, dK, dG, tot, nseq, Ls, s);
    if (D == 128) return gate_grad_t<__bf16, 128>(Q, dQ, K, dK, dG, tot, nseq, Ls, s);
  } else {
    if (D == 64) return gate_grad_t<float, 64>(Q, dQ, K, dK, dG, tot, nseq, Ls, s);
    if (D == 128) return gate_grad_t<float, 128>(Q, dQ, K, dK, dG, tot, nseq, Ls, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace la
