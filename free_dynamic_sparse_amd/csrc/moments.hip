// Pooled-key moments and routing thresholds for Sol-Attn (gfx950).
//
// Method: "Sol-Attn: Accelerating Video Generation Inference via On-the-Fly
// Attention Sparsification", method section, query-dependent threshold
// routing (Eq. 4) with the row statistics obtained from the first and second
// moments of the pooled keys (the moment identity derived in Appendix B):
// the proxy row shat_i = scale * Qbar_i Kbar^T has mean scale * Qbar_i . m
// and variance scale^2 * Qbar_i^T Sigma Qbar_i, so all thresholds cost
// O(N d^2) without the N x N proxy map.
//
// Two small kernels, each with a fixed reduction order (deterministic):
//   kcov_kernel    m = (1/N) sum_j Kbar_j and Sigma: one 32x32 tile of Sigma
//                  per workgroup, upper-triangle tiles only (each is also
//                  written to its mirror, so Sigma is exactly symmetric).  The
//                  workgroup first forms the means of its 64 dimensions
//                  (float64 sums), then the d x d update of the centred
//                  products as float64 MFMAs (v_mfma_f64_16x16x4f64: exact
//                  products of the float32 centred values, float64 sums), one
//                  16x16 sub-tile per wave, 4 pooled keys per MFMA
//   tau_kernel     mu_i, sigma_i, tau_i for 32 query blocks per workgroup:
//                  Y = Qbar Sigma by float32 MFMAs (v_mfma_f32_32x32x2f32,
//                  one 32-column slab of Y per wave), then
//                  sigma_i^2 = scale^2 sum_c Qbar_ic Y_ic in a fixed order

#include <math.h>

#include "common.hpp"
#include "launch.hpp"

namespace solattn {
namespace {

typedef double f64x4 __attribute__((ext_vector_type(4)));

// Upper-triangle tile y (row tile tr <= column tile tc) of a T x T tiling.
__device__ __forceinline__ void upper_tile(int y, int T, int* tr, int* tc) {
  int r = 0;
  while (y >= T - r) {
    y -= T - r;
    ++r;
  }
  *tr = r;
  *tc = r + y;
}

template <int D>
__global__ __launch_bounds__(256) void kcov_kernel(const float* __restrict__ kbar,
                                                   float* __restrict__ kmean,
                                                   float* __restrict__ kcov, uint32_t N) {
  constexpr int T = D / 32;   // 32-wide tiles per dimension
  constexpr int PH = 4;       // row phases of the mean pass
  constexpr int UNROLL = 8;   // rows (mean pass) or MFMA steps (update) in flight per thread
  const uint32_t bh = blockIdx.x;
  int tr, tc;
  upper_tile((int)blockIdx.y, T, &tr, &tc);
  const int r0 = 32 * tr, c0 = 32 * tc;
  const float* src = kbar + (size_t)bh * N * D;
  __shared__ double part[PH][64];
  __shared__ float mloc[64];  // means of dimensions r0 .. r0+31, then c0 .. c0+31

  // ---- means: thread (phase, column) sums rows phase, phase + 4, ... in order
  {
    const int col = threadIdx.x % 64, ph = threadIdx.x / 64;
    const float* p = src + (col < 32 ? r0 + col : c0 + col - 32);
    double s = 0.0;
    uint32_t j = ph;
    for (; j + PH * (UNROLL - 1) < N; j += PH * UNROLL) {
      float x[UNROLL];
#pragma unroll
      for (int u = 0; u < UNROLL; ++u) x[u] = p[(size_t)(j + PH * u) * D];
#pragma unroll
      for (int u = 0; u < UNROLL; ++u) s += (double)x[u];
    }
    for (; j < N; j += PH) s += (double)p[(size_t)j * D];
    part[ph][col] = s;
  }
  __syncthreads();
  if (threadIdx.x < 64) {
    double t = 0.0;
#pragma unroll
    for (int q = 0; q < PH; ++q) t += part[q][threadIdx.x];
    const float m = (float)(t / (double)N);
    mloc[threadIdx.x] = m;
    if (tr == tc && threadIdx.x < 32) kmean[(size_t)bh * D + r0 + threadIdx.x] = m;
  }
  __syncthreads();

  // ---- d x d update: wave w owns the 16x16 sub-tile (w / 2, w % 2) of the
  // tile.  Per MFMA, lane l contributes the centred value of pooled key
  // 4 s + l / 16 in row dimension dr (A operand, row l % 16, k = l / 16) and in
  // column dimension dc (B operand, column l % 16, k = l / 16); keys past N
  // contribute 0.
  const int w = threadIdx.x / 64, l = threadIdx.x % 64;
  const int sr = w / 2, sc = w % 2, i16 = l % 16, kq = l / 16;
  const int dr = r0 + 16 * sr + i16, dc = c0 + 16 * sc + i16;
  const float mr = mloc[16 * sr + i16], mc = mloc[32 + 16 * sc + i16];
  f64x4 acc = {0.0, 0.0, 0.0, 0.0};
  const uint32_t steps = (N + 3) / 4;
  for (uint32_t s0 = 0; s0 < steps; s0 += UNROLL) {
    float xa[UNROLL], xb[UNROLL];
#pragma unroll
    for (int u = 0; u < UNROLL; ++u) {
      // keys past N read the last key (in bounds) and are then zeroed, so
      // that every load of the group is in flight at once
      const uint32_t j = 4 * (s0 + u) + kq;
      const size_t jr = (size_t)(j < N ? j : N - 1) * D;
      xa[u] = src[jr + dr];
      xb[u] = src[jr + dc];
    }
#pragma unroll
    for (int u = 0; u < UNROLL; ++u) {
      const bool in = 4 * (s0 + u) + kq < N;
      xa[u] = in ? xa[u] - mr : 0.f;
      xb[u] = in ? xb[u] - mc : 0.f;
    }
#pragma unroll
    for (int u = 0; u < UNROLL; ++u)
      acc = __builtin_amdgcn_mfma_f64_16x16x4f64((double)xa[u], (double)xb[u], acc, 0, 0, 0);
  }
  // result register e of lane l: column l % 16 and row l / 16 + 4 e of the
  // sub-tile (the float64 MFMA's result layout, checked on the device)
  float* dst = kcov + (size_t)bh * D * D;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const int row = r0 + 16 * sr + kq + 4 * e, col = c0 + 16 * sc + i16;
    const float v = (float)(acc[e] / (double)N);
    dst[(size_t)row * D + col] = v;
    if (tr != tc) dst[(size_t)col * D + row] = v;
  }
}

// mu_i, sigma_i and tau_i for G = 32 query blocks per workgroup, D / 32 waves.
// Wave w forms the slab Y[:, 32 w .. 32 w + 31] of Y = Qbar Sigma (A = the
// blocks' Qbar rows from LDS, lane l holding block l % 32 and dimension
// 2 s + l / 32; B = Sigma rows 2 s, 2 s + 1 from memory), multiplies it by the
// matching Qbar entries and sums over its 32 columns (lane butterfly, fixed
// order); the waves' partial sums are then added in wave order.
template <int D>
__global__ __launch_bounds__(2 * D) void tau_kernel(const float* __restrict__ qbar,
                                                    const float* __restrict__ kmean,
                                                    const float* __restrict__ kcov,
                                                    float* __restrict__ tau, float* __restrict__ mu,
                                                    float* __restrict__ sigma, uint32_t N,
                                                    float scale, float beta) {
  constexpr int NT = 2 * D, G = 32, W = D / 32;
  const uint32_t bh = blockIdx.x;
  const uint32_t i0 = blockIdx.y * G;
  const int t = threadIdx.x, w = t / 64, l = t % 64, h = l / 32, l32 = l % 32;

  __shared__ float qs[G][D + 1];
  __shared__ float ms[D];
  __shared__ float part[W][G];
  for (int e = t; e < G * D; e += NT) {
    const int g = e / D, c = e % D;
    const uint32_t i = i0 + g;
    qs[g][c] = i < N ? qbar[((size_t)bh * N + i) * D + c] : 0.f;
  }
  for (int c = t; c < D; c += NT) ms[c] = kmean[(size_t)bh * D + c];
  __syncthreads();

  const float* cov = kcov + (size_t)bh * D * D + 32 * w + l32;
  f32x16 acc;
#pragma unroll
  for (int r = 0; r < 16; ++r) acc[r] = 0.f;
#pragma unroll 8
  for (int s = 0; s < D / 2; ++s)
    acc = __builtin_amdgcn_mfma_f32_32x32x2f32(qs[l32][2 * s + h], cov[(size_t)(2 * s + h) * D],
                                               acc, 0, 0, 0);
  // lane l holds Y[i][c], c = 32 w + l % 32, i = mfma_row(r, l / 32)
  const int c = 32 * w + l32;
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    float v = acc[r] * qs[mfma_row(r, h)][c];
#pragma unroll
    for (int o = 16; o >= 1; o /= 2) v += __shfl_xor(v, o);
    if (l32 == 0) part[w][mfma_row(r, h)] = v;
  }
  __syncthreads();

  if (t < G) {
    const uint32_t i = i0 + t;
    float qf = 0.f;
#pragma unroll
    for (int x = 0; x < W; ++x) qf += part[x][t];
    float md = 0.f;
#pragma unroll 8
    for (int r = 0; r < D; ++r) md = fmaf(qs[t][r], ms[r], md);
    if (i < N) {
      const float mu_i = scale * md;
      const float sigma_i = sqrtf(fmaxf(scale * scale * qf, 0.f));
      float tau_i;
      if (beta == -INFINITY)
        tau_i = -INFINITY;
      else if (beta == INFINITY)
        tau_i = INFINITY;
      else if (sigma_i == 0.f)
        tau_i = -INFINITY;  // constant proxy row: every block passes the >= test
      else
        tau_i = mu_i + beta * sigma_i;
      const size_t o = (size_t)bh * N + i;
      tau[o] = tau_i;
      if (mu) mu[o] = mu_i;
      if (sigma) sigma[o] = sigma_i;
    }
  }
}

template <int D>
hipError_t launch_moments_t(const Shape& s, const float* qbar, const float* kbar, float* kmean,
                            float* kcov, float* tau, float* mu, float* sigma, hipStream_t stream) {
  const uint32_t bh = (uint32_t)s.bh, N = (uint32_t)s.N;
  constexpr int T = D / 32;
  hipLaunchKernelGGL((kcov_kernel<D>), dim3(bh, T * (T + 1) / 2), dim3(256), 0, stream, kbar,
                     kmean, kcov, N);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((tau_kernel<D>), dim3(bh, (N + 31) / 32), dim3(2 * D), 0, stream, qbar,
                     kmean, kcov, tau, mu, sigma, N, s.scale, s.beta);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_moments(const Shape& s, const float* qbar, const float* kbar, float* kmean,
                          float* kcov, float* tau, float* mu, float* sigma, hipStream_t stream) {
  if (s.d == 128) return launch_moments_t<128>(s, qbar, kbar, kmean, kcov, tau, mu, sigma, stream);
  if (s.d == 64) return launch_moments_t<64>(s, qbar, kbar, kmean, kcov, tau, mu, sigma, stream);
  return hipErrorInvalidValue;
}

}  // namespace solattn
