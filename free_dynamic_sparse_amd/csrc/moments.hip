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
//   kcov_kernel    m = (1/N) sum_j Kbar_j and Sigma, one 32x32 tile of Sigma
//                  per workgroup (which first forms the means of its 64
//                  dimensions), float64 sums of centred products staged
//                  through LDS
//   tau_kernel     mu_i, sigma_i, tau_i; each thread keeps half a row of
//                  Sigma in registers and the workgroup walks 32 query blocks

#include <math.h>

#include "common.hpp"
#include "launch.hpp"

namespace solattn {
namespace {

// Sigma, one 32x32 tile per workgroup, and m.  The workgroup first forms the
// means of its 32 row-dimensions and 32 column-dimensions (float64 sums over
// the head's pooled keys in 8 fixed row phases, combined in a fixed order,
// rounded to float32), then the centred products of those dimensions in
// float64, staging 64 pooled keys at a time through LDS.  The diagonal tiles
// also write m.  The head's pooled keys stay in L2 between the two passes.
template <int D>
__global__ __launch_bounds__(256) void kcov_kernel(const float* __restrict__ kbar,
                                                   float* __restrict__ kmean,
                                                   float* __restrict__ kcov, uint32_t N) {
  constexpr int T = D / 32;  // tiles per dimension
  constexpr int RB = 64;     // pooled keys staged per step
  constexpr int PH = 256 / 32;  // row phases of the mean pass
  const uint32_t bh = blockIdx.x;
  const int r0 = 32 * (blockIdx.y / T);
  const int c0 = 32 * (blockIdx.y % T);
  const float* src = kbar + (size_t)bh * N * D;
  __shared__ float sr[RB][33];
  __shared__ float sc[RB][33];
  __shared__ double part[2][PH][32];
  __shared__ float mr[32], mc[32];

  {
    const int ph = threadIdx.x / 32, col = threadIdx.x % 32;
    double s_r = 0.0, s_c = 0.0;
    for (uint32_t j = ph; j < N; j += PH) {
      s_r += (double)src[(size_t)j * D + r0 + col];
      s_c += (double)src[(size_t)j * D + c0 + col];
    }
    part[0][ph][col] = s_r;
    part[1][ph][col] = s_c;
    __syncthreads();
    if (threadIdx.x < 64) {
      const int which = threadIdx.x / 32;
      double t = 0.0;
#pragma unroll
      for (int q = 0; q < PH; ++q) t += part[which][q][col];
      const float m = (float)(t / (double)N);
      if (which == 0) {
        mr[col] = m;
        if (r0 == c0) kmean[(size_t)bh * D + r0 + col] = m;
      } else {
        mc[col] = m;
      }
    }
    __syncthreads();
  }

  const int ta = threadIdx.x / 16, tb = threadIdx.x % 16;
  double acc[2][2] = {{0.0, 0.0}, {0.0, 0.0}};
  for (uint32_t j0 = 0; j0 < N; j0 += RB) {
    for (int e = threadIdx.x; e < RB * 32; e += 256) {
      const int jj = e / 32, col = e % 32;
      const uint32_t j = j0 + jj;
      float vr = 0.f, vc = 0.f;
      if (j < N) {
        vr = src[(size_t)j * D + r0 + col] - mr[col];
        vc = src[(size_t)j * D + c0 + col] - mc[col];
      }
      sr[jj][col] = vr;
      sc[jj][col] = vc;
    }
    __syncthreads();
#pragma unroll 4
    for (int jj = 0; jj < RB; ++jj) {
      const double a0 = sr[jj][2 * ta], a1 = sr[jj][2 * ta + 1];
      const double b0 = sc[jj][2 * tb], b1 = sc[jj][2 * tb + 1];
      acc[0][0] += a0 * b0;
      acc[0][1] += a0 * b1;
      acc[1][0] += a1 * b0;
      acc[1][1] += a1 * b1;
    }
    __syncthreads();
  }
  float* dst = kcov + (size_t)bh * D * D;
#pragma unroll
  for (int x = 0; x < 2; ++x)
#pragma unroll
    for (int y = 0; y < 2; ++y)
      dst[(size_t)(r0 + 2 * ta + x) * D + c0 + 2 * tb + y] = (float)(acc[x][y] / (double)N);
}

// mu_i, sigma_i and tau_i for 32 query blocks per workgroup.  Each thread
// keeps half a row r of Sigma in registers and forms (Sigma Qbar_i)_r for the
// 32 blocks; the per-dimension terms Qbar_ir (Sigma Qbar_i)_r and Qbar_ir m_r
// go to LDS, and TPG threads per block then sum them over r in a fixed order
// (a run of D / TPG dimensions each, then lane exchanges).
template <int D>
__global__ __launch_bounds__(2 * D) void tau_kernel(const float* __restrict__ qbar,
                                                    const float* __restrict__ kmean,
                                                    const float* __restrict__ kcov,
                                                    float* __restrict__ tau, float* __restrict__ mu,
                                                    float* __restrict__ sigma, uint32_t N,
                                                    float scale, float beta) {
  constexpr int NT = 2 * D, HALF = D / 2, G = 32;
  constexpr int TPG = NT / G;      // threads per query block in the final sums
  constexpr int RUN = D / TPG;     // dimensions summed by each of them
  static_assert(TPG * RUN == D && (TPG & (TPG - 1)) == 0, "reduction shape");
  const uint32_t bh = blockIdx.x;
  const uint32_t i0 = blockIdx.y * G;
  const int t = threadIdx.x, r = t / 2, h = t % 2;

  // half a row of Sigma per thread, kept in registers
  float srow[HALF];
  const float* cov = kcov + (size_t)bh * D * D + (size_t)r * D + h * HALF;
#pragma unroll
  for (int e = 0; e < HALF; ++e) srow[e] = cov[e];

  __shared__ float qs[G][D];
  __shared__ float ms[D];
  __shared__ float pq[G][D + 1];  // Qbar_ir (Sigma Qbar_i)_r
  __shared__ float pm[G][D + 1];  // Qbar_ir m_r
  for (int e = t; e < G * D; e += NT) {
    const int g = e / D, c = e % D;
    const uint32_t i = i0 + g;
    qs[g][c] = i < N ? qbar[((size_t)bh * N + i) * D + c] : 0.f;
  }
  for (int c = t; c < D; c += NT) ms[c] = kmean[(size_t)bh * D + c];
  __syncthreads();

  for (int g = 0; g < G; ++g) {
    const float* qv = qs[g];
    float y = 0.f;
#pragma unroll
    for (int e = 0; e < HALF; ++e) y = fmaf(srow[e], qv[h * HALF + e], y);
    const float other = __shfl_xor(y, 1);
    if (h == 0) {
      pq[g][r] = (y + other) * qv[r];  // (Sigma Qbar)_r, the two halves in a fixed order
      pm[g][r] = ms[r] * qv[r];
    }
  }
  __syncthreads();

  const int g = t / TPG, part = t % TPG;
  float qf = 0.f, md = 0.f;
#pragma unroll
  for (int e = 0; e < RUN; ++e) {
    qf += pq[g][part * RUN + e];
    md += pm[g][part * RUN + e];
  }
#pragma unroll
  for (int o = TPG / 2; o >= 1; o /= 2) {
    qf += __shfl_xor(qf, o);
    md += __shfl_xor(md, o);
  }
  const uint32_t i = i0 + g;
  if (part == 0 && i < N) {
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

template <int D>
hipError_t launch_moments_t(const Shape& s, const float* qbar, const float* kbar, float* kmean,
                            float* kcov, float* tau, float* mu, float* sigma, hipStream_t stream) {
  const uint32_t bh = (uint32_t)s.bh, N = (uint32_t)s.N;
  hipLaunchKernelGGL((kcov_kernel<D>), dim3(bh, (D / 32) * (D / 32)), dim3(256), 0, stream, kbar,
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
