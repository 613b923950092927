// Block pooling for Sol-Attn (gfx950).
//
// Method: "Sol-Attn: Accelerating Video Generation Inference via On-the-Fly
// Attention Sparsification", method section: the block proxies of Eq. 3
// (Qbar_i, Kbar_j = means of the block's rows) and the summed values Vhat_j
// used by the approximate terms of Eqs. 9-10.
//
// One workgroup per (b, h, block): 256 threads read the block's Q, K and V
// rows as coalesced 16-byte loads (each thread owns one 8-column segment of
// a row and walks rows with a fixed stride), issue all of them before the
// first add, accumulate in float32 registers, and reduce the row phases
// through LDS in a fixed order.  The pass is bound by HBM reads:
// 3 * n_j * d * 2 bytes per block, streamed with non-temporal loads (7 %
// faster at the Wan shape than cached loads).

#include "common.hpp"
#include "launch.hpp"

namespace solattn {
namespace {

constexpr int kPoolThreads = 256;

template <int D, int BLK>
__global__ __launch_bounds__(kPoolThreads) void pool_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
    const uint16_t* __restrict__ v, float* __restrict__ qbar, float* __restrict__ kbar,
    float* __restrict__ vhat, int64_t L, uint32_t N, uint32_t items) {
  constexpr int SEG = D / 8;                // 16-byte segments per row
  constexpr int RPS = kPoolThreads / SEG;   // rows covered by one step of all threads
  constexpr int STEPS = BLK / RPS;
  static_assert(BLK % RPS == 0, "block must be a multiple of the row stride");

  const uint32_t item = xcd_contiguous_item(blockIdx.x, items);  // (b*H + h)*N + j
  const uint32_t bh = item / N;
  const uint32_t j = item - bh * N;
  const int64_t row0 = (int64_t)j * BLK;
  const int n = (int)((L - row0) < BLK ? (L - row0) : BLK);
  const int seg = threadIdx.x % SEG;
  const int r = threadIdx.x / SEG;
  const size_t base = ((size_t)bh * L + row0) * D + seg * 8;

  float acc[3][8];
#pragma unroll
  for (int t = 0; t < 3; ++t)
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[t][e] = 0.f;

  const uint16_t* src[3] = {q + base, k + base, v + base};
  u32x4 w[STEPS][3];
#pragma unroll
  for (int s = 0; s < STEPS; ++s) {
    const int row = r + s * RPS;
#pragma unroll
    for (int t = 0; t < 3; ++t)
      w[s][t] = row < n ? __builtin_nontemporal_load(
                              reinterpret_cast<const u32x4*>(src[t] + (size_t)row * D))
                        : u32x4{0u, 0u, 0u, 0u};
  }
#pragma unroll
  for (int s = 0; s < STEPS; ++s)
#pragma unroll
    for (int t = 0; t < 3; ++t)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        acc[t][2 * e] += bf16_bits_to_f32(w[s][t][e] & 0xffffu);
        acc[t][2 * e + 1] += bf16_bits_to_f32(w[s][t][e] >> 16);
      }

  __shared__ float red[RPS][3 * D];
#pragma unroll
  for (int t = 0; t < 3; ++t)
#pragma unroll
    for (int e = 0; e < 8; ++e) red[r][t * D + seg * 8 + e] = acc[t][e];
  __syncthreads();

  for (int c = threadIdx.x; c < 3 * D; c += kPoolThreads) {
    float s = 0.f;
    for (int p = 0; p < RPS; ++p) s += red[p][c];
    const int t = c / D;
    const size_t o = (size_t)item * D + (c - t * D);
    if (t == 0)
      qbar[o] = s / (float)n;
    else if (t == 1)
      kbar[o] = s / (float)n;
    else
      vhat[o] = s;
  }
}

template <int D, int BLK>
hipError_t launch_pool_t(const Shape& s, const void* q, const void* k, const void* v,
                         float* qbar, float* kbar, float* vhat, hipStream_t stream) {
  const uint32_t items = (uint32_t)(s.bh * s.N);
  hipLaunchKernelGGL((pool_kernel<D, BLK>), dim3(items), dim3(kPoolThreads), 0, stream,
                     static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(k),
                     static_cast<const uint16_t*>(v), qbar, kbar, vhat, s.L, (uint32_t)s.N,
                     items);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_pool(const Shape& s, const void* q, const void* k, const void* v, float* qbar,
                       float* kbar, float* vhat, hipStream_t stream) {
  if (s.d == 128 && s.block == 128) return launch_pool_t<128, 128>(s, q, k, v, qbar, kbar, vhat, stream);
  if (s.d == 128 && s.block == 64) return launch_pool_t<128, 64>(s, q, k, v, qbar, kbar, vhat, stream);
  if (s.d == 64 && s.block == 128) return launch_pool_t<64, 128>(s, q, k, v, qbar, kbar, vhat, stream);
  if (s.d == 64 && s.block == 64) return launch_pool_t<64, 64>(s, q, k, v, qbar, kbar, vhat, stream);
  return hipErrorInvalidValue;
}

}  // namespace solattn
