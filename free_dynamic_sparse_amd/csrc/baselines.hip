// Routing baselines over the materialised proxy map (gfx950): the map
// itself, and top-k / top-p selection of each row.
//
// Method context: "Sol-Attn: Accelerating Video Generation Inference via
// On-the-Fly Attention Sparsification", method section after Eq. 4 and the
// experiments' Figures 5(b) and 7.  The page contrasts its threshold routing
// with top-k routing (a fixed budget per query block) and top-p routing (the
// shortest run of a row's largest scores whose softmax mass reaches p); both
// build the N x N proxy map shat_ij = scale * Qbar_i . Kbar_j and traverse it,
// top-p with a cumulative sum over the sorted scores.  These kernels are those
// baselines, for selection-latency and density-spread comparisons; the
// Sol-Attn forward does not use them.

#include <math.h>

#include "common.hpp"
#include "launch.hpp"

namespace solattn {
namespace {

// ------------------------------------------------------------ proxy map

constexpr int kMapTile = 64;  // a 64 x 64 tile of the map per workgroup
constexpr int kMapThreads = 256;
constexpr int kMapPad = 4;    // keeps 16-byte alignment of the transposed rows

// shat[bh][i][j] = scale * Qbar_i . Kbar_j, a float32 FMA chain in order of d.
// Each thread computes a 4 x 4 block of the tile from transposed LDS copies
// of the 64 pooled queries and 64 pooled keys.
template <int D>
__global__ __launch_bounds__(kMapThreads) void proxy_map_kernel(const float* qbar,
                                                                const float* kbar, float* shat,
                                                                uint32_t N, float scale) {
  __shared__ __attribute__((aligned(16))) float qt[D][kMapTile + kMapPad];
  __shared__ __attribute__((aligned(16))) float kt[D][kMapTile + kMapPad];
  const uint32_t tiles = (N + kMapTile - 1) / kMapTile;
  const size_t bh = blockIdx.x / (tiles * tiles);
  const uint32_t t = blockIdx.x % (tiles * tiles);
  const uint32_t i0 = (t / tiles) * kMapTile, j0 = (t % tiles) * kMapTile;
  const float* qh = qbar + bh * N * D;
  const float* kh = kbar + bh * N * D;
  const int tid = threadIdx.x;
  for (int e = tid; e < kMapTile * D; e += kMapThreads) {
    const int r = e / D, d = e % D;
    qt[d][r] = (i0 + r < N) ? qh[(size_t)(i0 + r) * D + d] : 0.f;
    kt[d][r] = (j0 + r < N) ? kh[(size_t)(j0 + r) * D + d] : 0.f;
  }
  __syncthreads();
  const int ty = tid / 16, tx = tid % 16;
  float acc[4][4];
#pragma unroll
  for (int r = 0; r < 4; ++r)
#pragma unroll
    for (int c = 0; c < 4; ++c) acc[r][c] = 0.f;
#pragma unroll 4
  for (int d = 0; d < D; ++d) {
    const f32x4 a = *reinterpret_cast<const f32x4*>(&qt[d][4 * ty]);
    const f32x4 b = *reinterpret_cast<const f32x4*>(&kt[d][4 * tx]);
#pragma unroll
    for (int r = 0; r < 4; ++r)
#pragma unroll
      for (int c = 0; c < 4; ++c) acc[r][c] = __builtin_fmaf(a[r], b[c], acc[r][c]);
  }
  float* out = shat + bh * (size_t)N * N;
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const uint32_t i = i0 + 4 * ty + r;
    if (i >= N) continue;
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const uint32_t j = j0 + 4 * tx + c;
      if (j < N) out[(size_t)i * N + j] = scale * acc[r][c];
    }
  }
}

// ------------------------------------------------------------ selection

constexpr int kSelThreads = 256;

// 32-bit key whose ascending order is the descending order of the score
// (-0 is folded onto +0 so the two compare equal, as floats do).
__device__ __forceinline__ uint32_t descending_key(float s) {
  const uint32_t u = __float_as_uint(s + 0.f);
  const uint32_t asc = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
  return ~asc;
}
__device__ __forceinline__ float key_score(uint32_t key) {
  const uint32_t asc = ~key;
  return __uint_as_float((asc & 0x80000000u) ? (asc & 0x7fffffffu) : ~asc);
}

// One workgroup per proxy row (b, h, i).  The row's N entries are sorted in
// LDS as 64-bit keys (descending score, then increasing block index: the
// tie rule) with a bitonic network over P = 2^ceil(log2 N) slots; the first
// `count` entries are the selected blocks:
//   top-k: count = min(k, N);
//   top-p: w_r = exp(s_r - s_0) over the sorted scores, cumulative sums in
//          float32 (sequential within each thread's run, then the runs'
//          offsets), count = 1 + #{r : cum_r < p * cum_{N-1}} (N for p = 1).
// Dynamic LDS: P keys (8 bytes), P floats for top-p, ceil(N/32) bitmap words.
template <bool TOPP>
__global__ __launch_bounds__(kSelThreads) void select_kernel(const float* shat, uint32_t N,
                                                             uint32_t P, uint32_t k,
                                                             float top_p, uint64_t* sel_mask,
                                                             int32_t* sel_count) {
  extern __shared__ __attribute__((aligned(16))) char sel_smem[];
  uint64_t* keys = reinterpret_cast<uint64_t*>(sel_smem);
  float* cum = reinterpret_cast<float*>(sel_smem + (size_t)P * 8);
  const uint32_t words = (N + 31) / 32;
  uint32_t* bits = reinterpret_cast<uint32_t*>(sel_smem + (size_t)P * (TOPP ? 12 : 8));
  __shared__ float run_total[kSelThreads];
  __shared__ uint32_t below;
  const size_t row = blockIdx.x;
  const float* sr = shat + row * N;
  const uint32_t tid = threadIdx.x;

  for (uint32_t e = tid; e < P; e += kSelThreads)
    keys[e] = e < N ? (((uint64_t)descending_key(sr[e]) << 32) | e) : ~0ull;
  for (uint32_t w = tid; w < words; w += kSelThreads) bits[w] = 0u;
  if (tid == 0) below = 0u;
  __syncthreads();

  // bitonic sort, ascending
  for (uint32_t size = 2; size <= P; size <<= 1) {
    for (uint32_t stride = size >> 1; stride > 0; stride >>= 1) {
      for (uint32_t t = tid; t < P / 2; t += kSelThreads) {
        const uint32_t lo = 2 * stride * (t / stride) + (t % stride);
        const uint32_t hi = lo + stride;
        const bool ascending = (lo & size) == 0;
        const uint64_t a = keys[lo], b = keys[hi];
        if ((a > b) == ascending) {
          keys[lo] = b;
          keys[hi] = a;
        }
      }
      __syncthreads();
    }
  }

  uint32_t count;
  if (!TOPP) {
    count = k < N ? k : N;
  } else if (top_p >= 1.f) {
    count = N;  // mass 1 is reached only by the whole row
  } else {
    // this thread's run [r0, r1) of the sorted order
    const uint32_t per = (N + kSelThreads - 1) / kSelThreads;
    const uint32_t r0 = tid * per < N ? tid * per : N;
    const uint32_t r1 = r0 + per < N ? r0 + per : N;
    const float s0 = key_score((uint32_t)(keys[0] >> 32));
    float run = 0.f;
    for (uint32_t r = r0; r < r1; ++r) {
      run += expf(key_score((uint32_t)(keys[r] >> 32)) - s0);
      cum[r] = run;
    }
    run_total[tid] = run;
    __syncthreads();
    if (tid == 0) {
      float acc = 0.f;
      for (int t = 0; t < kSelThreads; ++t) {
        const float x = run_total[t];
        run_total[t] = acc;  // exclusive offsets
        acc += x;
      }
    }
    __syncthreads();
    const float offset = run_total[tid];
    for (uint32_t r = r0; r < r1; ++r) cum[r] += offset;
    __syncthreads();
    const float thr = top_p * cum[N - 1];
    uint32_t n_below = 0;
    for (uint32_t r = r0; r < r1; ++r) n_below += cum[r] < thr ? 1u : 0u;
    if (n_below) atomicAdd(&below, n_below);
    __syncthreads();
    count = below + 1 < N ? below + 1 : N;
  }

  for (uint32_t r = tid; r < count; r += kSelThreads) {
    const uint32_t j = (uint32_t)(keys[r] & 0xffffffffu);
    atomicOr(&bits[j / 32], 1u << (j % 32));
  }
  __syncthreads();
  const uint32_t w64 = (N + 63) / 64;
  for (uint32_t w = tid; w < w64; w += kSelThreads) {
    const uint32_t lo = bits[2 * w];
    const uint32_t hi = 2 * w + 1 < words ? bits[2 * w + 1] : 0u;
    sel_mask[row * w64 + w] = ((uint64_t)hi << 32) | lo;
  }
  if (sel_count != nullptr && tid == 0) sel_count[row] = (int32_t)count;
}

uint32_t pow2_at_least(uint32_t n) {
  uint32_t p = 1;
  while (p < n) p <<= 1;
  return p;
}

template <bool TOPP>
hipError_t launch_select(const Shape& s, const float* shat, uint32_t k, float top_p,
                         uint64_t* sel_mask, int32_t* sel_count, hipStream_t stream) {
  const uint32_t N = (uint32_t)s.N;
  const uint32_t P = pow2_at_least(N < 2 ? 2 : N);
  const size_t lds = (size_t)P * (TOPP ? 12 : 8) + 4 * (size_t)((N + 31) / 32);
  hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&select_kernel<TOPP>),
                                     hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(select_kernel<TOPP>, dim3((uint32_t)(s.bh * s.N)), dim3(kSelThreads), lds,
                     stream, shat, N, P, k, top_p, sel_mask, sel_count);
  return hipGetLastError();
}

}  // namespace

int64_t select_max_blocks() { return 8192; }

int64_t proxy_map_workgroups(const Shape& s) {
  const int64_t tiles = (s.N + kMapTile - 1) / kMapTile;
  return s.bh * tiles * tiles;
}

hipError_t launch_proxy_map(const Shape& s, const float* qbar, const float* kbar, float* shat,
                            hipStream_t stream) {
  const uint32_t N = (uint32_t)s.N;
  const uint32_t tiles = (N + kMapTile - 1) / kMapTile;
  const dim3 grid((uint32_t)(s.bh * tiles * tiles));
  if (s.d == 128) {
    hipLaunchKernelGGL(proxy_map_kernel<128>, grid, dim3(kMapThreads), 0, stream, qbar, kbar,
                       shat, N, s.scale);
  } else if (s.d == 64) {
    hipLaunchKernelGGL(proxy_map_kernel<64>, grid, dim3(kMapThreads), 0, stream, qbar, kbar,
                       shat, N, s.scale);
  } else {
    return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_select_topk(const Shape& s, const float* shat, int64_t k, uint64_t* sel_mask,
                              int32_t* sel_count, hipStream_t stream) {
  const uint32_t kk = (uint32_t)(k < s.N ? k : s.N);
  return launch_select<false>(s, shat, kk, 1.f, sel_mask, sel_count, stream);
}

hipError_t launch_select_topp(const Shape& s, const float* shat, float top_p,
                              uint64_t* sel_mask, int32_t* sel_count, hipStream_t stream) {
  return launch_select<true>(s, shat, 0u, top_p, sel_mask, sel_count, stream);
}

}  // namespace solattn
