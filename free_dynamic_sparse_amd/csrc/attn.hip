// Fused Sol-Attn forward and the dense comparison kernel (gfx950).
//
// Method: "Sol-Attn: Accelerating Video Generation Inference via On-the-Fly
// Attention Sparsification", method section: chunk-wise streaming
// thresholding (Eqs. 6-7), zeroth-order approximation of unselected blocks
// with the combined denominator and numerator (Eqs. 9-10), the token-to-block
// score tile (Eq. 11, Figure 4) and the nested-loop kernel (Algorithm 3.2).
//
// Work decomposition.  One workgroup serves a pair of neighbouring query
// blocks (2p, 2p+1) of one head: waves [0, QW) own block 2p, waves [QW, 2QW)
// own block 2p+1, one wave per 32 query rows.  Each group keeps its own
// routing threshold, selected set and online-softmax state.  Neighbouring
// blocks select nearly the same key blocks, so a key block in either set is
// loaded into LDS once and consumed by whichever group selected it; the two
// groups also put two waves on every SIMD, so one group's softmax (VALU)
// overlaps the other's MFMA work.
//
// MFMA layout (v_mfma_f32_32x32x16_bf16), computed transposed so each lane
// owns one query:
//   S^T = K Q^T      A = K rows from LDS, B = Q^T held in registers;
//                    lane l holds query l%32 and 16 keys per 32x32 tile, so
//                    the softmax row max / sum is lane-local plus one
//                    exchange with lane l^32;
//   O^T += V^T P^T   A = V^T via the LDS transpose read (ds_read_b64_tr_b16)
//                    of row-major V, B = P^T straight from the S^T registers.
// K and V blocks travel global -> LDS with direct-to-LDS loads
// (global_load_lds_dwordx4, 1 KB per wave instruction) into XOR-swizzled
// tiles; the next selected block's K is fetched while this block's softmax
// and P V run, its V while the next S^T is computed.
//
// Outer loop, per chunk of C pooled keys (staged 32 at a time as float32):
//   * routing: every wave computes shat_ij = scale * Qbar_i . Kbar_j in
//     float32 for both groups and ballots shat_ij >= tau_i.  Every wave runs
//     the same instructions on the same data, so the masks agree across the
//     workgroup without communication.  (The page reads these scores off the
//     token-to-block tile as column means; the mean is the same number, and
//     the direct float32 dot keeps the decision far inside the tie band that
//     a bf16 tile would not.)
//   * approximation: the token-to-block tile scale * Q_i KC^T on MFMA (KC
//     rounded to bf16); each group's unselected columns update its online
//     softmax with weight n_j and value Vhat_j (VC).
// Inner loop: the chunk's selected key blocks, exact attention.  Exact and
// approximate terms share one running max, denominator and accumulator.

#include <math.h>

#include "common.hpp"
#include "launch.hpp"

namespace solattn {
namespace {

typedef short v4i16 __attribute__((ext_vector_type(4)));
typedef short v8i16 __attribute__((ext_vector_type(8)));
#define LDS_PTR(T, p) ((__attribute__((address_space(3))) T*)(p))

template <int D, int BLK>
struct Cfg {
  static constexpr int QW = BLK / 32;       // waves per query block
  static constexpr int WAVES = 2 * QW;      // a pair of query blocks
  static constexpr int NT = WAVES * kWave;  // = 4 * BLK (launch bounds)
  static constexpr int KS = D / 16;         // k-steps of Q K^T (contraction over d)
  static constexpr int MT = BLK / 32;       // 32-key tiles of S^T
  static constexpr int DT = D / 32;         // 32-wide d tiles of O^T
  static constexpr int PK = BLK / 16;       // k-steps of P V (contraction over keys)
  static constexpr int SEGS = D / 8;        // 16-byte segments in a bf16 row
  static constexpr int ROW = 2 * D;         // bytes per bf16 row
  static constexpr int TILE = BLK * ROW;    // bytes per K or V tile
  static constexpr int DMA = TILE / 1024 / WAVES;  // 1 KB loads per wave per tile
  static constexpr int ROWS_1K = 1024 / ROW;       // tile rows per 1 KB load
  static constexpr int SUB = 32;            // pooled rows staged at a time
  static constexpr int CROW = 4 * D + 16;   // bytes per float32 pooled row (16 B pad)
  static_assert(DMA * WAVES * 1024 == TILE, "tile must split into whole 1 KB loads");
};

// XOR swizzles of the 16-byte segments of tile row r (no padding possible
// with lane-linear direct-to-LDS writes).  K: the A-operand reads of 16
// consecutive rows hit 16 distinct segments.  V: each transpose read covers
// 8 rows x 64 bytes; rows r..r+3 land in disjoint 64-byte bank ranges.
template <int SEGS>
__device__ __forceinline__ int swz_k(int r) { return r % SEGS; }
template <int SEGS>
__device__ __forceinline__ int swz_v(int r) { return (4 * (r % 4)) % SEGS; }

struct AttnArgs {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  const float* qbar;
  const float* kbar;
  const float* vhat;
  const float* tau;
  uint16_t* out;
  uint64_t* sel_mask;
  int32_t* sel_count;
  int64_t L;
  uint32_t N;
  uint32_t pairs;    // ceil(N / 2)
  uint32_t per_xcd;  // pairs per XCD slab: ceil(pairs / 8)
  int chunk;
  float scale;
  float c_log2;      // scale * log2(e): logits enter exp2 in this unit
  uint32_t exact_only;
};

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Wait until at most N of this wave's vector-memory loads are outstanding.
template <int N>
__device__ __forceinline__ void wait_vm() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}
// Workgroup barrier that does not wait for outstanding direct-to-LDS loads.
__device__ __forceinline__ void barrier_lds() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// Issue this wave's share of the direct-to-LDS loads of one K or V tile.
// Rows >= nkeys re-read row nkeys-1 (finite data that the softmax masks).
template <int D, int BLK, bool IS_V>
__device__ __forceinline__ void dma_tile(char* tile, const uint16_t* gblk, int nkeys, int wave,
                                         int lane) {
  using C = Cfg<D, BLK>;
#pragma unroll
  for (int c = 0; c < C::DMA; ++c) {
    const int chunk = wave + c * C::WAVES;
    const int row = chunk * C::ROWS_1K + lane / C::SEGS;
    const int pos = lane % C::SEGS;
    const int seg = pos ^ (IS_V ? swz_v<C::SEGS>(row) : swz_k<C::SEGS>(row));
    const int grow = row < nkeys ? row : nkeys - 1;
    const uint16_t* src = gblk + (size_t)grow * D + seg * 8;
    __builtin_amdgcn_global_load_lds((void*)src, LDS_PTR(void, tile + chunk * 1024), 16, 0, 0);
  }
}

// S^T (keys x this wave's 32 queries) = K Q^T for the key tile in LDS.
template <int D, int BLK>
__device__ __forceinline__ void qk_tile(const char* ktile, const bf16x8* qreg, f32x16* s,
                                        int lane) {
  using C = Cfg<D, BLK>;
  const int h = lane / 32, l32 = lane % 32;
#pragma unroll
  for (int mt = 0; mt < C::MT; ++mt)
#pragma unroll
    for (int r = 0; r < 16; ++r) s[mt][r] = 0.f;
#pragma unroll
  for (int ks = 0; ks < C::KS; ++ks) {
#pragma unroll
    for (int mt = 0; mt < C::MT; ++mt) {
      const int row = 32 * mt + l32;
      const int seg = (2 * ks + h) ^ swz_k<C::SEGS>(row);
      const bf16x8 ka = *reinterpret_cast<const bf16x8*>(ktile + row * C::ROW + seg * 16);
      s[mt] = mfma32x32x16(ka, qreg[ks], s[mt]);
    }
    // keep at most one k-step of operands in flight (register budget)
    __builtin_amdgcn_sched_barrier(0);
  }
}

// Online-softmax update with the exact scores of one key block (nkeys valid
// keys); leaves P^T (unnormalised, float) in s.
template <int D, int BLK>
__device__ __forceinline__ void softmax_block(f32x16* s, int nkeys, float c, float& m_run,
                                              float& l_run, f32x16* o, int lane) {
  using C = Cfg<D, BLK>;
  const int h = lane / 32;
  if (nkeys < BLK) {
#pragma unroll
    for (int mt = 0; mt < C::MT; ++mt)
#pragma unroll
      for (int r = 0; r < 16; ++r)
        if (32 * mt + mfma_row(r, h) >= nkeys) s[mt][r] = -INFINITY;
  }
  float mx = -INFINITY;
#pragma unroll
  for (int mt = 0; mt < C::MT; ++mt)
#pragma unroll
    for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[mt][r]);
  mx = wave_max_pair(mx);
  const float m_new = fmaxf(m_run, mx * c);
  const float alpha = fast_exp2(m_run - m_new);
  float psum = 0.f;
#pragma unroll
  for (int mt = 0; mt < C::MT; ++mt)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const float p = fast_exp2(__builtin_fmaf(s[mt][r], c, -m_new));
      s[mt][r] = p;
      psum += p;
    }
  l_run = l_run * alpha + psum;
  m_run = m_new;
  if (__ballot(alpha != 1.f)) {
#pragma unroll
    for (int dt = 0; dt < C::DT; ++dt) o[dt] *= alpha;
  }
}

// O^T += V^T P^T for the value tile in LDS.
template <int D, int BLK>
__device__ __forceinline__ void pv_tile(const char* vtile, const f32x16* s, f32x16* o, int lane) {
  using C = Cfg<D, BLK>;
  const int g = lane / 16, j = lane % 16;
#pragma unroll
  for (int kk = 0; kk < C::PK; ++kk) {
    const int mt = kk / 2, hf = kk % 2;
    float pv[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) pv[e] = s[mt][8 * hf + e];
    const bf16x8 pb = pack_bf16x8(pv);
    const int row = 16 * kk + 4 * (g / 2) + j / 4;
#pragma unroll
    for (int dt = 0; dt < C::DT; ++dt) {
      const int col = 32 * dt + 16 * (g % 2) + 4 * (j % 4);
      const char* p0 =
          vtile + row * C::ROW + ((col / 8) ^ swz_v<C::SEGS>(row)) * 16 + (col % 8) * 2;
      // keys 16kk + 4h + {0..3} and 16kk + 8 + 4h + {0..3} for d = 32dt + lane%32
      const v4i16 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(LDS_PTR(v4i16, p0));
      const v4i16 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(LDS_PTR(v4i16, p0 + 8 * C::ROW));
      const v8i16 both = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
      o[dt] = mfma32x32x16(__builtin_bit_cast(bf16x8, both), pb, o[dt]);
    }
    __builtin_amdgcn_sched_barrier(0);
  }
}

// Copy pooled rows [j0, j0 + rows) of Kbar and Vhat (float32) to LDS; the
// rest of the SUB staged rows are zero so readers need no bounds checks.
template <int D, int BLK>
__device__ __forceinline__ void stage_pooled(char* kch, char* vch, const float* kbar_h,
                                             const float* vhat_h, uint32_t j0, int rows,
                                             int tid) {
  using C = Cfg<D, BLK>;
  constexpr int P = D / 4;  // 16-byte pieces per row
  constexpr int IT = (C::SUB * P + C::NT - 1) / C::NT;
#pragma unroll
  for (int it = 0; it < IT; ++it) {
    const int idx = tid + it * C::NT;
    const int jj = idx / P, pc = idx % P;
    if (jj < C::SUB) {
      f32x4 kk = {0.f, 0.f, 0.f, 0.f}, vv = {0.f, 0.f, 0.f, 0.f};
      if (jj < rows) {
        const size_t gofs = (size_t)(j0 + jj) * D + pc * 4;
        kk = *reinterpret_cast<const f32x4*>(kbar_h + gofs);
        vv = *reinterpret_cast<const f32x4*>(vhat_h + gofs);
      }
      *reinterpret_cast<f32x4*>(kch + jj * C::CROW + pc * 16) = kk;
      *reinterpret_cast<f32x4*>(vch + jj * C::CROW + pc * 16) = vv;
    }
  }
}

// Routing of up to 32 staged pooled keys for both query blocks of the pair:
// bit jj of mask g is set iff pooled key jj (< rows) has shat >= tau_g.
template <int D, int BLK>
__device__ __forceinline__ void route_sub(const char* kch, const float (*qbar_s)[D], int rows,
                                          float tau0, float tau1, float scale, int lane,
                                          uint32_t* m0, uint32_t* m1) {
  using C = Cfg<D, BLK>;
  constexpr int HALF = D / 2;
  const int h = lane / 32, jj = lane % 32;
  float p0 = 0.f, p1 = 0.f;
  if (jj < rows) {
    const float* kr = reinterpret_cast<const float*>(kch + jj * C::CROW) + h * HALF;
#pragma unroll
    for (int e = 0; e < HALF; e += 4) {
      const f32x4 kv = *reinterpret_cast<const f32x4*>(kr + e);
      const f32x4 q0 = *reinterpret_cast<const f32x4*>(&qbar_s[0][h * HALF + e]);
      const f32x4 q1 = *reinterpret_cast<const f32x4*>(&qbar_s[1][h * HALF + e]);
#pragma unroll
      for (int x = 0; x < 4; ++x) {
        p0 = __builtin_fmaf(q0[x], kv[x], p0);
        p1 = __builtin_fmaf(q1[x], kv[x], p1);
      }
    }
  }
  const float o0 = __shfl_xor(p0, 32), o1 = __shfl_xor(p1, 32);
  const float d0 = (h == 0) ? (p0 + o0) : (o0 + p0);
  const float d1 = (h == 0) ? (p1 + o1) : (o1 + p1);
  *m0 = (uint32_t)__ballot((jj < rows) && (scale * d0 >= tau0));
  *m1 = (uint32_t)__ballot((jj < rows) && (scale * d1 >= tau1));
}

// Zeroth-order terms of the staged pooled keys whose bit is set in unsel
// (Eqs. 9-10): logits from the token-to-block tile, weight n_j in the
// denominator, Vhat_j in the numerator.  jbase = index of staged row 0.
template <int D, int BLK>
__device__ __forceinline__ void approx_sub(const char* kch, const char* vch, const bf16x8* qreg,
                                           uint32_t unsel, uint32_t jbase, uint32_t N,
                                           int n_last, float c, float& m_run, float& l_run,
                                           f32x16* o, int lane) {
  using C = Cfg<D, BLK>;
  const int h = lane / 32, l32 = lane % 32;
  f32x16 t;
#pragma unroll
  for (int r = 0; r < 16; ++r) t[r] = 0.f;
#pragma unroll
  for (int ks = 0; ks < C::KS; ++ks) {
    // staged row l32 (finite; zero past the staged rows) feeds this lane's A operand
    const float* src = reinterpret_cast<const float*>(kch + l32 * C::CROW) + 16 * ks + 8 * h;
    const bf16x8 ka = pack_bf16x8(*reinterpret_cast<const f32x4*>(src),
                                  *reinterpret_cast<const f32x4*>(src + 4));
    t = mfma32x32x16(ka, qreg[ks], t);
  }
  float mx = -INFINITY;
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    if (!((unsel >> mfma_row(r, h)) & 1u)) t[r] = -INFINITY;
    mx = fmaxf(mx, t[r]);
  }
  mx = wave_max_pair(mx);
  const float m_new = fmaxf(m_run, mx * c);
  const float alpha = fast_exp2(m_run - m_new);
  float lsum = 0.f;
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    const float p = fast_exp2(__builtin_fmaf(t[r], c, -m_new));
    t[r] = p;
    const float w = (jbase + mfma_row(r, h) == N - 1) ? (float)n_last : (float)BLK;
    lsum = __builtin_fmaf(w, p, lsum);
  }
  l_run = l_run * alpha + lsum;
  m_run = m_new;
#pragma unroll
  for (int dt = 0; dt < C::DT; ++dt) o[dt] *= alpha;
#pragma unroll
  for (int hf = 0; hf < 2; ++hf) {
    float pv[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) pv[e] = t[8 * hf + e];
    const bf16x8 pb = pack_bf16x8(pv);
#pragma unroll
    for (int dt = 0; dt < C::DT; ++dt) {
      float vv[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        // columns outside unsel carry p = 0 against finite staged values
        const int jr = mfma_row(8 * hf + e, h);
        vv[e] = reinterpret_cast<const float*>(vch + jr * C::CROW)[32 * dt + l32];
      }
      o[dt] = mfma32x32x16(pack_bf16x8(vv), pb, o[dt]);
    }
  }
}

// Exact attention over the key blocks j0 + bit of `both` (in increasing
// order); this wave's group takes the blocks whose bit is set in `mine`.
// K/V of the next block are prefetched while the current one is consumed.
template <int D, int BLK>
__device__ __forceinline__ void exact_blocks(char* ktile, char* vtile, const uint16_t* kh,
                                             const uint16_t* vh, int64_t L, uint32_t j0,
                                             uint64_t both, uint64_t mine, const bf16x8* qreg,
                                             float c, float& m_run, float& l_run, f32x16* o,
                                             int wave, int lane) {
  using C = Cfg<D, BLK>;
  if (both == 0) return;
  auto nkeys_of = [&](uint32_t j) {
    const int64_t rem = L - (int64_t)j * BLK;
    return (int)(rem < BLK ? rem : BLK);
  };
  wait_vm<0>();
  uint32_t j = j0 + (uint32_t)__builtin_ctzll(both);
  both &= both - 1;
  dma_tile<D, BLK, false>(ktile, kh + (size_t)j * BLK * D, nkeys_of(j), wave, lane);
  dma_tile<D, BLK, true>(vtile, vh + (size_t)j * BLK * D, nkeys_of(j), wave, lane);
  f32x16 s[C::MT];
  while (true) {
    const bool has_next = both != 0;
    const uint32_t jn = has_next ? j0 + (uint32_t)__builtin_ctzll(both) : 0u;
    const bool active = (mine >> (j - j0)) & 1ull;
    const int nk = nkeys_of(j);
    wait_vm<C::DMA>();  // this block's K has landed (its V may still be in flight)
    barrier_lds();
    if (active) qk_tile<D, BLK>(ktile, qreg, s, lane);
    barrier_lds();      // every wave is done with K
    if (has_next)
      dma_tile<D, BLK, false>(ktile, kh + (size_t)jn * BLK * D, nkeys_of(jn), wave, lane);
    if (active) softmax_block<D, BLK>(s, nk, c, m_run, l_run, o, lane);
    if (has_next)
      wait_vm<C::DMA>();  // V has landed (the next K may still be in flight)
    else
      wait_vm<0>();
    barrier_lds();
    if (active) pv_tile<D, BLK>(vtile, s, o, lane);
    barrier_lds();      // every wave is done with V
    if (!has_next) break;
    dma_tile<D, BLK, true>(vtile, vh + (size_t)jn * BLK * D, nkeys_of(jn), wave, lane);
    j = jn;
    both &= both - 1;
  }
}

template <int D, int BLK, bool FUSED>
__global__ __launch_bounds__(4 * BLK) void attn_kernel(AttnArgs a) {
  using C = Cfg<D, BLK>;
  __shared__ __attribute__((aligned(1024))) char ktile[C::TILE];
  __shared__ __attribute__((aligned(1024))) char vtile[C::TILE];
  __shared__ __attribute__((aligned(16))) char kch[FUSED ? C::SUB * C::CROW : 16];
  __shared__ __attribute__((aligned(16))) char vch[FUSED ? C::SUB * C::CROW : 16];
  __shared__ __attribute__((aligned(16))) float qbar_s[2][D];

  const int tid = threadIdx.x, lane = tid % kWave, wave = tid / kWave;
  const int grp = wave / C::QW;  // which block of the pair
  const int h = lane / 32, l32 = lane % 32;
  uint32_t bh, pair;
  if (!head_striped_item(blockIdx.x, a.pairs, a.per_xcd, &bh, &pair)) return;
  const uint32_t N = a.N;
  const uint32_t i_g = 2 * pair + grp;       // this group's query block
  const bool grp_on = i_g < N;               // block 2p+1 may not exist
  const bool pair1_on = 2 * pair + 1 < N;
  const int64_t L = a.L;
  const int n_i =
      grp_on ? (int)((L - (int64_t)i_g * BLK) < BLK ? (L - (int64_t)i_g * BLK) : BLK) : 0;
  const int n_last = (int)(L - (int64_t)(N - 1) * BLK);
  const size_t head = (size_t)bh * (size_t)L * D;
  const uint16_t* qh = a.q + head;
  const uint16_t* kh = a.k + head;
  const uint16_t* vh = a.v + head;

  // Q^T operand: this lane's query row, 8 consecutive d per k-step.
  const int qrow = (wave % C::QW) * 32 + l32;
  bf16x8 qreg[C::KS];
#pragma unroll
  for (int ks = 0; ks < C::KS; ++ks) {
    u32x4 w = {0u, 0u, 0u, 0u};
    if (qrow < n_i)
      w = *reinterpret_cast<const u32x4*>(qh + ((size_t)i_g * BLK + qrow) * D + 16 * ks + 8 * h);
    qreg[ks] = __builtin_bit_cast(bf16x8, w);
  }

  float m_run = -INFINITY, l_run = 0.f;
  f32x16 o[C::DT];
#pragma unroll
  for (int dt = 0; dt < C::DT; ++dt)
#pragma unroll
    for (int r = 0; r < 16; ++r) o[dt][r] = 0.f;

  if constexpr (FUSED) {
    const uint32_t item0 = bh * N + 2 * pair;
    const float tau0 = a.tau[item0];
    const float tau1 = pair1_on ? a.tau[item0 + 1] : INFINITY;
    for (int cc = tid; cc < 2 * D; cc += C::NT) {
      const int g = cc / D;
      qbar_s[g][cc % D] = (g == 0 || pair1_on) ? a.qbar[(size_t)(item0 + g) * D + cc % D] : 0.f;
    }
    const float* kbar_h = a.kbar + (size_t)bh * N * D;
    const float* vhat_h = a.vhat + (size_t)bh * N * D;
    const uint32_t chunk = (uint32_t)a.chunk;
    const uint32_t T = (N + chunk - 1) / chunk;
    const uint32_t W = (N + 63) / 64;
    // the group's first wave keeps the debug bitmap (wave-uniform); lane 0 stores
    const bool writer = grp_on && (wave % C::QW) == 0;
    uint64_t* mrow = (a.sel_mask && writer) ? a.sel_mask + (size_t)(bh * N + i_g) * W : nullptr;
    uint32_t cur_word = 0;
    uint64_t cur_bits = 0;
    int count = 0;
    for (uint32_t t = 0; t < T; ++t) {
      const uint32_t j0 = t * chunk;
      const int cvalid = (int)((N - j0) < chunk ? (N - j0) : chunk);
      uint64_t mask0 = 0, mask1 = 0;
      for (int sb = 0; sb < cvalid; sb += C::SUB) {
        const int rows = (cvalid - sb) < C::SUB ? (cvalid - sb) : C::SUB;
        __syncthreads();  // previous readers of the staging buffers are done
        stage_pooled<D, BLK>(kch, vch, kbar_h, vhat_h, j0 + sb, rows, tid);
        __syncthreads();
        uint32_t s0, s1;
        route_sub<D, BLK>(kch, qbar_s, rows, tau0, tau1, a.scale, lane, &s0, &s1);
        mask0 |= (uint64_t)s0 << sb;
        mask1 |= (uint64_t)s1 << sb;
        const uint32_t mine_s = grp == 0 ? s0 : s1;
        const uint32_t valid = rows >= 32 ? 0xffffffffu : ((1u << rows) - 1u);
        const uint32_t unsel = valid & ~mine_s;
        if (grp_on && !a.exact_only && unsel)
          approx_sub<D, BLK>(kch, vch, qreg, unsel, j0 + sb, N, n_last, a.c_log2, m_run, l_run,
                             o, lane);
      }
      if (!pair1_on) mask1 = 0;
      const uint64_t mine = grp == 0 ? mask0 : mask1;
      if (mrow) {
        // append this chunk's bits to the row bitmap (chunks arrive in order)
        const uint32_t word = j0 / 64, sh = j0 % 64;
        if (word != cur_word) {
          if (lane == 0) mrow[cur_word] = cur_bits;
          cur_word = word;
          cur_bits = 0;
        }
        cur_bits |= mine << sh;
        if (sh + (uint32_t)cvalid > 64) {
          if (lane == 0) mrow[cur_word] = cur_bits;
          cur_word = word + 1;
          cur_bits = mine >> (64 - sh);
        }
      }
      count += __builtin_popcountll(mine);
      exact_blocks<D, BLK>(ktile, vtile, kh, vh, L, j0, mask0 | mask1, mine, qreg, a.c_log2,
                           m_run, l_run, o, wave, lane);
    }
    if (mrow && lane == 0) mrow[cur_word] = cur_bits;
    if (a.sel_count && writer && lane == 0) a.sel_count[bh * N + i_g] = count;
  } else {
    for (uint32_t j0 = 0; j0 < N; j0 += 64) {
      const uint32_t n = (N - j0) < 64 ? (N - j0) : 64;
      const uint64_t all = n >= 64 ? ~0ull : ((1ull << n) - 1ull);
      exact_blocks<D, BLK>(ktile, vtile, kh, vh, L, j0, all, grp_on ? all : 0ull, qreg,
                           a.c_log2, m_run, l_run, o, wave, lane);
    }
  }

  // O = N / D: combine the two lane halves of the denominator.
  const float ltot = l_run + __shfl_xor(l_run, 32);
  const float inv = ltot > 0.f ? 1.f / ltot : 0.f;
  if (qrow < n_i) {
    uint16_t* orow = a.out + head + ((size_t)i_g * BLK + qrow) * D;
#pragma unroll
    for (int dt = 0; dt < C::DT; ++dt)
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) {
        const int d0 = 32 * dt + 8 * r4 + 4 * h;
        const bf16 b0 = (bf16)(o[dt][4 * r4 + 0] * inv), b1 = (bf16)(o[dt][4 * r4 + 1] * inv);
        const bf16 b2 = (bf16)(o[dt][4 * r4 + 2] * inv), b3 = (bf16)(o[dt][4 * r4 + 3] * inv);
        uint2 st;
        st.x = (uint32_t)__builtin_bit_cast(uint16_t, b0) |
               ((uint32_t)__builtin_bit_cast(uint16_t, b1) << 16);
        st.y = (uint32_t)__builtin_bit_cast(uint16_t, b2) |
               ((uint32_t)__builtin_bit_cast(uint16_t, b3) << 16);
        *reinterpret_cast<uint2*>(orow + d0) = st;
      }
  }
}

template <bool FUSED>
hipError_t launch_attn(const Shape& s, AttnArgs a, hipStream_t stream) {
  a.L = s.L;
  a.N = (uint32_t)s.N;
  a.pairs = (uint32_t)((s.N + 1) / 2);
  a.per_xcd = (a.pairs + kXcds - 1) / kXcds;
  a.chunk = s.chunk;
  a.scale = s.scale;
  a.c_log2 = s.scale * kLog2e;
  const dim3 grid((uint32_t)(kXcds * a.per_xcd * s.bh));
#define SOLATTN_LAUNCH(DD, BB)                                                               \
  if (s.d == DD && s.block == BB) {                                                          \
    hipLaunchKernelGGL((attn_kernel<DD, BB, FUSED>), grid, dim3(Cfg<DD, BB>::NT), 0, stream, \
                       a);                                                                   \
    return hipGetLastError();                                                                \
  }
  SOLATTN_LAUNCH(128, 128)
  SOLATTN_LAUNCH(128, 64)
  SOLATTN_LAUNCH(64, 128)
  SOLATTN_LAUNCH(64, 64)
#undef SOLATTN_LAUNCH
  return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_fwd(const Shape& s, const void* q, const void* k, const void* v,
                      const float* qbar, const float* kbar, const float* vhat, const float* tau,
                      void* out, uint64_t* sel_mask, int32_t* sel_count, hipStream_t stream) {
  AttnArgs a{};
  a.q = static_cast<const uint16_t*>(q);
  a.k = static_cast<const uint16_t*>(k);
  a.v = static_cast<const uint16_t*>(v);
  a.qbar = qbar;
  a.kbar = kbar;
  a.vhat = vhat;
  a.tau = tau;
  a.out = static_cast<uint16_t*>(out);
  a.sel_mask = sel_mask;
  a.sel_count = sel_count;
  a.exact_only = (s.flags & 1u) ? 1u : 0u;
  return launch_attn<true>(s, a, stream);
}

hipError_t launch_dense(const Shape& s, const void* q, const void* k, const void* v, void* out,
                        hipStream_t stream) {
  AttnArgs a{};
  a.q = static_cast<const uint16_t*>(q);
  a.k = static_cast<const uint16_t*>(k);
  a.v = static_cast<const uint16_t*>(v);
  a.out = static_cast<uint16_t*>(out);
  return launch_attn<false>(s, a, stream);
}

}  // namespace solattn
