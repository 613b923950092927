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
// threshold, selected set and online-softmax state.  Neighbouring blocks
// select nearly the same key blocks, so a key block in either set is loaded
// into LDS once and used by whichever group selected it; the two groups also
// put two waves on every SIMD, so one wave's softmax (VALU) can overlap the
// other's MFMA work.
//
// The nested loop of Algorithm 3.2, pipelined for latency:
//   * outer loop (routing and approximation), run over all chunks first:
//     the chunk's pooled keys Kbar_j and summed values Vhat_j are staged in
//     LDS; every wave computes shat_ij = scale * Qbar_i . Kbar_j in float32
//     for both groups and ballots shat_ij >= tau_i (the same instructions on
//     the same data in every wave, so the masks agree without communication;
//     the page reads these scores off the token-to-block tile as column
//     means, the same number, which a bf16 tile could not resolve inside the
//     tie band); the selected bits go to an on-chip bitmap; the unselected
//     columns of the token-to-block tile scale * Q_i KC^T (MFMA, KC in bf16)
//     update the group's online softmax with weight n_j and value Vhat_j.
//   * inner loops (exact attention), then run back to back over the selected
//     blocks of all chunks in order, so that the next block's K/V are always
//     in flight: K and V are double-buffered in LDS, loaded with direct-to-LDS
//     loads (global_load_lds_dwordx4, 1 KB per wave instruction) into
//     XOR-swizzled tiles, one workgroup barrier per key block.
// Exact and approximate terms share one running max, denominator and
// accumulator; the order in which they enter is immaterial to the result.
//
// MFMA layout (v_mfma_f32_32x32x16_bf16), computed transposed so each lane
// owns one query:
//   S^T = K Q^T      A = K rows from LDS, B = Q^T held in registers;
//                    lane l holds query l%32 and 16 keys per 32x32 tile, so
//                    the softmax row max / sum is lane-local plus one
//                    exchange with lane l^32;
//   O^T += V^T P^T   A = V^T via the LDS transpose read (ds_read_b64_tr_b16)
//                    of row-major V, B = P^T packed to bf16 straight from
//                    the S^T result registers.

#include <math.h>

#include "common.hpp"
#include "launch.hpp"

namespace solattn {
namespace {

typedef short v4i16 __attribute__((ext_vector_type(4)));
typedef short v8i16 __attribute__((ext_vector_type(8)));
#define LDS_PTR(T, p) ((__attribute__((address_space(3))) T*)(p))

// Largest number of blocks per head the fused kernel keeps selection bits for.
constexpr int kMaxBlocks = 8192;

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
  static constexpr int PROW = 4 * D;        // bytes per float32 pooled row
  static constexpr int PSEGS = D / 4;       // 16-byte segments in a pooled row
  static_assert(DMA * WAVES * 1024 == TILE, "tile must split into whole 1 KB loads");
  static_assert(SUB * PROW <= TILE, "a staged sub-chunk must fit one tile buffer");
};

// XOR swizzles of 16-byte segments (rows are written lane-linearly by the
// direct-to-LDS loads, so padding is not available).  K: the A-operand
// reads of 16 consecutive rows hit 16 distinct segments.  V: each transpose
// read covers 8 rows x 64 bytes; rows r..r+3 land in disjoint 64-byte bank
// ranges.  Pooled rows: the 32 routing lanes read 32 distinct segments.
template <int SEGS>
__device__ __forceinline__ int swz_k(int r) { return r % SEGS; }
template <int SEGS>
__device__ __forceinline__ int swz_v(int r) { return (4 * (r % 4)) % SEGS; }
template <int PSEGS>
__device__ __forceinline__ int swz_p(int r) { return r % PSEGS; }

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

// The running max is only raised when a score exceeds it by more than
// 2^kLazyRescale (log2 units); below that, probabilities up to 2^8 simply
// enter the float32 sums and the bf16 P operand and the O^T rescale is
// skipped.  Normalising by the same denominator keeps the result exact.
constexpr float kLazyRescale = 8.f;

template <int DT>
__device__ __forceinline__ void raise_max(float mx, float& m_run, float& l_run, f32x16* o) {
  if (__ballot(mx > m_run + kLazyRescale)) {
    const float m_new = fmaxf(m_run, mx);
    const float alpha = fast_exp2(m_run - m_new);
    l_run *= alpha;
    m_run = m_new;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) o[dt] *= alpha;
  }
}

// Sum of the eight bf16 values of p (two per v_dot2_f32_bf16) added to acc.
__device__ __forceinline__ float sum_bf16x8(bf16x8 p, float acc) {
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
  bf16x2 one;
  one[0] = (bf16)1.f;
  one[1] = (bf16)1.f;
#pragma unroll
  for (int e = 0; e < 8; e += 2) {
    bf16x2 pr;
    pr[0] = p[e];
    pr[1] = p[e + 1];
    acc = __builtin_amdgcn_fdot2_f32_bf16(pr, one, acc, false);
  }
  return acc;
}

// ---------------------------------------------------------------- exact path

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

template <int D, int BLK>
__device__ __forceinline__ void dma_block(char* ktile, char* vtile, const uint16_t* kh,
                                          const uint16_t* vh, uint32_t j, int nkeys, int wave,
                                          int lane) {
  dma_tile<D, BLK, false>(ktile, kh + (size_t)j * BLK * D, nkeys, wave, lane);
  dma_tile<D, BLK, true>(vtile, vh + (size_t)j * BLK * D, nkeys, wave, lane);
}

// One key block of exact attention for this wave's 32 queries: S^T = K Q^T,
// online-softmax update, O^T += V^T P^T.  The exponentials of P V k-step
// kk + 1 are independent of the MFMAs of step kk, so the two overlap.
template <int D, int BLK>
__device__ __forceinline__ void exact_block(const char* ktile, const char* vtile,
                                            const bf16x8* qreg, int nkeys, float c,
                                            float& m_run, float& l_run, f32x16* o, int lane) {
  using C = Cfg<D, BLK>;
  const int h = lane / 32, l32 = lane % 32;
  f32x16 s[C::MT];
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
  }
  if (nkeys < BLK) {
    const int lim = nkeys - 4 * h;  // key 32mt + 8(r/4) + 4h + r%4 is valid iff < nkeys
#pragma unroll
    for (int mt = 0; mt < C::MT; ++mt)
#pragma unroll
      for (int r = 0; r < 16; ++r)
        if (32 * mt + 8 * (r / 4) + (r % 4) >= lim) s[mt][r] = -INFINITY;
  }
  float mx = -INFINITY;
#pragma unroll
  for (int mt = 0; mt < C::MT; ++mt)
#pragma unroll
    for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[mt][r]);
  mx = wave_max_pair(mx);
  raise_max<C::DT>(mx * c, m_run, l_run, o);
  float psum = 0.f;
  const int g = lane / 16, j = lane % 16;
#pragma unroll
  for (int kk = 0; kk < C::PK; ++kk) {
    const int mt = kk / 2, hf = kk % 2;
    float pv[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) pv[e] = fast_exp2(__builtin_fmaf(s[mt][8 * hf + e], c, -m_run));
    const bf16x8 pk = pack_bf16x8(pv);
    psum = sum_bf16x8(pk, psum);
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
      o[dt] = mfma32x32x16(__builtin_bit_cast(bf16x8, both), pk, o[dt]);
    }
  }
  l_run += psum;
}

// Iterates, in increasing order, over the blocks whose bit is set in the
// union of the two groups' bitmaps (wave-uniform state).
struct BlockWalker {
  const uint32_t* b0;
  const uint32_t* b1;
  uint32_t words;  // 32-bit words in each bitmap
  uint32_t w;      // current word
  uint32_t rem;    // bits of word w not yet returned
  __device__ __forceinline__ bool next(uint32_t* j) {
    while (rem == 0) {
      if (++w >= words) return false;
      rem = __builtin_amdgcn_readfirstlane(b0[w] | b1[w]);
    }
    const uint32_t bit = (uint32_t)__builtin_ctz(rem);
    rem &= rem - 1;
    *j = 32 * w + bit;
    return true;
  }
};

// Exact attention over every block of the union bitmap (or all N blocks
// when `bits` is null: the dense kernel), double-buffered.  Group grp takes
// the blocks whose bit is set in its own bitmap.
template <int D, int BLK>
__device__ __forceinline__ void exact_phase(char* k0, char* v0, char* k1, char* v1,
                                            const uint32_t (*bits)[kMaxBlocks / 32],
                                            uint32_t N, int64_t L, const uint16_t* kh,
                                            const uint16_t* vh, bool grp_on, int grp,
                                            const bf16x8* qreg, float c, float& m_run,
                                            float& l_run, f32x16* o, int wave, int lane) {
  auto nkeys_of = [&](uint32_t j) {
    const int64_t rem = L - (int64_t)j * BLK;
    return (int)(rem < BLK ? rem : BLK);
  };
  auto active_for = [&](uint32_t j) {
    if (!grp_on) return false;
    if (bits == nullptr) return true;
    return ((bits[grp][j / 32] >> (j % 32)) & 1u) != 0u;
  };
  // dense: all blocks in order; fused: the union bitmap
  uint32_t dense_next = 0;
  BlockWalker wk{bits ? bits[0] : nullptr, bits ? bits[1] : nullptr, (N + 31) / 32, 0u, 0u};
  if (bits) wk.rem = __builtin_amdgcn_readfirstlane(bits[0][0] | bits[1][0]);
  auto next = [&](uint32_t* j) {
    if (bits) return wk.next(j);
    if (dense_next >= N) return false;
    *j = dense_next++;
    return true;
  };
  uint32_t j;
  if (!next(&j)) return;
  dma_block<D, BLK>(k0, v0, kh, vh, j, nkeys_of(j), wave, lane);
  while (true) {
    // even step: compute from buffer 0, prefetch into buffer 1
    uint32_t jn;
    bool more = next(&jn);
    wait_vm<0>();
    barrier_lds();  // block j is in buffer 0; everyone is done with buffer 1
    if (more) dma_block<D, BLK>(k1, v1, kh, vh, jn, nkeys_of(jn), wave, lane);
    if (active_for(j)) exact_block<D, BLK>(k0, v0, qreg, nkeys_of(j), c, m_run, l_run, o, lane);
    if (!more) break;
    j = jn;
    // odd step: compute from buffer 1, prefetch into buffer 0
    more = next(&jn);
    wait_vm<0>();
    barrier_lds();
    if (more) dma_block<D, BLK>(k0, v0, kh, vh, jn, nkeys_of(jn), wave, lane);
    if (active_for(j)) exact_block<D, BLK>(k1, v1, qreg, nkeys_of(j), c, m_run, l_run, o, lane);
    if (!more) break;
    j = jn;
  }
  barrier_lds();  // buffers free for whoever comes next
}

// ---------------------------------------------------------- routing / approx

// Stage pooled rows [j0, j0 + rows) of Kbar into kst and Vhat into vst
// (float32, swizzled 16-byte segments); the rest of the SUB rows are zero so
// readers need no bounds checks.
template <int D, int BLK>
__device__ __forceinline__ void stage_pooled(char* kst, char* vst, const float* kbar_h,
                                             const float* vhat_h, uint32_t j0, int rows,
                                             int tid) {
  using C = Cfg<D, BLK>;
  constexpr int IT = (C::SUB * C::PSEGS + C::NT - 1) / C::NT;
#pragma unroll
  for (int it = 0; it < IT; ++it) {
    const int idx = tid + it * C::NT;
    const int jj = idx / C::PSEGS, sg = idx % C::PSEGS;
    if (jj < C::SUB) {
      f32x4 kk = {0.f, 0.f, 0.f, 0.f}, vv = {0.f, 0.f, 0.f, 0.f};
      if (jj < rows) {
        const size_t gofs = (size_t)(j0 + jj) * D + sg * 4;
        kk = *reinterpret_cast<const f32x4*>(kbar_h + gofs);
        vv = *reinterpret_cast<const f32x4*>(vhat_h + gofs);
      }
      const int at = jj * C::PROW + (sg ^ swz_p<C::PSEGS>(jj)) * 16;
      *reinterpret_cast<f32x4*>(kst + at) = kk;
      *reinterpret_cast<f32x4*>(vst + at) = vv;
    }
  }
}

template <int D, int BLK>
__device__ __forceinline__ const float* pooled_at(const char* st, int row, int col) {
  using C = Cfg<D, BLK>;
  return reinterpret_cast<const float*>(st + row * C::PROW +
                                        ((col / 4) ^ swz_p<C::PSEGS>(row)) * 16) +
         (col % 4);
}

// Routing of up to 32 staged pooled keys for both query blocks of the pair:
// bit jj of mask g is set iff pooled key jj (< rows) has shat >= tau_g.
template <int D, int BLK>
__device__ __forceinline__ void route_sub(const char* kst, const float (*qbar_s)[D], int rows,
                                          float tau0, float tau1, float scale, int lane,
                                          uint32_t* m0, uint32_t* m1) {
  constexpr int HALF = D / 2;
  const int h = lane / 32, jj = lane % 32;
  float p0 = 0.f, p1 = 0.f;
#pragma unroll
  for (int e = 0; e < HALF; e += 4) {
    const f32x4 kv = *reinterpret_cast<const f32x4*>(pooled_at<D, BLK>(kst, jj, h * HALF + e));
    const f32x4 q0 = *reinterpret_cast<const f32x4*>(&qbar_s[0][h * HALF + e]);
    const f32x4 q1 = *reinterpret_cast<const f32x4*>(&qbar_s[1][h * HALF + e]);
#pragma unroll
    for (int x = 0; x < 4; ++x) {
      p0 = __builtin_fmaf(q0[x], kv[x], p0);
      p1 = __builtin_fmaf(q1[x], kv[x], p1);
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
__device__ __forceinline__ void approx_sub(const char* kst, const char* vst, const bf16x8* qreg,
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
    const f32x4 a0 = *reinterpret_cast<const f32x4*>(pooled_at<D, BLK>(kst, l32, 16 * ks + 8 * h));
    const f32x4 a1 =
        *reinterpret_cast<const f32x4*>(pooled_at<D, BLK>(kst, l32, 16 * ks + 8 * h + 4));
    t = mfma32x32x16(pack_bf16x8(a0, a1), qreg[ks], t);
  }
  float mx = -INFINITY;
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    if (!((unsel >> mfma_row(r, h)) & 1u)) t[r] = -INFINITY;
    mx = fmaxf(mx, t[r]);
  }
  mx = wave_max_pair(mx);
  raise_max<C::DT>(mx * c, m_run, l_run, o);
  float lsum = 0.f;
#pragma unroll
  for (int hf = 0; hf < 2; ++hf) {
    float pv[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) pv[e] = fast_exp2(__builtin_fmaf(t[8 * hf + e], c, -m_run));
    const bf16x8 pk = pack_bf16x8(pv);
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      // weight n_j of the block behind pooled key jbase + row (bf16 P, as the numerator)
      const float w = (jbase + mfma_row(8 * hf + e, h) == N - 1) ? (float)n_last : (float)BLK;
      lsum = __builtin_fmaf(w, (float)pk[e], lsum);
    }
#pragma unroll
    for (int dt = 0; dt < C::DT; ++dt) {
      float vv[8];
#pragma unroll
      for (int e = 0; e < 8; ++e)  // columns outside unsel carry p = 0 against finite values
        vv[e] = *pooled_at<D, BLK>(vst, mfma_row(8 * hf + e, h), 32 * dt + l32);
      o[dt] = mfma32x32x16(pack_bf16x8(vv), pk, o[dt]);
    }
  }
  l_run += lsum;
}

// ------------------------------------------------------------------ kernel

template <int D, int BLK, bool FUSED>
__global__ __launch_bounds__(4 * BLK) void attn_kernel(AttnArgs a) {
  using C = Cfg<D, BLK>;
  __shared__ __attribute__((aligned(1024))) char k0[C::TILE];
  __shared__ __attribute__((aligned(1024))) char v0[C::TILE];
  __shared__ __attribute__((aligned(1024))) char k1[C::TILE];
  __shared__ __attribute__((aligned(1024))) char v1[C::TILE];
  __shared__ uint32_t selbits[FUSED ? 2 : 1][FUSED ? kMaxBlocks / 32 : 1];
  __shared__ __attribute__((aligned(16))) float qbar_s[FUSED ? 2 : 1][D];

  const int tid = threadIdx.x, lane = tid % kWave, wave = tid / kWave;
  const int grp = wave / C::QW;  // which block of the pair
  const int h = lane / 32, l32 = lane % 32;
  uint32_t bh, pair;
  if (!head_striped_item(blockIdx.x, a.pairs, a.per_xcd, &bh, &pair)) return;
  const uint32_t N = a.N;
  const uint32_t i_g = 2 * pair + grp;  // this group's query block
  const bool grp_on = i_g < N;          // block 2p+1 may not exist
  const bool pair1_on = 2 * pair + 1 < N;
  const int64_t L = a.L;
  const int n_i =
      grp_on ? (int)((L - (int64_t)i_g * BLK) < BLK ? (L - (int64_t)i_g * BLK) : BLK) : 0;
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
    // ---- outer loop: routing and approximation over every chunk
    const uint32_t item0 = bh * N + 2 * pair;
    const float tau0 = a.tau[item0];
    const float tau1 = pair1_on ? a.tau[item0 + 1] : INFINITY;
    for (int cc = tid; cc < 2 * D; cc += C::NT) {
      const int gq = cc / D;
      qbar_s[gq][cc % D] =
          (gq == 0 || pair1_on) ? a.qbar[(size_t)(item0 + gq) * D + cc % D] : 0.f;
    }
    const uint32_t words = (N + 31) / 32;
    for (uint32_t w = tid; w < 2 * words; w += C::NT) selbits[w / words][w % words] = 0u;
    const float* kbar_h = a.kbar + (size_t)bh * N * D;
    const float* vhat_h = a.vhat + (size_t)bh * N * D;
    const int n_last = (int)(L - (int64_t)(N - 1) * BLK);
    const uint32_t chunk = (uint32_t)a.chunk;
    for (uint32_t j0 = 0; j0 < N; j0 += chunk) {
      const int cvalid = (int)((N - j0) < chunk ? (N - j0) : chunk);
      for (int sb = 0; sb < cvalid; sb += C::SUB) {
        const int rows = (cvalid - sb) < C::SUB ? (cvalid - sb) : C::SUB;
        const uint32_t jb = j0 + sb;  // pooled key of staged row 0
        __syncthreads();  // previous readers of the staging buffers are done
        stage_pooled<D, BLK>(k1, v1, kbar_h, vhat_h, jb, rows, tid);
        __syncthreads();
        uint32_t s0, s1;
        route_sub<D, BLK>(k1, qbar_s, rows, tau0, tau1, a.scale, lane, &s0, &s1);
        if (!pair1_on) s1 = 0u;
        if (tid == 0) {  // append to the bitmaps (single writer, in order)
          const uint32_t wd = jb / 32, sh = jb % 32;
          selbits[0][wd] |= s0 << sh;
          selbits[1][wd] |= s1 << sh;
          if (sh != 0 && sh + (uint32_t)rows > 32) {
            selbits[0][wd + 1] |= s0 >> (32 - sh);
            selbits[1][wd + 1] |= s1 >> (32 - sh);
          }
        }
        const uint32_t mine = grp == 0 ? s0 : s1;
        const uint32_t valid = rows >= 32 ? 0xffffffffu : ((1u << rows) - 1u);
        const uint32_t unsel = valid & ~mine;
        if (grp_on && !a.exact_only && unsel)
          approx_sub<D, BLK>(k1, v1, qreg, unsel, jb, N, n_last, a.c_log2, m_run, l_run, o,
                             lane);
      }
    }
    __syncthreads();  // bitmaps complete; staging buffers free

    // debug outputs: the group's first wave writes its row of the bitmap
    if (grp_on && (wave % C::QW) == 0) {
      const uint32_t W64 = (N + 63) / 64;
      int count = 0;
      for (uint32_t w = lane; w < W64; w += kWave) {
        const uint32_t lo = selbits[grp][2 * w];
        const uint32_t hi = (2 * w + 1 < words) ? selbits[grp][2 * w + 1] : 0u;
        if (a.sel_mask)
          a.sel_mask[(size_t)(bh * N + i_g) * W64 + w] = ((uint64_t)hi << 32) | lo;
        count += __builtin_popcount(lo) + __builtin_popcount(hi);
      }
      if (a.sel_count) {
#pragma unroll
        for (int off = 32; off >= 1; off >>= 1) count += __shfl_xor(count, off);
        if (lane == 0) a.sel_count[bh * N + i_g] = count;
      }
    }

    // ---- inner loops: exact attention over the selected blocks, in order
    exact_phase<D, BLK>(k0, v0, k1, v1, selbits, N, L, kh, vh, grp_on, grp, qreg, a.c_log2,
                        m_run, l_run, o, wave, lane);
  } else {
    exact_phase<D, BLK>(k0, v0, k1, v1, nullptr, N, L, kh, vh, grp_on, grp, qreg, a.c_log2,
                        m_run, l_run, o, wave, lane);
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

int64_t fused_max_blocks() { return kMaxBlocks; }

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
