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
// The nested loop of Algorithm 3.2, reordered for latency (the selected set
// is the union of the chunks' sets, so the order changes nothing):
//   * routing and approximation, one pass over the pooled keys, 64 at a
//     time (32 with 64-token blocks): the float32 rows of Kbar and Vhat are loaded once (whole
//     128-byte lines per instruction, the next 64 rows in flight meanwhile);
//     the routing scores shat_ij = scale * Qbar_i . Kbar_j are formed from
//     them in float32 for both query blocks and tested against the
//     thresholds, and the decisions go to on-chip bitmaps (the page reads
//     these scores off the token-to-block tile as column means: the same
//     numbers, which a bf16 tile could not resolve inside the tie band); the
//     same registers are stored to LDS as bf16 tiles (Kbar as high and low
//     parts in the K layout, Vhat in the V layout), and the token-to-block
//     tile scale * Q_i KC^T (MFMA, high plus low part) gives the logits of
//     the unselected columns, which enter the group's online softmax with
//     weight n_j and value Vhat_j;
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

#include <mutex>

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
  static constexpr int SEGS = D / 8;        // 16-byte segments in a bf16 row
  static constexpr int ROW = 2 * D;         // bytes per bf16 row
  static constexpr int TILE = BLK * ROW;    // bytes per K or V tile
  static constexpr int DMA = TILE / 1024 / WAVES;  // 1 KB loads per wave per tile
  static constexpr int ROWS_1K = 1024 / ROW;       // tile rows per 1 KB load
  // pooled rows staged at a time: a K tile holds two sub-chunks (the high
  // bf16 parts of one, the low parts in its second half)
  static constexpr int SUB = BLK >= 128 ? 64 : 32;
  // One LDS array: K tiles first so that every K read address fits the
  // 16-bit instruction offset, then V tiles, then the routing state.
  static constexpr int K0 = 0, K1 = TILE, V0 = 2 * TILE, V1 = 3 * TILE;
  static constexpr int BITS = 4 * TILE;                      // 2 x kMaxBlocks bits
  static constexpr int QBAR = BITS + 2 * (kMaxBlocks / 8);  // 2 x D floats
  // Low bf16 parts of the staged pooled keys (the token-to-block tile runs on
  // Kbar = high + low): the unused second half of each K tile when a tile
  // holds two sub-chunks' rows, else a region of their own.
  static constexpr bool LO_IN_K = BLK >= 2 * SUB;
  static constexpr int LOX = QBAR + 2 * D * 4;
  static constexpr int KLO0 = LO_IN_K ? K0 + SUB * ROW : LOX;
  static constexpr int KLO1 = LO_IN_K ? K1 + SUB * ROW : LOX + SUB * ROW;
  static constexpr int SMEM_FUSED = LO_IN_K ? LOX : LOX + 2 * SUB * ROW;
  static constexpr int SMEM_DENSE = 4 * TILE;
  static_assert(DMA * WAVES * 1024 == TILE, "tile must split into whole 1 KB loads");
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
  const uint64_t* sel_in;  // given selections (masked mode) or null (threshold routing)
  float* out_f32;          // if set: O in float32 here instead of bf16 in out
  float* lse2;             // if set: per row, log2 of the softmax denominator in logit units
                           // (m + log2 l, the scale of the 2^(c s - m) weights)
  uint32_t* queue;   // fused kernel: kXcds work-queue counters, kQueueStride apart
  int64_t L;
  uint32_t N;
  uint32_t pairs;    // ceil(N / 2)
  uint32_t per_xcd;  // pairs per XCD slab (dense kernel): ceil(pairs / 8)
  uint32_t queue_len;  // entries per work queue (fused kernel): ceil(runs / 8) * run
  uint32_t run;        // pairs per run of the work queues
  uint32_t runs_per_head;  // ceil(pairs / run)
  uint32_t runs;       // B * H * runs_per_head
  float scale;
  float c_log2;      // scale * log2(e): logits enter exp2 in this unit
  uint32_t exact_only;
};

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }


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

// Direct-to-LDS loads of K and V tiles (global_load_lds_dwordx4: each lane
// fetches 16 bytes from global memory and the wave writes them to 1 KB of
// LDS at M0 + 16 * lane).  The loads are issued from inline assembly so the
// compiler does not track them: its waitcnt pass cannot tell the buffer being
// filled from the one being read and would otherwise wait for every
// outstanding prefetch before the first LDS read of a block.  The caller
// waits explicitly (s_waitcnt vmcnt) before a workgroup barrier, and no other
// vector-memory load may be outstanding while a prefetch is in flight.
template <int D, int BLK>
struct TileDma {
  using C = Cfg<D, BLK>;
  uint32_t koff[C::DMA];  // byte offset in a full tile of this lane's 16 bytes (K swizzle)
  uint32_t voff[C::DMA];  // same with the V swizzle

  __device__ __forceinline__ static int row_of(int wave, int lane, int c) {
    return (wave + c * C::WAVES) * C::ROWS_1K + lane / C::SEGS;
  }
  __device__ __forceinline__ static uint32_t offset(int row, int lane, bool is_v) {
    const int seg = (lane % C::SEGS) ^ (is_v ? swz_v<C::SEGS>(row) : swz_k<C::SEGS>(row));
    return (uint32_t)((row * D + seg * 8) * 2);
  }
  __device__ __forceinline__ void init(int wave, int lane) {
#pragma unroll
    for (int c = 0; c < C::DMA; ++c) {
      const int row = row_of(wave, lane, c);
      koff[c] = offset(row, lane, false);
      voff[c] = offset(row, lane, true);
    }
  }
  __device__ __forceinline__ static void load(uint32_t voffset, const uint16_t* sbase,
                                              uint32_t lds) {
    lds_dma_16b(voffset, sbase, lds);
  }
  // K and V of key block j (nkeys valid rows) into the tiles at LDS byte
  // addresses lds_k / lds_v.  Rows >= nkeys re-read row nkeys - 1 (finite
  // data that the softmax masks).
  __device__ __forceinline__ void block(uint32_t lds_k, uint32_t lds_v, const uint16_t* kh,
                                        const uint16_t* vh, uint32_t j, int nkeys, int wave,
                                        int lane) const {
    const uint16_t* kb = kh + (size_t)j * BLK * D;
    const uint16_t* vb = vh + (size_t)j * BLK * D;
    if (nkeys == BLK) {
#pragma unroll
      for (int c = 0; c < C::DMA; ++c)
        load(koff[c], kb, lds_k + (uint32_t)(wave + c * C::WAVES) * 1024u);
#pragma unroll
      for (int c = 0; c < C::DMA; ++c)
        load(voff[c], vb, lds_v + (uint32_t)(wave + c * C::WAVES) * 1024u);
    } else {
#pragma unroll
      for (int c = 0; c < C::DMA; ++c) {
        const int row = row_of(wave, lane, c);
        const int back = row < nkeys ? 0 : row - (nkeys - 1);
        load(koff[c] - (uint32_t)(back * D * 2), kb, lds_k + (uint32_t)(wave + c * C::WAVES) * 1024u);
      }
#pragma unroll
      for (int c = 0; c < C::DMA; ++c) {
        const int row = row_of(wave, lane, c);
        const int back = row < nkeys ? 0 : row - (nkeys - 1);
        load(voff[c] - (uint32_t)(back * D * 2), vb, lds_v + (uint32_t)(wave + c * C::WAVES) * 1024u);
      }
    }
  }
};


// Per-lane byte offsets, within a tile, of this lane's MFMA operand reads.
// They do not depend on the 32-key tile mt or the P V k-step kk (the
// swizzles repeat with period 16 rows for K and 4 rows for V), which enter
// as compile-time offsets.
template <int D, int BLK>
struct LaneOffsets {
  using C = Cfg<D, BLK>;
  uint32_t k[C::KS];  // K row 32 mt + lane % 32, d = 16 ks + 8 (lane / 32) .. + 7
  uint32_t v[C::DT];  // transpose-read address for d tile dt (rows 16 kk + ...) in V buffer 0
  __device__ __forceinline__ void init(int lane) {
    const int h = lane / 32, l32 = lane % 32;
#pragma unroll
    for (int ks = 0; ks < C::KS; ++ks)
      k[ks] = (uint32_t)(l32 * C::ROW + ((2 * ks + h) ^ swz_k<C::SEGS>(l32)) * 16);
    const int g = lane / 16, j = lane % 16;
    const int r0 = 4 * (g / 2) + j / 4;
#pragma unroll
    for (int dt = 0; dt < C::DT; ++dt) {
      const int col = 32 * dt + 16 * (g % 2) + 4 * (j % 4);
      v[dt] = (uint32_t)(C::V0 + r0 * C::ROW + ((col / 8) ^ swz_v<C::SEGS>(r0)) * 16 +
                         (col % 8) * 2);
    }
  }
};

// S^T tile mt (keys 32 mt .. 32 mt + 31 of the block) = K Q^T for this
// wave's 32 queries: lane l holds query l % 32 against keys
// 32 mt + mfma_row(r, l / 32).
template <int D, int BLK>
__device__ __forceinline__ f32x16 score_tile(const char* ktile, const LaneOffsets<D, BLK>& off,
                                             const bf16x8* qreg, int mt) {
  using C = Cfg<D, BLK>;
  f32x16 acc;
#pragma unroll
  for (int r = 0; r < 16; ++r) acc[r] = 0.f;
#pragma unroll
  for (int ks = 0; ks < C::KS; ++ks) {
    const bf16x8 ka =
        *reinterpret_cast<const bf16x8*>(ktile + 32 * mt * C::ROW + off.k[ks]);
    acc = mfma32x32x16(ka, qreg[ks], acc);
  }
  return acc;
}

// acc + the S^T tile mt of a second K-layout tile (the low parts of the
// staged pooled keys).
template <int D, int BLK>
__device__ __forceinline__ f32x16 score_tile_add(const char* ktile,
                                                 const LaneOffsets<D, BLK>& off,
                                                 const bf16x8* qreg, int mt, f32x16 acc) {
  using C = Cfg<D, BLK>;
#pragma unroll
  for (int ks = 0; ks < C::KS; ++ks) {
    const bf16x8 ka =
        *reinterpret_cast<const bf16x8*>(ktile + 32 * mt * C::ROW + off.k[ks]);
    acc = mfma32x32x16(ka, qreg[ks], acc);
  }
  return acc;
}

// V^T operand fragments of P V k-step kk (keys 16 kk + {4h..4h+3,
// 8+4h..8+4h+3}, the keys whose probabilities a tile's pk holds), one per
// 32-wide d tile.  vtile points V1 - V0 bytes past the start of V buffer 0
// for buffer 1 (the lane offsets include V0), so every address below is a
// lane offset plus a compile-time constant.
template <int D, int BLK>
struct VFrag {
  using C = Cfg<D, BLK>;
  bf16x8 a[C::DT];
  __device__ __forceinline__ void fetch(const char* vtile, const LaneOffsets<D, BLK>& off,
                                        int kk) {
#pragma unroll
    for (int dt = 0; dt < C::DT; ++dt) {
      const char* p0 = vtile + 16 * kk * C::ROW + off.v[dt];
      // keys 16kk + 4h + {0..3} and 16kk + 8 + 4h + {0..3} for d = 32dt + lane%32
      const v4i16 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(LDS_PTR(v4i16, p0));
      const v4i16 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(LDS_PTR(v4i16, p0 + 8 * C::ROW));
      a[dt] = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
    }
  }
  // O^T += V^T P^T for this k-step
  __device__ __forceinline__ void apply(bf16x8 pk, f32x16* o) const {
#pragma unroll
    for (int dt = 0; dt < C::DT; ++dt) o[dt] = mfma32x32x16(a[dt], pk, o[dt]);
  }
};

template <int D, int BLK>
__device__ __forceinline__ void pv_step(const char* vtile, const LaneOffsets<D, BLK>& off,
                                        bf16x8 pk, int kk, f32x16* o) {
  VFrag<D, BLK> f;
  f.fetch(vtile, off, kk);
  f.apply(pk, o);
}

// Probabilities of one S^T tile against the running max: p = 2^(c s - m),
// packed to bf16 for the P V product; returns the row-partial sum of the
// packed values (what the numerator sees).
__device__ __forceinline__ float tile_probs(const f32x16& s, float c, float m, bf16x8* pk0,
                                            bf16x8* pk1) {
  float p[16];
#pragma unroll
  for (int e = 0; e < 16; ++e) p[e] = fast_exp2(__builtin_fmaf(s[e], c, -m));
  *pk0 = pack_bf16x8(p);
  *pk1 = pack_bf16x8(p + 8);
  return sum_bf16x8(*pk1, sum_bf16x8(*pk0, 0.f));
}

// A tile's probabilities may exceed 1 by up to this factor before the
// running max is raised (they stay far from float32 overflow; bf16 and
// float32 keep their relative precision at any magnitude).
constexpr float kMaxTileSum = 0x1p40f;

// One key block of exact attention for this wave's 32 queries, streamed in
// 32-key tiles: the scores of tile mt + 1 (MFMA) are computed while tile
// mt's probabilities (VALU) are formed, and tile mt then enters O^T.  The
// running max is not recomputed per tile: the probabilities are formed
// against the current max and only when a tile's sum leaves [0, 2^40] (or
// is not finite, as on the very first tile) is the max raised to the tile's
// maximum, the state rescaled and the tile redone.  Normalising by the same
// denominator keeps the result exact whatever reference max is used.
// TAIL: the block has nkeys < BLK valid keys (the last block of a head);
// a separate instantiation keeps the masking out of the common path's basic
// blocks so the scheduler can interleave tile mt + 1's MFMAs with tile mt's
// exponentials.
template <int D, int BLK, bool TAIL>
__device__ __forceinline__ void exact_block(const char* ktile, const char* vtile,
                                            const LaneOffsets<D, BLK>& off, const bf16x8* qreg,
                                            int nkeys, float c, float& m_run, float& l_run,
                                            f32x16* o, int lane) {
  using C = Cfg<D, BLK>;
  const int h = lane / 32;
  f32x16 s = score_tile<D, BLK>(ktile, off, qreg, 0);
#pragma unroll
  for (int mt = 0; mt < C::MT; ++mt) {
    f32x16 s_next;
    if (mt + 1 < C::MT) s_next = score_tile<D, BLK>(ktile, off, qreg, mt + 1);
    // this tile's V operands, fetched ahead so the softmax below covers the
    // LDS latency
    VFrag<D, BLK> va, vb;
    va.fetch(vtile, off, 2 * mt);
    vb.fetch(vtile, off, 2 * mt + 1);
    if (TAIL) {
      const int lim = nkeys - 32 * mt - 4 * h;  // key 32mt + 8(r/4) + 4h + r%4 valid iff < nkeys
#pragma unroll
      for (int r = 0; r < 16; ++r)
        if (8 * (r / 4) + (r % 4) >= lim) s[r] = -INFINITY;
    }
    bf16x8 pk0, pk1;
    float ps = tile_probs(s, c, m_run, &pk0, &pk1);
    if (__builtin_expect(__ballot(!(ps <= kMaxTileSum)) != 0, 0)) {
      float mx = -INFINITY;
#pragma unroll
      for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[r]);
      mx = wave_max_pair(mx) * c;
      float m_new = fmaxf(m_run, mx);
      if (m_new == -INFINITY) m_new = 0.f;  // nothing valid yet: any finite reference
      const float alpha = fast_exp2(m_run - m_new);
      l_run *= alpha;
#pragma unroll
      for (int dt = 0; dt < C::DT; ++dt) o[dt] *= alpha;
      m_run = m_new;
      ps = tile_probs(s, c, m_run, &pk0, &pk1);
    }
    l_run += ps;
    va.apply(pk0, o);
    vb.apply(pk1, o);
    if (mt + 1 < C::MT) s = s_next;
  }
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
// when `bits` is null: the dense kernel), double-buffered in LDS: block j is
// computed from one buffer while block j+1 streams into the other, one
// workgroup barrier per block.  Group grp takes the blocks whose bit is set
// in its own bitmap.  Only the last block of a head can be partial; it is
// always the last one visited and is computed after the loop, so the loop
// body carries no masking.
template <int D, int BLK>
__device__ __forceinline__ void exact_phase(char* smem, const uint32_t (*bits)[kMaxBlocks / 32],
                                            uint32_t N, int64_t L, const uint16_t* kh,
                                            const uint16_t* vh, bool grp_on, int grp,
                                            const bf16x8* qreg, float c, float& m_run,
                                            float& l_run, f32x16* o, int wave, int lane) {
  using C = Cfg<D, BLK>;
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
  settle_vm();
  LaneOffsets<D, BLK> off;
  off.init(lane);
  TileDma<D, BLK> dma;
  dma.init(wave, lane);
  const uint32_t base = lds_addr(smem);
  const uint32_t lk0 = base + C::K0, lv0 = base + C::V0;
  const uint32_t lk1 = base + C::K1, lv1 = base + C::V1;
  uint32_t j;
  if (!next(&j)) return;
  dma.block(lk0, lv0, kh, vh, j, nkeys_of(j), wave, lane);
  bool tail = false;
  int tail_buf = 0;
  while (true) {
    // even step: compute from buffer 0, prefetch into buffer 1
    uint32_t jn;
    bool more = next(&jn);
    wait_vm<0>();
    barrier_lds();  // block j is in buffer 0; everyone is done with buffer 1
    if (more) dma.block(lk1, lv1, kh, vh, jn, nkeys_of(jn), wave, lane);
    if (nkeys_of(j) < BLK) { tail = true; tail_buf = 0; break; }
    if (active_for(j))
      exact_block<D, BLK, false>(smem + C::K0, smem, off, qreg, BLK, c, m_run, l_run, o, lane);
    if (!more) break;
    j = jn;
    // odd step: compute from buffer 1, prefetch into buffer 0
    more = next(&jn);
    wait_vm<0>();
    barrier_lds();
    if (more) dma.block(lk0, lv0, kh, vh, jn, nkeys_of(jn), wave, lane);
    if (nkeys_of(j) < BLK) { tail = true; tail_buf = 1; break; }
    if (active_for(j))
      exact_block<D, BLK, false>(smem + C::K1, smem + (C::V1 - C::V0), off, qreg, BLK, c, m_run,
                                 l_run, o, lane);
    if (!more) break;
    j = jn;
  }
  if (tail && active_for(j)) {
    const int kb = tail_buf ? C::K1 : C::K0, vb = tail_buf ? C::V1 - C::V0 : 0;
    exact_block<D, BLK, true>(smem + kb, smem + vb, off, qreg, nkeys_of(j), c, m_run, l_run, o,
                              lane);
  }
  barrier_lds();  // buffers free for whoever comes next
}

// ---------------------------------------------------------- routing / approx

// x from lane l's partner under a DPP lane permutation within rows of 16 lanes.
template <int CTRL>
__device__ __forceinline__ float dpp_move(float x) {
  return __builtin_bit_cast(
      float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x), CTRL, 0xf, 0xf, false));
}
constexpr int kDppQuadXor1 = 0xB1;     // quad_perm [1, 0, 3, 2]: lane i <-> i ^ 1
constexpr int kDppQuadXor2 = 0x4E;     // quad_perm [2, 3, 0, 1]: lane i <-> i ^ 2
constexpr int kDppHalfMirror = 0x141;  // row_half_mirror: lane i <-> 7 - i within 8 lanes

// One thread's share of a sub-chunk of SUB pooled rows (Kbar and Vhat,
// float32 in global memory), held in registers between its load and its use:
// TPR consecutive threads share a row, thread q of them holding the float4
// pieces q, q + TPR, q + 2 TPR, ... of it (so each load instruction reads
// whole 128-byte lines).  From these registers come
//   * the routing decisions of the staged rows for both query blocks, and
//   * the bf16 copies in the K-tile layout (so score_tile reads them as
//     32-key tiles) and in the V-tile layout (so pv_step reads them as 16-key
//     k-steps).
// Rows past the head's last block are 0.
template <int D, int BLK>
struct PooledStage {
  using C = Cfg<D, BLK>;
  static constexpr int E = D * C::SUB / C::NT;  // elements of one row per thread
  static constexpr int F4 = E / 4;              // float4 pieces per thread per array
  static constexpr int TPR = D / E;             // threads per row
  static constexpr int RPW = kWave / TPR;       // rows per wave
  static_assert(TPR == 4 || TPR == 8, "routing reduction covers 4 or 8 lanes");
  static_assert(F4 * 4 == E && TPR * C::SUB == C::NT, "sub-chunk must split evenly");
  f32x4 k[F4], v[F4];
  __device__ __forceinline__ void load(const float* kbar_h, const float* vhat_h, uint32_t jb,
                                       uint32_t N, int tid) {
    const int row = tid / TPR, q = tid % TPR;
    typedef const __attribute__((address_space(1))) f32x4 gf32x4;
    if (jb + C::SUB <= N) {
      // every staged row exists (all sub-chunks but possibly the last)
#pragma unroll
      for (int c = 0; c < F4; ++c) {
        const size_t g = (size_t)(jb + row) * D + 4 * (q + TPR * c);
        k[c] = *(gf32x4*)(kbar_h + g);
        v[c] = *(gf32x4*)(vhat_h + g);
      }
      return;
    }
#pragma unroll
    for (int c = 0; c < F4; ++c) {
      f32x4 kk = {0.f, 0.f, 0.f, 0.f}, vv = {0.f, 0.f, 0.f, 0.f};
      if (jb + row < N) {
        const size_t g = (size_t)(jb + row) * D + 4 * (q + TPR * c);
        kk = *(gf32x4*)(kbar_h + g);
        vv = *(gf32x4*)(vhat_h + g);
      }
      k[c] = kk;
      v[c] = vv;
    }
  }
  // Routing (Eq. 4) of the staged rows jb .. jb + SUB - 1: row j is selected
  // for group g iff scale * Qbar_g . Kbar_j >= tau_g, with the dot product in
  // float32 (each thread's pieces, then summed over the row's TPR lanes).
  // The wave's RPW rows give RPW bits per group, written to the groups'
  // bitmaps (bits viewed as bytes; sub-chunk sb = bytes 8 sb .. 8 sb + 7).
  __device__ __forceinline__ void route(uint8_t* bits0, uint8_t* bits1, const float (*qbar_s)[D],
                                        float tau0, float tau1, float scale, uint32_t jb,
                                        uint32_t N, int tid, int lane, int wave) const {
    const int q = tid % TPR;
    float d0 = 0.f, d1 = 0.f;
#pragma unroll
    for (int c = 0; c < F4; ++c) {
      const f32x4 a0 = *reinterpret_cast<const f32x4*>(&qbar_s[0][4 * (q + TPR * c)]);
      const f32x4 a1 = *reinterpret_cast<const f32x4*>(&qbar_s[1][4 * (q + TPR * c)]);
#pragma unroll
      for (int x = 0; x < 4; ++x) {
        d0 = __builtin_fmaf(a0[x], k[c][x], d0);
        d1 = __builtin_fmaf(a1[x], k[c][x], d1);
      }
    }
    // Sum over the row's lanes: the first exchange pairs each lane of the
    // lower half with one of the upper half; the lower half keeps group 0's
    // partial sums and the upper half group 1's, so one exchange serves both.
    const bool upper = (lane & (TPR / 2)) != 0;
    const float send = upper ? d0 : d1;
    float t = upper ? d1 : d0;
    t += (TPR == 8) ? dpp_move<kDppHalfMirror>(send) : dpp_move<kDppQuadXor2>(send);
    if (TPR == 8) t += dpp_move<kDppQuadXor2>(t);
    t += dpp_move<kDppQuadXor1>(t);
    const uint32_t j = jb + (uint32_t)(tid / TPR);
    const uint64_t b = __ballot(j < N && scale * t >= (upper ? tau1 : tau0));
    // row rr of the wave: group 0 in lane TPR rr, group 1 in lane TPR rr + TPR / 2
    uint32_t s0 = 0u, s1 = 0u;
#pragma unroll
    for (int rr = 0; rr < RPW; ++rr) {
      s0 |= (uint32_t)((b >> (TPR * rr)) & 1u) << rr;
      s1 |= (uint32_t)((b >> (TPR * rr + TPR / 2)) & 1u) << rr;
    }
    if (lane == 0) {
      const uint32_t byte = (jb / 8) + (uint32_t)wave * (RPW / 8);
      if (RPW == 8) {
        bits0[byte] = (uint8_t)s0;
        bits1[byte] = (uint8_t)s1;
      } else {
        *reinterpret_cast<uint16_t*>(bits0 + byte) = (uint16_t)s0;
        *reinterpret_cast<uint16_t*>(bits1 + byte) = (uint16_t)s1;
      }
    }
  }
  // Kbar as bf16 high part (kt) and low part x - high (klo), both in the K
  // layout; Vhat as bf16 in the V layout.
  __device__ __forceinline__ void store(char* kt, char* klo, char* vt, int tid) const {
    const int row = tid / TPR, q = tid % TPR;
#pragma unroll
    for (int c = 0; c < F4; ++c) {
      const int d = 4 * (q + TPR * c);
      const int byte = (d % 8) * 2;
      typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
      typedef float f32x2 __attribute__((ext_vector_type(2)));
      typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
      // two floats to one packed pair (RNE), one conversion instruction
      auto pack2 = [](float a, float b) {
        return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2){a, b}, bf16x2));
      };
      auto pack4 = [&](f32x4 x) {
        u32x2 r;
        r[0] = pack2(x[0], x[1]);
        r[1] = pack2(x[2], x[3]);
        return r;
      };
      // high parts, and the low parts x - high from the packed high bits
      const u32x2 hi = pack4(k[c]);
      f32x4 low;
#pragma unroll
      for (int e = 0; e < 2; ++e) {
        low[2 * e] = k[c][2 * e] - __uint_as_float(hi[e] << 16);
        low[2 * e + 1] = k[c][2 * e + 1] - __uint_as_float(hi[e] & 0xFFFF0000u);
      }
      const int koff = row * C::ROW + ((d / 8) ^ swz_k<C::SEGS>(row)) * 16 + byte;
      *reinterpret_cast<u32x2*>(kt + koff) = hi;
      *reinterpret_cast<u32x2*>(klo + koff) = pack4(low);
      *reinterpret_cast<u32x2*>(vt + row * C::ROW + ((d / 8) ^ swz_v<C::SEGS>(row)) * 16 + byte) =
          pack4(v[c]);
    }
  }
};

// Zeroth-order terms (Eqs. 9-10) of staged rows 32 half .. 32 half + 31
// whose bit is set in unsel, for this wave's 32 queries: logits
// scale * q_r . Kbar_j from the token-to-block tile (Eq. 11; MFMA on Kbar
// split into bf16 high and low parts, so that the logits keep about 16
// significant bits: a single bf16 Kbar would move a logit of size |a| by
// about |a| 2^-9, which matters where large approximate logits dominate a
// row), denominator weight n_j, numerator Vhat_j.  jb = pooled key of the
// first of those rows.
template <int D, int BLK>
__device__ __forceinline__ void approx_sub(const char* kt, const char* klo, const char* vt,
                                           const LaneOffsets<D, BLK>& off, const bf16x8* qreg,
                                           int half, uint32_t unsel, uint32_t jb, uint32_t N,
                                           int n_last, float c, float& m_run, float& l_run,
                                           f32x16* o, int lane) {
  using C = Cfg<D, BLK>;
  const int h = lane / 32;
  f32x16 t = score_tile_add<D, BLK>(klo, off, qreg, half, score_tile<D, BLK>(kt, off, qreg, half));
  // register r of lane l holds staged row 8 (r / 4) + 4 (l / 32) + r % 4:
  // its unselected bit, for both halves of the wave, as a wave-uniform lane
  // mask (scalar work), applied with one select per register
  float mx = -INFINITY;
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    const int pos = 8 * (r / 4) + r % 4;
    const uint32_t lo = 0u - ((unsel >> pos) & 1u), hi = 0u - ((unsel >> (pos + 4)) & 1u);
    if (!__builtin_amdgcn_inverse_ballot_w64(((uint64_t)hi << 32) | lo)) t[r] = -INFINITY;
    mx = fmaxf(mx, t[r]);
  }
  mx = wave_max_pair(mx);
  raise_max<C::DT>(mx * c, m_run, l_run, o);
  bf16x8 pk0, pk1;
  tile_probs(t, c, m_run, &pk0, &pk1);
  // denominator weights n_j (on the bf16 P, as the numerator sees it): BLK
  // for every pooled key but the head's last, which weighs n_last
  float lsum = (float)BLK * sum_bf16x8(pk1, sum_bf16x8(pk0, 0.f));
  const int rel = (int)(N - 1 - jb) - 4 * h;  // the last key's row, in this lane's numbering
  if (n_last != BLK && N - 1 - jb < 32u) {
#pragma unroll
    for (int r = 0; r < 16; ++r)
      if (rel == 8 * (r / 4) + r % 4)
        lsum -= (float)(BLK - n_last) * (float)(r < 8 ? pk0[r] : pk1[r - 8]);
  }
  pv_step<D, BLK>(vt, off, pk0, 2 * half, o);
  pv_step<D, BLK>(vt, off, pk1, 2 * half + 1, o);
  l_run += lsum;
}

// The outer loop over the pooled keys, SUB at a time (64; 32 with 64-token
// blocks, so that a K tile still holds a sub-chunk's high and low parts), for both query
// blocks of the pair.  Per sub-chunk:
//   * routing (Eq. 4 with the chunk-wise streaming test, Eqs. 6-7):
//     shat_gj = scale * Qbar_g . Kbar_j >= tau_g in float32, with the dot
//     products formed from the same coalesced float32 loads that feed the
//     staging; the selected bits of the sub-chunk go to the group's on-chip
//     bitmap (the page reads these scores off the token-to-block tile as
//     column means: the same numbers, which a bf16 tile could not resolve
//     inside the tie band);
//   * approximation: the unselected columns of the token-to-block tile enter
//     the group's online softmax with weight n_j and value Vhat_j (skipped in
//     exact-only mode).
// The next sub-chunk's rows are loaded into registers while the current one
// is used; staging buffers alternate between the two K / V tile buffers,
// which are free until the exact phase starts, so each sub-chunk costs one
// workgroup barrier.  On return both groups' bitmaps are complete and the
// tile buffers are free.  With route false the bitmaps are given (filled
// before the call) and only the approximation runs.
template <int D, int BLK>
__device__ __forceinline__ void route_approx_phase(
    char* smem, uint32_t (*bits)[kMaxBlocks / 32], const float (*qbar_s)[D], const float* kbar_h,
    const float* vhat_h, uint32_t N, int n_last, float tau0, float tau1, float scale,
    bool route, bool approx, bool grp_on, int grp, const bf16x8* qreg, float c, float& m_run,
    float& l_run, f32x16* o, int tid, int wave, int lane) {
  using C = Cfg<D, BLK>;
  static_assert((C::SUB == 64 || C::SUB == 32) && 2 * C::SUB <= BLK,
                "a staged sub-chunk is one or two 32-bit words per group");
  constexpr int HALVES = C::SUB / 32;
  using Stage = PooledStage<D, BLK>;
  const uint32_t nsub = (N + C::SUB - 1) / C::SUB;
  uint8_t* const bits0 = reinterpret_cast<uint8_t*>(bits[0]);
  uint8_t* const bits1 = reinterpret_cast<uint8_t*>(bits[1]);
  LaneOffsets<D, BLK> off;
  off.init(lane);
  Stage st;
  st.load(kbar_h, vhat_h, 0, N, tid);
  int buf = 0;
  for (uint32_t sb = 0; sb < nsub; ++sb) {
    char* kt = smem + (buf ? C::K1 : C::K0);
    char* klo = smem + (buf ? C::KLO1 : C::KLO0);
    char* vt = smem + (buf ? C::V1 : C::V0);
    if (route) st.route(bits0, bits1, qbar_s, tau0, tau1, scale, sb * C::SUB, N, tid, lane, wave);
    st.store(kt, klo, vt, tid);
    if (sb + 1 < nsub) st.load(kbar_h, vhat_h, (sb + 1) * C::SUB, N, tid);
    __syncthreads();  // staged rows and their bits visible; the other buffer's readers are done
    if (approx && grp_on) {
#pragma unroll
      for (int half = 0; half < HALVES; ++half) {
        const uint32_t base = sb * C::SUB + 32 * half;
        const uint32_t rem = base < N ? N - base : 0u;
        const uint32_t valid = rem >= 32u ? ~0u : ((1u << rem) - 1u);
        const uint32_t u =
            valid & ~__builtin_amdgcn_readfirstlane(bits[grp][sb * HALVES + half]);
        if (u)
          approx_sub<D, BLK>(kt, klo, vt - C::V0, off, qreg, half, u, base, N, n_last, c, m_run,
                             l_run, o, lane);
      }
    }
    buf ^= 1;
  }
  __syncthreads();  // bitmaps complete; staging buffers free
}

// ------------------------------------------------------------------ kernel

// ------------------------------------------------------------- work queue

// Work items of the fused kernel are pairs of query blocks.  They are cut
// into runs of `run` consecutive pairs of one head (twice the workgroups an
// XCD holds, or the whole head if it has fewer pairs), and the runs, head
// after head, are dealt round-robin to kXcds queues (run g to queue g mod 8),
// so a queue's items are neighbouring query blocks of one head at a time and
// the XCDs work on the same one or two heads at any moment.  A persistent
// workgroup of XCD x (workgroup id mod 8, the order in which the dispatcher
// deals workgroups to XCDs) takes items from queue x with an atomic counter,
// in order, and once that queue is empty from the others in turn.
// Query-dependent budgets make items unequal; a workgroup that finishes early
// takes the next item at once, and no CU waits for a workgroup to be
// dispatched.  Runs longer than the XCD's workgroup count keep more of the
// items running at once on an XCD neighbours of each other, whose selected
// key blocks overlap (an L2 model on Wan selections: hit rate 0.54 with one
// slab of ceil(pairs / 8) per XCD and head, 0.59 with runs of 64).  An item
// is computed the same way wherever it runs, so the output does not depend on
// which workgroup takes it.
constexpr uint32_t kQueueStride = 32;  // u32 between counters: one 128-byte line each
constexpr uint32_t kNoItem = 0xFFFFFFFFu;

struct WorkQueue {
  uint32_t* ctr;
  uint32_t len;    // entries per queue: ceil(runs / 8) * run
  uint32_t run;    // pairs per run
  uint32_t rph;    // runs per head
  uint32_t runs;   // runs in all
  uint32_t pairs;  // pairs per head
  // Next item (bh * pairs + pair) for a workgroup of XCD home, or kNoItem.
  __device__ uint32_t take(uint32_t home) const {
    for (uint32_t v = 0; v < kXcds; ++v) {
      const uint32_t qx = (home + v) % kXcds;
      for (;;) {
        const uint32_t idx = __hip_atomic_fetch_add(ctr + qx * kQueueStride, 1u,
                                                    __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        if (idx >= len) break;
        const uint32_t k = idx / run, slot = idx - k * run;
        const uint32_t g = qx + kXcds * k;  // the run this entry belongs to
        if (g >= runs) break;               // and every later entry of this queue too
        const uint32_t bh = g / rph, pair = (g - bh * rph) * run + slot;
        if (pair < pairs) return bh * pairs + pair;  // else: past a head's last pair
      }
    }
    return kNoItem;
  }
};

__global__ void queue_reset_kernel(uint32_t* ctr) {
  if (threadIdx.x < kXcds)
    __hip_atomic_store(ctr + threadIdx.x * kQueueStride, 0u, __ATOMIC_RELAXED,
                       __HIP_MEMORY_SCOPE_AGENT);
}

// ------------------------------------------------------------------ kernels

// x, through an empty volatile asm: the compiler cannot move what is derived
// from it out of the loop the asm sits in.  Per-lane offsets derived from the
// thread id inside a persistent loop are then recomputed per item instead of
// occupying registers across the whole loop.
__device__ __forceinline__ int loop_local(int x) {
  asm volatile("" : "+v"(x));
  return x;
}

// One work item: the query-block pair (2 pair, 2 pair + 1) of head bh.
// wq (persistent fused kernel only): once the item's exact phase is done,
// thread 0 takes the workgroup's next item from the queues and, after the
// item's output is written, leaves it in *next_slot (LDS).
template <int D, int BLK, bool FUSED>
__device__ __forceinline__ void attn_item(const AttnArgs& a, char* smem, uint32_t bh,
                                          uint32_t pair, const WorkQueue* wq = nullptr,
                                          uint32_t home = 0, uint32_t* next_slot = nullptr) {
  using C = Cfg<D, BLK>;
  auto selbits = reinterpret_cast<uint32_t(*)[kMaxBlocks / 32]>(smem + C::BITS);
  auto qbar_s = reinterpret_cast<float(*)[D]>(smem + C::QBAR);

  const int tid = loop_local((int)threadIdx.x), lane = tid % kWave;
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);  // wave-uniform
  const int grp = wave / C::QW;  // which block of the pair
  const int h = lane / 32, l32 = lane % 32;
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
      w = *gbl(reinterpret_cast<const u32x4*>(qh + ((size_t)i_g * BLK + qrow) * D + 16 * ks +
                                              8 * h));
    qreg[ks] = __builtin_bit_cast(bf16x8, w);
  }

  float m_run = -INFINITY, l_run = 0.f;
  f32x16 o[C::DT];
#pragma unroll
  for (int dt = 0; dt < C::DT; ++dt)
#pragma unroll
    for (int r = 0; r < 16; ++r) o[dt][r] = 0.f;

  if constexpr (FUSED) {
    // ---- outer loop: routing and approximation, sub-chunk by sub-chunk
    const uint32_t item0 = bh * N + 2 * pair;
    const bool route = a.sel_in == nullptr;
    float tau0 = INFINITY, tau1 = INFINITY;
    if (route) {
      tau0 = gbl(a.tau)[item0];
      tau1 = pair1_on ? gbl(a.tau)[item0 + 1] : INFINITY;
      for (int cc = tid; cc < 2 * D; cc += C::NT) {
        const int gq = cc / D;
        qbar_s[gq][cc % D] =
            (gq == 0 || pair1_on) ? gbl(a.qbar)[(size_t)(item0 + gq) * D + cc % D] : 0.f;
      }
    } else {
      // masked mode: the two query blocks' given rows, with any bit at or
      // past N cleared so that the walk never visits a block that does not exist
      const uint32_t W64 = (N + 63) / 64;
      for (uint32_t e = tid; e < 2 * W64; e += C::NT) {
        const uint32_t gq = e / W64, w = e % W64;
        uint64_t word =
            (gq == 0 || pair1_on) ? gbl(a.sel_in)[(size_t)(item0 + gq) * W64 + w] : 0ull;
        const uint32_t rows = N - 64 * w;
        if (rows < 64u) word &= (1ull << rows) - 1ull;
        selbits[gq][2 * w] = (uint32_t)word;
        selbits[gq][2 * w + 1] = (uint32_t)(word >> 32);
      }
    }
    const uint32_t words = (N + 31) / 32;
    const float* kbar_h = a.kbar + (size_t)bh * N * D;
    const float* vhat_h = a.vhat + (size_t)bh * N * D;
    __syncthreads();
    route_approx_phase<D, BLK>(smem, selbits, qbar_s, kbar_h, vhat_h, N,
                               (int)(L - (int64_t)(N - 1) * BLK), tau0, tau1, a.scale, route,
                               !a.exact_only, grp_on, grp, qreg, a.c_log2, m_run, l_run, o, tid,
                               wave, lane);

    // debug outputs: the group's first wave writes its row of the bitmap
    if (grp_on && (wave % C::QW) == 0) {
      const uint32_t W64 = (N + 63) / 64;
      int count = 0;
      for (uint32_t w = lane; w < W64; w += kWave) {
        const uint32_t lo = selbits[grp][2 * w];
        const uint32_t hi = (2 * w + 1 < words) ? selbits[grp][2 * w + 1] : 0u;
        if (a.sel_mask)
          gbl(a.sel_mask)[(size_t)(bh * N + i_g) * W64 + w] = ((uint64_t)hi << 32) | lo;
        count += __builtin_popcount(lo) + __builtin_popcount(hi);
      }
      if (a.sel_count) {
#pragma unroll
        for (int off = 32; off >= 1; off >>= 1) count += __shfl_xor(count, off);
        if (lane == 0) gbl(a.sel_count)[bh * N + i_g] = count;
      }
    }

    // ---- inner loops: exact attention over the selected blocks, in order
    exact_phase<D, BLK>(smem, selbits, N, L, kh, vh, grp_on, grp, qreg, a.c_log2,
                        m_run, l_run, o, wave, lane);
  } else {
    exact_phase<D, BLK>(smem, nullptr, N, L, kh, vh, grp_on, grp, qreg, a.c_log2,
                        m_run, l_run, o, wave, lane);
  }

  // The next item is taken here, not at the item's start: taken at the start,
  // a workgroup would run items in the order in which it finished the items
  // before, which spreads the items running at once on an XCD further apart
  // in the queue and costs L2 hits (measured: 50 GB against 41 GB fetched
  // from beyond L2 per launch at the Wan shape).  Its latency overlaps the
  // output stores below.
  uint32_t next = kNoItem;
  if (wq != nullptr && tid == 0) next = wq->take(home);

  // O = N / D: combine the two lane halves of the denominator.
  const float ltot = l_run + __shfl_xor(l_run, 32);
  const float inv = ltot > 0.f ? 1.f / ltot : 0.f;
  if (a.lse2 != nullptr && qrow < n_i && h == 0)
    gbl(a.lse2)[(size_t)bh * L + (size_t)i_g * BLK + qrow] = m_run + __builtin_amdgcn_logf(ltot);
  if (a.out_f32 != nullptr) {
    if (qrow < n_i) {
      float* orow = a.out_f32 + head + ((size_t)i_g * BLK + qrow) * D;
#pragma unroll
      for (int dt = 0; dt < C::DT; ++dt)
#pragma unroll
        for (int r4 = 0; r4 < 4; ++r4) {
          f32x4 st;
#pragma unroll
          for (int e = 0; e < 4; ++e) st[e] = o[dt][4 * r4 + e] * inv;
          *gbl(reinterpret_cast<f32x4*>(orow + 32 * dt + 8 * r4 + 4 * h)) = st;
        }
    }
  } else if (qrow < n_i) {
    uint16_t* orow = a.out + head + ((size_t)i_g * BLK + qrow) * D;
#pragma unroll
    for (int dt = 0; dt < C::DT; ++dt)
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) {
        const int d0 = 32 * dt + 8 * r4 + 4 * h;
        typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
        typedef float f32x2 __attribute__((ext_vector_type(2)));
        typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
        u32x2 st;
#pragma unroll
        for (int e = 0; e < 2; ++e) {
          const f32x2 pr = {o[dt][4 * r4 + 2 * e] * inv, o[dt][4 * r4 + 2 * e + 1] * inv};
          st[e] = __builtin_bit_cast(uint32_t, __builtin_convertvector(pr, bf16x2));
        }
        *gbl(reinterpret_cast<u32x2*>(orow + d0)) = st;
      }
  }
  if (wq != nullptr && tid == 0) *next_slot = next;
}

// Both attention kernels are held to 256 registers per lane (two waves per
// SIMD): with 64-token blocks a workgroup has only four waves, one per SIMD,
// and without the cap the compiler spends the whole register file on one wave
// per SIMD, leaving no second wave to overlap one wave's softmax with the
// other's MFMAs (measured at the Wan shape with 64-token blocks: fused 31.7 ->
// 20.8 ms, dense 145 -> 106 ms, outputs bitwise equal).

// The dense comparison kernel: one workgroup per item, head-striped.
template <int D, int BLK>
__global__ __launch_bounds__(4 * BLK) __attribute__((amdgpu_waves_per_eu(2)))
void attn_dense_kernel(AttnArgs a) {
  using C = Cfg<D, BLK>;
  __shared__ __attribute__((aligned(1024))) char smem[C::SMEM_DENSE];
  uint32_t bh, pair;
  if (!head_striped_item(blockIdx.x, a.pairs, a.per_xcd, &bh, &pair)) return;
  attn_item<D, BLK, false>(a, smem, bh, pair);
}

// The fused Sol-Attn kernel: persistent workgroups draining the work queues.
// Each item hands the next one to the whole workgroup through LDS at its end.
template <int D, int BLK>
__global__ __launch_bounds__(4 * BLK) __attribute__((amdgpu_waves_per_eu(2)))
void attn_fused_kernel(AttnArgs a) {
  using C = Cfg<D, BLK>;
  __shared__ __attribute__((aligned(1024))) char smem[C::SMEM_FUSED + 16];
  uint32_t* slot = reinterpret_cast<uint32_t*>(smem + C::SMEM_FUSED);
  const WorkQueue wq{a.queue, a.queue_len, a.run, a.runs_per_head, a.runs, a.pairs};
  const uint32_t home = blockIdx.x % kXcds;
  if (threadIdx.x == 0) slot[0] = wq.take(home);
  __syncthreads();
  uint32_t item = slot[0];
  // The arguments are read again from the kernel-argument segment for every
  // item (scalar loads, through a pointer the compiler cannot see to be loop
  // invariant), so they are not held in scalar registers across the item
  // loop; held there, they left too few for the item itself and about 46
  // were spilled to vector-register lanes (measured: 16.76 -> 16.29 ms at the
  // Wan shape, outputs bitwise equal).
  typedef const __attribute__((address_space(4))) uint32_t KWord;
  KWord* const kargs = (KWord*)__builtin_amdgcn_kernarg_segment_ptr();
  static_assert(sizeof(AttnArgs) % 4 == 0, "the arguments are copied as whole words");
  while (item != kNoItem) {
    KWord* kp = kargs;
    asm volatile("" : "+s"(kp));
    AttnArgs ai;
#pragma unroll
    for (int i = 0; i < (int)(sizeof(AttnArgs) / 4); ++i)
      reinterpret_cast<uint32_t*>(&ai)[i] = kp[i];
    const uint32_t bh = item / ai.pairs;
    // slot[0] is rewritten only after this item's exact phase, which every
    // wave reaches after many barriers: by then all have read it
    attn_item<D, BLK, true>(ai, smem, bh, item - bh * ai.pairs, &wq, home, slot);
    __syncthreads();
    item = slot[0];
  }
}

// Workgroups of the persistent fused kernel on the current device: every CU
// times the kernel's occupancy, found once per device and instantiation.
// Plain static storage (no allocation), so the allocation-free entry point
// can use it too.
constexpr int kMaxDevices = 64;
std::mutex g_grid_mu;
int g_grid[kMaxDevices][4];

hipError_t persistent_grid(const void* kernel, int threads, int inst, uint32_t* grid) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_grid_mu);
  if (g_grid[dev][inst] == 0) {
    int cus = 0, occ = 0;
    e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
    if (e != hipSuccess) return e;
    e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&occ, kernel, threads, 0);
    if (e != hipSuccess) return e;
    g_grid[dev][inst] = (cus > 0 ? cus : 1) * (occ > 0 ? occ : 1);
  }
  *grid = (uint32_t)g_grid[dev][inst];
  return hipSuccess;
}

template <bool FUSED>
hipError_t launch_attn(const Shape& s, AttnArgs a, hipStream_t stream) {
  a.L = s.L;
  a.N = (uint32_t)s.N;
  a.pairs = (uint32_t)((s.N + 1) / 2);
  a.per_xcd = (a.pairs + kXcds - 1) / kXcds;
  a.scale = s.scale;
  a.c_log2 = s.scale * kLog2e;
  const uint64_t items = (uint64_t)s.bh * a.pairs;
#define SOLATTN_LAUNCH(DD, BB, INST)                                                           \
  if (s.d == DD && s.block == BB) {                                                            \
    if (!FUSED) {                                                                              \
      const dim3 grid((uint32_t)(kXcds * a.per_xcd * s.bh));                                   \
      hipLaunchKernelGGL((attn_dense_kernel<DD, BB>), grid, dim3(Cfg<DD, BB>::NT), 0, stream,  \
                         a);                                                                   \
      return hipGetLastError();                                                                \
    }                                                                                          \
    uint32_t grid = 0;                                                                         \
    hipError_t e = persistent_grid(reinterpret_cast<const void*>(&attn_fused_kernel<DD, BB>),  \
                                   Cfg<DD, BB>::NT, INST, &grid);                              \
    if (e != hipSuccess) return e;                                                             \
    if (items < grid) grid = (uint32_t)items;                                                  \
    a.run = 2 * ((grid + kXcds - 1) / kXcds);                                                  \
    if (a.run > a.pairs) a.run = a.pairs;                                                      \
    a.runs_per_head = (a.pairs + a.run - 1) / a.run;                                           \
    a.runs = (uint32_t)(s.bh * a.runs_per_head);                                               \
    a.queue_len = (a.runs + kXcds - 1) / kXcds * a.run;                                        \
    hipLaunchKernelGGL(queue_reset_kernel, dim3(1), dim3(kWave), 0, stream, a.queue);          \
    e = hipGetLastError();                                                                     \
    if (e != hipSuccess) return e;                                                             \
    hipLaunchKernelGGL((attn_fused_kernel<DD, BB>), dim3(grid), dim3(Cfg<DD, BB>::NT), 0,      \
                       stream, a);                                                             \
    return hipGetLastError();                                                                  \
  }
  SOLATTN_LAUNCH(128, 128, 0)
  SOLATTN_LAUNCH(128, 64, 1)
  SOLATTN_LAUNCH(64, 128, 2)
  SOLATTN_LAUNCH(64, 64, 3)
#undef SOLATTN_LAUNCH
  return hipErrorInvalidValue;
}

}  // namespace

int64_t fused_max_blocks() { return kMaxBlocks; }

size_t fwd_workspace_bytes() { return (size_t)kXcds * kQueueStride * sizeof(uint32_t); }

hipError_t launch_fwd(const Shape& s, const void* q, const void* k, const void* v,
                      const float* qbar, const float* kbar, const float* vhat, const float* tau,
                      const uint64_t* sel_in, void* out, uint64_t* sel_mask, int32_t* sel_count,
                      float* out_f32, float* lse2, void* workspace, hipStream_t stream) {
  AttnArgs a{};
  a.queue = static_cast<uint32_t*>(workspace);
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
  a.sel_in = sel_in;
  a.out_f32 = out_f32;
  a.lse2 = lse2;
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
