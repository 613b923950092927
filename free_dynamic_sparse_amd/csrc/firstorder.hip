// First-order term of the unselected blocks (gfx950).
//
// Method context: "Sol-Attn: Accelerating Video Generation Inference via
// On-the-Fly Attention Sparsification", method section: the Taylor expansion
// of an unselected block's exponential score matrix around the row-wise mean
// score within the block (the expansion before Eqs. 9-10), of which the page
// keeps the zeroth-order term.  The next term is exp(c_r) (S_rt - c_r), with
// S_rt = scale q_r . k_t and centre c_r = scale q_r . Kbar_j.  Summed over the
// block's keys it adds nothing to the denominator (c_r is the mean of S_rt
// over them); with the keys' values it adds exp(c_r) scale C_j^T q_r to the
// numerator, where
//   C_j = sum over block j's valid tokens t of (k_t - Kbar_j) v_t^T   (d x d).
//
// Two kernels:
//   * kv_moments_kernel: C_j = K_j^T V_j - Kbar_j Vhat_j^T of every block
//     (the same sum, since Vhat_j is the sum of the block's values): the
//     products of the exact bf16 keys and values accumulate in float32 on
//     MFMA and the pooled outer product is subtracted in float32, so the only
//     rounding of note is the final bf16 store, with the value dimension as
//     rows (kvc[j][b][a] = C_j[a][b]) so that a 16-byte row segment is an
//     MFMA operand fragment;
//   * fo_kernel: after the fused forward has written O in float32, the row's
//     log2 denominator lse2_r (in logit units, 2^lse2_r = sum of the row's
//     2^(c s) weights) and the selection bitmaps, every row gains
//       sum over j in U_i of 2^(c_log2 q_r.Kbar_j - lse2_r) scale C_j^T q_r
//     and is rounded to bf16 once.  Its cost is an MFMA product of
//     2 n_i d^2 FLOPs per (query block, unselected block): half an exact
//     block when d equals the block size.
//
// fo_kernel layout.  One workgroup of 8 waves serves G consecutive query
// blocks of one head (G = 2 for 128-token blocks, 4 for 64), one wave per 32
// query rows.  It walks the union of the G blocks' unselected sets; each
// C_j of the union is streamed into LDS once (direct-to-LDS loads, one
// workgroup barrier per block) and used by the groups that did not select j,
// with the loads running two blocks ahead (three buffers).
// MFMA layout as in the fused kernel, transposed so that each
// lane owns one query:
//   T^T = C_j^T Q^T   A = rows of kvc_j from LDS, B = Q^T in registers;
//   O^T += w_j T^T    w_j = the lane's own weight, a per-lane scalar.
// The weights of 32 pooled keys at a time come from one MFMA tile of
// Kbar (split into bf16 high and low parts, so the logits carry about 16
// significant bits) against Q^T, through a per-wave LDS table.

#include <math.h>

#include "common.hpp"
#include "launch.hpp"

namespace solattn {
namespace {

// ------------------------------------------------------------ C_j

template <int D, int BLK>
struct KvCfg {
  static constexpr int NT = 256;
  static constexpr int WAVES = NT / kWave;
  static constexpr int KS = BLK / 16;   // k-steps over the tokens
  static constexpr int TD = D / 32;     // 32-wide tiles per dimension
  static constexpr int SEGS = D / 8;    // 16-byte segments in a bf16 row of K or V
  static constexpr int ROW = 2 * D;     // bytes per bf16 row
};

typedef short kv_v4i16 __attribute__((ext_vector_type(4)));

// XOR swizzle of a row's 16-byte segments: rows r .. r + 3 land in disjoint
// 64-byte bank ranges for the transposed reads below.
__device__ __forceinline__ int kv_swz(int r, int segs) { return (4 * (r % 4)) % segs; }

// One workgroup per block j of one head.  The block's keys and values are
// staged row-major in LDS (16-byte writes, zero past the n_j valid tokens)
// and read back transposed (ds_read_b64_tr_b16): lane l gets dimension
// 32 t + l % 32 and the eight tokens 16 kk + 4 (l / 32) + {0..3, 8..11} of
// k-step kk, the same tokens for both operands, so each MFMA contracts over
// the 16 tokens of its k-step.  Tile by tile,
//   out^T[a][b] = sum_t k_t[a] v_t[b] - Kbar_j[a] Vhat_j[b]
// with A = key rows, B = value rows.  Centring the keys before the product
// would round each k_t - Kbar_j to bf16; this form multiplies exact bf16
// inputs and cancels the mean in float32 instead.
template <int D, int BLK>
__global__ __launch_bounds__(256) void kv_moments_kernel(const uint16_t* k, const uint16_t* v,
                                                         const float* kbar, const float* vhat,
                                                         uint16_t* kvc, int64_t L, uint32_t N) {
  using C = KvCfg<D, BLK>;
  __shared__ __attribute__((aligned(16))) char k_s[BLK * C::ROW];
  __shared__ __attribute__((aligned(16))) char v_s[BLK * C::ROW];
  const uint32_t item = blockIdx.x;  // bh * N + j
  const uint32_t j = item % N;
  const size_t bh = item / N;
  const int64_t rem = L - (int64_t)j * BLK;
  const int n = (int)(rem < BLK ? rem : BLK);
  const uint16_t* kb = k + ((size_t)bh * L + (size_t)j * BLK) * D;
  const uint16_t* vb = v + ((size_t)bh * L + (size_t)j * BLK) * D;
  const int tid = threadIdx.x;

  for (int e = tid; e < BLK * C::SEGS; e += C::NT) {
    const int t = e / C::SEGS, sg = e % C::SEGS;
    u32x4 kw = {0u, 0u, 0u, 0u}, vw = {0u, 0u, 0u, 0u};
    if (t < n) {
      kw = *reinterpret_cast<const u32x4*>(kb + (size_t)t * D + 8 * sg);
      vw = *reinterpret_cast<const u32x4*>(vb + (size_t)t * D + 8 * sg);
    }
    const int off = t * C::ROW + ((sg ^ kv_swz(t, C::SEGS)) * 16);
    *reinterpret_cast<u32x4*>(k_s + off) = kw;
    *reinterpret_cast<u32x4*>(v_s + off) = vw;
  }
  __syncthreads();

  const float* km = kbar + (size_t)item * D;
  const float* vs = vhat + (size_t)item * D;
  const int wave = tid / kWave, lane = tid % kWave;
  const int h = lane / 32, l32 = lane % 32;
  const int g = lane / 16, jj = lane % 16, r0 = 4 * (g / 2) + jj / 4;
  // transposed fragment of dimension tile t, k-step kk
  auto frag = [&](const char* tile, int t, int kk) -> bf16x8 {
    const int col = 32 * t + 16 * (g % 2) + 4 * (jj % 4);
    const char* p0 = tile + (16 * kk + r0) * C::ROW +
                     ((col / 8) ^ kv_swz(r0, C::SEGS)) * 16 + (col % 8) * 2;
    typedef __attribute__((address_space(3))) kv_v4i16 lds_v4i16;
    const kv_v4i16 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16*)(p0));
    const kv_v4i16 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16*)(p0 + 8 * C::ROW));
    return __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
  };
  for (int tile = wave; tile < C::TD * C::TD; tile += C::WAVES) {
    const int ta = tile / C::TD, tb = tile % C::TD;
    f32x16 acc;
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[r] = 0.f;
#pragma unroll
    for (int kk = 0; kk < C::KS; ++kk) acc = mfma32x32x16(frag(k_s, ta, kk), frag(v_s, tb, kk), acc);
    // pooled values first (a later load would otherwise wait for the stores)
    const float vb_sum = vs[32 * tb + l32];
    f32x4 m[4];
#pragma unroll
    for (int r4 = 0; r4 < 4; ++r4)
      m[r4] = *reinterpret_cast<const f32x4*>(km + 32 * ta + 8 * r4 + 4 * h);
    // lane: value dim b = 32 tb + l32; key dims a = 32 ta + mfma_row(r, h),
    // four consecutive per group of four registers
    uint16_t* orow = kvc + ((size_t)item * D + 32 * tb + l32) * D + 32 * ta;
#pragma unroll
    for (int r4 = 0; r4 < 4; ++r4) {
      bf16 c[4];
#pragma unroll
      for (int e = 0; e < 4; ++e)
        c[e] = (bf16)__builtin_fmaf(-m[r4][e], vb_sum, acc[4 * r4 + e]);
      uint2 st;
      st.x = (uint32_t)__builtin_bit_cast(uint16_t, c[0]) |
             ((uint32_t)__builtin_bit_cast(uint16_t, c[1]) << 16);
      st.y = (uint32_t)__builtin_bit_cast(uint16_t, c[2]) |
             ((uint32_t)__builtin_bit_cast(uint16_t, c[3]) << 16);
      *reinterpret_cast<uint2*>(orow + 8 * r4 + 4 * h) = st;
    }
  }
}

// ------------------------------------------------------------ correction

// Largest N the correction kernel keeps per-block selection words for in LDS
// (the entry point allows N <= 8192, the fused kernel's own limit).
constexpr int kFoMaxBlocks = 8192;
constexpr int kFoMaxGroups = kFoMaxBlocks / 32;

template <int D, int BLK>
struct FoCfg {
  static constexpr int QW = BLK / 32;          // waves per query block
  static constexpr int WAVES = 8;
  static constexpr int G = WAVES / QW;         // query blocks per workgroup
  static constexpr int NT = WAVES * kWave;
  static constexpr int KS = D / 16;            // k-steps over d
  static constexpr int DT = D / 32;            // 32-wide d tiles of O^T
  static constexpr int SEGS = D / 8;           // 16-byte segments per bf16 row
  static constexpr int ROW = 2 * D;            // bytes per bf16 row
  static constexpr int CT = D * ROW;           // bytes of one bf16 C_j tile
  static constexpr int DMA = CT / 1024 / WAVES;  // 1 KB loads per wave per tile
  static constexpr int ROWS_1K = 1024 / ROW;
  static constexpr int KB = 32 * ROW;          // 32 staged pooled keys, bf16
  static constexpr int WT = 32 * 32 * 4;       // one wave's weight table (32 keys x 32 rows)
  static constexpr int NBUF = 3;               // C_j buffers: loads run two blocks ahead
  static constexpr int C0 = 0, KHI = NBUF * CT, KLO = KHI + KB, WTAB = KLO + KB;
  // unselected words, u32 [1 + G][kFoMaxGroups]: the union of the G blocks',
  // then each block's own
  static constexpr int SELW = WTAB + WAVES * WT;
  static constexpr int SMEM = SELW + (1 + G) * kFoMaxGroups * 4;
  static_assert(DMA >= 1 && DMA * WAVES * 1024 == CT, "a C_j tile splits into whole 1 KB loads");
};

struct FoArgs {
  const uint16_t* q;
  const float* kbar;
  const uint16_t* kvc;
  const uint64_t* sel;
  const float* lse2;
  const float* o32;
  uint16_t* out;
  int64_t L;
  uint32_t N;
  uint32_t tuples;   // ceil(N / G) workgroup items per head
  uint32_t per_xcd;  // items per XCD slab: ceil(tuples / 8)
  float scale;
  float c_log2;      // scale * log2(e)
};

__device__ __forceinline__ const uint16_t* uniform_ptr(const uint16_t* p) {
  const uint64_t u = (uint64_t)(uintptr_t)p;
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)u);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(u >> 32));
  return reinterpret_cast<const uint16_t*>((uintptr_t)(((uint64_t)hi << 32) | (uint64_t)lo));
}

template <int D, int BLK>
__global__ __launch_bounds__(512) void fo_kernel(FoArgs a) {
  using C = FoCfg<D, BLK>;
  __shared__ __attribute__((aligned(1024))) char smem[C::SMEM];
  const int tid = threadIdx.x, lane = tid % kWave;
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
  const int grp = wave / C::QW;
  const int h = lane / 32, l32 = lane % 32;
  uint32_t bh, tup;
  if (!head_striped_item(blockIdx.x, a.tuples, a.per_xcd, &bh, &tup)) return;
  const uint32_t N = a.N;
  const int64_t L = a.L;
  const uint32_t i0 = tup * C::G;
  const uint32_t i_g = i0 + grp;
  const bool grp_on = i_g < N;
  const int n_i =
      grp_on ? (int)((L - (int64_t)i_g * BLK) < BLK ? (L - (int64_t)i_g * BLK) : BLK) : 0;
  const int qrow = (wave % C::QW) * 32 + l32;
  const bool row_on = qrow < n_i;
  const size_t head = (size_t)bh * (size_t)L * D;
  const size_t row_g = (size_t)i_g * BLK + qrow;  // token index of this lane's query

  bf16x8 qreg[C::KS];
#pragma unroll
  for (int ks = 0; ks < C::KS; ++ks) {
    u32x4 w = {0u, 0u, 0u, 0u};
    if (row_on) w = *reinterpret_cast<const u32x4*>(a.q + head + row_g * D + 16 * ks + 8 * h);
    qreg[ks] = __builtin_bit_cast(bf16x8, w);
  }
  // rows past the block get weight 2^-inf = 0
  const float lse2 = row_on ? a.lse2[(size_t)bh * L + row_g] : INFINITY;

  f32x16 o[C::DT];
#pragma unroll
  for (int dt = 0; dt < C::DT; ++dt)
#pragma unroll
    for (int r = 0; r < 16; ++r) o[dt][r] = 0.f;

  const uint32_t W64 = (N + 63) / 64;
  const uint32_t ngb = (N + 31) / 32;  // groups of 32 pooled keys
  const uint64_t* selh = a.sel + (size_t)bh * N * W64;
  // Unselected blocks of query block i among pooled keys 32 gb .. 32 gb + 31.
  auto unsel_word = [&](uint32_t i, uint32_t gb) -> uint32_t {
    if (i >= N) return 0u;
    const uint64_t w = selh[(size_t)i * W64 + gb / 2];
    const uint32_t s = (uint32_t)(w >> (32 * (gb % 2)));
    const uint32_t rem = N - 32 * gb;
    const uint32_t valid = rem >= 32u ? ~0u : ((1u << rem) - 1u);
    return ~s & valid;
  };
  // The tuple's unselected words go to LDS once, so that walking them later
  // issues no vector-memory load (whose wait would also wait for the C_j
  // loads in flight).
  uint32_t* usel = reinterpret_cast<uint32_t*>(smem + C::SELW);
  for (uint32_t gb = (uint32_t)tid; gb < ngb; gb += C::NT) {
    uint32_t u = 0u;
#pragma unroll
    for (int g = 0; g < C::G; ++g) {
      const uint32_t w = unsel_word(i0 + g, gb);
      usel[(1 + g) * kFoMaxGroups + gb] = w;
      u |= w;
    }
    usel[gb] = u;
  }
  __syncthreads();
  auto union_word = [&](uint32_t gb) -> uint32_t {
    return __builtin_amdgcn_readfirstlane(usel[gb]);
  };
  // Smallest j >= from unselected by any block of the tuple, or N.
  auto next_block = [&](uint32_t from) -> uint32_t {
    uint32_t gb = from / 32;
    if (gb >= ngb) return N;
    uint32_t u = union_word(gb) & (~0u << (from % 32));
    while (u == 0u) {
      if (++gb >= ngb) return N;
      u = union_word(gb);
    }
    return 32 * gb + (uint32_t)__builtin_ctz(u);
  };

  // per-lane byte offsets: DMA sources (swizzled) and operand reads
  uint32_t doff[C::DMA];
#pragma unroll
  for (int c = 0; c < C::DMA; ++c) {
    const int row = (wave + c * C::WAVES) * C::ROWS_1K + lane / C::SEGS;
    doff[c] = (uint32_t)(row * C::ROW + (((lane % C::SEGS) ^ (row % C::SEGS)) * 16));
  }
  uint32_t aoff[C::KS];  // row l32, logical segment 2 ks + h
#pragma unroll
  for (int ks = 0; ks < C::KS; ++ks)
    aoff[ks] = (uint32_t)(l32 * C::ROW + (((2 * ks + h) ^ (l32 % C::SEGS)) * 16));
  const uint32_t lbase = lds_addr(smem);
  const uint16_t* kvc_h = a.kvc + (size_t)bh * N * D * D;
  auto issue = [&](uint32_t j, int buf) {
    const uint16_t* src = uniform_ptr(kvc_h + (size_t)j * D * D);
    const uint32_t dst = lbase + (uint32_t)(C::C0 + buf * C::CT);
#pragma unroll
    for (int c = 0; c < C::DMA; ++c)
      lds_dma_16b(doff[c], src, dst + (uint32_t)(wave + c * C::WAVES) * 1024u);
  };
  float* wtab = reinterpret_cast<float*>(smem + C::WTAB + wave * C::WT);  // [32 keys][32 rows]
  const float* kbar_h = a.kbar + (size_t)bh * N * D;

  settle_vm();
  uint32_t j = next_block(0);
  uint32_t jn = j < N ? next_block(j + 1) : N;
  if (j < N) issue(j, 0);
  if (jn < N) issue(jn, 1);
  int buf = 0;
  uint32_t staged = ~0u, own = 0u;
  while (j < N) {
    const uint32_t gb = j / 32;
    if (gb != staged) {
      // Kbar rows 32 gb .. 32 gb + 31 as bf16 high and low parts, K layout
      if (tid < 32 * C::SEGS) {
        const int r = tid / C::SEGS, sg = tid % C::SEGS;
        const uint32_t jr = 32 * gb + (uint32_t)r;
        f32x4 x0 = {0.f, 0.f, 0.f, 0.f}, x1 = {0.f, 0.f, 0.f, 0.f};
        if (jr < N) {
          x0 = *reinterpret_cast<const f32x4*>(kbar_h + (size_t)jr * D + 8 * sg);
          x1 = *reinterpret_cast<const f32x4*>(kbar_h + (size_t)jr * D + 8 * sg + 4);
        }
        bf16x8 hi, lo;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float x = e < 4 ? x0[e] : x1[e - 4];
          hi[e] = (bf16)x;
          lo[e] = (bf16)(x - (float)hi[e]);
        }
        const int off = r * C::ROW + ((sg ^ (r % C::SEGS)) * 16);
        *reinterpret_cast<bf16x8*>(smem + C::KHI + off) = hi;
        *reinterpret_cast<bf16x8*>(smem + C::KLO + off) = lo;
      }
      barrier_lds();
      own = __builtin_amdgcn_readfirstlane(grp_on ? usel[(1 + grp) * kFoMaxGroups + gb] : 0u);
      if (own) {
        // logits of the 32 staged keys for this wave's 32 queries:
        // lane = query l32, register r = key mfma_row(r, h)
        f32x16 s;
#pragma unroll
        for (int r = 0; r < 16; ++r) s[r] = 0.f;
#pragma unroll
        for (int ks = 0; ks < C::KS; ++ks)
          s = mfma32x32x16(*reinterpret_cast<const bf16x8*>(smem + C::KHI + aoff[ks]), qreg[ks],
                           s);
#pragma unroll
        for (int ks = 0; ks < C::KS; ++ks)
          s = mfma32x32x16(*reinterpret_cast<const bf16x8*>(smem + C::KLO + aoff[ks]), qreg[ks],
                           s);
#pragma unroll
        for (int r = 0; r < 16; ++r)
          wtab[mfma_row(r, h) * 32 + l32] =
              a.scale * __builtin_amdgcn_exp2f(__builtin_fmaf(s[r], a.c_log2, -lse2));
      }
      staged = gb;
    }
    const uint32_t jnn = jn < N ? next_block(jn + 1) : N;
    // C_j (buffer buf) has landed once at most the next block's loads are
    // outstanding; after the barrier everyone is done with block j - 1's
    // buffer, which takes the block after next.
    if (jn < N)
      wait_vm<C::DMA>();
    else
      wait_vm<0>();
    barrier_lds();
    if (jnn < N) issue(jnn, buf == 0 ? C::NBUF - 1 : buf - 1);
    if ((own >> (j % 32)) & 1u) {
      const char* ct = smem + C::C0 + buf * C::CT;
      const float w = wtab[(j % 32) * 32 + l32];
#pragma unroll
      for (int dt = 0; dt < C::DT; ++dt) {
        f32x16 t;
#pragma unroll
        for (int r = 0; r < 16; ++r) t[r] = 0.f;
#pragma unroll
        for (int ks = 0; ks < C::KS; ++ks)
          t = mfma32x32x16(*reinterpret_cast<const bf16x8*>(ct + 32 * dt * C::ROW + aoff[ks]),
                           qreg[ks], t);
#pragma unroll
        for (int r = 0; r < 16; ++r) o[dt][r] = __builtin_fmaf(w, t[r], o[dt][r]);
      }
    }
    buf = buf + 1 == C::NBUF ? 0 : buf + 1;
    j = jn;
    jn = jnn;
  }

  if (row_on) {
    // all loads first: the stores to out could alias o32 as far as the
    // compiler knows, which would otherwise serialise every load
    const float* src = a.o32 + head + row_g * D;
    uint16_t* dst = a.out + head + row_g * D;
    f32x4 xs[C::DT][4];
#pragma unroll
    for (int dt = 0; dt < C::DT; ++dt)
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4)
        xs[dt][r4] = *reinterpret_cast<const f32x4*>(src + 32 * dt + 8 * r4 + 4 * h);
#pragma unroll
    for (int dt = 0; dt < C::DT; ++dt)
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) {
        const int d0 = 32 * dt + 8 * r4 + 4 * h;
        const f32x4 x = xs[dt][r4];
        uint2 st;
        st.x = (uint32_t)__builtin_bit_cast(uint16_t, (bf16)(x[0] + o[dt][4 * r4 + 0])) |
               ((uint32_t)__builtin_bit_cast(uint16_t, (bf16)(x[1] + o[dt][4 * r4 + 1])) << 16);
        st.y = (uint32_t)__builtin_bit_cast(uint16_t, (bf16)(x[2] + o[dt][4 * r4 + 2])) |
               ((uint32_t)__builtin_bit_cast(uint16_t, (bf16)(x[3] + o[dt][4 * r4 + 3])) << 16);
        *reinterpret_cast<uint2*>(dst + d0) = st;
      }
  }
}

}  // namespace

hipError_t launch_kv_moments(const Shape& s, const void* k, const void* v, const float* kbar,
                             const float* vhat, void* kvc, hipStream_t stream) {
  const dim3 grid((uint32_t)(s.bh * s.N));
  const uint16_t* kk = static_cast<const uint16_t*>(k);
  const uint16_t* vv = static_cast<const uint16_t*>(v);
  uint16_t* out = static_cast<uint16_t*>(kvc);
  const uint32_t N = (uint32_t)s.N;
#define SOLATTN_KV(DD, BB)                                                                  \
  if (s.d == DD && s.block == BB) {                                                         \
    hipLaunchKernelGGL((kv_moments_kernel<DD, BB>), grid, dim3(256), 0, stream, kk, vv, kbar, \
                       vhat, out, s.L, N);                                                  \
    return hipGetLastError();                                                               \
  }
  SOLATTN_KV(128, 128)
  SOLATTN_KV(128, 64)
  SOLATTN_KV(64, 128)
  SOLATTN_KV(64, 64)
#undef SOLATTN_KV
  return hipErrorInvalidValue;
}

hipError_t launch_first_order(const Shape& s, const void* q, const float* kbar, const void* kvc,
                              const uint64_t* sel_mask, const float* lse2, const float* o32,
                              void* out, hipStream_t stream) {
  if (s.N > kFoMaxBlocks) return hipErrorInvalidValue;
  FoArgs a{};
  a.q = static_cast<const uint16_t*>(q);
  a.kbar = kbar;
  a.kvc = static_cast<const uint16_t*>(kvc);
  a.sel = sel_mask;
  a.lse2 = lse2;
  a.o32 = o32;
  a.out = static_cast<uint16_t*>(out);
  a.L = s.L;
  a.N = (uint32_t)s.N;
  a.scale = s.scale;
  a.c_log2 = s.scale * kLog2e;
#define SOLATTN_FO(DD, BB)                                                                  \
  if (s.d == DD && s.block == BB) {                                                         \
    a.tuples = (a.N + FoCfg<DD, BB>::G - 1) / FoCfg<DD, BB>::G;                             \
    a.per_xcd = (a.tuples + kXcds - 1) / kXcds;                                             \
    const dim3 grid((uint32_t)(kXcds * a.per_xcd * s.bh));                                  \
    hipLaunchKernelGGL((fo_kernel<DD, BB>), grid, dim3(FoCfg<DD, BB>::NT), 0, stream, a);   \
    return hipGetLastError();                                                               \
  }
  SOLATTN_FO(128, 128)
  SOLATTN_FO(128, 64)
  SOLATTN_FO(64, 128)
  SOLATTN_FO(64, 64)
#undef SOLATTN_FO
  return hipErrorInvalidValue;
}

}  // namespace solattn
