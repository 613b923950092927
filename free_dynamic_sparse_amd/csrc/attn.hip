// Fused Sol-Attn forward and the dense comparison kernel (gfx950).
//
// Method: "Sol-Attn: Accelerating Video Generation Inference via On-the-Fly
// Attention Sparsification", method section: chunk-wise streaming
// thresholding (Eqs. 6-7), zeroth-order approximation of unselected blocks
// with the combined denominator and numerator (Eqs. 9-10), the token-to-block
// score tile (Eq. 11, Figure 4) and the nested-loop kernel (Algorithm 3.2).
//
// One workgroup per (b, h, query block i), one wave per 32 query rows.
// Everything is computed transposed so that each lane owns one query:
//   S^T = K Q^T      v_mfma_f32_32x32x16_bf16, A = K rows from LDS,
//                    B = Q^T held in registers for the whole kernel;
//                    lane l holds query l%32 and 16 keys per 32x32 tile, so
//                    the row max / sum of the online softmax is a lane-local
//                    reduction plus one exchange with lane l^32;
//   O^T += V^T P^T   A = V^T from LDS (stored transposed, keys permuted to
//                    the order in which P^T sits in the S^T result
//                    registers), B = P^T straight from those registers.
// Per chunk of C pooled keys (the outer loop):
//   * routing: every wave computes shat_ij = scale * Qbar_i . Kbar_j in
//     float32 for the chunk's columns and ballots shat_ij >= tau_i into a
//     64-bit mask.  Every wave runs the same instructions on the same data,
//     so the mask is identical across the workgroup without a barrier.
//     (The page obtains these scores as column means of the token-to-block
//     tile; the mean is the same number, and the direct float32 dot keeps the
//     decision accurate to far below the tie band that a bf16 tile allows.)
//   * approximation: the token-to-block tile scale * Q_i KC^T comes from
//     MFMA (KC rounded to bf16); its unselected columns update the online
//     softmax with weight n_j and value Vhat_j (VC).
// Inner loop: the chunk's selected key blocks, exact attention.
// Both paths share one running max, denominator and accumulator.

#include <math.h>

#include "common.hpp"
#include "launch.hpp"

namespace solattn {
namespace {

template <int D, int BLK>
struct Cfg {
  static constexpr int WAVES = BLK / 32;   // one wave per 32 query rows
  static constexpr int NT = WAVES * kWave;  // = 2 * BLK (launch bounds)
  static constexpr int KS = D / 16;        // k-steps of Q K^T (contraction over d)
  static constexpr int MT = BLK / 32;      // 32-key tiles of S^T
  static constexpr int DT = D / 32;        // 32-wide d tiles of O^T
  static constexpr int PK = BLK / 16;      // k-steps of P V (contraction over keys)
  static constexpr int KROW = 2 * D + 16;  // LDS bytes per K row (16 B pad: no bank conflicts)
  static constexpr int VROW = 2 * BLK + 16;  // LDS bytes per V^T row
  static constexpr int CMAX = 64;          // largest chunk
  static constexpr int CROW = 4 * D + 16;  // LDS bytes per float32 pooled row
  static constexpr int TILE_BYTES = BLK * KROW + D * VROW;
  static constexpr int CHUNK_BYTES = 2 * CMAX * CROW;
  static constexpr int MAIN_BYTES = TILE_BYTES > CHUNK_BYTES ? TILE_BYTES : CHUNK_BYTES;
  static constexpr int SMEM = MAIN_BYTES + 4 * D;  // + Qbar_i
};

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
  uint32_t per_xcd;  // query blocks per XCD slab: ceil(N / 8)
  int chunk;
  float scale;
  float c_log2;  // scale * log2(e): logits enter exp2 in this unit
  uint32_t exact_only;
};

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Position of key kappa inside its 16-key group in the V^T tile: swap bits 2
// and 3, so that positions [8h, 8h+8) hold the keys that lanes of half h
// carry in registers 0..7 of an S^T result (keys 8(e/4) + 4h + e%4).
__device__ __forceinline__ int vt_pos(int kappa) {
  return (kappa & ~12) | ((kappa & 4) << 1) | ((kappa & 8) >> 1);
}

// Copy key block rows [0, nkeys) to LDS: K row-major (padded rows), V
// transposed with the key order above.  Rows >= nkeys are written as zeros.
template <int D, int BLK>
__device__ __forceinline__ void stage_kv(char* ktile, char* vtile, const uint16_t* kblk,
                                         const uint16_t* vblk, int nkeys, int tid) {
  using C = Cfg<D, BLK>;
  constexpr int SEG = D / 8;
  constexpr int KIT = BLK * SEG / C::NT;
  constexpr int VIT = (BLK / 2) * SEG / C::NT;
  static_assert(KIT * C::NT == BLK * SEG && VIT * C::NT == (BLK / 2) * SEG, "tiling");
  const u32x4 zero = {0u, 0u, 0u, 0u};
  u32x4 kv[KIT], va[VIT], vb[VIT];
#pragma unroll
  for (int it = 0; it < KIT; ++it) {
    const int idx = tid + it * C::NT;
    const int row = idx / SEG, seg = idx % SEG;
    kv[it] = row < nkeys ? *reinterpret_cast<const u32x4*>(kblk + (size_t)row * D + seg * 8) : zero;
  }
#pragma unroll
  for (int it = 0; it < VIT; ++it) {
    const int idx = tid + it * C::NT;
    const int pp = idx % (BLK / 2), g = idx / (BLK / 2);
    const int r0 = 2 * pp;
    va[it] = r0 < nkeys ? *reinterpret_cast<const u32x4*>(vblk + (size_t)r0 * D + g * 8) : zero;
    vb[it] = r0 + 1 < nkeys ? *reinterpret_cast<const u32x4*>(vblk + (size_t)(r0 + 1) * D + g * 8)
                            : zero;
  }
#pragma unroll
  for (int it = 0; it < KIT; ++it) {
    const int idx = tid + it * C::NT;
    const int row = idx / SEG, seg = idx % SEG;
    *reinterpret_cast<u32x4*>(ktile + row * C::KROW + seg * 16) = kv[it];
  }
#pragma unroll
  for (int it = 0; it < VIT; ++it) {
    const int idx = tid + it * C::NT;
    const int pp = idx % (BLK / 2), g = idx / (BLK / 2);
    const int key = 2 * pp;
    const int pos = (key & ~15) | vt_pos(key & 15);
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const uint32_t ev = (va[it][w] & 0xffffu) | (vb[it][w] << 16);
      const uint32_t od = (va[it][w] >> 16) | (vb[it][w] & 0xffff0000u);
      *reinterpret_cast<uint32_t*>(vtile + (8 * g + 2 * w) * C::VROW + pos * 2) = ev;
      *reinterpret_cast<uint32_t*>(vtile + (8 * g + 2 * w + 1) * C::VROW + pos * 2) = od;
    }
  }
}

// Copy pooled rows [j0, j0 + cvalid) of Kbar and Vhat (float32) to LDS.
template <int D, int BLK>
__device__ __forceinline__ void stage_chunk(char* kchunk, char* vchunk, const float* kbar_h,
                                            const float* vhat_h, uint32_t j0, int cvalid,
                                            int tid) {
  using C = Cfg<D, BLK>;
  constexpr int P = D / 4;  // 16-byte pieces per row
  for (int idx = tid; idx < cvalid * P; idx += C::NT) {
    const int jj = idx / P, pc = idx % P;
    const size_t g = (size_t)(j0 + jj) * D + pc * 4;
    const f32x4 kk = *reinterpret_cast<const f32x4*>(kbar_h + g);
    const f32x4 vv = *reinterpret_cast<const f32x4*>(vhat_h + g);
    *reinterpret_cast<f32x4*>(kchunk + jj * C::CROW + pc * 16) = kk;
    *reinterpret_cast<f32x4*>(vchunk + jj * C::CROW + pc * 16) = vv;
  }
}

// Exact attention of the wave's 32 queries against the key block in LDS,
// folded into the online-softmax state (m_run in log2 units, l_run = this
// lane's half of the denominator, o = O^T accumulators).
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
      const bf16x8 ka = *reinterpret_cast<const bf16x8*>(
          ktile + (32 * mt + l32) * C::KROW + (16 * ks + 8 * h) * 2);
      s[mt] = mfma32x32x16(ka, qreg[ks], s[mt]);
    }
  }
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
#pragma unroll
  for (int dt = 0; dt < C::DT; ++dt) o[dt] *= alpha;
#pragma unroll
  for (int kk = 0; kk < C::PK; ++kk) {
    const int mt = kk / 2, hf = kk % 2;
    float pv[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) pv[e] = s[mt][8 * hf + e];
    const bf16x8 pb = pack_bf16x8(pv);
#pragma unroll
    for (int dt = 0; dt < C::DT; ++dt) {
      const bf16x8 va = *reinterpret_cast<const bf16x8*>(
          vtile + (32 * dt + l32) * C::VROW + (16 * kk + 8 * h) * 2);
      o[dt] = mfma32x32x16(va, pb, o[dt]);
    }
  }
}

// Routing of one chunk: bit jj of the result is set iff pooled key j0 + jj
// (jj < cvalid) has shat >= tau_i.  Identical in every wave.
template <int D, int BLK>
__device__ __forceinline__ uint64_t route_chunk(const char* kchunk, const float* qbar_s,
                                                int cvalid, float tau_i, float scale, int lane) {
  using C = Cfg<D, BLK>;
  constexpr int HALF = D / 2;
  const int h = lane / 32, l32 = lane % 32;
  uint64_t mask = 0;
#pragma unroll
  for (int ct = 0; ct < C::CMAX / 32; ++ct) {
    if (32 * ct >= cvalid) break;
    const int jj = 32 * ct + l32;
    float part = 0.f;
    if (jj < cvalid) {
      const float* kr = reinterpret_cast<const float*>(kchunk + jj * C::CROW) + h * HALF;
      const float* qr = qbar_s + h * HALF;
#pragma unroll
      for (int e = 0; e < HALF; e += 4) {
        const f32x4 kv = *reinterpret_cast<const f32x4*>(kr + e);
        const f32x4 qv = *reinterpret_cast<const f32x4*>(qr + e);
        part = __builtin_fmaf(qv[0], kv[0], part);
        part = __builtin_fmaf(qv[1], kv[1], part);
        part = __builtin_fmaf(qv[2], kv[2], part);
        part = __builtin_fmaf(qv[3], kv[3], part);
      }
    }
    const float other = __shfl_xor(part, 32);
    const float dot = (h == 0) ? (part + other) : (other + part);
    const bool sel = (jj < cvalid) && (scale * dot >= tau_i);
    const uint64_t b = __ballot(sel);
    mask |= (b & 0xffffffffull) << (32 * ct);
  }
  return mask;
}

// Zeroth-order terms of the chunk's unselected columns (Eqs. 9-10): logits
// from the token-to-block tile, weight n_j in the denominator, Vhat_j in the
// numerator.
template <int D, int BLK>
__device__ __forceinline__ void approx_chunk(const char* kchunk, const char* vchunk,
                                             const bf16x8* qreg, uint64_t unsel, int cvalid,
                                             uint32_t j0, uint32_t N, int n_last, float c,
                                             float& m_run, float& l_run, f32x16* o, int lane) {
  using C = Cfg<D, BLK>;
  constexpr int CT = C::CMAX / 32;
  const int h = lane / 32, l32 = lane % 32;
  const int nct = (cvalid + 31) / 32;
  f32x16 t[CT];
  float mx = -INFINITY;
#pragma unroll
  for (int ct = 0; ct < CT; ++ct) {
    if (ct >= nct) break;
#pragma unroll
    for (int r = 0; r < 16; ++r) t[ct][r] = 0.f;
    const int jj = 32 * ct + l32;
#pragma unroll
    for (int ks = 0; ks < C::KS; ++ks) {
      bf16x8 ka;
      if (jj < cvalid) {
        const float* src = reinterpret_cast<const float*>(kchunk + jj * C::CROW) + 16 * ks + 8 * h;
        ka = pack_bf16x8(*reinterpret_cast<const f32x4*>(src),
                         *reinterpret_cast<const f32x4*>(src + 4));
      } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) ka[e] = (bf16)0.f;
      }
      t[ct] = mfma32x32x16(ka, qreg[ks], t[ct]);
    }
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int jr = 32 * ct + mfma_row(r, h);
      if (!((unsel >> jr) & 1ull)) t[ct][r] = -INFINITY;
      mx = fmaxf(mx, t[ct][r]);
    }
  }
  mx = wave_max_pair(mx);
  const float m_new = fmaxf(m_run, mx * c);
  const float alpha = fast_exp2(m_run - m_new);
  float lsum = 0.f;
#pragma unroll
  for (int ct = 0; ct < CT; ++ct) {
    if (ct >= nct) break;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int jr = 32 * ct + mfma_row(r, h);
      const float p = fast_exp2(__builtin_fmaf(t[ct][r], c, -m_new));
      t[ct][r] = p;
      const float w = (j0 + jr == N - 1) ? (float)n_last : (float)BLK;
      lsum = __builtin_fmaf(w, p, lsum);
    }
  }
  l_run = l_run * alpha + lsum;
  m_run = m_new;
#pragma unroll
  for (int dt = 0; dt < C::DT; ++dt) o[dt] *= alpha;
#pragma unroll
  for (int ct = 0; ct < CT; ++ct) {
    if (ct >= nct) break;
#pragma unroll
    for (int hf = 0; hf < 2; ++hf) {
      float pv[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) pv[e] = t[ct][8 * hf + e];
      const bf16x8 pb = pack_bf16x8(pv);
#pragma unroll
      for (int dt = 0; dt < C::DT; ++dt) {
        float vv[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int jr = 32 * ct + mfma_row(8 * hf + e, h);
          vv[e] = jr < cvalid
                      ? reinterpret_cast<const float*>(vchunk + jr * C::CROW)[32 * dt + l32]
                      : 0.f;
        }
        o[dt] = mfma32x32x16(pack_bf16x8(vv), pb, o[dt]);
      }
    }
  }
}

template <int D, int BLK, bool FUSED>
__global__ __launch_bounds__(2 * BLK) void attn_kernel(AttnArgs a) {
  using C = Cfg<D, BLK>;
  __shared__ __attribute__((aligned(16))) char smem[C::SMEM];
  char* ktile = smem;
  char* vtile = smem + BLK * C::KROW;
  char* kchunk = smem;  // the chunk stage reuses the tile buffers
  char* vchunk = smem + C::CMAX * C::CROW;
  float* qbar_s = reinterpret_cast<float*>(smem + C::MAIN_BYTES);

  const int tid = threadIdx.x, lane = tid % kWave, wave = tid / kWave;
  const int h = lane / 32, l32 = lane % 32;
  uint32_t bh, i;
  if (!head_striped_item(blockIdx.x, a.N, a.per_xcd, &bh, &i)) return;
  const uint32_t item = bh * a.N + i;  // (b*H + h)*N + i
  const int64_t L = a.L;
  const int n_i = (int)((L - (int64_t)i * BLK) < BLK ? (L - (int64_t)i * BLK) : BLK);
  const int n_last = (int)(L - (int64_t)(a.N - 1) * BLK);
  const size_t head = (size_t)bh * (size_t)L * D;
  const uint16_t* qh = a.q + head;
  const uint16_t* kh = a.k + head;
  const uint16_t* vh = a.v + head;

  // Q^T operand: this lane's query row, 8 consecutive d per k-step.
  const int qrow = wave * 32 + l32;
  bf16x8 qreg[C::KS];
#pragma unroll
  for (int ks = 0; ks < C::KS; ++ks) {
    u32x4 w = {0u, 0u, 0u, 0u};
    if (qrow < n_i)
      w = *reinterpret_cast<const u32x4*>(qh + ((size_t)i * BLK + qrow) * D + 16 * ks + 8 * h);
    qreg[ks] = __builtin_bit_cast(bf16x8, w);
  }

  float m_run = -INFINITY, l_run = 0.f;
  f32x16 o[C::DT];
#pragma unroll
  for (int dt = 0; dt < C::DT; ++dt)
#pragma unroll
    for (int r = 0; r < 16; ++r) o[dt][r] = 0.f;

  if constexpr (FUSED) {
    const float tau_i = a.tau[item];
    for (int cc = tid; cc < D; cc += C::NT) qbar_s[cc] = a.qbar[(size_t)item * D + cc];
    const float* kbar_h = a.kbar + (size_t)bh * a.N * D;
    const float* vhat_h = a.vhat + (size_t)bh * a.N * D;
    const uint32_t chunk = (uint32_t)a.chunk;
    const uint32_t T = (a.N + chunk - 1) / chunk;
    const uint32_t W = (a.N + 63) / 64;
    uint64_t* mrow = a.sel_mask ? a.sel_mask + (size_t)item * W : nullptr;
    uint32_t cur_word = 0;
    uint64_t cur_bits = 0;
    int count = 0;
    for (uint32_t t = 0; t < T; ++t) {
      const uint32_t j0 = t * chunk;
      const int cvalid = (int)((a.N - j0) < chunk ? (a.N - j0) : chunk);
      stage_chunk<D, BLK>(kchunk, vchunk, kbar_h, vhat_h, j0, cvalid, tid);
      __syncthreads();
      uint64_t mask = route_chunk<D, BLK>(kchunk, qbar_s, cvalid, tau_i, a.scale, lane);
      const uint64_t valid = cvalid >= 64 ? ~0ull : ((1ull << cvalid) - 1ull);
      const uint64_t unsel = valid & ~mask;
      if (!a.exact_only && unsel)
        approx_chunk<D, BLK>(kchunk, vchunk, qreg, unsel, cvalid, j0, a.N, n_last, a.c_log2,
                             m_run, l_run, o, lane);
      if (mrow) {
        // append this chunk's bits to the row bitmap (chunks arrive in order)
        const uint32_t word = j0 / 64, sh = j0 % 64;
        if (word != cur_word) {
          if (tid == 0) mrow[cur_word] = cur_bits;
          cur_word = word;
          cur_bits = 0;
        }
        cur_bits |= mask << sh;
        if (sh + (uint32_t)cvalid > 64) {
          if (tid == 0) mrow[cur_word] = cur_bits;
          cur_word = word + 1;
          cur_bits = mask >> (64 - sh);
        }
      }
      count += __builtin_popcountll(mask);
      __syncthreads();
      while (mask) {
        const uint32_t jj = (uint32_t)__builtin_ctzll(mask);
        mask &= mask - 1;
        const uint32_t j = j0 + jj;
        const int nk = (int)((L - (int64_t)j * BLK) < BLK ? (L - (int64_t)j * BLK) : BLK);
        stage_kv<D, BLK>(ktile, vtile, kh + (size_t)j * BLK * D, vh + (size_t)j * BLK * D, nk,
                         tid);
        __syncthreads();
        exact_block<D, BLK>(ktile, vtile, qreg, nk, a.c_log2, m_run, l_run, o, lane);
        __syncthreads();
      }
    }
    if (mrow && tid == 0) mrow[cur_word] = cur_bits;
    if (a.sel_count && tid == 0) a.sel_count[item] = count;
  } else {
    for (uint32_t j = 0; j < a.N; ++j) {
      const int nk = (int)((L - (int64_t)j * BLK) < BLK ? (L - (int64_t)j * BLK) : BLK);
      stage_kv<D, BLK>(ktile, vtile, kh + (size_t)j * BLK * D, vh + (size_t)j * BLK * D, nk, tid);
      __syncthreads();
      exact_block<D, BLK>(ktile, vtile, qreg, nk, a.c_log2, m_run, l_run, o, lane);
      __syncthreads();
    }
  }

  // O = N / D: combine the two lane halves of the denominator.
  const float ltot = l_run + __shfl_xor(l_run, 32);
  const float inv = ltot > 0.f ? 1.f / ltot : 0.f;
  if (qrow < n_i) {
    uint16_t* orow = a.out + head + ((size_t)i * BLK + qrow) * D;
#pragma unroll
    for (int dt = 0; dt < C::DT; ++dt)
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) {
        const int d0 = 32 * dt + 8 * r4 + 4 * h;
        uint32_t w0, w1;
        {
          const bf16 b0 = (bf16)(o[dt][4 * r4 + 0] * inv), b1 = (bf16)(o[dt][4 * r4 + 1] * inv);
          const bf16 b2 = (bf16)(o[dt][4 * r4 + 2] * inv), b3 = (bf16)(o[dt][4 * r4 + 3] * inv);
          w0 = (uint32_t)__builtin_bit_cast(uint16_t, b0) |
               ((uint32_t)__builtin_bit_cast(uint16_t, b1) << 16);
          w1 = (uint32_t)__builtin_bit_cast(uint16_t, b2) |
               ((uint32_t)__builtin_bit_cast(uint16_t, b3) << 16);
        }
        uint2 st;
        st.x = w0;
        st.y = w1;
        *reinterpret_cast<uint2*>(orow + d0) = st;
      }
  }
}

template <bool FUSED>
hipError_t launch_attn(const Shape& s, AttnArgs a, hipStream_t stream) {
  a.L = s.L;
  a.N = (uint32_t)s.N;
  a.per_xcd = (uint32_t)((s.N + kXcds - 1) / kXcds);
  a.chunk = s.chunk;
  a.scale = s.scale;
  a.c_log2 = s.scale * kLog2e;
  const dim3 grid((uint32_t)(kXcds * a.per_xcd * s.bh));
#define SOLATTN_LAUNCH(DD, BB)                                                              \
  if (s.d == DD && s.block == BB) {                                                         \
    hipLaunchKernelGGL((attn_kernel<DD, BB, FUSED>), grid, dim3(Cfg<DD, BB>::NT), 0, stream, \
                       a);                                                                  \
    return hipGetLastError();                                                               \
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
