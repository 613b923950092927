// Host-side launchers of the Sol-Attn kernels.  Arguments are already
// validated by the C ABI layer (solattn_api.cpp) when these run.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace solattn {

struct Shape {
  int64_t bh;     // B * H
  int64_t L;      // tokens per head
  int d;          // head dim (64 or 128)
  int block;      // tokens per block (64 or 128)
  int64_t N;      // ceil(L / block)
  int chunk;      // pooled keys per routing chunk (1..64)
  float beta;
  float scale;    // softmax scale (> 0)
  uint32_t flags;
};

hipError_t launch_pool(const Shape& s, const void* q, const void* k, const void* v, float* qbar,
                       float* kbar, float* vhat, hipStream_t stream);

hipError_t launch_moments(const Shape& s, const float* qbar, const float* kbar, float* kmean,
                          float* kcov, float* tau, float* mu, float* sigma, hipStream_t stream);

// Largest N = ceil(L / block) the fused kernel keeps on-chip selection bits for.
int64_t fused_max_blocks();

// Device workspace of the fused kernel (its work-queue counters), in bytes;
// the same for every problem.
size_t fwd_workspace_bytes();

// sel_in null: threshold routing from qbar and tau.  Otherwise the given
// selections (qbar and tau unused).  out_f32, if set, receives O in float32
// instead of out; lse2, if set, the log2 of each row's softmax denominator in
// units of scale * log2(e) * q.k (f32 [bh, L]).  workspace: fwd_workspace_bytes()
// of device memory, 256-byte aligned, reset in-stream by every launch.
hipError_t launch_fwd(const Shape& s, const void* q, const void* k, const void* v,
                      const float* qbar, const float* kbar, const float* vhat, const float* tau,
                      const uint64_t* sel_in, void* out, uint64_t* sel_mask, int32_t* sel_count,
                      float* out_f32, float* lse2, void* workspace, hipStream_t stream);

// First-order term of the unselected blocks.
// kvc[bh][j][b][a] = sum over block j's valid tokens t of v_t[b] (k_t[a] - Kbar_j[a]), bf16,
// formed as K_j^T V_j - Kbar_j Vhat_j^T.
hipError_t launch_kv_moments(const Shape& s, const void* k, const void* v, const float* kbar,
                             const float* vhat, void* kvc, hipStream_t stream);
// out = bf16(o32 + sum over j unselected (sel_mask) of 2^(c q.Kbar_j - lse2) scale C_j^T q)
// row by row; o32, lse2 and sel_mask as written by launch_fwd.
hipError_t launch_first_order(const Shape& s, const void* q, const float* kbar, const void* kvc,
                              const uint64_t* sel_mask, const float* lse2, const float* o32,
                              void* out, hipStream_t stream);

hipError_t launch_dense(const Shape& s, const void* q, const void* k, const void* v, void* out,
                        hipStream_t stream);

// Routing baselines over the materialised proxy map.
int64_t select_max_blocks();                      // largest N a proxy row may have
int64_t proxy_map_workgroups(const Shape& s);     // grid size of launch_proxy_map

hipError_t launch_proxy_map(const Shape& s, const float* qbar, const float* kbar, float* shat,
                            hipStream_t stream);

hipError_t launch_select_topk(const Shape& s, const float* shat, int64_t k, uint64_t* sel_mask,
                              int32_t* sel_count, hipStream_t stream);

hipError_t launch_select_topp(const Shape& s, const float* shat, float top_p,
                              uint64_t* sel_mask, int32_t* sel_count, hipStream_t stream);

}  // namespace solattn
