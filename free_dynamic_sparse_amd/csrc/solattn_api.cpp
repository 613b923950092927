// C ABI of the Sol-Attn library: argument checks first, then launches.
// Every check runs before any HIP call, so a bad argument never reaches the
// device and the error paths can be exercised on a machine without a GPU.

#include <math.h>
#include <stdint.h>

#include "solattn.h"
#include "launch.hpp"
#include "noalloc.hpp"

namespace {

constexpr int64_t kMaxSeqLen = int64_t(1) << 22;
constexpr int64_t kMaxGrid = (int64_t(1) << 31) - 1;

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
bool aligned256(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 255u) == 0; }
bool ok_ptr(const void* p) { return p != nullptr && aligned16(p); }
bool ok_opt_ptr(const void* p) { return p == nullptr || aligned16(p); }

// Shape checks shared by every entry point.  Sets *empty for B*H == 0 or L == 0.
int check_shape(const solattn_problem_t* p, solattn::Shape* s, bool* empty) {
  if (p == nullptr) return SOLATTN_E_INVALID_ARG;
  if (p->reserved != 0 || (p->flags & ~SOLATTN_FLAG_EXACT_ONLY) != 0) return SOLATTN_E_INVALID_ARG;
  if (p->batch < 0 || p->heads < 0 || p->seq_len < 0 || p->seq_len > kMaxSeqLen)
    return SOLATTN_E_INVALID_ARG;
  if (p->head_dim != 64 && p->head_dim != 128) return SOLATTN_E_UNSUPPORTED;
  if (p->block != 64 && p->block != 128) return SOLATTN_E_UNSUPPORTED;
  if (isnan(p->scale) || isinf(p->scale)) return SOLATTN_E_INVALID_ARG;
  if (p->batch > 0 && p->heads > kMaxGrid / p->batch) return SOLATTN_E_INVALID_ARG;
  const int64_t bh = p->batch * p->heads;
  const int64_t N = (p->seq_len + p->block - 1) / p->block;
  // the attention grid holds 8 * ceil(N / 8) workgroups per (b, h)
  if (N > 0 && bh > kMaxGrid / (N + 8)) return SOLATTN_E_INVALID_ARG;
  s->bh = bh;
  s->L = p->seq_len;
  s->d = (int)p->head_dim;
  s->block = p->block;
  s->N = N;
  s->chunk = p->chunk;
  s->beta = p->beta;
  s->scale = p->scale > 0.f ? p->scale : (float)(1.0 / sqrt((double)p->head_dim));
  s->flags = p->flags;
  *empty = (bh == 0 || N == 0);
  return SOLATTN_OK;
}

int check_routing(const solattn_problem_t* p) {
  if (isnan(p->beta)) return SOLATTN_E_INVALID_ARG;
  if (p->chunk < 1 || p->chunk > 64) return SOLATTN_E_UNSUPPORTED;
  return SOLATTN_OK;
}

int from_hip(hipError_t e) { return e == hipSuccess ? SOLATTN_OK : SOLATTN_E_HIP; }

// The fused forward's workspace: its work-queue counters.
int check_workspace(const void* ws, size_t bytes, size_t need) {
  if (ws == nullptr || !aligned256(ws) || bytes < need) return SOLATTN_E_WORKSPACE;
  return SOLATTN_OK;
}

// Regions of the first-order workspace, each starting on a 256-byte boundary:
// the fused kernel's work-queue counters, its selection bitmaps
// (u64 [bh, N, ceil(N/64)]), its per-row log2 denominators (f32 [bh, L]) and
// its float32 output (f32 [bh, L, d]).
struct FirstOrderLayout {
  size_t queue, sel, lse2, o32, total;
};

FirstOrderLayout first_order_layout(const solattn::Shape& s) {
  auto up = [](size_t x) { return (x + 255u) & ~(size_t)255u; };
  const size_t w64 = (size_t)((s.N + 63) / 64);
  FirstOrderLayout l;
  l.queue = 0;
  l.sel = up(solattn::fwd_workspace_bytes());
  l.lse2 = l.sel + up((size_t)s.bh * (size_t)s.N * w64 * 8u);
  l.o32 = l.lse2 + up((size_t)s.bh * (size_t)s.L * 4u);
  l.total = l.o32 + up((size_t)s.bh * (size_t)s.L * (size_t)s.d * 4u);
  return l;
}

}  // namespace

extern "C" {

int solattn_pool(const solattn_problem_t* p, const void* q, const void* k, const void* v,
                 float* qbar, float* kbar, float* vhat, void* stream) {
  solattn::Shape s;
  bool empty = false;
  int rc = check_shape(p, &s, &empty);
  if (rc != SOLATTN_OK) return rc;
  if (empty) return SOLATTN_OK;
  if (!ok_ptr(q) || !ok_ptr(k) || !ok_ptr(v) || !ok_ptr(qbar) || !ok_ptr(kbar) || !ok_ptr(vhat))
    return SOLATTN_E_INVALID_ARG;
  return from_hip(solattn::launch_pool(s, q, k, v, qbar, kbar, vhat,
                                       static_cast<hipStream_t>(stream)));
}

int solattn_moments(const solattn_problem_t* p, const float* qbar, const float* kbar,
                    float* kmean, float* kcov, float* tau, float* mu, float* sigma,
                    void* stream) {
  solattn::Shape s;
  bool empty = false;
  int rc = check_shape(p, &s, &empty);
  if (rc != SOLATTN_OK) return rc;
  if (isnan(p->beta)) return SOLATTN_E_INVALID_ARG;
  if (empty) return SOLATTN_OK;
  if (!ok_ptr(qbar) || !ok_ptr(kbar) || !ok_ptr(kmean) || !ok_ptr(kcov) || !ok_ptr(tau) ||
      !ok_opt_ptr(mu) || !ok_opt_ptr(sigma))
    return SOLATTN_E_INVALID_ARG;
  return from_hip(solattn::launch_moments(s, qbar, kbar, kmean, kcov, tau, mu, sigma,
                                          static_cast<hipStream_t>(stream)));
}

size_t solattn_fwd_workspace_bytes(const solattn_problem_t* p) {
  solattn::Shape s;
  bool empty = false;
  if (check_shape(p, &s, &empty) != SOLATTN_OK || empty) return 0;
  return solattn::fwd_workspace_bytes();
}

int solattn_fwd(const solattn_problem_t* p, const void* q, const void* k, const void* v,
                const float* qbar, const float* kbar, const float* vhat, const float* tau,
                void* out, void* workspace, size_t workspace_bytes, uint64_t* sel_mask,
                int32_t* sel_count, void* stream) {
  solattn::Shape s;
  bool empty = false;
  int rc = check_shape(p, &s, &empty);
  if (rc != SOLATTN_OK) return rc;
  rc = check_routing(p);
  if (rc != SOLATTN_OK) return rc;
  if (s.N > solattn::fused_max_blocks()) return SOLATTN_E_UNSUPPORTED;
  if (empty) return SOLATTN_OK;
  if (!ok_ptr(q) || !ok_ptr(k) || !ok_ptr(v) || !ok_ptr(qbar) || !ok_ptr(kbar) ||
      !ok_ptr(vhat) || !ok_ptr(tau) || !ok_ptr(out) || !ok_opt_ptr(sel_mask) ||
      !ok_opt_ptr(sel_count))
    return SOLATTN_E_INVALID_ARG;
  rc = check_workspace(workspace, workspace_bytes, solattn::fwd_workspace_bytes());
  if (rc != SOLATTN_OK) return rc;
  return from_hip(solattn::launch_fwd(s, q, k, v, qbar, kbar, vhat, tau, nullptr, out, sel_mask,
                                      sel_count, nullptr, nullptr, workspace,
                                      static_cast<hipStream_t>(stream)));
}

int solattn_fwd_noalloc(const solattn_problem_t* p, const void* q, const void* k, const void* v,
                        const float* qbar, const float* kbar, const float* vhat, const float* tau,
                        void* out, uint64_t* sel_mask, int32_t* sel_count, void* stream) {
  solattn::Shape s;
  bool empty = false;
  int rc = check_shape(p, &s, &empty);
  if (rc != SOLATTN_OK) return rc;
  rc = check_routing(p);
  if (rc != SOLATTN_OK) return rc;
  if (s.N > solattn::fused_max_blocks()) return SOLATTN_E_UNSUPPORTED;
  if (empty) return SOLATTN_OK;
  if (!ok_ptr(q) || !ok_ptr(k) || !ok_ptr(v) || !ok_ptr(qbar) || !ok_ptr(kbar) ||
      !ok_ptr(vhat) || !ok_ptr(tau) || !ok_ptr(out) || !ok_opt_ptr(sel_mask) ||
      !ok_opt_ptr(sel_count))
    return SOLATTN_E_INVALID_ARG;
  // the scratch array must hold what solattn_fwd's workspace would
  if (solattn::fwd_workspace_bytes() > solattn::noalloc_scratch_bytes())
    return SOLATTN_E_WORKSPACE;
  void* scratch = nullptr;
  if (solattn::noalloc_scratch(&scratch) != hipSuccess) return SOLATTN_E_HIP;
  return from_hip(solattn::launch_fwd(s, q, k, v, qbar, kbar, vhat, tau, nullptr, out, sel_mask,
                                      sel_count, nullptr, nullptr, scratch,
                                      static_cast<hipStream_t>(stream)));
}

int solattn_fwd_masked(const solattn_problem_t* p, const void* q, const void* k, const void* v,
                       const float* kbar, const float* vhat, const uint64_t* sel_in, void* out,
                       void* workspace, size_t workspace_bytes, void* stream) {
  solattn::Shape s;
  bool empty = false;
  int rc = check_shape(p, &s, &empty);
  if (rc != SOLATTN_OK) return rc;
  if (s.N > solattn::fused_max_blocks()) return SOLATTN_E_UNSUPPORTED;
  if (empty) return SOLATTN_OK;
  if (!ok_ptr(q) || !ok_ptr(k) || !ok_ptr(v) || !ok_ptr(kbar) || !ok_ptr(vhat) ||
      !ok_ptr(sel_in) || !ok_ptr(out))
    return SOLATTN_E_INVALID_ARG;
  rc = check_workspace(workspace, workspace_bytes, solattn::fwd_workspace_bytes());
  if (rc != SOLATTN_OK) return rc;
  return from_hip(solattn::launch_fwd(s, q, k, v, nullptr, kbar, vhat, nullptr, sel_in, out,
                                      nullptr, nullptr, nullptr, nullptr, workspace,
                                      static_cast<hipStream_t>(stream)));
}

int solattn_kv_moments(const solattn_problem_t* p, const void* k, const void* v,
                       const float* kbar, const float* vhat, void* kvc, void* stream) {
  solattn::Shape s;
  bool empty = false;
  int rc = check_shape(p, &s, &empty);
  if (rc != SOLATTN_OK) return rc;
  if (empty) return SOLATTN_OK;
  if (!ok_ptr(k) || !ok_ptr(v) || !ok_ptr(kbar) || !ok_ptr(vhat) || !ok_ptr(kvc))
    return SOLATTN_E_INVALID_ARG;
  return from_hip(solattn::launch_kv_moments(s, k, v, kbar, vhat, kvc,
                                             static_cast<hipStream_t>(stream)));
}

size_t solattn_fwd_first_order_workspace(const solattn_problem_t* p) {
  solattn::Shape s;
  bool empty = false;
  if (check_shape(p, &s, &empty) != SOLATTN_OK || empty) return 0;
  return first_order_layout(s).total;
}

int solattn_fwd_first_order(const solattn_problem_t* p, const void* q, const void* k,
                            const void* v, const float* qbar, const float* kbar,
                            const float* vhat, const void* kvc, const float* tau, void* out,
                            void* workspace, size_t workspace_bytes, void* stream) {
  solattn::Shape s;
  bool empty = false;
  int rc = check_shape(p, &s, &empty);
  if (rc != SOLATTN_OK) return rc;
  rc = check_routing(p);
  if (rc != SOLATTN_OK) return rc;
  if (p->flags & SOLATTN_FLAG_EXACT_ONLY) return SOLATTN_E_INVALID_ARG;
  if (s.N > solattn::fused_max_blocks()) return SOLATTN_E_UNSUPPORTED;
  if (empty) return SOLATTN_OK;
  if (!ok_ptr(q) || !ok_ptr(k) || !ok_ptr(v) || !ok_ptr(qbar) || !ok_ptr(kbar) ||
      !ok_ptr(vhat) || !ok_ptr(kvc) || !ok_ptr(tau) || !ok_ptr(out))
    return SOLATTN_E_INVALID_ARG;
  const FirstOrderLayout l = first_order_layout(s);
  rc = check_workspace(workspace, workspace_bytes, l.total);
  if (rc != SOLATTN_OK) return rc;
  char* ws = static_cast<char*>(workspace);
  uint64_t* sel = reinterpret_cast<uint64_t*>(ws + l.sel);
  float* lse2 = reinterpret_cast<float*>(ws + l.lse2);
  float* o32 = reinterpret_cast<float*>(ws + l.o32);
  const hipStream_t st = static_cast<hipStream_t>(stream);
  hipError_t e = solattn::launch_fwd(s, q, k, v, qbar, kbar, vhat, tau, nullptr, nullptr, sel,
                                     nullptr, o32, lse2, ws + l.queue, st);
  if (e != hipSuccess) return SOLATTN_E_HIP;
  return from_hip(solattn::launch_first_order(s, q, kbar, kvc, sel, lse2, o32, out, st));
}

int solattn_dense_fwd(const solattn_problem_t* p, const void* q, const void* k, const void* v,
                      void* out, void* stream) {
  solattn::Shape s;
  bool empty = false;
  int rc = check_shape(p, &s, &empty);
  if (rc != SOLATTN_OK) return rc;
  if (empty) return SOLATTN_OK;
  if (!ok_ptr(q) || !ok_ptr(k) || !ok_ptr(v) || !ok_ptr(out)) return SOLATTN_E_INVALID_ARG;
  return from_hip(solattn::launch_dense(s, q, k, v, out, static_cast<hipStream_t>(stream)));
}

int solattn_proxy_map(const solattn_problem_t* p, const float* qbar, const float* kbar,
                      float* shat, void* stream) {
  solattn::Shape s;
  bool empty = false;
  int rc = check_shape(p, &s, &empty);
  if (rc != SOLATTN_OK) return rc;
  if (empty) return SOLATTN_OK;
  if (solattn::proxy_map_workgroups(s) > kMaxGrid) return SOLATTN_E_INVALID_ARG;
  if (!ok_ptr(qbar) || !ok_ptr(kbar) || !ok_ptr(shat)) return SOLATTN_E_INVALID_ARG;
  return from_hip(solattn::launch_proxy_map(s, qbar, kbar, shat,
                                            static_cast<hipStream_t>(stream)));
}

int solattn_select_topk(const solattn_problem_t* p, const float* shat, int64_t k,
                        uint64_t* sel_mask, int32_t* sel_count, void* stream) {
  solattn::Shape s;
  bool empty = false;
  int rc = check_shape(p, &s, &empty);
  if (rc != SOLATTN_OK) return rc;
  if (k < 1) return SOLATTN_E_INVALID_ARG;
  if (s.N > solattn::select_max_blocks()) return SOLATTN_E_UNSUPPORTED;
  if (empty) return SOLATTN_OK;
  if (!ok_ptr(shat) || !ok_ptr(sel_mask) || !ok_opt_ptr(sel_count)) return SOLATTN_E_INVALID_ARG;
  return from_hip(solattn::launch_select_topk(s, shat, k, sel_mask, sel_count,
                                              static_cast<hipStream_t>(stream)));
}

int solattn_select_topp(const solattn_problem_t* p, const float* shat, float top_p,
                        uint64_t* sel_mask, int32_t* sel_count, void* stream) {
  solattn::Shape s;
  bool empty = false;
  int rc = check_shape(p, &s, &empty);
  if (rc != SOLATTN_OK) return rc;
  if (!(top_p > 0.f && top_p <= 1.f)) return SOLATTN_E_INVALID_ARG;
  if (s.N > solattn::select_max_blocks()) return SOLATTN_E_UNSUPPORTED;
  if (empty) return SOLATTN_OK;
  if (!ok_ptr(shat) || !ok_ptr(sel_mask) || !ok_opt_ptr(sel_count)) return SOLATTN_E_INVALID_ARG;
  return from_hip(solattn::launch_select_topp(s, shat, top_p, sel_mask, sel_count,
                                              static_cast<hipStream_t>(stream)));
}

const char* solattn_strerror(int code) {
  switch (code) {
    case SOLATTN_OK:
      return "ok";
    case SOLATTN_E_INVALID_ARG:
      return "invalid argument (null or misaligned pointer, bad shape, NaN beta or scale, "
             "k < 1, top_p outside (0, 1], or the first-order forward asked for in "
             "exact-only mode)";
    case SOLATTN_E_UNSUPPORTED:
      return "unsupported configuration (head_dim and block must be 64 or 128, chunk 1..64, "
             "and solattn_fwd and the top-k / top-p selections need ceil(seq_len / block) "
             "<= 8192)";
    case SOLATTN_E_HIP:
      return "HIP launch failed";
    case SOLATTN_E_WORKSPACE:
      return "workspace missing, not 256-byte aligned, or smaller than the entry point's "
             "workspace size (solattn_fwd_workspace_bytes, solattn_fwd_first_order_workspace)";
    default:
      return "unknown error code";
  }
}

int solattn_version(void) { return 300; }

}  // extern "C"
