/*
 * solattn.h - C ABI of the Sol-Attn sparse-attention forward pass on AMD
 * Instinct MI355X (gfx950).
 *
 * Method: "Sol-Attn: Accelerating Video Generation Inference via On-the-Fly
 * Attention Sparsification" (arXiv 2607.24027).  One forward call is
 *   solattn_pool     -> block proxies Qbar, Kbar and summed values Vhat
 *   solattn_moments  -> pooled-key moments and per-query-block thresholds tau
 *   solattn_fwd      -> the fused nested-loop attention kernel
 * and solattn_dense_fwd is plain dense softmax attention on the same core,
 * kept as the in-house comparison point.  solattn_proxy_map with
 * solattn_select_topk / solattn_select_topp are the top-k and top-p routing
 * baselines the page compares its routing with.  solattn_kv_moments with
 * solattn_fwd_first_order keep the first-order term of the expansion whose
 * zeroth-order term the page uses for unselected blocks.
 *
 * Conventions shared by every entry point
 * - Tensors are contiguous row-major device memory.  Q, K, V and O are
 *   bfloat16 [B, H, L, d]; pooled and per-block arrays are float32.
 * - Blocks: N = ceil(L / block) query blocks and N key blocks per (b, h);
 *   block j holds tokens [j*block, min(L, (j+1)*block)), n_j of them.
 * - Every device pointer must be 16-byte aligned.  The caller owns every
 *   buffer; the library never allocates, frees or synchronises.
 * - Calls are asynchronous on `stream` (a hipStream_t; NULL is the null
 *   stream).  All arguments are checked before any HIP call, so a bad
 *   argument returns an error without touching the device.  A device fault
 *   shows at the caller's next synchronisation.
 * - B*H == 0 or L == 0 is a valid empty problem: the call returns
 *   SOLATTN_OK and launches nothing.
 * - Calls that write the same output buffers and overlap on one device
 *   race; calls on distinct buffers may overlap freely.
 */
#ifndef SOLATTN_H_
#define SOLATTN_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Return codes. */
#define SOLATTN_OK 0
#define SOLATTN_E_INVALID_ARG (-1) /* null pointer, bad shape, NaN beta, misalignment */
#define SOLATTN_E_UNSUPPORTED (-2) /* head_dim, block or chunk outside the built set */
#define SOLATTN_E_HIP (-3)         /* a HIP launch failed; see hipGetLastError */
#define SOLATTN_E_WORKSPACE (-4)   /* workspace NULL, not 256-byte aligned, or too small */

/* solattn_problem_t.flags */
#define SOLATTN_FLAG_EXACT_ONLY 1u /* drop the approximation of unselected blocks */

/*
 * Problem description (host memory, read during the call only).
 *  batch, heads, seq_len  B, H, L; each >= 0, L <= 2^22, B*H < 2^31.
 *  head_dim               d: 64 or 128.
 *  block                  tokens per block, 64 or 128 (the page uses square
 *                         block x block tiles for queries and keys alike).
 *  chunk                  C, pooled keys per routing chunk, 1..64.  On the
 *                         page C changes the schedule, never the result
 *                         (method section, chunk-wise streaming
 *                         thresholding: the selected set is the union of
 *                         the chunks' sets).  Here it is validated and has
 *                         no other effect: the fused kernel routes 64 pooled
 *                         keys per step (32 with 64-token blocks) whatever its
 *                         value, and every output bit is the same for every C.
 *  beta                   standardized cutoff of tau_i = mu_i + beta*sigma_i
 *                         (Eq. 4).  Any finite value; -INFINITY selects every
 *                         block, +INFINITY none.  NaN is rejected.
 *  scale                  softmax scale; <= 0 means 1/sqrt(head_dim).
 *  flags                  SOLATTN_FLAG_* bits; unknown bits are rejected.
 *  reserved               must be 0.
 */
typedef struct solattn_problem {
  int64_t batch;
  int64_t heads;
  int64_t seq_len;
  int64_t head_dim;
  int32_t block;
  int32_t chunk;
  float beta;
  float scale;
  uint32_t flags;
  uint32_t reserved;
} solattn_problem_t;

/*
 * Block pooling (method section, block proxies of Eq. 3 and the summed
 * values Vhat_j of Eqs. 9-10).
 *   q, k, v  in:  bf16 [B, H, L, d]
 *   qbar     out: f32 [B, H, N, d]  Qbar_i = mean of block i's query rows
 *   kbar     out: f32 [B, H, N, d]  Kbar_j = mean of block j's key rows
 *   vhat     out: f32 [B, H, N, d]  Vhat_j = sum of block j's value rows
 * A ragged last block is pooled over its n_j valid tokens.  Accumulation is
 * float32 in a fixed order, so results are deterministic.  Reads 3*B*H*L*d
 * bf16 once.
 */
int solattn_pool(const solattn_problem_t* p, const void* q, const void* k, const void* v,
                 float* qbar, float* kbar, float* vhat, void* stream);

/*
 * Pooled-key moments and routing thresholds (method section, query-dependent
 * threshold routing, Eq. 4, with the moment identity of Appendix B).
 *   qbar, kbar  in:  f32 [B, H, N, d]  from solattn_pool
 *   kmean       out: f32 [B, H, d]     m = (1/N) sum_j Kbar_j
 *   kcov        out: f32 [B, H, d, d]  (1/N) sum_j (Kbar_j - m)(Kbar_j - m)^T
 *   tau         out: f32 [B, H, N]     tau_i = mu_i + beta*sigma_i
 *   mu, sigma   out: f32 [B, H, N], each may be NULL
 *               mu_i = scale*Qbar_i.m, sigma_i = scale*sqrt(Qbar_i^T Sigma Qbar_i):
 *               mean and population std of the proxy row scale*Qbar_i Kbar^T,
 *               without building the N x N map.
 * tau_i is -INFINITY when beta is -INFINITY or sigma_i == 0 (a constant row:
 * every block passes the >= test), +INFINITY when beta is +INFINITY.
 * m and Sigma accumulate in float64 (Sigma is exactly symmetric); mu and sigma
 * in float32.  Every sum has a fixed order, so results are deterministic.
 */
int solattn_moments(const solattn_problem_t* p, const float* qbar, const float* kbar,
                    float* kmean, float* kcov, float* tau, float* mu, float* sigma,
                    void* stream);

/*
 * The fused Sol-Attn forward (method section: chunk-wise streaming
 * thresholding, Eqs. 6-7; zeroth-order approximation and the combined
 * denominator and numerator, Eqs. 9-10; the token-to-block tile, Eq. 11;
 * the nested-loop kernel of Algorithm 3.2 and Figure 4).
 *   q, k, v    in:  bf16 [B, H, L, d]
 *   qbar       in:  f32 [B, H, N, d]  from solattn_pool (routing scores)
 *   kbar, vhat in:  f32 [B, H, N, d]  from solattn_pool (KC and VC chunks)
 *   tau        in:  f32 [B, H, N]     from solattn_moments
 *   out        out: bf16 [B, H, L, d]
 *   workspace  device memory of workspace_bytes >= solattn_fwd_workspace_bytes(p)
 *              bytes, 256-byte aligned, owned by the caller; its contents on
 *              entry do not matter.  It holds the counters of the work queues
 *              from which persistent workgroups take pairs of query blocks
 *              (per-row budgets |S_i| depend on the query, method section,
 *              Eq. 4, so items take unequal time); a kernel in the same
 *              stream clears them at the start of every call, so the call
 *              can be captured in a HIP graph.  Calls that share a workspace
 *              and overlap race.  NULL, misaligned or too small:
 *              SOLATTN_E_WORKSPACE.
 *   sel_mask   out, may be NULL: u64 [B, H, N, ceil(N/64)]; bit (j mod 64) of
 *              word j/64 of row (b, h, i) is set iff block j is in S_i.
 *   sel_count  out, may be NULL: i32 [B, H, N], |S_i|.
 * For query block i the kernel scans the pooled keys 64 at a time (32 with
 * 64-token blocks): the
 * proxy score shat_ij = scale*Qbar_i.Kbar_j is compared with tau_i on chip;
 * selected blocks get exact attention, unselected blocks the zeroth-order
 * term (n_j * exp(centre) in the denominator, exp(centre) * Vhat_j in the
 * numerator, centre = scale*q_r.Kbar_j), all in one online softmax.
 * Nothing about the selection is written to memory unless sel_mask or
 * sel_count is given.  With SOLATTN_FLAG_EXACT_ONLY unselected blocks are
 * dropped and a row with no selected block outputs 0.
 * Limit: N = ceil(L / block) <= 8192 (the selection bits of a query block
 * stay on chip); larger N returns SOLATTN_E_UNSUPPORTED.
 */
int solattn_fwd(const solattn_problem_t* p, const void* q, const void* k, const void* v,
                const float* qbar, const float* kbar, const float* vhat, const float* tau,
                void* out, void* workspace, size_t workspace_bytes, uint64_t* sel_mask,
                int32_t* sel_count, void* stream);

/* Workspace bytes solattn_fwd and solattn_fwd_masked need (the same for
 * every problem: 1 KiB); 0 for an empty or invalid problem, whose call needs
 * none. */
size_t solattn_fwd_workspace_bytes(const solattn_problem_t* p);

/*
 * solattn_fwd for callers that cannot allocate device memory (code under HIP
 * graph capture, tight serving loops, harnesses that forbid allocation): the
 * same kernels, arguments and results, with the work-queue counters in a
 * file-scope device array of the library (1 KiB, the most solattn_fwd's
 * workspace ever needs; each GPU the library runs on holds one copy until
 * the process ends) instead of a caller's workspace.  A problem needing more
 * would return SOLATTN_E_WORKSPACE.  The call allocates and frees nothing;
 * the caller still passes every input and output.  Every call on one GPU
 * shares that GPU's array, which the call clears in-stream before use:
 * calls that overlap on one GPU (different streams, or concurrent host
 * threads) race and must be serialised by the caller.
 */
int solattn_fwd_noalloc(const solattn_problem_t* p, const void* q, const void* k, const void* v,
                        const float* qbar, const float* kbar, const float* vhat, const float* tau,
                        void* out, uint64_t* sel_mask, int32_t* sel_count, void* stream);

/*
 * The fused forward with the selected sets given instead of routed: the
 * same kernel and arithmetic as solattn_fwd (exact attention over the given
 * blocks, the zeroth-order terms of every other block unless
 * SOLATTN_FLAG_EXACT_ONLY), for comparing routing rules at identical block
 * indices (the page's comparisons at identical selections, experiments
 * section, Figures 7 and 8).
 *   q, k, v    in:  bf16 [B, H, L, d]
 *   kbar, vhat in:  f32 [B, H, N, d]  from solattn_pool
 *   sel_in     in:  u64 [B, H, N, ceil(N/64)], solattn_fwd's sel_mask layout
 *              (e.g. from solattn_select_topk / solattn_select_topp); bits
 *              at or past N are ignored
 *   out        out: bf16 [B, H, L, d]
 *   workspace  as for solattn_fwd
 * beta and chunk are ignored.  Same limit as solattn_fwd (N <= 8192).
 */
int solattn_fwd_masked(const solattn_problem_t* p, const void* q, const void* k, const void* v,
                       const float* kbar, const float* vhat, const uint64_t* sel_in, void* out,
                       void* workspace, size_t workspace_bytes, void* stream);

/*
 * First-order term of the unselected blocks.  The page expands an
 * unselected block's exponential score matrix exp(S_ij) around the
 * row-wise mean score within the block, c_r = scale*q_r.Kbar_j, and keeps
 * the zeroth-order term (method section, the expansion before Eqs. 9-10).
 * The first-order term exp(c_r)*(S_rt - c_r) sums to zero over the block's
 * keys, so the denominator is unchanged, and adds
 * exp(c_r) * scale * q_r^T C_j to the numerator, with the block moment
 *   C_j = sum over block j's valid tokens t of (k_t - Kbar_j) v_t^T  (d x d).
 *
 * solattn_kv_moments: C_j of every block.
 *   k, v        in:  bf16 [B, H, L, d]
 *   kbar, vhat  in:  f32 [B, H, N, d]  from solattn_pool
 *   kvc         out: bf16 [B, H, N, d, d], value dimension first:
 *                    element [b][h][j][e][a] is C_j[a][e] (key dim a, value dim e)
 * Formed as K_j^T V_j - Kbar_j Vhat_j^T: products of the bf16 inputs
 * accumulate in float32, the pooled outer product is subtracted in float32
 * and the result is rounded to bf16 once.  beta, chunk and flags are
 * ignored.
 *
 * solattn_fwd_first_order: solattn_fwd (threshold routing, exact selected
 * blocks, zeroth-order unselected blocks) with the first-order term of every
 * unselected block added, so that row r of query block i is
 *   O_r = (N_r + sum_{j in U_i} exp(c_rj) scale q_r^T C_j) / D_r
 * with N_r and D_r the zeroth-order numerator and denominator (Eqs. 9-10).
 *   q, k, v, qbar, kbar, vhat, tau, out  as for solattn_fwd
 *   kvc        in: bf16 [B, H, N, d, d] from solattn_kv_moments
 *   workspace  device scratch of workspace_bytes >=
 *              solattn_fwd_first_order_workspace(p) bytes, 256-byte aligned;
 *              its contents on entry do not matter and are overwritten (the
 *              fused kernel's work-queue counters, and the selection
 *              bitmaps, the per-row denominators and O in float32, passed
 *              between the two kernels of the call)
 * Two kernels: the fused forward writes float32 O, its log denominators and
 * the bitmaps to the workspace; a second kernel adds the first-order terms
 * (an MFMA product C_j^T q_r per query row and unselected block: 2 n_i d^2
 * FLOPs per block pair) and rounds O to bf16 once.  Calls that share a
 * workspace race.  SOLATTN_FLAG_EXACT_ONLY is refused
 * (SOLATTN_E_INVALID_ARG): the first-order term extends the zeroth-order
 * one.  A workspace that is NULL, misaligned or smaller than required is
 * SOLATTN_E_WORKSPACE.  Same limit as solattn_fwd (N <= 8192).
 *
 * solattn_fwd_first_order_workspace: the workspace size in bytes; 0 for an
 * empty or invalid problem.
 */
int solattn_kv_moments(const solattn_problem_t* p, const void* k, const void* v,
                       const float* kbar, const float* vhat, void* kvc, void* stream);
size_t solattn_fwd_first_order_workspace(const solattn_problem_t* p);
int solattn_fwd_first_order(const solattn_problem_t* p, const void* q, const void* k,
                            const void* v, const float* qbar, const float* kbar,
                            const float* vhat, const void* kvc, const float* tau, void* out,
                            void* workspace, size_t workspace_bytes, void* stream);
/*
 * Dense softmax attention softmax(scale * Q K^T) V on the same MFMA core,
 * block by block with one online softmax (no routing).  This is an in-house
 * comparison point with no definition on the page (the page compares with
 * dense FlashAttention-3 on its own hardware); it is textbook attention, the
 * limit beta = -inf of the method.  beta, chunk and flags are ignored; block
 * picks the tile size.
 *   q, k, v in: bf16 [B, H, L, d];  out: bf16 [B, H, L, d]
 */
int solattn_dense_fwd(const solattn_problem_t* p, const void* q, const void* k, const void* v,
                      void* out, void* stream);

/*
 * Routing baselines the page compares threshold routing with (method section
 * after Eq. 4; the selection-latency comparison of Figure 5(b) and the
 * density spread of Figure 7).  Not part of the Sol-Attn forward: they
 * materialise the N x N proxy map that the method never builds.
 *
 * solattn_proxy_map: shat_ij = scale * Qbar_i . Kbar_j (Eq. 3) for every
 * query block i and key block j of each (b, h).
 *   qbar, kbar in:  f32 [B, H, N, d]  from solattn_pool
 *   shat       out: f32 [B, H, N, N]
 * Float32 dot products in order of d.  beta, chunk and flags are ignored.
 * B*H*ceil(N/64)^2 must stay below 2^31.
 */
int solattn_proxy_map(const solattn_problem_t* p, const float* qbar, const float* kbar,
                      float* shat, void* stream);

/*
 * solattn_select_topk: top-k routing, S_i = the k largest entries of proxy
 * row i (all N when k >= N); equal scores are taken in increasing block
 * index.  solattn_select_topp: top-p routing, S_i = the shortest run of row
 * i's largest entries (same order) whose softmax mass reaches top_p, with
 * weights w_j = exp(shat_ij) / sum_l exp(shat_il) over the row's N blocks,
 * at least one block; top_p = 1 selects the whole row.  Cumulative sums are
 * float32 over the sorted row.
 *   shat       in:  f32 [B, H, N, N]  from solattn_proxy_map
 *   k          >= 1 (else SOLATTN_E_INVALID_ARG)
 *   top_p      in (0, 1] (else SOLATTN_E_INVALID_ARG; NaN included)
 *   sel_mask   out: u64 [B, H, N, ceil(N/64)], the same bitmap layout as
 *              solattn_fwd's sel_mask
 *   sel_count  out, may be NULL: i32 [B, H, N], |S_i|
 * Limit: N <= 8192 (a row is sorted in on-chip memory); larger N returns
 * SOLATTN_E_UNSUPPORTED.
 */
int solattn_select_topk(const solattn_problem_t* p, const float* shat, int64_t k,
                        uint64_t* sel_mask, int32_t* sel_count, void* stream);
int solattn_select_topp(const solattn_problem_t* p, const float* shat, float top_p,
                        uint64_t* sel_mask, int32_t* sel_count, void* stream);

/* Static text for a return code. */
const char* solattn_strerror(int code);

/* Library version, major*10000 + minor*100 + patch. */
int solattn_version(void);

#ifdef __cplusplus
}
#endif

#endif /* SOLATTN_H_ */
