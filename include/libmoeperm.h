/*
 * libmoeperm -- single-GPU MoE expert hot path for MI355X (gfx950 / CDNA4):
 * token permute, rank-major -> expert-major reorder, grouped SwiGLU GEMM,
 * weighted unpermute-combine and the unpermute backward.
 *
 * Conventions shared by every call
 * --------------------------------
 *  - Every tensor pointer is DEVICE memory owned by the caller. The library
 *    never allocates, frees or keeps a pointer past the call.
 *  - Token / expert rows are contiguous row-major bfloat16, passed as void*
 *    (uint16 bit patterns). Row pointers must be 16-byte aligned and the row
 *    length H a multiple of 8 (rows move as 16-byte vectors). Index tensors are
 *    int32, probabilities and coefficients float32, 4-byte aligned.
 *  - Every call only ENQUEUES work on `stream` and returns without a host
 *    synchronisation: outputs are valid when the stream reaches that point.
 *    Nothing in the path reads a device value back to the host; buffers are
 *    sized at their capacity (T*K rows for a permute) instead.
 *  - Arguments are validated on the host before anything is enqueued. On any
 *    status other than MOE_OK nothing was enqueued (MOE_ERR_HIP: a launch
 *    failed; earlier launches of the same call may have been enqueued).
 *  - Data-dependent problems that cannot be seen without a device read
 *    (an expert id out of range, a row index outside a buffer) are not errors:
 *    such a slot is dropped (no row, contributes 0), never an out-of-bounds
 *    access.
 *  - Workspaces are caller-allocated device memory of at least the size the
 *    matching *_workspace_size call returns; their contents are undefined
 *    afterwards. Calls that share one workspace on one stream are fine; calls
 *    that overlap in time must use different workspaces.
 *  - The library holds no global state, and calls are re-entrant, with one
 *    exception: moe_permute_noalloc keeps its count table in a device array
 *    that the library owns (one per GPU, 64 KiB).
 *
 * Source passages (page title, then section):
 *  [EP]  "Coverage for hyper_parallel/core/expert_parallel/expert_parallel.py"
 *        -- _generate_permute_indices, _permute, _unpermute.
 *  [CV2] "torch_npu.npu_moe_distribute_combine_v2" -- 功能说明 / 计算公式
 *        (the combine sum and the special-expert formulas), 参数说明,
 *        约束说明.
 *  [UNP] "[sync] PR-40312: Update moe token unpermute DTensor support" --
 *        主要改动 (npu_moe_token_unpermute and its grad_v2).
 *  [GMM] "feat(moe): NPU平台 EP experts forward计算改用 NPU grouped matmul"
 *        -- PR description (grouped matmul + swiglu; permute as x[idx]).
 */
#ifndef LIBMOEPERM_H
#define LIBMOEPERM_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum moe_status {
    MOE_OK = 0,
    MOE_ERR_INVALID_ARG = 1, /* bad size, null or misaligned pointer */
    MOE_ERR_UNSUPPORTED = 2, /* legal on the pages but outside this library (H % 8, K > 16) */
    MOE_ERR_WORKSPACE = 3,   /* workspace null or smaller than required */
    MOE_ERR_HIP = 4          /* a HIP launch or runtime call failed */
} moe_status_t;

/* Static, human-readable name of a status. Never NULL. */
const char* moe_status_str(moe_status_t status);

/* Version of this ABI (bumped on any signature change). */
int32_t moe_abi_version(void);

/* Limits enforced by the host checks. */
#define MOE_MAX_TOPK 16         /* [CV2] 约束说明: 0 < K <= 16 */
#define MOE_MAX_EXPERTS 1024    /* [CV2] 参数说明 moe_expert_num: [1, 1024] */
#define MOE_MAX_DERED_CELLS (1 << 22)  /* oep_size * num_experts of the deredundency count table */
#define MOE_MAX_REORDER_BLOCKS 65536 /* R * E_local */

/* ------------------------------------------------------------------------
 * moe_permute -- stable expert-major token permute.
 *
 * [EP] _permute (x[permuted_indices]) and _generate_permute_indices (order
 * inside a block kept); [GMM] (permute as advanced indexing x[idx]).
 * Slots s = t*K + k (row-major expert_ids [T,K]) with 0 <= id < E are
 * bucketed by id, stably: the row of slot s is
 *     expert_offsets[id] + #{ s' < s : id(s') == id }.
 * Slots whose id is outside [0, E) (special experts of [CV2], which own no
 * row) get row_of_slot = -1, and so do slots outside the active mask.
 *
 *  x              bf16 [T, H]                       in  (may be NULL iff permuted is NULL)
 *  expert_ids     int32 [T, K]                      in
 *  active_mask    uint8 [T] or [T, K]               in  (nullable: every slot takes part)
 *  mask_per_slot  0: active_mask is [T], one flag per token; 1: [T, K], one per slot
 *                 ([CV2] 参数说明 x_active_mask: nonzero = the token / slot takes
 *                 part in the exchange; a [T] mask should hold its trues first,
 *                 but any pattern is applied flag by flag)
 *  permuted       bf16 [T*K, H] capacity            out rows [0, N) written, N = expert_offsets[E];
 *                                                       NULL: index maps only
 *  sorted_slot    int32 [T*K]                       out row -> slot, -1 for rows [N, T*K)
 *  row_of_slot    int32 [T*K]                       out slot -> row, -1 for non-real slots
 *  expert_counts  int32 [E]                         out rows per expert
 *  expert_offsets int32 [E+1]                       out exclusive prefix, [E] = N
 *  workspace      >= moe_permute_workspace_size(T, K, E)
 * Errors: INVALID_ARG for T < 0, K outside [1,16], E outside [1,1024], H <= 0,
 * T*K > INT32_MAX, mask_per_slot not 0 or 1, a required pointer NULL or
 * misaligned; UNSUPPORTED for H % 8 != 0; WORKSPACE if too small.
 * ------------------------------------------------------------------------ */
moe_status_t moe_permute_workspace_size(int64_t T, int32_t K, int32_t E, size_t* bytes);
moe_status_t moe_permute(const void* x, const int32_t* expert_ids, const uint8_t* active_mask,
                         int32_t mask_per_slot, int64_t T, int32_t H, int32_t K,
                         int32_t num_experts, void* permuted, int32_t* sorted_slot,
                         int32_t* row_of_slot, int32_t* expert_counts, int32_t* expert_offsets,
                         void* workspace, size_t workspace_bytes, hipStream_t stream);

/* ------------------------------------------------------------------------
 * moe_permute_rows -- the row move of the permute alone, for a routing that
 * is already resolved.
 *
 * [EP] _permute (x gathered by precomputed permuted_indices): every token's
 * row is copied to the rows its slots own,
 *     permuted[row_of_slot[t*K + k]] = x[t]   for row_of_slot[t*K + k] in [0, N),
 * e.g. a second [T, H] tensor moved with the routing of an earlier
 * moe_permute call. Rows that no slot names are left as they are; slots
 * outside [0, N) are skipped.
 *
 *  x            bf16 [T, H]    in
 *  row_of_slot  int32 [T, K]   in  (moe_permute's output)
 *  permuted     bf16 [N, H]    out
 * Errors: INVALID_ARG for T < 0, K outside [1,16], T*K > INT32_MAX, H <= 0, N
 * outside [0, INT32_MAX], a required pointer NULL or misaligned; UNSUPPORTED
 * for H % 8 != 0.
 * ------------------------------------------------------------------------ */
moe_status_t moe_permute_rows(const void* x, const int32_t* row_of_slot, int64_t T, int32_t H,
                              int32_t K, int64_t N, void* permuted, hipStream_t stream);

/* ------------------------------------------------------------------------
 * moe_permute_noalloc -- moe_permute without a workspace argument, for
 * callers that cannot allocate device memory: code under HIP graph capture,
 * tight serving loops, harnesses that forbid hipMalloc.
 *
 * Same arguments, outputs and checks as moe_permute, minus the workspace. The
 * count table lives in a 64 KiB device array of the library, one per GPU,
 * kept until the process ends; the call allocates nothing. Every table size
 * the permute's planner makes fits (at most 16,384 int32 entries); a larger
 * one would be refused with MOE_ERR_WORKSPACE. The first call on a GPU looks
 * up that GPU's array (MOE_ERR_HIP if the lookup fails). Calls on one GPU
 * share its array: calls on the same stream are fine, calls that overlap in
 * time on different streams of one GPU race and must not be issued.
 * ------------------------------------------------------------------------ */
moe_status_t moe_permute_noalloc(const void* x, const int32_t* expert_ids,
                                 const uint8_t* active_mask, int32_t mask_per_slot, int64_t T,
                                 int32_t H, int32_t K, int32_t num_experts, void* permuted,
                                 int32_t* sorted_slot, int32_t* row_of_slot,
                                 int32_t* expert_counts, int32_t* expert_offsets,
                                 hipStream_t stream);

/* ------------------------------------------------------------------------
 * moe_rank_to_expert_reorder -- receive buffer, rank-major -> expert-major.
 *
 * [EP] _generate_permute_indices + _permute. The received rows are laid out
 * as blocks (r, e) in r-major order, block (r, e) holding counts[r*E_local+e]
 * rows. Expert compute wants blocks in (e, r) order; order inside a block is
 * kept. perm[i] is the source row of destination row i (the page's
 * permuted_indices); inv_perm is its inverse.
 *
 *  x_rank_major      bf16 [N, H]        in  (NULL iff y_expert_major is NULL)
 *  counts            int32 [R*E_local]  in  device; must be >= 0 (negative reads as 0)
 *  N                 row capacity of x / y / perm / inv_perm; the rows used are
 *                    total = sum(counts). Destination rows [total, N) get perm = -1
 *                    and are not written; inv_perm[j] = -1 for j in [total, N).
 *                    A destination or source index >= N is dropped.
 *  y_expert_major    bf16 [N, H]        out (NULL: index maps only)
 *  perm              int32 [N]          out
 *  inv_perm          int32 [N]          out (nullable)
 *  tokens_per_expert int32 [E_local]    out sum over r of counts[r, e]
 *  expert_offsets    int32 [E_local+1]  out exclusive prefix of tokens_per_expert
 * Errors: INVALID_ARG for R < 1, E_local < 1, R*E_local > 65536, N < 0,
 * N > INT32_MAX, H <= 0 (when rows are moved), NULL / misaligned pointers;
 * UNSUPPORTED for H % 8 != 0; WORKSPACE if too small.
 * ------------------------------------------------------------------------ */
moe_status_t moe_rank_to_expert_reorder_workspace_size(int32_t R, int32_t E_local, size_t* bytes);
moe_status_t moe_rank_to_expert_reorder(const void* x_rank_major, const int32_t* counts, int32_t R,
                                        int32_t E_local, int64_t N, int32_t H,
                                        void* y_expert_major, int32_t* perm, int32_t* inv_perm,
                                        int32_t* tokens_per_expert, int32_t* expert_offsets,
                                        void* workspace, size_t workspace_bytes,
                                        hipStream_t stream);

/* ------------------------------------------------------------------------
 * moe_grouped_gemm_swiglu -- per-expert SwiGLU FFN over expert-major rows.
 *
 * [GMM] (one grouped matmul + swiglu over all expert groups instead of a
 * loop over experts). For each expert e and each row n in
 * [expert_offsets[e], expert_offsets[e+1]):
 *     g = x[n] . w_gate[e]     u = x[n] . w_up[e]      (fp32 accumulate)
 *     h[n] = bf16( silu(g) * u ),  silu(z) = z / (1 + exp(-z))
 *     y[n] = bf16( h[n] . w_down[e] )                  (fp32 accumulate)
 * bf16 MFMA with fp32 accumulation; g and u are never rounded before SwiGLU.
 * Empty experts cost nothing; rows past expert_offsets[E] are not written.
 *
 *  x               bf16 [N_cap, H]   in  expert-major (e.g. moe_permute's output)
 *  expert_offsets  int32 [E+1]       in  device; non-decreasing, [0] = 0, [E] <= N_cap
 *  w_gate, w_up    bf16 [E, H, I]    in
 *  w_down          bf16 [E, I, H]    in
 *  h               bf16 [N_cap, I]   out
 *  y               bf16 [N_cap, H]   out
 *  preact          fp32 [N_cap, 2I]  out (nullable, 16-byte aligned): when not
 *                  NULL, the pre-activations are kept for the backward, g in
 *                  columns [0, I) and u in [I, 2I) of each written row, exactly
 *                  the fp32 values the SwiGLU used (rows past
 *                  expert_offsets[E] are not written)
 * Errors: INVALID_ARG for E outside [1,1024], N_cap < 0 or > INT32_MAX,
 * H <= 0, I <= 0, NULL / misaligned pointers; UNSUPPORTED unless H % 64 == 0
 * and I % 64 == 0, and for H or I above 2^20; WORKSPACE if too small. Offsets that break the stated
 * contract are clamped on device to [0, N_cap] (no out-of-bounds access).
 * ------------------------------------------------------------------------ */
moe_status_t moe_grouped_gemm_swiglu_workspace_size(int32_t E, int64_t N_cap, int32_t H,
                                                    int32_t I, size_t* bytes);
moe_status_t moe_grouped_gemm_swiglu(const void* x, const int32_t* expert_offsets, int32_t E,
                                     int64_t N_cap, int32_t H, int32_t I, const void* w_gate,
                                     const void* w_up, const void* w_down, void* h, void* y,
                                     float* preact, void* workspace, size_t workspace_bytes,
                                     hipStream_t stream);

/* ------------------------------------------------------------------------
 * moe_grouped_gemm_swiglu_grad -- backward of moe_grouped_gemm_swiglu.
 *
 * [GMM] (the grouped matmul + swiglu of the forward, differentiated for
 * training). For each expert e and row n of its group, with dy = dL/dy:
 *     dh = dy . w_down[e]^T            g, u: the forward's preact, or recomputed from x
 *     s = 1 / (1 + exp(-g)),  dg = dh * u * s * (1 + g * (1 - s)),  du = dh * g * s
 *     dx[n] = dg . w_gate[e]^T + du . w_up[e]^T
 *     dw_gate[e] = sum_n x[n]^T dg,  dw_up[e] = sum_n x[n]^T du,
 *     dw_down[e] = sum_n h[n]^T dy[n]
 * bf16 MFMA with fp32 accumulation; dh and [dg | du] are kept in the
 * workspace as bf16; h is the forward's output (as stored). Experts without
 * rows get zero weight gradients; rows of dx past expert_offsets[E] are not
 * written.
 *
 *  x, expert_offsets, w_gate, w_up, w_down   as for moe_grouped_gemm_swiglu
 *  h        bf16 [N_cap, I]   in  the forward's h
 *  dy       bf16 [N_cap, H]   in
 *  dx       bf16 [N_cap, H]   out
 *  dw_gate, dw_up  bf16 [E, H, I]   out
 *  dw_down         bf16 [E, I, H]   out
 *  preact   fp32 [N_cap, 2I]  in (nullable, 16-byte aligned): the forward's
 *           pre-activations (moe_grouped_gemm_swiglu's preact, same x, weights
 *           and offsets). When given, the gate/up GEMM is not run again and dh
 *           is not stored: [dg | du] comes straight out of the dh GEMM. The
 *           results are the same bits either way; NULL recomputes g and u
 *           (2 N_cap H I more multiply-adds, no [N_cap, 2I] fp32 buffer).
 *  workspace  moe_grouped_gemm_swiglu_grad_workspace_size bytes, 256-byte
 *             aligned (about 6 * N_cap * I bytes: dh and [dg | du])
 * Errors: as moe_grouped_gemm_swiglu (INVALID_ARG, UNSUPPORTED unless
 * H % 64 == 0 and I % 64 == 0 or for H or I above 2^20, WORKSPACE).
 * ------------------------------------------------------------------------ */
moe_status_t moe_grouped_gemm_swiglu_grad_workspace_size(int32_t E, int64_t N_cap, int32_t H,
                                                         int32_t I, size_t* bytes);
moe_status_t moe_grouped_gemm_swiglu_grad(const void* x, const int32_t* expert_offsets, int32_t E,
                                          int64_t N_cap, int32_t H, int32_t I, const void* w_gate,
                                          const void* w_up, const void* w_down, const void* h,
                                          const void* dy, void* dx, void* dw_gate, void* dw_up,
                                          void* dw_down, const float* preact, void* workspace,
                                          size_t workspace_bytes, hipStream_t stream);

/* ------------------------------------------------------------------------
 * moe_unpermute_combine -- weighted top-K combine back to token order.
 *
 * [CV2] 计算公式: x = Sum(expert_scales * expert_out + shared_expert_x), with
 * the zero / copy / constant expert outputs Moe(ori_x) = 0, ori_x and
 * alpha_1 * ori_x + alpha_2 * const_expert_v; 参数说明 (expert_scales): the
 * shared expert carries no weight and is added once. [EP] _unpermute.
 *     out[t] = bf16( sum_k p[t,k] * v_k(t) + shared_x[t] )      (fp32 accumulate, k order)
 * with, for slot s = t*K + k and id = expert_ids[s]:
 *     id in [0, E)                 v = expert_out[row], row = row_of_slot[s], or
 *                                      row_map[row_of_slot[s]] when row_map != NULL
 *     id in [E, E+Z)               v = 0                      (zero expert)
 *     id in [E+Z, E+Z+C)           v = ori_x[t]               (copy expert)
 *     id in [E+Z+C, E+Z+C+Nc)      v = alpha1*ori_x[t] + alpha2*const_v[c], c = id-(E+Z+C)
 *     otherwise                    slot dropped
 * A routed slot whose row is outside [0, N) is dropped. row_map lets the
 * combine read a buffer that was reordered after the permute (for instance
 * by moe_rank_to_expert_reorder: row_map = inv_perm), fusing the inverse
 * reorder into the gather.
 *
 *  expert_out   bf16 [N, H]   in (may be NULL iff N == 0)
 *  row_of_slot  int32 [T*K]   in     row_map  int32 [N] in (nullable)
 *  expert_ids   int32 [T*K]   in     probs    fp32 [T*K] in (any sign, any sum)
 *  active_mask  uint8 [T] or [T*K] in (nullable), mask_per_slot as for
 *               moe_permute: a slot outside the mask adds no term (the shared
 *               row is still added)
 *  special      nullable: no special experts. Its ori_x is bf16 [T,H]
 *               (required if num_copy + num_const > 0); alpha1 / alpha2 are
 *               fp32 with element (t, c, h) at t*alpha_stride_t +
 *               c*alpha_stride_c + h*alpha_stride_h (per-token scalars:
 *               strides (1,0,0); the page's (const_num, H) layout: (0,H,1));
 *               const_v bf16 [num_const, H]. alpha*, const_v required if
 *               num_const > 0.
 *  shared_x     bf16 [T, H]   in (nullable)
 *  out          bf16 [T, H]   out
 * Errors: INVALID_ARG for T < 0, K outside [1,16], H <= 0, E < 1, N < 0,
 * negative special counts, E+Z+C+Nc >= 2^31-1 ([CV2] 约束说明), T*K >
 * INT32_MAX, N > INT32_MAX, missing ori_x / alpha / const_v ([CV2] 参数说明),
 * mask_per_slot not 0 or 1, NULL / misaligned pointers; UNSUPPORTED for
 * H % 8 != 0.
 * ------------------------------------------------------------------------ */
typedef struct moe_special_experts {
    int32_t num_zero;
    int32_t num_copy;
    int32_t num_const;
    const void* ori_x;
    const float* alpha1;
    const float* alpha2;
    int64_t alpha_stride_t;
    int64_t alpha_stride_c;
    int64_t alpha_stride_h;
    const void* const_v;
} moe_special_experts_t;

moe_status_t moe_unpermute_combine(const void* expert_out, int64_t N, const int32_t* row_of_slot,
                                   const int32_t* row_map, const int32_t* expert_ids,
                                   const float* probs, const uint8_t* active_mask,
                                   int32_t mask_per_slot, int64_t T, int32_t K, int32_t H,
                                   int32_t num_experts, const moe_special_experts_t* special,
                                   const void* shared_x, void* out, hipStream_t stream);

/* ------------------------------------------------------------------------
 * moe_unpermute_combine_grad -- backward of moe_unpermute_combine, special
 * and shared experts included.
 *
 * [CV2] 计算公式: the combine is out[t] = sum_k p[t,k] v_k(t) + shared[t]
 * with v_k an expert row, 0 (zero expert), ori_x[t] (copy expert) or
 * a1*ori_x[t] + a2*const_v[c] (const expert c, a* = alpha*(t, c, h)). Given
 * g = grad_out, this call returns the gradient of every input of that sum:
 *     d_expert_out[row] = bf16( p g[t] )       routed slot (row via row_map)
 *     d_probs[t,k]      = sum_h g[t,h] v_k(t,h)     (0 for zero / dropped slots)
 *     d_ori_x[t]        = bf16( sum_copy p g[t] + sum_const p a1 g[t] )
 *     d_alpha1(t,c,h)  += p g ori_x[t,h]     d_alpha2(t,c,h) += p g const_v[c,h]
 *     d_const_v[c]      = bf16( sum over tokens and slots of p a2 g[t] )
 * all accumulated in fp32. The shared term is added once with no weight
 * ([CV2] 参数说明), so its gradient is grad_out itself: there is no output
 * for it. Rows of d_expert_out that no slot references are not written.
 *
 * d_alpha1 / d_alpha2 have alpha's layout (the same strides); every element
 * alpha reads is written (0 where no slot uses it). Supported layouts for
 * them: each token owns its span (stride_h = 0, stride_t > 0,
 * (num_const-1)*stride_c < stride_t: per-token [T] or [T, num_const]), or
 * all tokens share it (stride_t = 0 with stride_h = 1 and stride_c >= H: the
 * page's [num_const, H]; or stride_h = 0: [num_const] or one scalar).
 * Sums over tokens (d_const_v, shared alpha layouts) go through fp32
 * per-segment partials in the workspace, added in a fixed order: the result
 * is deterministic.
 *
 *  grad_out      bf16 [T, H]   in          (the other inputs, active_mask
 *                                          included, as for the combine; slots
 *                                          outside the mask get d_probs = 0)
 *  d_expert_out  bf16 [N, H]   out (nullable: not computed)
 *  d_probs       fp32 [T*K]    out
 *  d_ori_x       bf16 [T, H]   out (nullable); zero rows for tokens without
 *                                  copy / const slots
 *  d_alpha1, d_alpha2  fp32, alpha's layout   out (nullable)
 *  d_const_v     bf16 [num_const, H]  out (nullable)
 *  workspace     moe_unpermute_combine_grad_workspace_size(T, H, num_const)
 *                bytes, 16-byte aligned; needed only when num_const > 0 and
 *                d_const_v or a shared-layout d_alpha is requested
 * Errors: as moe_unpermute_combine, plus NULL grad_out / d_probs and
 * misaligned outputs (INVALID_ARG); UNSUPPORTED for a d_alpha request with
 * any other alpha layout; WORKSPACE if the workspace is missing or small.
 * ------------------------------------------------------------------------ */
moe_status_t moe_unpermute_combine_grad_workspace_size(int64_t T, int32_t H, int32_t num_const,
                                                      size_t* bytes);
moe_status_t moe_unpermute_combine_grad(
    const void* grad_out, const void* expert_out, int64_t N, const int32_t* row_of_slot,
    const int32_t* row_map, const int32_t* expert_ids, const float* probs,
    const uint8_t* active_mask, int32_t mask_per_slot, int64_t T, int32_t K, int32_t H,
    int32_t num_experts, const moe_special_experts_t* special, void* d_expert_out,
    float* d_probs, void* d_ori_x, float* d_alpha1, float* d_alpha2, void* d_const_v,
    void* workspace, size_t workspace_bytes, hipStream_t stream);

/* ------------------------------------------------------------------------
 * moe_unpermute_grad -- backward of the routed part of the combine.
 *
 * [UNP] 主要改动: npu_moe_token_unpermute_grad_v2 returns the gradient of
 * permuted_tokens (hidden-dim sharded: elementwise in h) and of probs
 * (Partial(): a sum over h). For slot s = t*K + k with row = row_of_slot[s]
 * in [0, N):
 *     d_permuted[row] = bf16( p[s] * grad_out[t] )   correctly rounded product
 *     d_probs[s]      = sum_h grad_out[t,h] * permuted[row,h]   (fp32 accumulate)
 * Slots with row outside [0, N) get d_probs = 0 and write no row. Rows of
 * d_permuted that no slot references are not written.
 *
 *  grad_out    bf16 [T, H]   in      permuted  bf16 [N, H]  in
 *  row_of_slot int32 [T*K]   in      probs     fp32 [T*K]   in
 *  d_permuted  bf16 [N, H]   out     d_probs   fp32 [T*K]   out
 * Errors: INVALID_ARG for T < 0, K outside [1,16], H <= 0, N < 0, T*K or N >
 * INT32_MAX, NULL / misaligned pointers; UNSUPPORTED for H % 8 != 0.
 * ------------------------------------------------------------------------ */
moe_status_t moe_unpermute_grad(const void* grad_out, const void* permuted, int64_t N,
                                const int32_t* row_of_slot, const float* probs, int64_t T,
                                int32_t K, int32_t H, void* d_permuted, float* d_probs,
                                hipStream_t stream);

/* ------------------------------------------------------------------------
 * moe_permute_grad -- backward of moe_permute's row copy.
 *
 * [GMM] (fix 2 of the PR description): the permute is the advanced-index
 * gather x[idx], whose backward index_put accumulates the gradients of
 * repeated indices. Row row_of_slot[t*K + k] holds a copy of x[t], so
 *     d_x[t] = bf16( sum_k d_permuted[row_of_slot[t*K + k]] )   (fp32 accumulate, k order)
 * over the slots whose row is in [0, N); a token without such a slot gets 0.
 * (The combine with every weight 1 and no special or shared term.)
 *
 *  d_permuted  bf16 [N, H]   in (may be NULL iff N == 0)
 *  row_of_slot int32 [T*K]   in      d_x  bf16 [T, H]  out
 * Errors: INVALID_ARG for T < 0, K outside [1,16], H <= 0, N < 0, T*K or N >
 * INT32_MAX, NULL / misaligned pointers; UNSUPPORTED for H % 8 != 0.
 * ------------------------------------------------------------------------ */
moe_status_t moe_permute_grad(const void* d_permuted, int64_t N, const int32_t* row_of_slot,
                              int64_t T, int32_t K, int32_t H, void* d_x, hipStream_t stream);

/* ------------------------------------------------------------------------
 * moe_deredundency_dispatch_indices -- gather-view indices of one outer
 * expert range, ordered [iep_dst, local_expert, oep_source].
 *
 * [EP] _generate_deredundency_dispatch_indices. tokens_per_expert_by_source
 * [oep_size, num_experts] (device) describes each source rank's expert-major
 * routed buffer; the buffers are concatenated in source order (the gathered
 * buffer, G = sum of all counts rows). The selected experts are
 * e = expert_start + d*num_local_experts + l for d < iep_size,
 * l < num_local_experts; block (d, l, s) holds source s's rows of expert e, in
 * their order, and blocks follow in (d, l, s) order. indices[i] is the
 * gathered row of selected row i (int32 here: the page returns int64);
 * positions past the total get -1. counts_by_dest[d*num_local_experts + l]
 * sums expert e over the sources. Negative counts read as 0; the sum of all
 * counts must stay below 2^31.
 *
 *  tokens_per_expert_by_source int32 [oep_size * num_experts] in   device
 *  indices        int32 [capacity]                 out  -1 past the total
 *  counts_by_dest int32 [iep_size * num_local_experts] out
 *  total          int32 [1]                        out  (nullable) the number of selected rows
 * Errors: INVALID_ARG for oep_size, num_experts, iep_size or num_local_experts
 * < 1, expert_start < 0, expert_start + iep_size*num_local_experts >
 * num_experts, oep_size*num_experts > MOE_MAX_DERED_CELLS, capacity outside
 * [0, INT32_MAX], NULL / misaligned pointers; WORKSPACE if too small.
 * ------------------------------------------------------------------------ */
moe_status_t moe_deredundency_dispatch_indices_workspace_size(int32_t oep_size,
                                                             int32_t num_experts,
                                                             int32_t iep_size,
                                                             int32_t num_local_experts,
                                                             size_t* bytes);
moe_status_t moe_deredundency_dispatch_indices(
    const int32_t* tokens_per_expert_by_source, int32_t oep_size, int32_t num_experts,
    int32_t expert_start, int32_t iep_size, int32_t num_local_experts, int64_t capacity,
    int32_t* indices, int32_t* counts_by_dest, int32_t* total, void* workspace,
    size_t workspace_bytes, hipStream_t stream);

/* ------------------------------------------------------------------------
 * moe_deredundency_combine -- the whiteboard of the deredundency combine.
 *
 * [EP] _scale_by_router_coeff then _scatter_add_first_dim: outer_output row j
 * is scaled by router_coeff[j] and added into a zero [G, H] buffer at row
 * dispatch_indices[j]:
 *     whiteboard[r] = bf16( sum over j with dispatch_indices[j] == r of
 *                           router_coeff[j] * outer_output[j] ),  0 if no j names r
 * (router_coeff NULL: coefficient 1). A row named once holds the correctly
 * rounded product; a row named by several j holds their sum accumulated in
 * fp32 in ascending j, rounded once; either way the result does not depend on
 * scheduling. As in a zero buffer plus the rows, an exactly zero result is +0.
 * The indices of moe_deredundency_dispatch_indices name every row at most
 * once. Indices outside [0, G) are skipped. Every row of the whiteboard is
 * written once (no separate zero fill).
 *
 *  outer_output     bf16 [n, H]  in
 *  router_coeff     fp32 [n]     in  (nullable)
 *  dispatch_indices int32 [n]    in
 *  whiteboard       bf16 [G, H]  out
 *  workspace        moe_deredundency_combine_workspace_size(n, G) bytes
 * Errors: INVALID_ARG for n or G outside [0, INT32_MAX], H <= 0, NULL /
 * misaligned pointers; UNSUPPORTED for H % 8 != 0; WORKSPACE if too small.
 * ------------------------------------------------------------------------ */
moe_status_t moe_deredundency_combine_workspace_size(int64_t n, int64_t G, size_t* bytes);
moe_status_t moe_deredundency_combine(const void* outer_output, const float* router_coeff,
                                      const int32_t* dispatch_indices, int64_t n, int32_t H,
                                      int64_t G, void* whiteboard, void* workspace,
                                      size_t workspace_bytes, hipStream_t stream);

#ifdef __cplusplus
}
#endif
#endif /* LIBMOEPERM_H */
